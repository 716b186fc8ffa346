"""Python binding of libconvrot (the C ABI in include/convrot.h).

Argument marshalling only: PyTorch provides device memory and the current HIP
stream; every step of the forward path runs in the library's HIP kernels.
The functions carry the C names.  If the library has not been built the first
call raises -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libconvrot.so")

OK, EINVAL, EALIGN, EWORKSPACE, ELAYOUT, EUNSUPPORTED, EHIP = 0, -1, -2, -3, -4, -5, -6
F32, BF16, I8, I32 = 0, 1, 2, 3
OUT_MAJOR, IN_MAJOR = 0, 1
WEIGHTS_MAGIC = 0x38545243
WEIGHTS_VERSION = 2
ROT_REGULAR = 0x100          # rotation kind: regular H_4 Kronecker blocks
ROTATIONS = {"sylvester": 0, "regular": ROT_REGULAR}
FLAG_GELU = 1
FLAG_SWIGLU = 2
SWIGLU_PAIRS = 0x200         # weight flag: interleaved SwiGLU gate/up rows

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_p = ctypes.c_void_p
_c_sz = ctypes.c_size_t


class convrot_weights(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32),
        ("version", ctypes.c_uint32),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
        ("block", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("codes", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
    ]


_W = ctypes.POINTER(convrot_weights)

_SIGNATURES = {
    "convrot_status_string": (ctypes.c_char_p, [_c_int]),
    "convrot_last_hip_error": (_c_int, []),
    "convrot_version": (_c_int, []),
    "convrot_weights_packed_bytes": (_c_sz, [_c_i64, _c_i64, _c_int]),
    "convrot_prepare_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_int, _c_int, _c_int]),
    "convrot_linear_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_int]),
    "lowrank_convrot_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i64, _c_int]),
    "convrot_mlp_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i64, _c_int]),
    "lowrank_convrot_padded_rank": (_c_i64, [_c_i64, _c_int]),
    "lowrank_convrot_prepare_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_int, _c_int]),
    "lowrank_convrot_prepare_weights": (
        _c_int, [_c_p, _c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _W, _W, _c_p, _c_sz, _c_p]),
    "convrot_linear_prepare_weights": (
        _c_int, [_c_p, _c_int, _c_int, _c_p, _c_i64, _c_i64, _c_int, _W, _c_p, _c_sz, _c_p]),
    "convrot_linear_forward": (
        _c_int, [_c_p, _c_i64, _W, _c_p, _c_p, _c_int, _c_p, _c_sz, _c_p]),
    "convrot_linear_forward_noalloc": (
        _c_int, [_c_p, _c_i64, _W, _c_p, _c_p, _c_int, _c_p]),
    "lowrank_convrot_forward": (
        _c_int, [_c_p, _c_i64, _W, _W, _c_p, _c_p, _c_int, _c_p, _c_sz, _c_p]),
    "convrot_mlp_forward": (
        _c_int, [_c_p, _c_i64, _W, _c_p, _W, _c_p, _c_p, _c_int, _c_p, _c_sz, _c_p]),
    "convrot_rotate_quantize": (
        _c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_int, ctypes.c_uint32, _c_p, _c_p, _c_p]),
    "convrot_gemm_i32": (_c_int, [_c_p, _c_i64, _W, _c_p, _c_p]),
    "convrot_gemm_dequant": (
        _c_int, [_c_p, _c_p, _c_i64, _W, _c_p, _c_p, _c_int, ctypes.c_uint32, _c_p]),
    "convrot_lowrank_factor1": (_c_int, [_c_p, _c_p, _c_i64, _W, _c_p, _c_p, _c_p]),
    "convrot_swiglu_prepare_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_int, _c_int]),
    "convrot_swiglu_prepare_weights": (
        _c_int, [_c_p, _c_int, _c_p, _c_i64, _c_i64, _c_int, _W, _c_p, _c_sz, _c_p]),
    "convrot_swiglu_mlp_workspace_bytes": (
        _c_sz, [_c_i64, _c_i64, _c_i64, _c_i64, _c_int, _c_int]),
    "convrot_swiglu_mlp_forward": (
        _c_int, [_c_p, _c_i64, _W, _c_p, _W, _c_p, _c_p, _c_int, _c_p, _c_sz, _c_p]),
    "convrot_swiglu_bf16": (_c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p]),
    "convrot_silu_f32": (_c_int, [_c_p, _c_i64, _c_p, _c_p]),
    "lowrank_bf16_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64]),
    "lowrank_bf16_forward": (
        _c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_i64, _c_p, _c_p, _c_p,
                 ctypes.c_size_t, _c_p]),
    "convrot_gelu_bf16": (_c_int, [_c_p, _c_i64, _c_p, _c_p]),
    "convrot_probe_mfma_i8": (_c_int, [_c_i64, _c_p, _c_p, ctypes.POINTER(ctypes.c_int64),
                                       _c_p]),
    "convrot_probe_stream": (_c_int, [_c_p, _c_p, _c_i64, _c_int, _c_p]),
}

EXPORTED = tuple(_SIGNATURES)

_lib = None


class ConvRotError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = library()
        msg = lib.convrot_status_string(status).decode()
        extra = ""
        if status == EHIP:
            extra = f" (hipError {lib.convrot_last_hip_error()})"
        super().__init__(f"{fn} failed: {msg} [{status}]{extra}")
        self.status = status


def library():
    """Load libconvrot.so (built in-tree by ``w8a8_int8_rotated_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m w8a8_int8_rotated_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, rc: int):
    if rc != OK:
        raise ConvRotError(fn, rc)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_tag(dt: torch.dtype) -> int:
    return {torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8, torch.int32: I32}[dt]


def _torch_dtype(tag: int) -> torch.dtype:
    return {F32: torch.float32, BF16: torch.bfloat16}[tag]


def _on_device(device, **tensors):
    """Every tensor the library will dereference is a GPU tensor on `device`
    (any GPU when None).  Called after the shape and dtype checks, so a
    host-side caller sees those errors first."""
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda" or (device is not None and t.device != device):
            raise ValueError(f"{name} must be a GPU tensor on {device or 'the GPU'}, "
                             f"got {t.device}")


def _need(t, name: str, dtypes, shape):
    """Check a tensor argument before its pointer reaches the library: its
    dtype, exact shape and contiguity (the device is checked by _on_device)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(map(str, dtypes))}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _opt(t, name: str, dtypes, shape):
    return None if t is None else _need(t, name, dtypes, shape)


def _weights(W, name: str):
    if not isinstance(W, PreparedWeights):
        raise ValueError(f"{name} must be PreparedWeights from convrot_linear_prepare_weights")
    return W.codes.device


def _rows(X, name: str, K: int):
    """bf16 activations [M, K]; returns M."""
    if not isinstance(X, torch.Tensor) or X.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor [M, {K}]")
    _need(X, name, torch.bfloat16, (X.shape[0], K))
    return X.shape[0]


def _output(out, M: int, N: int, dtypes):
    return None if out is None else _need(out, "out", dtypes, (M, N))


def _check_workspace(nbytes: int, workspace):
    if workspace is None or nbytes == 0:
        return
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 \
            or workspace.dim() != 1 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    if workspace.numel() < nbytes:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {nbytes} needed")


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return None
    if workspace is not None:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ------------------------------------------------------------- sizing ----

def convrot_weights_packed_bytes(N: int, K: int, block: int) -> int:
    return library().convrot_weights_packed_bytes(N, K, block)


def convrot_prepare_workspace_bytes(N, K, block, w_dtype, layout) -> int:
    return library().convrot_prepare_workspace_bytes(N, K, block, w_dtype, layout)


def convrot_linear_workspace_bytes(M, K, N, block) -> int:
    return library().convrot_linear_workspace_bytes(M, K, N, block)


def lowrank_convrot_workspace_bytes(M, K, r, N, block) -> int:
    return library().lowrank_convrot_workspace_bytes(M, K, r, N, block)


def convrot_mlp_workspace_bytes(M, K, F, N, block) -> int:
    return library().convrot_mlp_workspace_bytes(M, K, F, N, block)


def lowrank_bf16_workspace_bytes(M, r) -> int:
    return library().lowrank_bf16_workspace_bytes(M, r)


# ----------------------------------------------------------- weights ----

class PreparedWeights:
    """A prepared weight: the C descriptor plus the tensors it points into."""

    def __init__(self, desc: convrot_weights, codes: torch.Tensor, scale: torch.Tensor):
        self.desc = desc
        self.codes = codes
        self.scale = scale

    @property
    def N(self):
        return self.desc.N

    @property
    def K(self):
        return self.desc.K

    @property
    def block(self):
        return self.desc.block

    def ref(self):
        return ctypes.byref(self.desc)


def convrot_linear_prepare_weights(W: torch.Tensor, block: int, layout: int = OUT_MAJOR,
                                   src_scale: torch.Tensor | None = None,
                                   stream=None, rotation: str = "sylvester") -> PreparedWeights:
    """Rotate + quantise + pack a weight (``[N, K]`` or ``[K, N]`` per layout)
    with the rotation kind ``'sylvester'`` or ``'regular'``."""
    lib = library()
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError("W must be a 2-D tensor")
    if layout not in (OUT_MAJOR, IN_MAJOR):
        raise ValueError("layout must be OUT_MAJOR or IN_MAJOR")
    if layout == OUT_MAJOR:
        N, K = W.shape
    else:
        K, N = W.shape
    if W.dtype not in (torch.float32, torch.bfloat16, torch.int8):
        raise ValueError(f"W must be float32, bfloat16 or int8 codes, got {W.dtype}")
    if (W.dtype == torch.int8) != (src_scale is not None):
        raise ValueError("src_scale is required for int8 codes and only for them")
    _opt(src_scale, "src_scale", torch.float32, (N,))
    if rotation not in ROTATIONS:
        raise ValueError(f"rotation must be one of {sorted(ROTATIONS)}")
    W = W.contiguous()
    _on_device(W.device, W=W, src_scale=src_scale)
    tag = _dtype_tag(W.dtype)
    nbytes = lib.convrot_weights_packed_bytes(N, K, block)
    if nbytes == 0:
        raise ConvRotError("convrot_linear_prepare_weights", EUNSUPPORTED)
    codes = torch.empty(nbytes, dtype=torch.int8, device=W.device)
    scale = torch.empty(N, dtype=torch.float32, device=W.device)
    desc = convrot_weights()
    desc.codes = codes.data_ptr()
    desc.scale = scale.data_ptr()
    desc.flags = ROTATIONS[rotation]
    wsb = lib.convrot_prepare_workspace_bytes(N, K, block, tag, layout)
    ws = _workspace(wsb, W.device, None)
    rc = lib.convrot_linear_prepare_weights(
        _ptr(W), tag, layout, _ptr(src_scale), N, K, block, ctypes.byref(desc), _ptr(ws),
        wsb, _stream(stream))
    _check("convrot_linear_prepare_weights", rc)
    pw = PreparedWeights(desc, codes, scale)
    pw._ws = ws  # keep alive until the stream has consumed it
    return pw


def lowrank_padded_rank(r: int, block: int) -> int:
    """The rank a low-rank pair is stored with (lowrank_convrot_padded_rank)."""
    return library().lowrank_convrot_padded_rank(r, block)


def convrot_lowrank_prepare(A: torch.Tensor, B: torch.Tensor, block: int, stream=None,
                            rotation: str = "sylvester"):
    """Prepare a low-rank pair W ~ B . A, A [r, K] and B [N, r] (output-major,
    float32 or bfloat16) with lowrank_convrot_prepare_weights, which pads the
    rank with zero rows of A and zero columns of B to
    lowrank_padded_rank(r, block).  Returns two PreparedWeights."""
    lib = library()
    for t, name in ((A, "A"), (B, "B")):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError(f"{name} must be a 2-D tensor")
    r, K = A.shape
    N = B.shape[0]
    if A.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"A must be float32 or bfloat16, got {A.dtype}")
    B = B.contiguous()
    _need(B, "B", A.dtype, (N, r))
    if rotation not in ROTATIONS:
        raise ValueError(f"rotation must be one of {sorted(ROTATIONS)}")
    A = A.contiguous()
    _on_device(A.device, A=A, B=B)
    tag = _dtype_tag(A.dtype)
    rp = lib.lowrank_convrot_padded_rank(r, block)
    na, nb = lib.convrot_weights_packed_bytes(rp, K, block), lib.convrot_weights_packed_bytes(N, rp, block)
    if rp == 0 or na == 0 or nb == 0:
        raise ConvRotError("lowrank_convrot_prepare_weights", EUNSUPPORTED)
    dev = A.device
    pws = []
    descs = []
    for n, nbytes in ((rp, na), (N, nb)):
        d = convrot_weights()
        codes = torch.empty(nbytes, dtype=torch.int8, device=dev)
        scale = torch.empty(n, dtype=torch.float32, device=dev)
        d.codes, d.scale, d.flags = codes.data_ptr(), scale.data_ptr(), ROTATIONS[rotation]
        descs.append(d)
        pws.append((codes, scale))
    wsb = lib.lowrank_convrot_prepare_workspace_bytes(r, K, N, block, tag)
    ws = _workspace(wsb, dev, None)
    rc = lib.lowrank_convrot_prepare_weights(
        _ptr(A), _ptr(B), tag, r, K, N, block, ctypes.byref(descs[0]), ctypes.byref(descs[1]),
        _ptr(ws), wsb, _stream(stream))
    _check("lowrank_convrot_prepare_weights", rc)
    pa = PreparedWeights(descs[0], *pws[0])
    pb = PreparedWeights(descs[1], *pws[1])
    pa._ws = pb._ws = ws    # keep alive until the stream has consumed it
    return pa, pb


# ----------------------------------------------------------- forward ----

def convrot_linear_forward(X: torch.Tensor, W: PreparedWeights, bias=None,
                           out_dtype: torch.dtype = torch.bfloat16, out=None,
                           workspace=None, stream=None) -> torch.Tensor:
    lib = library()
    dev = _weights(W, "W")
    M = _rows(X, "X", W.K)
    _opt(bias, "bias", torch.float32, (W.N,))
    _output(out, M, W.N, (torch.bfloat16, torch.float32))
    wsb = lib.convrot_linear_workspace_bytes(M, W.K, W.N, W.block)
    _check_workspace(wsb, workspace)
    _on_device(dev, X=X, bias=bias, out=out, workspace=workspace)
    if out is None:
        out = torch.empty((M, W.N), dtype=out_dtype, device=dev)
    ws = _workspace(wsb, dev, workspace)
    rc = lib.convrot_linear_forward(_ptr(X), M, W.ref(), _ptr(bias), _ptr(out),
                                    _dtype_tag(out.dtype), _ptr(ws),
                                    ws.numel() if ws is not None else 0, _stream(stream))
    _check("convrot_linear_forward", rc)
    return out


def convrot_linear_forward_noalloc(X: torch.Tensor, W: PreparedWeights, bias=None,
                                   out_dtype: torch.dtype = torch.bfloat16, out=None,
                                   stream=None) -> torch.Tensor:
    """convrot_linear_forward with the library's static device scratch as its
    workspace (the C call allocates nothing; pass `out` to allocate nothing
    here either).  Calls on one device must not overlap in time."""
    lib = library()
    dev = _weights(W, "W")
    M = _rows(X, "X", W.K)
    _opt(bias, "bias", torch.float32, (W.N,))
    _output(out, M, W.N, (torch.bfloat16, torch.float32))
    _on_device(dev, X=X, bias=bias, out=out)
    if out is None:
        out = torch.empty((M, W.N), dtype=out_dtype, device=dev)
    rc = lib.convrot_linear_forward_noalloc(_ptr(X), M, W.ref(), _ptr(bias), _ptr(out),
                                            _dtype_tag(out.dtype), _stream(stream))
    _check("convrot_linear_forward_noalloc", rc)
    return out


def lowrank_convrot_forward(X: torch.Tensor, A: PreparedWeights, B: PreparedWeights,
                            bias=None, out_dtype: torch.dtype = torch.bfloat16, out=None,
                            workspace=None, stream=None) -> torch.Tensor:
    lib = library()
    dev = _weights(A, "A")
    if _weights(B, "B") != dev:
        raise ValueError("A and B must be on the same device")
    M = _rows(X, "X", A.K)
    _opt(bias, "bias", torch.float32, (B.N,))
    _output(out, M, B.N, (torch.bfloat16, torch.float32))
    wsb = lib.lowrank_convrot_workspace_bytes(M, A.K, A.N, B.N, A.block)
    _check_workspace(wsb, workspace)
    _on_device(dev, X=X, bias=bias, out=out, workspace=workspace)
    if out is None:
        out = torch.empty((M, B.N), dtype=out_dtype, device=dev)
    ws = _workspace(wsb, dev, workspace)
    rc = lib.lowrank_convrot_forward(_ptr(X), M, A.ref(), B.ref(), _ptr(bias), _ptr(out),
                                     _dtype_tag(out.dtype), _ptr(ws),
                                     ws.numel() if ws is not None else 0, _stream(stream))
    _check("lowrank_convrot_forward", rc)
    return out


def convrot_mlp_forward(X: torch.Tensor, W_up: PreparedWeights, W_down: PreparedWeights,
                        bias_up=None, bias_down=None, out_dtype: torch.dtype = torch.bfloat16,
                        out=None, workspace=None, stream=None) -> torch.Tensor:
    lib = library()
    dev = _weights(W_up, "W_up")
    if _weights(W_down, "W_down") != dev:
        raise ValueError("W_up and W_down must be on the same device")
    M = _rows(X, "X", W_up.K)
    _opt(bias_up, "bias_up", torch.float32, (W_up.N,))
    _opt(bias_down, "bias_down", torch.float32, (W_down.N,))
    _output(out, M, W_down.N, (torch.bfloat16, torch.float32))
    wsb = lib.convrot_mlp_workspace_bytes(M, W_up.K, W_up.N, W_down.N, W_up.block)
    _check_workspace(wsb, workspace)
    _on_device(dev, X=X, bias_up=bias_up, bias_down=bias_down, out=out, workspace=workspace)
    if out is None:
        out = torch.empty((M, W_down.N), dtype=out_dtype, device=dev)
    ws = _workspace(wsb, dev, workspace)
    rc = lib.convrot_mlp_forward(_ptr(X), M, W_up.ref(), _ptr(bias_up), W_down.ref(),
                                 _ptr(bias_down), _ptr(out), _dtype_tag(out.dtype), _ptr(ws),
                                 ws.numel() if ws is not None else 0, _stream(stream))
    _check("convrot_mlp_forward", rc)
    return out


# ------------------------------------------------------------ SwiGLU ----

def convrot_swiglu_mlp_workspace_bytes(M, K, F, N, block_up, block_down) -> int:
    return library().convrot_swiglu_mlp_workspace_bytes(M, K, F, N, block_up, block_down)


def convrot_swiglu_prepare(W: torch.Tensor, block: int, src_scale: torch.Tensor | None = None,
                           stream=None, rotation: str = "sylvester") -> PreparedWeights:
    """Prepare a SwiGLU fc1 weight [2F, K] (gate rows, then up rows): float32 or
    bfloat16 weights, or int8 codes with src_scale [2F]; stored interleaved
    (SWIGLU_PAIRS) for the fused SwiGLU epilogue."""
    lib = library()
    if not isinstance(W, torch.Tensor) or W.dim() != 2 or W.shape[0] % 2:
        raise ValueError("W must be a 2-D tensor [2F, K]")
    N2, K = W.shape
    if W.dtype not in (torch.float32, torch.bfloat16, torch.int8):
        raise ValueError(f"W must be float32, bfloat16 or int8 codes, got {W.dtype}")
    if (W.dtype == torch.int8) != (src_scale is not None):
        raise ValueError("src_scale is required for int8 codes and only for them")
    _opt(src_scale, "src_scale", torch.float32, (N2,))
    if rotation not in ROTATIONS:
        raise ValueError(f"rotation must be one of {sorted(ROTATIONS)}")
    W = W.contiguous()
    _on_device(W.device, W=W, src_scale=src_scale)
    tag = _dtype_tag(W.dtype)
    nbytes = lib.convrot_weights_packed_bytes(N2, K, block)
    wsb = lib.convrot_swiglu_prepare_workspace_bytes(N2 // 2, K, block, tag)
    if nbytes == 0 or wsb == 0:
        raise ConvRotError("convrot_swiglu_prepare_weights", EUNSUPPORTED)
    codes = torch.empty(nbytes, dtype=torch.int8, device=W.device)
    scale = torch.empty(N2, dtype=torch.float32, device=W.device)
    desc = convrot_weights()
    desc.codes, desc.scale, desc.flags = codes.data_ptr(), scale.data_ptr(), ROTATIONS[rotation]
    ws = _workspace(wsb, W.device, None)
    rc = lib.convrot_swiglu_prepare_weights(_ptr(W), tag, _ptr(src_scale), N2 // 2, K, block,
                                            ctypes.byref(desc), _ptr(ws), wsb, _stream(stream))
    _check("convrot_swiglu_prepare_weights", rc)
    pw = PreparedWeights(desc, codes, scale)
    pw._ws = ws
    return pw


def convrot_swiglu_mlp_forward(X: torch.Tensor, W_gu: PreparedWeights, W_down: PreparedWeights,
                               bias_gu=None, bias_down=None,
                               out_dtype: torch.dtype = torch.bfloat16, out=None,
                               workspace=None, stream=None) -> torch.Tensor:
    """Y = linear(swiglu(linear(X; W_gu) + bias_gu); W_down) + bias_down."""
    lib = library()
    dev = _weights(W_gu, "W_gu")
    if _weights(W_down, "W_down") != dev:
        raise ValueError("W_gu and W_down must be on the same device")
    M = _rows(X, "X", W_gu.K)
    F = W_down.K
    _opt(bias_gu, "bias_gu", torch.float32, (W_gu.N,))
    _opt(bias_down, "bias_down", torch.float32, (W_down.N,))
    _output(out, M, W_down.N, (torch.bfloat16, torch.float32))
    wsb = lib.convrot_swiglu_mlp_workspace_bytes(M, W_gu.K, F, W_down.N, W_gu.block,
                                                 W_down.block)
    _check_workspace(wsb, workspace)
    _on_device(dev, X=X, bias_gu=bias_gu, bias_down=bias_down, out=out, workspace=workspace)
    if out is None:
        out = torch.empty((M, W_down.N), dtype=out_dtype, device=dev)
    ws = _workspace(wsb, dev, workspace)
    rc = lib.convrot_swiglu_mlp_forward(_ptr(X), M, W_gu.ref(), _ptr(bias_gu), W_down.ref(),
                                        _ptr(bias_down), _ptr(out), _dtype_tag(out.dtype),
                                        _ptr(ws), ws.numel() if ws is not None else 0,
                                        _stream(stream))
    _check("convrot_swiglu_mlp_forward", rc)
    return out


def convrot_swiglu_bf16(gu: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """g [M, F] = bf16(fp32(silu(gate)) * up) for gu [M, 2F] = gate | up."""
    lib = library()
    if not isinstance(gu, torch.Tensor) or gu.dim() != 2 or gu.shape[1] % 2:
        raise ValueError("gu must be a 2-D tensor [M, 2F]")
    M, F = gu.shape[0], gu.shape[1] // 2
    _need(gu, "gu", torch.bfloat16, (M, 2 * F))
    _opt(out, "out", torch.bfloat16, (M, F))
    _on_device(gu.device, gu=gu, out=out)
    if out is None:
        out = torch.empty((M, F), dtype=torch.bfloat16, device=gu.device)
    _check("convrot_swiglu_bf16", lib.convrot_swiglu_bf16(_ptr(gu), M, F, _ptr(out),
                                                          _stream(stream)))
    return out


def convrot_silu_f32(a: torch.Tensor, stream=None) -> torch.Tensor:
    """fp32(silu(a)) of bf16 values, as every SwiGLU path computes it."""
    lib = library()
    if not isinstance(a, torch.Tensor) or a.dtype != torch.bfloat16:
        raise ValueError("a must be a bf16 tensor")
    a = a.contiguous()
    _on_device(a.device, a=a)
    out = torch.empty(a.shape, dtype=torch.float32, device=a.device)
    _check("convrot_silu_f32", lib.convrot_silu_f32(_ptr(a), a.numel(), _ptr(out),
                                                    _stream(stream)))
    return out


def lowrank_bf16_forward(X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, bias=None,
                         out=None, workspace=None, stream=None) -> torch.Tensor:
    """Comparison variant: bf16(bf16(X . A^T) . B^T + bias), bf16 factors
    A [r, K] and B [N, r], no rotation or quantisation."""
    lib = library()
    for t, name in ((X, "X"), (A, "A"), (B, "B")):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError(f"{name} must be a 2-D tensor")
    M, K = X.shape
    r, N = A.shape[0], B.shape[0]
    dev = A.device
    _need(X, "X", torch.bfloat16, (M, K))
    _need(A, "A", torch.bfloat16, (r, K))
    _need(B, "B", torch.bfloat16, (N, r))
    _opt(bias, "bias", torch.float32, (N,))
    _output(out, M, N, torch.bfloat16)
    wsb = lib.lowrank_bf16_workspace_bytes(M, r)
    _check_workspace(wsb, workspace)
    _on_device(dev, X=X, A=A, B=B, bias=bias, out=out, workspace=workspace)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = _workspace(wsb, dev, workspace)
    rc = lib.lowrank_bf16_forward(_ptr(X), M, K, _ptr(A), r, _ptr(B), N, _ptr(bias), _ptr(out),
                                  _ptr(ws), ws.numel() if ws is not None else 0,
                                  _stream(stream))
    _check("lowrank_bf16_forward", rc)
    return out


# ------------------------------------------------------------- hooks ----

def padded_rows(M: int) -> int:
    """Rows of a K-tiled INT8 code buffer holding M rows (a multiple of 16)."""
    return (M + 15) // 16 * 16


def _codes(q, M: int, K: int, device):
    """A K-tiled code buffer for M rows of K codes: allocated as (Mp, K) int8
    on `device` when q is None, or a caller tensor checked to hold Mp * K
    bytes (its device is checked by the caller)."""
    Mp = padded_rows(M)
    if q is None:
        return torch.empty((Mp, K), dtype=torch.int8, device=device)
    if not isinstance(q, torch.Tensor) or q.dtype != torch.int8 or not q.is_contiguous() \
            or q.numel() < Mp * K:
        raise ValueError(f"K-tiled codes need a contiguous int8 tensor of {Mp * K} elements")
    return q


def convrot_rotate_quantize(X: torch.Tensor, block: int, q=None, s=None, stream=None,
                            rotation: str = "sylvester", gelu: bool = False):
    """Rotate + quantise the rows of X: (q, s), q the K-tiled codes (Mp, K).
    gelu: quantise bf16(GELU(X)) instead (bf16 X, 6144 < K <= 24576), as the
    MLP path does with its intermediate."""
    lib = library()
    if not isinstance(X, torch.Tensor) or X.dim() != 2:
        raise ValueError("X must be a 2-D tensor [M, K]")
    M, K = X.shape
    _need(X, "X", (torch.bfloat16, torch.float32), (M, K))
    q = _codes(q, M, K, X.device) if q is not None else None
    _opt(s, "s", torch.float32, (M,))
    if rotation not in ROTATIONS:
        raise ValueError(f"rotation must be one of {sorted(ROTATIONS)}")
    _on_device(X.device, X=X, q=q, s=s)
    if q is None:
        q = _codes(None, M, K, X.device)
    if s is None:
        s = torch.empty(M, dtype=torch.float32, device=X.device)
    flags = ROTATIONS[rotation] | (FLAG_GELU if gelu else 0)
    rc = lib.convrot_rotate_quantize(_ptr(X), _dtype_tag(X.dtype), M, K, block,
                                     flags, _ptr(q), _ptr(s), _stream(stream))
    _check("convrot_rotate_quantize", rc)
    return q, s


def convrot_gemm_i32(q_x: torch.Tensor, M: int, W: PreparedWeights, out=None, stream=None):
    """acc [M, N] int32 from K-tiled codes q_x of M rows."""
    lib = library()
    dev = _weights(W, "W")
    _codes(q_x, M, W.K, dev)
    _output(out, M, W.N, torch.int32)
    _on_device(dev, q_x=q_x, out=out)
    if out is None:
        out = torch.empty((M, W.N), dtype=torch.int32, device=dev)
    rc = lib.convrot_gemm_i32(_ptr(q_x), M, W.ref(), _ptr(out), _stream(stream))
    _check("convrot_gemm_i32", rc)
    return out


def convrot_gemm_dequant(q_x: torch.Tensor, s_x: torch.Tensor, W: PreparedWeights, bias=None,
                         out_dtype: torch.dtype = torch.bfloat16, out=None, gelu: bool = False,
                         swiglu: bool = False, stream=None):
    """Y [M, N] from K-tiled codes q_x and row scales s_x [M] (with swiglu, W a
    SwiGLU fc1 weight and Y = g [M, N/2])."""
    lib = library()
    dev = _weights(W, "W")
    if not isinstance(s_x, torch.Tensor) or s_x.dim() != 1:
        raise ValueError("s_x must be a 1-D tensor [M]")
    M = s_x.shape[0]
    _need(s_x, "s_x", torch.float32, (M,))
    _codes(q_x, M, W.K, dev)
    _opt(bias, "bias", torch.float32, (W.N,))
    ncols = W.N // 2 if swiglu else W.N
    _output(out, M, ncols, (torch.bfloat16, torch.float32))
    _on_device(dev, q_x=q_x, s_x=s_x, bias=bias, out=out)
    if out is None:
        out = torch.empty((M, ncols), dtype=out_dtype, device=dev)
    flags = (FLAG_GELU if gelu else 0) | (FLAG_SWIGLU if swiglu else 0)
    rc = lib.convrot_gemm_dequant(_ptr(q_x), _ptr(s_x), M, W.ref(), _ptr(bias), _ptr(out),
                                  _dtype_tag(out.dtype), flags, _stream(stream))
    _check("convrot_gemm_dequant", rc)
    return out


def convrot_lowrank_factor1(q_x: torch.Tensor, s_x: torch.Tensor, A: PreparedWeights,
                            q_h=None, s_h=None, stream=None):
    """Factor 1 of the low-rank chain with its output rotated and requantised:
    returns (q_h, s_h), q_h the K-tiled codes (Mp, r), s_h [M] f32."""
    lib = library()
    dev = _weights(A, "A")
    if not isinstance(s_x, torch.Tensor) or s_x.dim() != 1:
        raise ValueError("s_x must be a 1-D tensor [M]")
    M = s_x.shape[0]
    _need(s_x, "s_x", torch.float32, (M,))
    _codes(q_x, M, A.K, dev)
    if q_h is not None:
        _codes(q_h, M, A.N, dev)
    _opt(s_h, "s_h", torch.float32, (M,))
    _on_device(dev, q_x=q_x, s_x=s_x, q_h=q_h, s_h=s_h)
    q_h = _codes(q_h, M, A.N, dev)
    if s_h is None:
        s_h = torch.empty(M, dtype=torch.float32, device=dev)
    rc = lib.convrot_lowrank_factor1(_ptr(q_x), _ptr(s_x), M, A.ref(), _ptr(q_h), _ptr(s_h),
                                     _stream(stream))
    _check("convrot_lowrank_factor1", rc)
    return q_h, s_h


def convrot_gelu_bf16(u: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """bf16(GELU(u)) elementwise, as the MLP's up projection applies it."""
    lib = library()
    if not isinstance(u, torch.Tensor) or u.dtype != torch.bfloat16:
        raise ValueError("u must be a bf16 tensor")
    u = u.contiguous()
    _opt(out, "out", torch.bfloat16, tuple(u.shape))
    _on_device(u.device, u=u, out=out)
    if out is None:
        out = torch.empty_like(u)
    _check("convrot_gelu_bf16", lib.convrot_gelu_bf16(_ptr(u), u.numel(), _ptr(out),
                                                      _stream(stream)))
    return out


def convrot_probe_mfma_i8(iters: int, seed: torch.Tensor, sink: torch.Tensor,
                          stream=None) -> int:
    """Launch the INT8 MFMA rate probe; returns its INT8 operation count.
    seed: 4 KiB on the device (the operands it starts from); sink: 16 bytes."""
    lib = library()
    if seed.numel() * seed.element_size() < 4096 or sink.numel() * sink.element_size() < 16:
        raise ValueError("seed needs 4 KiB and sink 16 bytes")
    ops = ctypes.c_int64(0)
    _check("convrot_probe_mfma_i8", lib.convrot_probe_mfma_i8(
        iters, _ptr(seed), _ptr(sink), ctypes.byref(ops), _stream(stream)))
    return ops.value


def convrot_probe_stream(src, dst: torch.Tensor, mode: int, stream=None):
    """Streaming probe: mode 0 reads src's 16-byte items and writes 8 bytes
    per item into dst, mode 1 copies them, mode 2 (src None) only writes all
    of dst's 16-byte items."""
    lib = library()
    if mode == 2:
        n16 = dst.numel() * dst.element_size() // 16
    else:
        nbytes = src.numel() * src.element_size()
        n16 = nbytes // 16
        if nbytes % 16 or dst.numel() * dst.element_size() < n16 * (8 if mode == 0 else 16):
            raise ValueError("src must be whole 16-byte items and dst large enough")
    _check("convrot_probe_stream", lib.convrot_probe_stream(
        None if src is None else _ptr(src), _ptr(dst), n16, mode, _stream(stream)))
    return dst
