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
    "convrot_linear_prepare_weights": (
        _c_int, [_c_p, _c_int, _c_int, _c_p, _c_i64, _c_i64, _c_int, _W, _c_p, _c_sz, _c_p]),
    "convrot_linear_forward": (
        _c_int, [_c_p, _c_i64, _W, _c_p, _c_p, _c_int, _c_p, _c_sz, _c_p]),
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
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    if layout == OUT_MAJOR:
        N, K = W.shape
    else:
        K, N = W.shape
    W = W.contiguous()
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
    """The rank a low-rank pair is stored with: r rounded up to a multiple of
    128 (the contraction's K granularity) and of the Hadamard block b."""
    m = 256 if block == 256 else 128
    return (r + m - 1) // m * m


def convrot_lowrank_prepare(A: torch.Tensor, B: torch.Tensor, block: int, stream=None,
                            rotation: str = "sylvester"):
    """Prepare a low-rank pair W ~ B . A, A [r, K] and B [N, r] (output-major),
    padding the rank with zero rows of A and zero columns of B to
    lowrank_padded_rank(r, block), as the checkpoint loader pads ranks to a
    multiple of 64.  The padding leaves the product B . A unchanged; when r is
    already a multiple of b, the rotated and requantised intermediate of the
    real rank positions is unchanged too."""
    if A.dim() != 2 or B.dim() != 2 or B.shape[1] != A.shape[0]:
        raise ValueError("A must be [r, K] and B [N, r]")
    r = A.shape[0]
    rp = lowrank_padded_rank(r, block)
    if rp != r:
        A = torch.cat([A, A.new_zeros((rp - r, A.shape[1]))], dim=0)
        B = torch.cat([B, B.new_zeros((B.shape[0], rp - r))], dim=1)
    pa = convrot_linear_prepare_weights(A.contiguous(), block, stream=stream, rotation=rotation)
    pb = convrot_linear_prepare_weights(B.contiguous(), block, stream=stream, rotation=rotation)
    return pa, pb


# ----------------------------------------------------------- forward ----

def convrot_linear_forward(X: torch.Tensor, W: PreparedWeights, bias=None,
                           out_dtype: torch.dtype = torch.bfloat16, out=None,
                           workspace=None, stream=None) -> torch.Tensor:
    lib = library()
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, W.N), dtype=out_dtype, device=X.device)
    wsb = lib.convrot_linear_workspace_bytes(M, W.K, W.N, W.block)
    ws = _workspace(wsb, X.device, workspace)
    rc = lib.convrot_linear_forward(_ptr(X), M, W.ref(), _ptr(bias), _ptr(out),
                                    _dtype_tag(out.dtype), _ptr(ws),
                                    ws.numel() if ws is not None else 0, _stream(stream))
    _check("convrot_linear_forward", rc)
    return out


def lowrank_convrot_forward(X: torch.Tensor, A: PreparedWeights, B: PreparedWeights,
                            bias=None, out_dtype: torch.dtype = torch.bfloat16, out=None,
                            workspace=None, stream=None) -> torch.Tensor:
    lib = library()
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, B.N), dtype=out_dtype, device=X.device)
    wsb = lib.lowrank_convrot_workspace_bytes(M, A.K, A.N, B.N, A.block)
    ws = _workspace(wsb, X.device, workspace)
    rc = lib.lowrank_convrot_forward(_ptr(X), M, A.ref(), B.ref(), _ptr(bias), _ptr(out),
                                     _dtype_tag(out.dtype), _ptr(ws),
                                     ws.numel() if ws is not None else 0, _stream(stream))
    _check("lowrank_convrot_forward", rc)
    return out


def convrot_mlp_forward(X: torch.Tensor, W_up: PreparedWeights, W_down: PreparedWeights,
                        bias_up=None, bias_down=None, out_dtype: torch.dtype = torch.bfloat16,
                        out=None, workspace=None, stream=None) -> torch.Tensor:
    lib = library()
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, W_down.N), dtype=out_dtype, device=X.device)
    wsb = lib.convrot_mlp_workspace_bytes(M, W_up.K, W_up.N, W_down.N, W_up.block)
    ws = _workspace(wsb, X.device, workspace)
    rc = lib.convrot_mlp_forward(_ptr(X), M, W_up.ref(), _ptr(bias_up), W_down.ref(),
                                 _ptr(bias_down), _ptr(out), _dtype_tag(out.dtype), _ptr(ws),
                                 ws.numel() if ws is not None else 0, _stream(stream))
    _check("convrot_mlp_forward", rc)
    return out


def lowrank_bf16_forward(X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, bias=None,
                         out=None, workspace=None, stream=None) -> torch.Tensor:
    """Comparison variant: bf16(bf16(X . A^T) . B^T + bias), bf16 factors
    A [r, K] and B [N, r], no rotation or quantisation."""
    lib = library()
    for t in (X, A, B):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("X, A and B must be contiguous bf16")
    M, K = X.shape
    r, N = A.shape[0], B.shape[0]
    if A.shape[1] != K or B.shape[1] != r:
        raise ValueError("A must be [r, K] and B [N, r]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    wsb = lib.lowrank_bf16_workspace_bytes(M, r)
    ws = _workspace(wsb, X.device, workspace)
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
    """A K-tiled code buffer for M rows of K codes: allocated as (Mp, K) int8,
    or a caller tensor checked to hold Mp * K bytes."""
    Mp = padded_rows(M)
    if q is None:
        return torch.empty((Mp, K), dtype=torch.int8, device=device)
    if q.dtype != torch.int8 or not q.is_contiguous() or q.numel() < Mp * K:
        raise ValueError(f"K-tiled codes need a contiguous int8 tensor of {Mp * K} elements")
    return q


def convrot_rotate_quantize(X: torch.Tensor, block: int, q=None, s=None, stream=None,
                            rotation: str = "sylvester", gelu: bool = False):
    """Rotate + quantise the rows of X: (q, s), q the K-tiled codes (Mp, K).
    gelu: quantise bf16(GELU(X)) instead (bf16 X, 6144 < K <= 24576), as the
    MLP path does with its intermediate."""
    lib = library()
    M, K = X.shape
    q = _codes(q, M, K, X.device)
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
    _codes(q_x, M, W.K, None)
    if out is None:
        out = torch.empty((M, W.N), dtype=torch.int32, device=q_x.device)
    rc = lib.convrot_gemm_i32(_ptr(q_x), M, W.ref(), _ptr(out), _stream(stream))
    _check("convrot_gemm_i32", rc)
    return out


def convrot_gemm_dequant(q_x: torch.Tensor, s_x: torch.Tensor, W: PreparedWeights, bias=None,
                         out_dtype: torch.dtype = torch.bfloat16, out=None, gelu: bool = False,
                         stream=None):
    """Y [M, N] from K-tiled codes q_x and row scales s_x [M]."""
    lib = library()
    M = s_x.shape[0]
    _codes(q_x, M, W.K, None)
    if out is None:
        out = torch.empty((M, W.N), dtype=out_dtype, device=q_x.device)
    rc = lib.convrot_gemm_dequant(_ptr(q_x), _ptr(s_x), M, W.ref(), _ptr(bias), _ptr(out),
                                  _dtype_tag(out.dtype), FLAG_GELU if gelu else 0,
                                  _stream(stream))
    _check("convrot_gemm_dequant", rc)
    return out


def convrot_lowrank_factor1(q_x: torch.Tensor, s_x: torch.Tensor, A: PreparedWeights,
                            q_h=None, s_h=None, stream=None):
    """Factor 1 of the low-rank chain with its output rotated and requantised:
    returns (q_h, s_h), q_h the K-tiled codes (Mp, r), s_h [M] f32."""
    lib = library()
    M = s_x.shape[0]
    _codes(q_x, M, A.K, None)
    q_h = _codes(q_h, M, A.N, q_x.device)
    if s_h is None:
        s_h = torch.empty(M, dtype=torch.float32, device=q_x.device)
    rc = lib.convrot_lowrank_factor1(_ptr(q_x), _ptr(s_x), M, A.ref(), _ptr(q_h), _ptr(s_h),
                                     _stream(stream))
    _check("convrot_lowrank_factor1", rc)
    return q_h, s_h


def convrot_gelu_bf16(u: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """bf16(GELU(u)) elementwise, as the MLP's up projection applies it."""
    lib = library()
    if u.dtype != torch.bfloat16:
        raise ValueError("u must be bf16")
    u = u.contiguous()
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
