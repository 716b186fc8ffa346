"""numpy front end of the C oracle (``oracle/convrot_oracle.c``).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  bf16 tensors are
carried as ``numpy.uint16`` arrays holding the raw bfloat16 bits.

Each function names the step of the method it follows; the arithmetic itself
lives in the C file, whose header lists the page passages and the readings
taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32 = 0
BF16 = 1

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    _lib = open_library(_LIB_PATH)
    return _lib


def open_library(path):
    """Open a build of the oracle's C file and declare its signatures."""
    lib = ctypes.CDLL(path)
    sig = {
        "oracle_num_threads": (_c_int, []),
        "oracle_set_num_threads": (None, [_c_int]),
        "oracle_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "oracle_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "oracle_fwht_f32": (_c_int, [_c_p, _c_i64, _c_int]),
        "oracle_inv_sqrt_b": (ctypes.c_float, [_c_int]),
        "oracle_rowquant": (_c_int, [_c_p, _c_i64, _c_int, _c_p, _c_p]),
        "oracle_rotate_quantize_rows": (
            _c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_p, _c_p]),
        "oracle_prepare_weights_in_major": (
            _c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_int, _c_p, _c_p]),
        "oracle_gemm_i32": (_c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p]),
        "oracle_dequant": (
            _c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_int, _c_p]),
        "oracle_linear_forward": (
            _c_int, [_c_p, _c_i64, _c_i64, _c_int, _c_p, _c_p, _c_i64, _c_p,
                     _c_int, _c_p]),
        "oracle_lowrank_forward": (
            _c_int, [_c_p, _c_i64, _c_i64, _c_int, _c_p, _c_p, _c_i64, _c_p,
                     _c_p, _c_i64, _c_p, _c_int, _c_p, _c_p]),
        "oracle_gelu_f64": (ctypes.c_double, [ctypes.c_double]),
        "oracle_gelu_bf16": (None, [_c_p, _c_i64, _c_p]),
        "oracle_mlp_forward": (
            _c_int, [_c_p, _c_i64, _c_i64, _c_int, _c_p, _c_p, _c_i64, _c_p,
                     _c_p, _c_p, _c_i64, _c_p, _c_int, _c_p, _c_p, _c_p]),
        "oracle_fwht_regular_f32": (_c_int, [_c_p, _c_i64, _c_int]),
        "oracle_rotate_f32": (_c_int, [_c_p, _c_i64, _c_int, _c_int]),
        "oracle_rotate_quantize_rows_rot": (
            _c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_p, _c_p]),
        "oracle_prepare_weights_in_major_rot": (
            _c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_int, _c_int, _c_p, _c_p]),
        "oracle_linear_forward_rot": (
            _c_int, [_c_p, _c_i64, _c_i64, _c_int, _c_int, _c_p, _c_p, _c_i64, _c_p,
                     _c_int, _c_p]),
        "oracle_lowrank_forward_rot": (
            _c_int, [_c_p, _c_i64, _c_i64, _c_int, _c_int, _c_p, _c_p, _c_i64, _c_p,
                     _c_p, _c_i64, _c_p, _c_int, _c_p, _c_p]),
        "oracle_lowrank_bf16_forward": (
            _c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_i64, _c_p, _c_p, _c_p]),
        "oracle_silu_f64": (ctypes.c_double, [ctypes.c_double]),
        "oracle_silu_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "oracle_swiglu_bf16": (None, [_c_p, _c_i64, _c_i64, _c_p]),
        "oracle_swiglu_mlp_forward_rot": (
            _c_int, [_c_p, _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_p, _c_p, _c_i64, _c_p,
                     _c_p, _c_p, _c_i64, _c_p, _c_int, _c_p, _c_p, _c_p]),
        "oracle_mlp_forward_rot": (
            _c_int, [_c_p, _c_i64, _c_i64, _c_int, _c_int, _c_p, _c_p, _c_i64, _c_p,
                     _c_p, _c_p, _c_i64, _c_p, _c_int, _c_p, _c_p, _c_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _swap_library(lib):
    """Test hook: route every wrapper through another build (a planted
    mistake); returns the previous library so the caller can restore it."""
    global _lib
    prev = _load()
    _lib = lib
    return prev


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# rotation kinds: the Sylvester blocks (R1) or the regular H_4 Kronecker
# blocks of the Rung-Omega README (R8)
ROTATIONS = {"sylvester": 0, "regular": 1}


def _rot(rot: str) -> int:
    if rot not in ROTATIONS:
        raise ValueError(rot)
    return ROTATIONS[rot]


# ---------------------------------------------------------------- bf16 ----

def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits to fp32."""
    u16 = np.asarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x) -> np.ndarray:
    """Round-to-nearest-even narrowing to bf16 (element by element in C)."""
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    f = lib.oracle_f32_to_bf16
    for i in range(flat.size):
        out[i] = f(float(flat[i]))
    return out.reshape(x.shape)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel regions use."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's later parallel regions (timing only)."""
    _load().oracle_set_num_threads(int(n))


def inv_sqrt_b(b: int) -> np.float32:
    return np.float32(_load().oracle_inv_sqrt_b(int(b)))


# -------------------------------------------------------------- O1, O2 ----

def fwht(v, b: int, rot: str = "sylvester") -> np.ndarray:
    """O1: blockwise Sylvester FWHT of every row (fp32, ascending strides), or
    with rot='regular' the regular H_4 Kronecker blocks (R8)."""
    lib = _load()
    out = _c(v, np.float32).copy()
    K = out.shape[-1]
    rows = out.reshape(-1, K)
    for r in range(rows.shape[0]):
        row = np.ascontiguousarray(rows[r])
        _check(lib.oracle_rotate_f32(_ptr(row), K, int(b), _rot(rot)), "fwht")
        rows[r] = row
    return out


def rowquant(v, b: int):
    """O2 on rows that are already rotated: returns (codes int8, scale f32)."""
    lib = _load()
    v = _c(v, np.float32)
    K = v.shape[-1]
    rows = v.reshape(-1, K)
    q = np.empty(rows.shape, dtype=np.int8)
    s = np.empty(rows.shape[0], dtype=np.float32)
    for r in range(rows.shape[0]):
        row = np.ascontiguousarray(rows[r])
        qr = np.empty(K, dtype=np.int8)
        sr = np.empty(1, dtype=np.float32)
        _check(lib.oracle_rowquant(_ptr(row), K, int(b), _ptr(qr), _ptr(sr)),
               "rowquant")
        q[r] = qr
        s[r] = sr[0]
    return q.reshape(v.shape), s.reshape(v.shape[:-1])


# -------------------------------------------------------------- O3, O4 ----

def rotate_quantize(x, b: int, dtype: str, rot: str = "sylvester"):
    """O4 (activations, dtype='bf16' raw uint16) or O3 (weights, 'f32')."""
    lib = _load()
    if dtype == "bf16":
        x = _c(x, np.uint16)
        tag = BF16
    elif dtype == "f32":
        x = _c(x, np.float32)
        tag = F32
    else:
        raise ValueError(dtype)
    rows, K = x.shape
    q = np.empty((rows, K), dtype=np.int8)
    s = np.empty(rows, dtype=np.float32)
    _check(lib.oracle_rotate_quantize_rows_rot(_ptr(x), tag, rows, K, K, int(b), _rot(rot),
                                               _ptr(q), _ptr(s)), "rotate_quantize")
    return q, s


def prepare_weights(W, b: int, dtype: str = "f32", layout: str = "out_major",
                    rot: str = "sylvester"):
    """O3: codes and per-output scales of the rotated weight W . R^T.

    ``layout='out_major'`` takes W as [N, K]; ``'in_major'`` as [K, N]."""
    if layout == "out_major":
        return rotate_quantize(W, b, dtype, rot)
    if layout != "in_major":
        raise ValueError(layout)
    lib = _load()
    if dtype == "bf16":
        W = _c(W, np.uint16)
        tag = BF16
    else:
        W = _c(W, np.float32)
        tag = F32
    K, N = W.shape
    q = np.empty((N, K), dtype=np.int8)
    s = np.empty(N, dtype=np.float32)
    _check(lib.oracle_prepare_weights_in_major_rot(_ptr(W), tag, N, K, int(b), _rot(rot),
                                                   _ptr(q), _ptr(s)), "prepare")
    return q, s


# ---------------------------------------------------------- O5, O6, O7 ----

def gemm_i32(qx, qw) -> np.ndarray:
    """O5: exact int32 acc[m, n] = sum_k qx[m, k] qw[n, k]."""
    lib = _load()
    qx = _c(qx, np.int8)
    qw = _c(qw, np.int8)
    M, K = qx.shape
    N, K2 = qw.shape
    assert K == K2
    acc = np.empty((M, N), dtype=np.int32)
    _check(lib.oracle_gemm_i32(_ptr(qx), _ptr(qw), M, N, K, _ptr(acc)), "gemm")
    return acc


def dequant(acc, sx, sw, bias=None, out: str = "f32") -> np.ndarray:
    """O6/O7: y = ((float)acc * s_x) * s_w (+ bias), then fp32 or bf16."""
    lib = _load()
    acc = _c(acc, np.int32)
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    bias = None if bias is None else _c(bias, np.float32)
    M, N = acc.shape
    if out == "f32":
        y = np.empty((M, N), dtype=np.float32)
        tag = F32
    else:
        y = np.empty((M, N), dtype=np.uint16)
        tag = BF16
    _check(lib.oracle_dequant(_ptr(acc), _ptr(sx), _ptr(sw), _ptr(bias), M, N,
                              tag, _ptr(y)), "dequant")
    return y


def linear_forward(X_bf16, qw, sw, b: int, bias=None, out: str = "bf16",
                   rot: str = "sylvester"):
    """O4 -> O5 -> O6/O7 on bf16 activations [M, K]."""
    lib = _load()
    X = _c(X_bf16, np.uint16)
    qw = _c(qw, np.int8)
    sw = _c(sw, np.float32)
    bias = None if bias is None else _c(bias, np.float32)
    M, K = X.shape
    N = qw.shape[0]
    y = np.empty((M, N), dtype=np.float32 if out == "f32" else np.uint16)
    _check(lib.oracle_linear_forward_rot(_ptr(X), M, K, int(b), _rot(rot), _ptr(qw),
                                         _ptr(sw), N, _ptr(bias),
                                         F32 if out == "f32" else BF16, _ptr(y)),
           "linear_forward")
    return y


def lowrank_forward(X_bf16, qa, sa, qb, sb, b: int, bias=None,
                    out: str = "bf16", return_h: bool = False, rot: str = "sylvester"):
    """O8: h = bf16(linear(X; A)); y = linear(h; B, bias)."""
    lib = _load()
    X = _c(X_bf16, np.uint16)
    qa, sa = _c(qa, np.int8), _c(sa, np.float32)
    qb, sb = _c(qb, np.int8), _c(sb, np.float32)
    bias = None if bias is None else _c(bias, np.float32)
    M, K = X.shape
    r = qa.shape[0]
    N = qb.shape[0]
    assert qb.shape[1] == r
    y = np.empty((M, N), dtype=np.float32 if out == "f32" else np.uint16)
    h = np.empty((M, r), dtype=np.uint16)
    _check(lib.oracle_lowrank_forward_rot(_ptr(X), M, K, int(b), _rot(rot), _ptr(qa),
                                          _ptr(sa), r, _ptr(qb), _ptr(sb), N, _ptr(bias),
                                          F32 if out == "f32" else BF16, _ptr(y),
                                          _ptr(h)), "lowrank_forward")
    return (y, h) if return_h else y


def gelu_f64(z: float) -> float:
    return _load().oracle_gelu_f64(float(z))


def gelu_bf16(u_bf16) -> np.ndarray:
    """O9 activation: g = bf16(GELU_erf(float(u))), GELU in fp64."""
    lib = _load()
    u = _c(u_bf16, np.uint16)
    g = np.empty_like(u)
    lib.oracle_gelu_bf16(_ptr(u), u.size, _ptr(g))
    return g


def mlp_forward(X_bf16, qu, su, qd, sd, b: int, bias_up=None, bias_down=None,
                out: str = "bf16", return_intermediates: bool = False,
                rot: str = "sylvester"):
    """O9: u = bf16(linear(X; W_up)); g = GELU(u); y = linear(g; W_down)."""
    lib = _load()
    X = _c(X_bf16, np.uint16)
    qu, su = _c(qu, np.int8), _c(su, np.float32)
    qd, sd = _c(qd, np.int8), _c(sd, np.float32)
    bu = None if bias_up is None else _c(bias_up, np.float32)
    bd = None if bias_down is None else _c(bias_down, np.float32)
    M, K = X.shape
    F = qu.shape[0]
    N = qd.shape[0]
    assert qd.shape[1] == F
    y = np.empty((M, N), dtype=np.float32 if out == "f32" else np.uint16)
    u = np.empty((M, F), dtype=np.uint16)
    g = np.empty((M, F), dtype=np.uint16)
    _check(lib.oracle_mlp_forward_rot(_ptr(X), M, K, int(b), _rot(rot), _ptr(qu), _ptr(su),
                                      F, _ptr(bu), _ptr(qd), _ptr(sd), N, _ptr(bd),
                                      F32 if out == "f32" else BF16, _ptr(y),
                                      _ptr(u), _ptr(g)), "mlp_forward")
    return (y, u, g) if return_intermediates else y


def silu_f64(z: float) -> float:
    """R10: silu(z) = z / (1 + exp(-z)) in fp64."""
    return _load().oracle_silu_f64(float(z))


def silu_f32(a_bf16) -> np.ndarray:
    """R10: fp32(silu) of bf16 gate values (raw uint16 bits), element by element."""
    lib = _load()
    a = np.asarray(a_bf16, dtype=np.uint16)
    flat = a.reshape(-1)
    out = np.empty(flat.shape, dtype=np.float32)
    f = lib.oracle_silu_f32
    for i in range(flat.size):
        out[i] = f(int(flat[i]))
    return out.reshape(a.shape)


def swiglu_bf16(gu_bf16) -> np.ndarray:
    """R10: g = bf16(silu_f32(gate) * up) for the fc1 output gu [M, 2F]
    (gate = first F columns, up = last F)."""
    lib = _load()
    gu = _c(gu_bf16, np.uint16)
    M, F2 = gu.shape
    assert F2 % 2 == 0
    g = np.empty((M, F2 // 2), dtype=np.uint16)
    lib.oracle_swiglu_bf16(_ptr(gu), M, F2 // 2, _ptr(g))
    return g


def swiglu_mlp_forward(X_bf16, qgu, sgu, qd, sd, b_up: int, b_down: int, bias_gu=None,
                       bias_down=None, out: str = "bf16", return_intermediates: bool = False,
                       rot: str = "sylvester"):
    """R10: gu = bf16(linear(X; W_gu)) [M, 2F]; g = swiglu(gu); y = linear(g; W_down)."""
    lib = _load()
    X = _c(X_bf16, np.uint16)
    qgu, sgu = _c(qgu, np.int8), _c(sgu, np.float32)
    qd, sd = _c(qd, np.int8), _c(sd, np.float32)
    bu = None if bias_gu is None else _c(bias_gu, np.float32)
    bd = None if bias_down is None else _c(bias_down, np.float32)
    M, K = X.shape
    F2 = qgu.shape[0]
    assert F2 % 2 == 0
    F = F2 // 2
    N = qd.shape[0]
    assert qd.shape[1] == F
    y = np.empty((M, N), dtype=np.float32 if out == "f32" else np.uint16)
    gu = np.empty((M, F2), dtype=np.uint16)
    g = np.empty((M, F), dtype=np.uint16)
    _check(lib.oracle_swiglu_mlp_forward_rot(_ptr(X), M, K, int(b_up), int(b_down), _rot(rot),
                                             _ptr(qgu), _ptr(sgu), F, _ptr(bu), _ptr(qd),
                                             _ptr(sd), N, _ptr(bd),
                                             F32 if out == "f32" else BF16, _ptr(y), _ptr(gu),
                                             _ptr(g)), "swiglu_mlp_forward")
    return (y, gu, g) if return_intermediates else y


def lowrank_bf16_forward(X_bf16, A_bf16, B_bf16, bias=None, return_h: bool = False):
    """R9, the bf16 low-rank comparison variant: h = bf16(X . A^T),
    y = bf16(h . B^T + bias), each sum exact then rounded to fp32."""
    lib = _load()
    X = _c(X_bf16, np.uint16)
    A = _c(A_bf16, np.uint16)
    B = _c(B_bf16, np.uint16)
    bias = None if bias is None else _c(bias, np.float32)
    M, K = X.shape
    r, N = A.shape[0], B.shape[0]
    assert A.shape[1] == K and B.shape[1] == r
    y = np.empty((M, N), dtype=np.uint16)
    h = np.empty((M, r), dtype=np.uint16)
    _check(lib.oracle_lowrank_bf16_forward(_ptr(X), M, K, _ptr(A), r, _ptr(B), N, _ptr(bias),
                                           _ptr(y), _ptr(h)), "lowrank_bf16_forward")
    return (y, h) if return_h else y


__all__ = [
    "num_threads", "set_num_threads", "bf16_to_f32", "f32_to_bf16", "inv_sqrt_b", "fwht", "rowquant",
    "rotate_quantize", "prepare_weights", "gemm_i32", "dequant",
    "linear_forward", "lowrank_forward", "gelu_f64", "gelu_bf16", "mlp_forward",
    "lowrank_bf16_forward", "silu_f64", "silu_f32", "swiglu_bf16", "swiglu_mlp_forward",
]
