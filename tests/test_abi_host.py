"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every symbol include/convrot.h declares, sizes workspaces as documented, and
rejects bad arguments before launching anything.  Pointers below are fake
(never dereferenced): validation fails before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")


@pytest.fixture(scope="module")
def cr():
    from w8a8_int8_rotated_amd import convrot
    if not os.path.exists(convrot.LIB_PATH):
        pytest.fail("libconvrot.so not built (run __graft_entry__.build())")
    convrot.library()
    return convrot


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b((?:convrot|lowrank)_\w+)\s*\(", txt, flags=re.M)
    return sorted(set(names))


def test_header_declares_entry_points():
    names = declared_functions()
    for must in ("convrot_linear_prepare_weights", "convrot_linear_forward",
                 "lowrank_convrot_forward"):
        assert must in names


def test_every_declared_symbol_is_exported(cr):
    lib = ctypes.CDLL(cr.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding declares a signature for every one of them
    assert sorted(cr.EXPORTED) == declared_functions()


def test_internal_symbols_hidden(cr):
    out = os.popen(f"nm -D --defined-only {cr.LIB_PATH}").read()
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    api = set(declared_functions())
    assert exported >= api
    assert not [s for s in exported - api if "convrot" in s], exported - api


def test_status_strings(cr):
    lib = cr.library()
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.convrot_status_string(code)
    assert lib.convrot_status_string(-99) == b"unknown status"
    assert lib.convrot_version() >= 100
    assert lib.convrot_last_hip_error() == 0


def test_sizing(cr):
    assert cr.convrot_weights_packed_bytes(16128, 5376, 128) == 16128 * 5376
    assert cr.convrot_weights_packed_bytes(16, 5376, 96) == 0        # bad block
    assert cr.convrot_weights_packed_bytes(10, 5376, 128) == 0       # N % 16
    assert cr.convrot_weights_packed_bytes(16, 5440, 64) == 0        # K % 128
    assert cr.convrot_weights_packed_bytes(16, 65536 + 128, 128) == 0
    M, K, N = 38656, 5376, 16128
    ws = cr.convrot_linear_workspace_bytes(M, K, N, 128)
    assert ws >= M * K + 4 * M and ws % 256 == 0
    assert cr.convrot_linear_workspace_bytes(0, K, N, 128) == 0
    lr = cr.lowrank_convrot_workspace_bytes(M, K, 512, 5376, 128)
    assert lr >= M * K + M * 512 * 3 + 8 * M
    assert cr.lowrank_convrot_workspace_bytes(M, K, 500, 5376, 128) == 0
    mlp = cr.convrot_mlp_workspace_bytes(16384, 5376, 21504, 5376, 128)
    assert mlp >= 16384 * (5376 + 3 * 21504)
    assert cr.convrot_prepare_workspace_bytes(N, K, 128, cr.F32, cr.OUT_MAJOR) == 0
    assert cr.convrot_prepare_workspace_bytes(N, K, 128, cr.F32, cr.IN_MAJOR) >= 4 * N * K
    assert cr.convrot_prepare_workspace_bytes(N, K, 128, cr.I8, cr.IN_MAJOR) == 0


FAKE = 0x7f0000000000          # 16-byte aligned, never dereferenced
FAKE_ODD = FAKE + 8


def _desc(cr, N=512, K=512, block=128, magic=None, version=None):
    d = cr.convrot_weights()
    d.magic = cr.WEIGHTS_MAGIC if magic is None else magic
    d.version = cr.WEIGHTS_VERSION if version is None else version
    d.N, d.K, d.block, d.flags = N, K, block, 0
    d.codes, d.scale = FAKE, FAKE + 4096
    return d


def _fwd(cr, d, M=4, X=FAKE, Y=FAKE + 8192, ws=FAKE + 65536, ws_bytes=1 << 30, y=1, bias=None):
    return cr.library().convrot_linear_forward(X, M, ctypes.byref(d), bias, Y, y, ws,
                                               ws_bytes, None)


def test_forward_validation(cr):
    d = _desc(cr)
    assert _fwd(cr, _desc(cr, magic=0)) == cr.ELAYOUT
    assert _fwd(cr, _desc(cr, version=9)) == cr.ELAYOUT
    assert _fwd(cr, _desc(cr, block=100)) == cr.ELAYOUT
    assert _fwd(cr, d, M=-1) == cr.EINVAL
    assert _fwd(cr, d, M=0) == cr.OK                  # no-op, nothing launched
    assert _fwd(cr, d, X=None) == cr.EINVAL
    assert _fwd(cr, d, X=FAKE_ODD) == cr.EALIGN
    assert _fwd(cr, d, Y=FAKE_ODD) == cr.EALIGN
    assert _fwd(cr, d, ws=None) == cr.EWORKSPACE
    assert _fwd(cr, d, ws_bytes=16) == cr.EWORKSPACE
    assert _fwd(cr, d, y=cr.I8) == cr.EUNSUPPORTED
    big = _desc(cr, N=16, K=65536)
    assert _fwd(cr, big, M=40000) == cr.EUNSUPPORTED  # M*K beyond int32 offsets
    lib = cr.library()
    assert lib.convrot_linear_forward(FAKE, 4, None, None, FAKE, 1, FAKE, 1 << 20, None) \
        == cr.EINVAL


def test_prepare_validation(cr):
    lib = cr.library()
    d = cr.convrot_weights()
    d.codes, d.scale = FAKE, FAKE + 4096
    call = lambda **k: lib.convrot_linear_prepare_weights(
        k.get("W", FAKE), k.get("dt", cr.F32), k.get("layout", cr.OUT_MAJOR),
        k.get("scale", None), k.get("N", 512), k.get("K", 512), k.get("b", 128),
        ctypes.byref(k.get("d", d)), k.get("ws", None), k.get("wsb", 0), None)
    assert call(b=32) == cr.EINVAL
    assert call(K=384, b=256) == cr.EINVAL                    # K % b
    assert call(K=320, b=64) == cr.EUNSUPPORTED               # K % 128
    assert call(N=24) == cr.EUNSUPPORTED                      # N % 16
    assert call(dt=cr.I32) == cr.EUNSUPPORTED
    assert call(dt=cr.I8) == cr.EINVAL                        # import needs scales
    assert call(scale=FAKE) == cr.EINVAL                      # scales only for import
    assert call(layout=7) == cr.EINVAL
    assert call(W=FAKE_ODD) == cr.EALIGN
    assert call(layout=cr.IN_MAJOR) == cr.EWORKSPACE          # transpose staging
    e = cr.convrot_weights()
    assert call(d=e) == cr.EINVAL                             # codes/scale not set
    assert d.magic == 0                                       # nothing written on error


def test_lowrank_and_mlp_validation(cr):
    lib = cr.library()
    A, B = _desc(cr, N=256, K=512), _desc(cr, N=512, K=256)
    bad = _desc(cr, N=512, K=384)
    ok = lambda a, b_: lib.lowrank_convrot_forward(FAKE, 0, ctypes.byref(a), ctypes.byref(b_),
                                                   None, FAKE, 1, FAKE, 1 << 30, None)
    assert ok(A, B) == cr.OK                                   # M = 0
    assert ok(A, bad) == cr.ELAYOUT                            # r mismatch
    B64 = _desc(cr, N=512, K=256, block=64)
    assert ok(A, B64) == cr.ELAYOUT                            # block mismatch
    assert lib.lowrank_convrot_forward(FAKE, 8, ctypes.byref(A), ctypes.byref(B), None, FAKE,
                                       1, FAKE, 64, None) == cr.EWORKSPACE
    assert lib.convrot_mlp_forward(FAKE, 8, ctypes.byref(A), None, ctypes.byref(bad), None,
                                   FAKE, 1, FAKE, 1 << 30, None) == cr.ELAYOUT


def test_hook_validation(cr):
    lib = cr.library()
    rq = lambda x_dtype, K, flags, M=4: lib.convrot_rotate_quantize(
        FAKE, x_dtype, M, K, 128, flags, FAKE, FAKE, None)
    assert rq(cr.BF16, 512, 2) == cr.EUNSUPPORTED                  # unknown flag bit
    # GELU on load: bf16 rows with 6144 < K <= 24576 only
    assert rq(cr.BF16, 512, cr.FLAG_GELU) == cr.EUNSUPPORTED
    assert rq(cr.BF16, 6144, cr.FLAG_GELU) == cr.EUNSUPPORTED
    assert rq(cr.BF16, 24576 + 128, cr.FLAG_GELU) == cr.EUNSUPPORTED
    assert rq(cr.F32, 8192, cr.FLAG_GELU) == cr.EUNSUPPORTED
    assert rq(cr.BF16, 6144 + 128, cr.FLAG_GELU, M=0) == cr.OK
    assert rq(cr.BF16, 24576, cr.FLAG_GELU, M=0) == cr.OK
    assert lib.convrot_rotate_quantize(FAKE, cr.BF16, 4, 500, 128, 0, FAKE, FAKE, None) \
        == cr.EINVAL
    assert lib.convrot_rotate_quantize(FAKE, cr.I8, 4, 512, 128, 0, FAKE, FAKE, None) \
        == cr.EUNSUPPORTED
    assert lib.convrot_rotate_quantize(FAKE, cr.BF16, 0, 512, 128, 0, None, None, None) == cr.OK
    d = _desc(cr)
    assert lib.convrot_gemm_dequant(FAKE, FAKE, 4, ctypes.byref(d), None, FAKE, cr.F32,
                                    cr.FLAG_GELU, None) == cr.EUNSUPPORTED
    assert lib.convrot_gemm_dequant(FAKE, FAKE, 4, ctypes.byref(d), None, FAKE, cr.BF16, 4,
                                    None) == cr.EUNSUPPORTED
    # the SwiGLU epilogue needs a weight prepared as SwiGLU pairs, and a plain
    # forward refuses such a weight
    assert lib.convrot_gemm_dequant(FAKE, FAKE, 4, ctypes.byref(d), None, FAKE, cr.BF16,
                                    cr.FLAG_SWIGLU, None) == cr.ELAYOUT
    dp = _desc(cr)
    dp.flags = cr.SWIGLU_PAIRS
    assert lib.convrot_linear_forward(FAKE, 4, ctypes.byref(dp), None, FAKE, cr.BF16, FAKE,
                                      1 << 30, None) == cr.ELAYOUT
    assert lib.convrot_gemm_dequant(FAKE, FAKE, 4, ctypes.byref(dp), None, FAKE, cr.F32,
                                    cr.FLAG_SWIGLU, None) == cr.EUNSUPPORTED
    assert lib.convrot_swiglu_mlp_forward(FAKE, 4, ctypes.byref(d), None, ctypes.byref(d), None,
                                          FAKE, cr.BF16, FAKE, 1 << 30, None) == cr.ELAYOUT
    assert lib.convrot_gemm_i32(FAKE_ODD, 4, ctypes.byref(d), FAKE, None) == cr.EALIGN
    f1 = lambda d, M=4, qx=FAKE, sx=FAKE, qh=FAKE, sh=FAKE: lib.convrot_lowrank_factor1(
        qx, sx, M, ctypes.byref(d), qh, sh, None)
    assert f1(_desc(cr, N=640)) == cr.EUNSUPPORTED             # r > 512
    assert f1(_desc(cr, block=256)) == cr.EUNSUPPORTED         # block 256
    assert f1(_desc(cr, magic=0)) == cr.ELAYOUT
    assert f1(_desc(cr), M=0, qx=None, sx=None, qh=None, sh=None) == cr.OK
    assert f1(_desc(cr), qh=None) == cr.EINVAL
    assert f1(_desc(cr), M=-1) == cr.EINVAL
    assert f1(_desc(cr, N=256, block=64), sh=FAKE_ODD) == cr.EALIGN
    assert lib.convrot_gelu_bf16(FAKE, -1, FAKE, None) == cr.EINVAL


def test_rotation_kind_validation(cr):
    """The regular H_4 rotation exists for b = 64 and 256 only; unknown kind
    bits are rejected; chained weights must share the kind."""
    lib = cr.library()
    R = cr.ROT_REGULAR
    rq = lambda flags, block, M=0: lib.convrot_rotate_quantize(
        None, cr.BF16, M, 512, block, flags, None, None, None)
    assert rq(R, 64) == cr.OK and rq(R, 256) == cr.OK
    assert rq(R, 128) == cr.EINVAL
    assert rq(0x200, 64) == cr.EUNSUPPORTED
    # descriptors
    reg = lambda **kw: _flag(_desc(cr, **kw), R)
    assert _fwd(cr, reg(block=128)) == cr.ELAYOUT
    assert _fwd(cr, _flag(_desc(cr), 0x200)) == cr.ELAYOUT
    assert _fwd(cr, reg(block=64), M=0) == cr.OK
    A, B = reg(N=256, K=512, block=64), _desc(cr, N=512, K=256, block=64)
    assert lib.lowrank_convrot_forward(FAKE, 8, ctypes.byref(A), ctypes.byref(B), None, FAKE,
                                       1, FAKE, 1 << 30, None) == cr.ELAYOUT
    up, down = reg(N=256, K=512, block=64), _desc(cr, N=512, K=256, block=64)
    assert lib.convrot_mlp_forward(FAKE, 8, ctypes.byref(up), None, ctypes.byref(down), None,
                                   FAKE, 1, FAKE, 1 << 30, None) == cr.ELAYOUT
    assert lib.convrot_lowrank_factor1(FAKE, FAKE, 4, ctypes.byref(reg(N=256, block=64)), FAKE,
                                       FAKE, None) == cr.EUNSUPPORTED
    # prepare: the kind is requested through out->flags
    d = cr.convrot_weights()
    d.codes, d.scale, d.flags = FAKE, FAKE + 4096, R
    assert lib.convrot_linear_prepare_weights(FAKE, cr.F32, cr.OUT_MAJOR, None, 64, 512, 128,
                                              ctypes.byref(d), None, 0, None) == cr.EINVAL
    d.flags = 0x200
    assert lib.convrot_linear_prepare_weights(FAKE, cr.F32, cr.OUT_MAJOR, None, 64, 512, 64,
                                              ctypes.byref(d), None, 0, None) == cr.EINVAL


def test_lowrank_bf16_validation(cr):
    lib = cr.library()
    f = lambda M=8, K=512, r=64, N=256, X=FAKE, ws=FAKE, wsb=1 << 20: lib.lowrank_bf16_forward(
        X, M, K, FAKE, r, FAKE, N, None, FAKE, ws, wsb, None)
    assert f(M=0, X=None, ws=None, wsb=0) == cr.OK
    assert f(M=-1) == cr.EINVAL
    assert f(K=500) == cr.EUNSUPPORTED
    assert f(r=96) == cr.EUNSUPPORTED
    assert f(N=250) == cr.EUNSUPPORTED
    assert f(X=None) == cr.EINVAL
    assert f(X=FAKE_ODD) == cr.EALIGN
    assert f(ws=None) == cr.EWORKSPACE
    assert f(wsb=100) == cr.EWORKSPACE
    assert lib.lowrank_bf16_workspace_bytes(8, 64) >= 8 * 64 * 2


def _flag(d, flags):
    d.flags = flags
    return d


def test_gelu_and_probe_validation(cr):
    lib = cr.library()
    assert lib.convrot_gelu_bf16(None, 0, None, None) == cr.OK
    assert lib.convrot_gelu_bf16(None, 4, FAKE, None) == cr.EINVAL
    assert lib.convrot_gelu_bf16(FAKE, -1, FAKE, None) == cr.EINVAL
    ops = ctypes.c_int64(0)
    mfma = lambda it=10, seed=FAKE, sink=FAKE, o=ctypes.byref(ops): lib.convrot_probe_mfma_i8(
        it, seed, sink, o, None)
    assert mfma(it=0) == cr.EINVAL
    assert mfma(it=(1 << 24) + 1) == cr.EINVAL
    assert mfma(seed=None) == cr.EINVAL
    assert mfma(o=None) == cr.EINVAL
    assert mfma(sink=FAKE_ODD) == cr.EALIGN
    stream = lambda src=FAKE, dst=FAKE, n=64, mode=0: lib.convrot_probe_stream(src, dst, n, mode,
                                                                               None)
    assert stream(n=0, src=None, dst=None) == cr.OK
    assert stream(n=-1) == cr.EINVAL
    assert stream(mode=3) == cr.EINVAL
    assert stream(mode=0, src=None) == cr.EINVAL
    assert stream(dst=None) == cr.EINVAL
    assert stream(src=FAKE_ODD) == cr.EALIGN


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    """No silent fallback: a missing library raises on first use."""
    from w8a8_int8_rotated_amd import convrot
    monkeypatch.setattr(convrot, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(convrot, "_lib", None)
    with pytest.raises(ImportError):
        convrot.library()


def test_call_log(cr):
    """CONVROT_LOG=1 makes the main entry points print their name, shape and
    status to stderr (checked on calls that fail validation, so nothing is
    launched)."""
    import subprocess
    import sys
    code = ("import ctypes; from w8a8_int8_rotated_amd import convrot as cr; "
            "lib = cr.library(); "
            "print(lib.convrot_linear_forward(None, 4, None, None, None, 1, None, 0, None)); "
            "print(lib.lowrank_convrot_forward(None, -1, None, None, None, None, 1, None, 0, None))")
    env = dict(os.environ, CONVROT_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "[convrot] convrot_linear_forward M=4 N=0 K=0 -> invalid argument" in r.stderr
    assert "[convrot] lowrank_convrot_forward M=-1" in r.stderr
    env["CONVROT_LOG"] = "0"
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=120)
    assert "[convrot]" not in r.stderr
