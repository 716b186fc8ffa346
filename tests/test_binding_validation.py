"""Host-only tests of the Python binding's argument checks: a tensor whose
dtype, shape, contiguity or device does not match what the C ABI will
dereference is rejected with ValueError before any pointer reaches the
library.  CPU tensors stand in for device ones; shape and dtype are checked
before the device, so each mistake is seen on its own, and a well-formed call
with host tensors fails on the device check (nothing is ever launched)."""
import os

import pytest
import torch


@pytest.fixture(scope="module")
def cr():
    from w8a8_int8_rotated_amd import convrot
    if not os.path.exists(convrot.LIB_PATH):
        pytest.fail("libconvrot.so not built (run __graft_entry__.build())")
    convrot.library()
    return convrot


def fake_weights(cr, N, K, block=128):
    """A prepared-weight descriptor over host tensors (never dereferenced)."""
    d = cr.convrot_weights()
    d.magic, d.version, d.N, d.K, d.block, d.flags = (cr.WEIGHTS_MAGIC, cr.WEIGHTS_VERSION,
                                                      N, K, block, 0)
    codes = torch.zeros(N * K, dtype=torch.int8)
    scale = torch.ones(N, dtype=torch.float32)
    return cr.PreparedWeights(d, codes, scale)


M, K, N = 32, 256, 64
bf, f32 = torch.bfloat16, torch.float32


def X_ok():
    return torch.zeros((M, K), dtype=bf)


@pytest.mark.parametrize("case,kw,msg", [
    ("x_dtype", dict(X=torch.zeros((M, K), dtype=f32)), "X must be torch.bfloat16"),
    ("x_short_k", dict(X=torch.zeros((M, K - 128), dtype=bf)), "X must have shape"),
    ("x_1d", dict(X=torch.zeros(M * K, dtype=bf)), "X must be a 2-D tensor"),
    ("x_strided", dict(X=torch.zeros((K, M), dtype=bf).t()), "X must be contiguous"),
    ("out_small", dict(out=torch.zeros((M - 1, N), dtype=bf)), "out must have shape"),
    ("out_dtype", dict(out=torch.zeros((M, N), dtype=torch.float16)), "out must be"),
    ("out_strided", dict(out=torch.zeros((N, M), dtype=bf).t()), "out must be contiguous"),
    ("bias_dtype", dict(bias=torch.zeros(N, dtype=bf)), "bias must be torch.float32"),
    ("bias_len", dict(bias=torch.zeros(N - 16, dtype=f32)), "bias must have shape"),
    ("ws_small", dict(workspace=torch.zeros(64, dtype=torch.uint8)), "workspace holds"),
    ("ws_dtype", dict(workspace=torch.zeros(1 << 20, dtype=torch.int32)), "workspace must be"),
    ("host_tensors", dict(), "must be a GPU tensor"),
])
def test_linear_forward_rejects(cr, case, kw, msg):
    W = fake_weights(cr, N, K)
    args = dict(X=X_ok(), bias=None, out=None, workspace=None)
    args.update(kw)
    X = args.pop("X")
    with pytest.raises(ValueError, match=msg):
        cr.convrot_linear_forward(X, W, **args)


def test_weights_must_be_prepared(cr):
    with pytest.raises(ValueError, match="PreparedWeights"):
        cr.convrot_linear_forward(X_ok(), torch.zeros((N, K), dtype=torch.int8))


def test_lowrank_forward_rejects(cr):
    r = 128
    A, B = fake_weights(cr, r, K), fake_weights(cr, N, r)
    with pytest.raises(ValueError, match="X must have shape"):
        cr.lowrank_convrot_forward(torch.zeros((M, r), dtype=bf), A, B)
    with pytest.raises(ValueError, match="bias must have shape"):
        cr.lowrank_convrot_forward(X_ok(), A, B, bias=torch.zeros(r, dtype=f32))
    with pytest.raises(ValueError, match="out must have shape"):
        cr.lowrank_convrot_forward(X_ok(), A, B, out=torch.zeros((M, r), dtype=bf))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        cr.lowrank_convrot_forward(X_ok(), A, B)


def test_mlp_forward_rejects(cr):
    F = 512
    Wu, Wd = fake_weights(cr, F, K), fake_weights(cr, N, F)
    with pytest.raises(ValueError, match="bias_up must have shape"):
        cr.convrot_mlp_forward(X_ok(), Wu, Wd, bias_up=torch.zeros(N, dtype=f32))
    with pytest.raises(ValueError, match="bias_down must be torch.float32"):
        cr.convrot_mlp_forward(X_ok(), Wu, Wd, bias_down=torch.zeros(N, dtype=torch.float64))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        cr.convrot_mlp_forward(X_ok(), Wu, Wd)


def test_hooks_reject(cr):
    W = fake_weights(cr, N, K)
    q = torch.zeros((cr.padded_rows(M), K), dtype=torch.int8)
    with pytest.raises(ValueError, match="s_x must be torch.float32"):
        cr.convrot_gemm_dequant(q, torch.zeros(M, dtype=bf), W)
    with pytest.raises(ValueError, match="K-tiled codes need"):
        cr.convrot_gemm_dequant(q[:M - 1], torch.zeros(M, dtype=f32), W)
    with pytest.raises(ValueError, match="K-tiled codes need"):
        cr.convrot_gemm_i32(q.view(-1)[: M * K - 1], M, W)
    with pytest.raises(ValueError, match="s must have shape"):
        cr.convrot_rotate_quantize(X_ok(), 128, q=q, s=torch.zeros(M + 1, dtype=f32))
    with pytest.raises(ValueError, match="X must be"):
        cr.convrot_rotate_quantize(torch.zeros((M, K), dtype=torch.float16), 128)
    with pytest.raises(ValueError, match="u must be a bf16 tensor"):
        cr.convrot_gelu_bf16(torch.zeros(16, dtype=f32))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        cr.convrot_gemm_dequant(q, torch.zeros(M, dtype=f32), W)


def test_prepare_rejects(cr):
    with pytest.raises(ValueError, match="src_scale is required"):
        cr.convrot_linear_prepare_weights(torch.zeros((N, K), dtype=torch.int8), 128)
    with pytest.raises(ValueError, match="W must be float32"):
        cr.convrot_linear_prepare_weights(torch.zeros((N, K), dtype=torch.float64), 128)
    with pytest.raises(ValueError, match="src_scale must have shape"):
        cr.convrot_linear_prepare_weights(torch.zeros((N, K), dtype=torch.int8), 128,
                                          src_scale=torch.zeros(N + 1, dtype=f32))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        cr.convrot_linear_prepare_weights(torch.zeros((N, K), dtype=f32), 128)
