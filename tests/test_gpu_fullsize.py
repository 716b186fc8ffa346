"""GPU parity at the full workload sizes, through the same entry points and
launch configurations the benchmark times.  Rotate+quantise codes and scales
are compared on every row; outputs (and INT32 accumulators) on sampled rows
that include the first and last rows and both sides of tile edges -- rows are
independent, so the oracle computes exactly those rows."""
import numpy as np
import pytest
import torch

import oracle
from w8a8_int8_rotated_amd import workloads as wl
from gpu_util import (announce, assert_output_parity, bf16_bits, dev, host, padded_rows,
                      sample_rows, tile,
                      to_dev, to_dev_bf16, untile)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cr():
    from w8a8_int8_rotated_amd import convrot
    convrot.library()
    return convrot


def _prep(cr, W, b):
    pw = cr.convrot_linear_prepare_weights(to_dev(W), b)
    q_ref, s_ref = oracle.prepare_weights(W, b)
    assert np.array_equal(untile(pw.codes, *q_ref.shape), q_ref), "weight codes"
    assert np.array_equal(host(pw.scale), s_ref), "weight scales"
    return pw, q_ref, s_ref


def test_qkv_38656_fullsize(cr):
    """M=38656, K=5376, N=16128, Student-t(4) activations, bf16 out."""
    w = wl.WORKLOADS["qkv_38656"]
    announce(w.description)
    x, W = w.activations(), w.weight()
    pw, qw, sw = _prep(cr, W, w.block)
    X = to_dev_bf16(x)
    y = cr.convrot_linear_forward(X, pw)
    qx, sx = cr.convrot_rotate_quantize(X, w.block)
    torch.cuda.synchronize()
    qx_ref, sx_ref = oracle.rotate_quantize(x, w.block, "bf16")
    assert np.array_equal(host(sx), sx_ref), "row scales, all rows"
    assert np.array_equal(untile(qx, w.M, w.K), qx_ref), "codes, all rows"
    rows = sample_rows(w.M, 64)
    y_ref = oracle.linear_forward(x[rows], qw, sw, w.block, out="bf16")
    yr = bf16_bits(y[torch.from_numpy(rows).cuda()])
    assert assert_output_parity(yr, y_ref, "bf16", "qkv_38656 sampled rows") == 0
    # INT32 accumulators from the full-size launch: one row in every 256-row
    # tile (at an offset that walks through the tile) plus the sampled rows
    acc = cr.convrot_gemm_i32(qx, w.M, pw)
    tiles = (w.M + 255) // 256
    per_tile = np.minimum(np.arange(tiles) * 256 + (np.arange(tiles) * 37) % 256, w.M - 1)
    arows = np.unique(np.concatenate([per_tile, rows]))
    got = host(acc[torch.from_numpy(arows).cuda()])
    del acc
    want = oracle.gemm_i32(qx_ref[arows], qw)
    bad = int(np.count_nonzero(got != want))
    print(f"[parity] qkv_38656 INT32: {bad} differ on {len(arows)} rows "
          f"(every one of {tiles} m-tiles)", flush=True)
    assert bad == 0


def test_lowrank_38656_fullsize(cr):
    """M=38656, K=5376 -> r=512 -> N=5376, 2% outlier channels x25."""
    w = wl.WORKLOADS["lowrank_38656"]
    announce(w.description)
    x, A, B = w.activations(), w.weight("w"), w.weight("w2")
    pa, qa, sa = _prep(cr, A, w.block)
    pb, qb, sb = _prep(cr, B, w.block)
    y = cr.lowrank_convrot_forward(to_dev_bf16(x), pa, pb)
    rows = sample_rows(w.M, 64)
    y_ref = oracle.lowrank_forward(x[rows], qa, sa, qb, sb, w.block, out="bf16")
    yr = bf16_bits(y[torch.from_numpy(rows).cuda()])
    assert assert_output_parity(yr, y_ref, "bf16", "lowrank_38656 sampled rows") == 0


def test_mlp_16384_fullsize(cr):
    """up M=16384 K=5376 N=21504, GELU, down K=21504 N=5376: bit-exact, since
    the device applies the oracle's GELU map (checked on all bf16 inputs)."""
    w = wl.WORKLOADS["mlp_16384"]
    announce(w.description)
    x, Wu, Wd = w.activations(), w.weight("w"), w.weight("w2")
    pu, qu, su = _prep(cr, Wu, w.block)
    pd, qd, sd = _prep(cr, Wd, w.block)
    y = cr.convrot_mlp_forward(to_dev_bf16(x), pu, pd)
    rows = sample_rows(w.M, 48)
    y_ref = oracle.mlp_forward(x[rows], qu, su, qd, sd, w.block, out="bf16")
    yr = bf16_bits(y[torch.from_numpy(rows).cuda()])
    assert assert_output_parity(yr, y_ref, "bf16", "mlp_16384 sampled rows") == 0


def test_qk_38656_small_k(cr):
    """Small-K GEMM at the attention QK shape (K = head_dim = 128, one Hadamard
    block per row): M = N = 38656, sampled output rows and INT32 rows."""
    w = wl.WORKLOADS["qk_38656"]
    announce(w.description)
    x, W = w.activations(), w.weight()
    pw, qw, sw = _prep(cr, W, w.block)
    X = to_dev_bf16(x)
    y = cr.convrot_linear_forward(X, pw)
    qx, sx = cr.convrot_rotate_quantize(X, w.block)
    torch.cuda.synchronize()
    qx_ref, sx_ref = oracle.rotate_quantize(x, w.block, "bf16")
    assert np.array_equal(untile(qx, w.M, w.K), qx_ref) and np.array_equal(host(sx), sx_ref)
    rows = sample_rows(w.M, 48)
    y_ref = oracle.linear_forward(x[rows], qw, sw, w.block, out="bf16")
    yr = bf16_bits(y[torch.from_numpy(rows).cuda()])
    assert assert_output_parity(yr, y_ref, "bf16", "qk_38656 sampled rows") == 0
    acc = cr.convrot_gemm_i32(to_dev(tile(qx_ref[rows[:8]])), 8, pw)
    assert np.array_equal(host(acc), oracle.gemm_i32(qx_ref[rows[:8]], qw))


def test_max_rows_32bit_offsets(cr):
    """The most rows the entry points accept at K = 5376: the padded code
    matrix is just under 2^31 bytes (M = 399449, ragged in its last 16-row
    block; M + 16 would pass 2^31 and is rejected).  N = 256, bf16 out.
    Codes and row scales of the sampled rows (the last 20 rows included) and
    their outputs against the oracle, so every 32-bit offset near the limit
    is exercised."""
    K, N, b = 5376, 256, 128
    M = 399449
    assert padded_rows(M) * K < 2**31 <= padded_rows(M + 16) * K
    announce(f"largest row count M={M} K={K} N={N} b={b}")
    # seeded N(0,1) activations drawn on the device in chunks (4.3 GB of
    # bf16), 1% of channels x30; the oracle gets the same bytes back
    gen = torch.Generator(device=dev()).manual_seed(0)
    X = torch.empty((M, K), dtype=torch.bfloat16, device=dev())
    for r0 in range(0, M, 65536):
        r1 = min(M, r0 + 65536)
        X[r0:r1] = torch.randn((r1 - r0, K), generator=gen, device=dev()).to(torch.bfloat16)
    hot = np.random.default_rng(1).choice(K, size=54, replace=False)
    X[:, torch.from_numpy(hot).to(dev())] *= 30
    W = np.random.default_rng(2).normal(0.0, 0.02, (N, K)).astype(np.float32)
    pw, qw, sw = _prep(cr, W, b)
    y = cr.convrot_linear_forward(X, pw)
    qx, sx = cr.convrot_rotate_quantize(X, b)
    torch.cuda.synchronize()
    rows = np.union1d(sample_rows(M, 64), np.arange(M - 20, M))
    rows_d = torch.from_numpy(rows).to(dev())
    x_rows = bf16_bits(X[rows_d])
    qx_ref, sx_ref = oracle.rotate_quantize(x_rows, b, "bf16")
    assert np.array_equal(host(sx[rows_d]), sx_ref), "row scales"
    blocks = host(qx.view(-1, 16 * K)[torch.from_numpy(rows // 16).to(dev())])
    got = np.stack([untile(blk, 16, K)[r % 16] for blk, r in zip(blocks, rows)])
    assert np.array_equal(got, qx_ref), "codes of the sampled rows"
    y_ref = oracle.linear_forward(x_rows, qw, sw, b, out="bf16")
    assert assert_output_parity(bf16_bits(y[rows_d]), y_ref, "bf16",
                                f"M={M} sampled rows") == 0


def test_max_rows_gelu_on_load(cr):
    """The MLP entry point at the most rows it accepts for F = 24576, the
    longest intermediate rows that rotquant applies GELU to as it loads them:
    the padded codes of g are just under 2^31 bytes (M = 87369, ragged in the
    last 16-row block), u is 4.3 GB.  Sampled outputs (the last 20 rows
    included) against the oracle."""
    K, F, N, b = 256, 24576, 160, 128
    M = 87369
    assert padded_rows(M) * F < 2**31 <= padded_rows(M + 16) * F
    announce(f"largest row count, GELU on load: M={M} K={K} F={F} N={N} b={b}")
    gen = torch.Generator(device=dev()).manual_seed(3)
    X = (torch.randn((M, K), generator=gen, device=dev()) * 2).to(torch.bfloat16)
    rng = np.random.default_rng(4)
    Wu = rng.normal(0.0, 0.06, (F, K)).astype(np.float32)
    Wd = rng.normal(0.0, 0.02, (N, F)).astype(np.float32)
    pu, qu, su = _prep(cr, Wu, b)
    pd, qd, sd = _prep(cr, Wd, b)
    y = cr.convrot_mlp_forward(X, pu, pd)
    torch.cuda.synchronize()
    rows = np.union1d(sample_rows(M, 48), np.arange(M - 20, M))
    rows_d = torch.from_numpy(rows).to(dev())
    y_ref = oracle.mlp_forward(bf16_bits(X[rows_d]), qu, su, qd, sd, b, out="bf16")
    assert assert_output_parity(bf16_bits(y[rows_d]), y_ref, "bf16",
                                f"MLP M={M} F={F} sampled rows") == 0


def test_swiglu_16384_fullsize(cr):
    """SwiGLU MLP M=16384, fc1 K=5376 -> 2 x 21504 (b=128), fc2 21504 -> 5376
    with ConvRot64: fc1 codes on every row, g and the outputs on sampled rows,
    in the launch configuration the benchmark times."""
    w = wl.WORKLOADS["swiglu_16384"]
    announce(w.description)
    x, Wgu, Wd = w.activations(), w.weight("w"), w.weight("w2")
    F = w.ffn
    pgu = cr.convrot_swiglu_prepare(to_dev(Wgu), w.block)
    p = np.arange(2 * F)
    perm = np.where(p % 32 < 16, (p // 32) * 16 + p % 32, F + (p // 32) * 16 + p % 32 - 16)
    qgu, sgu = oracle.prepare_weights(Wgu, w.block)
    assert np.array_equal(host(pgu.scale), sgu[perm])
    pd, qd, sd = _prep(cr, Wd, w.down_block)
    X = to_dev_bf16(x)
    y = cr.convrot_swiglu_mlp_forward(X, pgu, pd)
    qx, sx = cr.convrot_rotate_quantize(X, w.block)
    g = cr.convrot_gemm_dequant(qx, sx, pgu, swiglu=True)
    torch.cuda.synchronize()
    rows = sample_rows(w.M, 24)
    y_ref, gu_ref, g_ref = oracle.swiglu_mlp_forward(x[rows], qgu, sgu, qd, sd, w.block,
                                                     w.down_block, out="bf16",
                                                     return_intermediates=True)
    gr = bf16_bits(g[torch.from_numpy(rows).cuda()])
    assert np.array_equal(gr, g_ref), int(np.count_nonzero(gr != g_ref))
    yr = bf16_bits(y[torch.from_numpy(rows).cuda()])
    assert assert_output_parity(yr, y_ref, "bf16", "swiglu_16384 sampled rows") == 0
