"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test names what it pins: the textbook Sylvester matrix (scipy), exact
integer identities of the Hadamard transform, a hand-worked example
(tests/golden/hand_b4.json), the quantiser's invariants, a brute-force integer
contraction, fp64 evaluations of the float identity (W R^T)(R x) = W x, and
the textbook rotation-free W8A8 at b = 1.  A plausible slip in the oracle (a
dropped 1/sqrt(b), a wrong butterfly sign or stride, a transposed operand, a
truncating round) breaks at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from w8a8_int8_rotated_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32_EPS = np.float32(2.0 ** -24)


def dense_h(b):
    """Sylvester Hadamard from scipy (the library routine), as float64."""
    return scipy.linalg.hadamard(b).astype(np.float64)


def blockdiag_apply(v64, b):
    """fp64 dense R-free rotation: each length-b block -> H_b . block."""
    H = dense_h(b)
    K = v64.shape[-1]
    blocks = v64.reshape(v64.shape[:-1] + (K // b, b))
    return (blocks @ H.T).reshape(v64.shape)


# ------------------------------------------------------------- Hadamard ----

@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_columns_are_sylvester(b):
    """FWHT(e_i) is column i of the textbook Sylvester H_b (exact)."""
    cols = oracle.fwht(np.eye(b, dtype=np.float32), b)  # row i = FWHT(e_i)
    assert np.array_equal(cols.T.astype(np.float64), dense_h(b))


@pytest.mark.parametrize("b", [2, 4, 64, 128, 256])
def test_hadamard_orthogonality(b):
    """H . H^T = b . I exactly (integers), with H built by the oracle."""
    H = oracle.fwht(np.eye(b, dtype=np.float32), b).T.astype(np.int64)
    assert np.array_equal(H @ H.T, b * np.eye(b, dtype=np.int64))


@pytest.mark.parametrize("b", [64, 128, 256])
def test_fwht_involution_and_dc(b):
    rng = np.random.default_rng(1)
    v = rng.integers(-8, 9, size=(3, 4 * b)).astype(np.float32)
    twice = oracle.fwht(oracle.fwht(v, b), b)
    assert np.array_equal(twice, b * v)                    # H.H = b.I
    ones = oracle.fwht(np.ones((1, b), np.float32), b)[0]  # H.1 = b.e0
    expect = np.zeros(b, np.float32)
    expect[0] = b
    assert np.array_equal(ones, expect)


@pytest.mark.parametrize("b", [64, 128, 256])
def test_fwht_fp32_vs_fp64_dense(b):
    """fp32 butterflies stay within the summation bound of fp64 dense H.v;
    bf16 inputs of modest spread are exact in fp64."""
    rng = np.random.default_rng(2)
    x = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(
        rng.standard_normal((8, 2 * b)).astype(np.float32)))
    got = oracle.fwht(x, b).astype(np.float64)
    ref = blockdiag_apply(x.astype(np.float64), b)
    stages = int(math.log2(b))
    absx = np.abs(x.astype(np.float64)).reshape(8, -1, b).sum(-1)
    bound = stages * float(F32_EPS) * 1.01 * np.repeat(absx, b, axis=1)
    assert np.all(np.abs(got - ref) <= bound)
    # and at least some rounding actually happened somewhere in fp32 vs fp64
    # only when b is large; otherwise the two agree exactly
    assert np.max(np.abs(got - ref)) <= np.max(bound)


# ------------------------------------------ regular H_4 Kronecker blocks ----
# The Rung-Omega README ("Technical Architecture Overview", item 1) rotates
# with the regular ("DC-balanced") orthogonal H_256 = H_4 (x) H_4 (x) H_4 (x)
# H_4; the reading takes H_4 = J - 2I.  These pins build the matrix with
# numpy.kron, independently of the oracle's digit-by-digit transform.

def regular_h(b):
    H4 = np.ones((4, 4)) - 2.0 * np.eye(4)
    H = np.ones((1, 1))
    while H.shape[0] < b:
        H = np.kron(H, H4)
    return H


@pytest.mark.parametrize("b", [4, 16, 64, 256])
def test_regular_columns(b):
    """Transform of e_i is column i of the Kronecker power of J - 2I (exact)."""
    cols = oracle.fwht(np.eye(b, dtype=np.float32), b, rot="regular")
    assert np.array_equal(cols.T.astype(np.float64), regular_h(b))


@pytest.mark.parametrize("b", [4, 64, 256])
def test_regular_hadamard_properties(b):
    """H H^T = b I, H symmetric, every row sums to sqrt(b) (regular), the
    all-ones vector maps to sqrt(b) times itself (DC stays DC) and applying
    the transform twice gives b v, all exact."""
    H = oracle.fwht(np.eye(b, dtype=np.float32), b, rot="regular").T.astype(np.int64)
    assert np.array_equal(H @ H.T, b * np.eye(b, dtype=np.int64))
    assert np.array_equal(H, H.T)
    root = int(round(math.sqrt(b)))
    assert np.all(H.sum(axis=1) == root)
    ones = oracle.fwht(np.ones((1, 2 * b), np.float32), b, rot="regular")
    assert np.array_equal(ones, np.full((1, 2 * b), root, np.float32))
    rng = np.random.default_rng(b)
    v = rng.integers(-8, 9, size=(3, 2 * b)).astype(np.float32)
    twice = oracle.fwht(oracle.fwht(v, b, rot="regular"), b, rot="regular")
    assert np.array_equal(twice, b * v)


@pytest.mark.parametrize("b", [64, 256])
def test_regular_fp32_vs_fp64_dense(b):
    """fp32 digit stages stay within a rounding bound of the fp64 dense
    product: each stage adds at most 4 roundings of magnitude <= the block's
    L1 norm, and H_4 amplifies earlier errors at most 4-fold."""
    rng = np.random.default_rng(5)
    x = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(
        rng.standard_normal((8, 2 * b)).astype(np.float32)))
    got = oracle.fwht(x, b, rot="regular").astype(np.float64)
    H = regular_h(b)
    ref = (x.astype(np.float64).reshape(8, -1, b) @ H.T).reshape(8, -1)
    k = int(round(math.log(b, 4)))
    l1 = np.abs(x.astype(np.float64)).reshape(8, -1, b).sum(-1)
    bound = 4 * float(F32_EPS) * 1.01 * (4 ** k - 1) / 3 * np.repeat(l1, b, axis=1)
    assert np.all(np.abs(got - ref) <= bound)


def test_regular_rejects_orders_not_powers_of_four():
    with pytest.raises(ValueError):
        oracle.fwht(np.zeros((1, 128), np.float32), 128, rot="regular")
    with pytest.raises(ValueError):
        oracle.rotate_quantize(np.zeros((1, 128), np.float32), 128, "f32", rot="regular")


# --------------------------------------------------- hand-worked example ----

def _rat(p):
    return p[0] / p[1]


def test_golden_hand_example_b4():
    g = json.load(open(os.path.join(GOLDEN, "hand_b4.json")))
    b = g["block"]
    x = np.array([g["x"]], np.float32)
    W = np.array(g["W"], np.float32)
    assert np.array_equal(oracle.fwht(x, b)[0], np.array(g["x_rotated"], np.float32))
    assert np.array_equal(oracle.fwht(W, b), np.array(g["w_rotated"], np.float32))
    xb = wl.f32_to_bf16_bits(x)
    qx, sx = oracle.rotate_quantize(xb, b, "bf16")
    assert qx[0].tolist() == g["x_codes"]
    assert sx[0] == np.float32(_rat(g["x_scale"]))
    qw, sw = oracle.prepare_weights(W, b)
    assert qw.tolist() == g["w_codes"]
    assert [float(s) for s in sw] == [float(np.float32(_rat(p))) for p in g["w_scale"]]
    acc = oracle.gemm_i32(qx, qw)
    assert acc[0].tolist() == g["acc"]
    y = oracle.linear_forward(xb, qw, sw, b, out="f32")[0].astype(np.float64)
    exact = np.array([_rat(p) for p in g["y_no_bias"]])
    ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(y - exact) <= 4 * ulp)
    bias = np.array(g["bias"], np.float32)
    yb = oracle.linear_forward(xb, qw, sw, b, bias=bias, out="f32")[0]
    assert np.all(np.abs(yb - (exact + bias)) <= 8 * ulp + 1e-7)
    # zero row: codes 0, scale 0, output = bias
    z = np.zeros((1, 4), np.uint16)
    qz, sz = oracle.rotate_quantize(z, b, "bf16")
    assert not qz.any() and sz[0] == 0
    yz = oracle.linear_forward(z, qw, sw, b, bias=bias, out="f32")[0]
    assert np.array_equal(yz, bias)
    # float product for orientation: the quantised result is close to W x
    assert np.allclose(y, g["Wx_float"], atol=0.03)


def _hexf(xs):
    return np.array([float.fromhex(x) for x in xs], np.float32)


def test_golden_fwht_stage_order():
    """The butterfly association (reading: strides ascending, each stage
    rounded once in fp32) against the hand-worked vectors of
    tests/golden/fwht_order.json: with one input at 1 and others at 2^-24 the
    rounding of 1 + 2^-24 (a tie, to even) depends on which stage runs first,
    and only the ascending order gives the recorded bits."""
    g = json.load(open(os.path.join(GOLDEN, "fwht_order.json")))
    for case in g["cases"]:
        b = case["block"]
        v = _hexf(case["v"])[None, :]
        got = oracle.fwht(v, b)[0]
        want = _hexf(case["ascending"])
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (b, got, want)
        for other in ("descending", "order_1_4_2"):
            if other in case:
                assert not np.array_equal(got, _hexf(case[other]))


# ------------------------------------------------------------- quantiser ----

def _rand_rows(rng, rows, K, scale=1.0):
    return (rng.standard_normal((rows, K)) * scale).astype(np.float32)


def test_rowquant_invariants():
    rng = np.random.default_rng(3)
    b = 128
    v = _rand_rows(rng, 16, 512, 3.0)
    v[3, 17] = 40.0
    q, s = oracle.rowquant(v, b)
    # max |q| = 127 at the argmax of |v|
    am = np.argmax(np.abs(v), axis=1)
    assert np.all(np.abs(q).max(axis=1) == 127)
    assert np.all(np.abs(q[np.arange(16), am]) == 127)
    assert np.all(np.sign(q[np.arange(16), am]) == np.sign(v[np.arange(16), am]))
    # codes never -128
    assert q.min() >= -127
    # odd symmetry
    qn, sn = oracle.rowquant(-v, b)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # exact power-of-two equivariance
    for j in (-3, 5):
        q2, s2 = oracle.rowquant(v * np.float32(2.0 ** j), b)
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, s * np.float32(2.0 ** j))
    # rounding error at most one half unit of the grid
    amax = np.abs(v).max(axis=1, keepdims=True)
    inv = np.float32(127.0) / amax
    t = (v * inv).astype(np.float64)
    assert np.all(np.abs(t - q) <= 0.5)
    # the scale carries 1/sqrt(b): q*s*sqrt(b) reconstructs v within step/2
    step = (amax / np.float32(127.0)).astype(np.float64)
    recon = q * (s[:, None].astype(np.float64) * math.sqrt(b))
    assert np.all(np.abs(recon - v) <= step / 2 * (1 + 1e-5) + 1e-12)


def test_rowquant_rne_ties():
    """v*inv landing on .5 rounds to even, not away from zero."""
    v = np.array([[1.0, 0.5, -0.5, 2.5 / 127, 3.5 / 127]], np.float32)
    q, _ = oracle.rowquant(v, 1)
    # amax = 1 -> inv = 127: 0.5*127 = 63.5 -> 64; -63.5 -> -64; 2.5 -> 2; 3.5 -> 4
    t = v[0] * np.float32(127.0)
    assert q[0, 1] == 64 and q[0, 2] == -64
    assert q[0, 3] == np.rint(t[3]) and q[0, 4] == np.rint(t[4])


@pytest.mark.parametrize("b", [64, 128, 256])
def test_one_hot_closed_form(b):
    """A one-hot block rotates to a +-1 column of H: codes +-127 and
    scale = fp32(1/127) * fp32(1/sqrt b) for a unit spike."""
    x = np.zeros((1, 2 * b), np.float32)
    i = 5
    x[0, b + i] = 1.0
    q, s = oracle.rotate_quantize(wl.f32_to_bf16_bits(x), b, "bf16")
    H = dense_h(b)
    assert np.array_equal(q[0, :b], np.zeros(b, np.int8))
    assert np.array_equal(q[0, b:].astype(np.float64), 127 * H[:, i])
    assert s[0] == np.float32(np.float32(1.0) / np.float32(127.0)) * np.float32(1 / math.sqrt(b))


def test_zero_and_nonfinite_rows():
    x = np.zeros((2, 256), np.uint16)
    q, s = oracle.rotate_quantize(x, 128, "bf16")
    assert not q.any() and not s.any()
    bad = np.zeros((1, 128), np.float32)
    bad[0, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.rotate_quantize(bad, 128, "f32")


def test_b1_is_textbook_w8a8():
    """At b = 1 there is no rotation: per-token x per-channel symmetric W8A8,
    written here independently in numpy."""
    rng = np.random.default_rng(4)
    M, K, N = 9, 40, 7
    x = wl.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xf = wl.bf16_bits_to_f32(x)

    def textbook(a):
        amax = np.abs(a).max(axis=1, keepdims=True).astype(np.float32)
        q = np.clip(np.rint(a * (np.float32(127) / amax)), -127, 127).astype(np.int8)
        return q, (amax[:, 0] / np.float32(127)).astype(np.float32)

    qx_t, sx_t = textbook(xf)
    qw_t, sw_t = textbook(W)
    qx, sx = oracle.rotate_quantize(x, 1, "bf16")
    qw, sw = oracle.prepare_weights(W, 1)
    assert np.array_equal(qx, qx_t) and np.array_equal(sx, sx_t)
    assert np.array_equal(qw, qw_t) and np.array_equal(sw, sw_t)
    acc_t = qx_t.astype(np.int64) @ qw_t.astype(np.int64).T
    y_t = (acc_t.astype(np.float32) * sx_t[:, None]) * sw_t[None, :]
    y = oracle.linear_forward(x, qw, sw, 1, out="f32")
    assert np.array_equal(y, y_t.astype(np.float32))


# ----------------------------------------------------------------- GEMM ----

def test_gemm_brute_force_tiny():
    rng = np.random.default_rng(5)
    M, N, K = 5, 6, 64
    a = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    w = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    acc = oracle.gemm_i32(a, w)
    for m in range(M):
        for n in range(N):
            s = 0
            for k in range(K):
                s += int(a[m, k]) * int(w[n, k])
            assert acc[m, n] == s


def test_gemm_extremes_and_numpy():
    rng = np.random.default_rng(6)
    M, N, K = 16, 16, 512
    a = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    w = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    a[0] = 127
    w[0] = -127
    acc = oracle.gemm_i32(a, w)
    assert np.array_equal(acc, a.astype(np.int64) @ w.astype(np.int64).T)
    assert acc[0, 0] == -K * 127 * 127


def test_gemm_rejects_overflowing_k():
    with pytest.raises(ValueError):
        oracle.gemm_i32(np.zeros((1, 133144 + 128), np.int8),
                        np.zeros((1, 133144 + 128), np.int8))


# ----------------------------------------------------- dequant, bf16 out ----

def test_dequant_vs_fp64():
    rng = np.random.default_rng(7)
    M, N = 12, 10
    acc = rng.integers(-3_000_000, 3_000_000, size=(M, N)).astype(np.int32)
    sx = rng.uniform(1e-4, 1e-2, M).astype(np.float32)
    sw = rng.uniform(1e-5, 1e-3, N).astype(np.float32)
    bias = rng.normal(0, 0.01, N).astype(np.float32)
    y = oracle.dequant(acc, sx, sw, bias, out="f32").astype(np.float64)
    ref = acc.astype(np.float64) * sx[:, None] * sw[None, :] + bias[None, :]
    mag = np.abs(acc.astype(np.float64) * sx[:, None] * sw[None, :]) + np.abs(bias)
    assert np.all(np.abs(y - ref) <= 4 * float(F32_EPS) * mag)
    # bf16 output = RNE of the fp32 output, checked with torch's narrowing
    import torch
    y32 = oracle.dequant(acc, sx, sw, bias, out="f32")
    yb = oracle.dequant(acc, sx, sw, bias, out="bf16")
    tb = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, tb)


def test_bf16_narrowing_matches_torch():
    import torch
    rng = np.random.default_rng(8)
    vals = np.concatenate([
        rng.standard_normal(2000).astype(np.float32) * 1e3,
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.3895314e38, 1e-40, -1e-40,
                  1.00390625, 1.01171875, 1.0078125 + 2 ** -24], np.float32),
        # exact ties between neighbours: odd and even keep bits
        (np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80C000], np.uint32)
         .view(np.float32)),
    ])
    got = oracle.f32_to_bf16(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    assert np.array_equal(got, wl.f32_to_bf16_bits(vals))


# ------------------------------------------ float identities end to end ----

def _bound_linear(xf64, W64, b, sx, sw):
    """Closed-form bound of |y - W x| for the quantised product.

    With x~ = R x and w~ = R w (fp64), and grid steps dx = s_x*sqrt(b)... the
    dequantised rotated operands are q*s, each within s/2 (+fp32 butterfly
    rounding) of x~, w~.  |sum x^ w^ - sum x~ w~| <= sum(|x~| dw + |w~| dx +
    dx dw) with dx = s_x/2, dw = s_w/2 per element."""
    r = 1.0 / math.sqrt(b)
    xt = blockdiag_apply(xf64, b) * r            # [M, K]
    wt = blockdiag_apply(W64, b) * r             # [N, K]
    dx = sx.astype(np.float64)[:, None] / 2 * 1.0001 + 1e-30
    dw = sw.astype(np.float64)[:, None] / 2 * 1.0001 + 1e-30
    K = xf64.shape[1]
    # fp32 rotation rounding, relative to the operand magnitude
    rot_x = np.log2(b) * 2 ** -24 * np.abs(xf64).reshape(xf64.shape[0], -1, b).sum(-1).max(-1) * r
    rot_w = np.log2(b) * 2 ** -24 * np.abs(W64).reshape(W64.shape[0], -1, b).sum(-1).max(-1) * r
    dx = dx + rot_x[:, None]
    dw = dw + rot_w[:, None]
    bound = (np.abs(xt).sum(1)[:, None] * dw.T
             + dx * np.abs(wt).sum(1)[None, :]
             + K * dx * dw.T)
    return bound


@pytest.mark.parametrize("b,rot", [(64, "sylvester"), (128, "sylvester"), (256, "sylvester"),
                                   (64, "regular"), (256, "regular")])
def test_rotation_identity_end_to_end(b, rot):
    """(W R^T)(R x) = W x: the oracle's output stays within the closed-form
    quantisation bound of the fp64 product W x, and is far tighter than what a
    missing 1/sqrt(b), a sign slip or a transposed operand would give."""
    w = wl.scaled("tiny", M=24, K=512, N=40, block=b)
    x = w.activations()
    W = w.weight()
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    ref = xf @ W.astype(np.float64).T
    qw, sw = oracle.prepare_weights(W, b, rot=rot)
    qx, sx = oracle.rotate_quantize(x, b, "bf16", rot=rot)
    y = oracle.linear_forward(x, qw, sw, b, out="f32", rot=rot).astype(np.float64)
    bound = _bound_linear(xf, W.astype(np.float64), b, sx, sw)
    assert np.all(np.abs(y - ref) <= bound + 1e-6 * np.abs(ref))
    # the worst-case bound is loose; the typical error is what an 8-bit grid
    # on rotated operands gives (~1%), far below the O(1) relative error of a
    # missing 1/sqrt(b) (factor sqrt(b)), a butterfly sign slip or a swapped
    # operand
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 0.03, rel


def test_undo_rotation_recovers_weights():
    """Dequantise the codes and undo the rotation: R (q s) ~ w within
    sqrt(b) s / 2 per element (the exactness the MLX card relies on)."""
    b = 128
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((6, 512)) * 0.02).astype(np.float32)
    q, s = oracle.prepare_weights(W, b)
    deq = q.astype(np.float64) * s[:, None].astype(np.float64)
    back = blockdiag_apply(deq, b) / math.sqrt(b)
    tol = math.sqrt(b) * s[:, None].astype(np.float64) / 2 * 1.001
    assert np.all(np.abs(back - W) <= tol)


def test_in_major_equals_out_major():
    rng = np.random.default_rng(10)
    W = (rng.standard_normal((48, 256)) * 0.02).astype(np.float32)
    q1, s1 = oracle.prepare_weights(W, 128, layout="out_major")
    q2, s2 = oracle.prepare_weights(np.ascontiguousarray(W.T), 128, layout="in_major")
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    Wb = wl.f32_to_bf16_bits(W)
    q3, s3 = oracle.prepare_weights(Wb, 128, dtype="bf16")
    q4, s4 = oracle.prepare_weights(np.ascontiguousarray(Wb.T), 128, dtype="bf16",
                                    layout="in_major")
    assert np.array_equal(q3, q4) and np.array_equal(s3, s4)


def test_lowrank_vs_dense_fp64():
    """Low-rank chain: y ~ B A x in fp64, within the composed bound."""
    b = 128
    w = wl.scaled("lowrank_38656", M=16, K=512, N=384, rank=256)
    x = w.activations()
    A = w.weight("w")
    B = w.weight("w2")
    qa, sa = oracle.prepare_weights(A, b)
    qb, sb = oracle.prepare_weights(B, b)
    y, h = oracle.lowrank_forward(x, qa, sa, qb, sb, b, out="f32", return_h=True)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    h_ref = xf @ A.astype(np.float64).T
    _, sx = oracle.rotate_quantize(x, b, "bf16")
    bound_h = _bound_linear(xf, A.astype(np.float64), b, sx, sa)
    hf = wl.bf16_bits_to_f32(h).astype(np.float64)
    assert np.all(np.abs(hf - h_ref) <= bound_h + np.abs(h_ref) * 2 ** -8)
    # second factor: bound from the actual h, plus B times the h error
    _, sh = oracle.rotate_quantize(h, b, "bf16")
    bound_y = _bound_linear(hf, B.astype(np.float64), b, sh, sb)
    y_ref = xf @ A.astype(np.float64).T @ B.astype(np.float64).T
    prop = np.abs(hf - h_ref) @ np.abs(B.astype(np.float64)).T
    assert np.all(np.abs(y.astype(np.float64) - y_ref) <= bound_y + prop + 1e-6)


def test_lowrank_is_two_chained_linears_with_bias():
    """O8 as the composition the workload names: h = bf16(linear(X; A)) with
    no bias, then linear(h; B) with the bias, bit for bit (the bias belongs
    to the second factor only; both outputs checked)."""
    b = 128
    w = wl.scaled("lowrank_38656", M=12, K=256, N=192, rank=128)
    x = w.activations()
    qa, sa = oracle.prepare_weights(w.weight("w"), b)
    qb, sb = oracle.prepare_weights(w.weight("w2"), b)
    bias = np.random.default_rng(41).normal(0, 0.5, 192).astype(np.float32)
    h_ref = oracle.linear_forward(x, qa, sa, b, bias=None, out="bf16")
    for out in ("f32", "bf16"):
        y, h = oracle.lowrank_forward(x, qa, sa, qb, sb, b, bias=bias, out=out, return_h=True)
        assert np.array_equal(h, h_ref)
        y_ref = oracle.linear_forward(h_ref, qb, sb, b, bias=bias, out=out)
        assert np.array_equal(y, y_ref)
        # the bias is really there: without it every output moves
        y_nb = oracle.linear_forward(h_ref, qb, sb, b, bias=None, out=out)
        assert not np.array_equal(y, y_nb)


def test_lowrank_vs_dense_error_report():
    """The comparison the low-rank workload names: the W8A8 low-rank chain
    (A [r, K], B [N, r]) against the dense W8A8 linear with W = B A (formed in
    fp64, stored fp32, prepared like any weight), both against the fp64
    product W x on the same rows.  The dense path stays inside its
    closed-form bound; both normwise errors are reported and stay at the
    scale of INT8 quantisation (a few percent), the chain's larger by the
    requantisation of h."""
    b = 128
    w = wl.scaled("lowrank_38656", M=24, K=1024, N=384, rank=256)
    x = w.activations()
    A, B = w.weight("w"), w.weight("w2")
    W = (B.astype(np.float64) @ A.astype(np.float64)).astype(np.float32)
    qa, sa = oracle.prepare_weights(A, b)
    qb, sb = oracle.prepare_weights(B, b)
    qw, sw = oracle.prepare_weights(W, b)
    y_lr = oracle.lowrank_forward(x, qa, sa, qb, sb, b, out="f32").astype(np.float64)
    y_d = oracle.linear_forward(x, qw, sw, b, out="f32").astype(np.float64)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    y64 = xf @ W.astype(np.float64).T
    _, sx = oracle.rotate_quantize(x, b, "bf16")
    bound = _bound_linear(xf, W.astype(np.float64), b, sx, sw)
    assert np.all(np.abs(y_d - y64) <= bound + np.abs(y64) * 2.0 ** -22)
    norm = lambda e: float(np.linalg.norm(e) / np.linalg.norm(y64))
    e_d, e_lr, e_between = norm(y_d - y64), norm(y_lr - y64), norm(y_lr - y_d)
    print(f"[report] normwise error vs fp64 W x: dense {e_d:.4f}, low-rank {e_lr:.4f}; "
          f"low-rank vs dense {e_between:.4f}")
    assert e_d < 0.03 and e_lr < 0.05 and e_d < e_lr


def test_lowrank_rejects_bad_rank():
    q = np.zeros((100, 128), np.int8)
    s = np.ones(100, np.float32)
    qb = np.zeros((8, 100), np.int8)
    with pytest.raises(ValueError):
        oracle.lowrank_forward(np.zeros((2, 128), np.uint16), q, s, qb,
                               np.ones(8, np.float32), 128)


# ----------------------------------------------------------------- GELU ----

def test_lowrank_bf16_variant_vs_numpy():
    """R9: the bf16 low-rank variant equals numpy's fp64 matmul of the same
    bf16 values, rounded to fp32 (plus bias) and then to bf16 by the
    workloads module's independent RNE narrowing; products of bf16 values and
    their sums are exact in fp64 at these exponent ranges."""
    rng = np.random.default_rng(17)
    M, K, r, N = 7, 256, 64, 48
    to_b = lambda a: wl.f32_to_bf16_bits(a.astype(np.float32))
    X = to_b(rng.standard_normal((M, K)))
    A = to_b(rng.standard_normal((r, K)) * 0.05)
    B = to_b(rng.standard_normal((N, r)) * 0.05)
    bias = rng.normal(0, 0.01, N).astype(np.float32)
    y, h = oracle.lowrank_bf16_forward(X, A, B, bias, return_h=True)
    f = lambda u: wl.bf16_bits_to_f32(u).astype(np.float64)
    h_ref = to_b((f(X) @ f(A).T).astype(np.float32))
    assert np.array_equal(h, h_ref)
    y_ref = to_b((f(h_ref) @ f(B).T).astype(np.float32) + bias)
    assert np.array_equal(y, y_ref)


def test_gelu_values():
    assert oracle.gelu_f64(0.0) == 0.0
    for z in (-3.0, -1.0, -0.25, 0.5, 1.0, 2.0, 7.0):
        ref = 0.5 * z * (1 + math.erf(z / math.sqrt(2)))
        assert abs(oracle.gelu_f64(z) - ref) <= 4e-16 * max(1, abs(z))
    assert abs(oracle.gelu_f64(1.0) - 0.8413447460685429) < 1e-15
    assert oracle.gelu_f64(40.0) == 40.0 and oracle.gelu_f64(-40.0) == -0.0


def test_gelu_bf16_and_mlp_chain():
    b = 128
    w = wl.scaled("mlp_16384", M=8, K=256, N=128, ffn=256)
    x = w.activations()
    Wu, Wd = w.weight("w"), w.weight("w2")
    qu, su = oracle.prepare_weights(Wu, b)
    qd, sd = oracle.prepare_weights(Wd, b)
    y, u, g = oracle.mlp_forward(x, qu, su, qd, sd, b, out="f32",
                                 return_intermediates=True)
    uf = wl.bf16_bits_to_f32(u).astype(np.float64)
    ref_g = 0.5 * uf * (1 + np.vectorize(math.erf)(uf / math.sqrt(2)))
    gf = wl.bf16_bits_to_f32(g).astype(np.float64)
    # g is the bf16 rounding of the exact GELU: within half a bf16 ulp
    assert np.all(np.abs(gf - ref_g) <= np.abs(ref_g) * 2 ** -8 + 1e-38)
    # the down projection of the oracle equals a linear on g
    y2 = oracle.linear_forward(g, qd, sd, b, out="f32")
    assert np.array_equal(y, y2)


def test_mlp_is_two_biased_linears_around_gelu():
    """O9 as a composition: u = bf16(linear(X; W_up) + bias_up), g =
    bf16(GELU(u)), y = linear(g; W_down) + bias_down, bit for bit, each bias
    on its own projection."""
    b = 128
    w = wl.scaled("mlp_16384", M=9, K=256, N=128, ffn=256)
    x = w.activations()
    qu, su = oracle.prepare_weights(w.weight("w"), b)
    qd, sd = oracle.prepare_weights(w.weight("w2"), b)
    rng = np.random.default_rng(43)
    bu = rng.normal(0, 0.5, 256).astype(np.float32)
    bd = rng.normal(0, 0.5, 128).astype(np.float32)
    y, u, g = oracle.mlp_forward(x, qu, su, qd, sd, b, bias_up=bu, bias_down=bd, out="f32",
                                 return_intermediates=True)
    u_ref = oracle.linear_forward(x, qu, su, b, bias=bu, out="bf16")
    assert np.array_equal(u, u_ref)
    assert not np.array_equal(u, oracle.linear_forward(x, qu, su, b, out="bf16"))
    assert np.array_equal(g, oracle.gelu_bf16(u_ref))
    y_ref = oracle.linear_forward(g, qd, sd, b, bias=bd, out="f32")
    assert np.array_equal(y, y_ref)
    assert not np.array_equal(y, oracle.linear_forward(g, qd, sd, b, out="f32"))


# ---------------------------------------------------------------- SwiGLU ----

def test_silu_values():
    """R10's activation against scipy's logistic function: silu(z) =
    z * expit(z) within two fp64 ulps, silu(0) = 0 with the sign of zero,
    and the odd-part identity silu(z) - silu(-z) = z."""
    import scipy.special
    zs = [-200.0, -40.0, -3.0, -1.0, -0.25, -1e-9, 1e-9, 0.5, 1.0, 2.0, 7.0, 40.0, 200.0]
    for z in zs:
        ref = z * scipy.special.expit(z)
        assert abs(oracle.silu_f64(z) - ref) <= 2 * np.spacing(abs(ref)) + 1e-300, z
        assert abs((oracle.silu_f64(z) - oracle.silu_f64(-z)) - z) <= 4e-16 * max(1.0, abs(z))
    assert oracle.silu_f64(0.0) == 0.0 and math.copysign(1.0, oracle.silu_f64(-0.0)) == -1.0
    assert abs(oracle.silu_f64(1.0) - 0.7310585786300049) < 1e-16


def test_silu_f32_every_bf16_pattern():
    """The fp32 activation of every finite bf16 gate equals fp32(z *
    expit(z)) from scipy, and the closed forms that bound it: z/2 for
    |z| < 2^-24, z for z >= 32, -0 for z <= -128."""
    import scipy.special
    a = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s = oracle.silu_f32(a)
    z = wl.bf16_bits_to_f32(a)
    fin = np.isfinite(z)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = (z.astype(np.float64) * scipy.special.expit(z.astype(np.float64))).astype(np.float32)
    assert np.array_equal(s[fin].view(np.uint32), ref[fin].view(np.uint32))
    tiny = fin & (np.abs(z) < 2.0 ** -24)
    assert np.array_equal(s[tiny].view(np.uint32), (z[tiny] * np.float32(0.5)).view(np.uint32))
    big = fin & (z >= 32)
    assert np.array_equal(s[big], z[big])
    neg = fin & (z <= -128)
    assert np.all(s[neg].view(np.uint32) == 0x80000000)


def test_swiglu_bf16_composition():
    """g = bf16(fp32(silu(gate)) * up) with the gate in the first half of the
    fc1 output and the up projection in the second, against scipy's logistic,
    numpy's fp32 product and the input recipe's RNE narrowing."""
    import scipy.special
    rng = np.random.default_rng(51)
    M, F = 7, 96
    gu = wl.f32_to_bf16_bits((rng.standard_normal((M, 2 * F)) * 3).astype(np.float32))
    gate = wl.bf16_bits_to_f32(gu[:, :F]).astype(np.float64)
    up = wl.bf16_bits_to_f32(gu[:, F:])
    s32 = (gate * scipy.special.expit(gate)).astype(np.float32)
    ref = wl.f32_to_bf16_bits(s32 * up)
    g = oracle.swiglu_bf16(gu)
    assert np.array_equal(g, ref)
    # up = 1 passes the activation through (rounded to bf16)
    gu1 = gu.copy()
    gu1[:, F:] = 0x3F80
    assert np.array_equal(oracle.swiglu_bf16(gu1), wl.f32_to_bf16_bits(s32))


def test_swiglu_mlp_is_linear_swiglu_linear():
    """R10 as a composition: gu = bf16(linear(X; W_gu) + bias_gu) with the
    fc1 block, g = swiglu(gu), y = linear(g; W_down) + bias_down with the fc2
    block (64, ConvRot64), bit for bit."""
    w = wl.scaled("swiglu_16384", M=9, K=256, N=128, ffn=256)
    x = w.activations()
    qgu, sgu = oracle.prepare_weights(w.weight("w"), w.block)
    qd, sd = oracle.prepare_weights(w.weight("w2"), w.down_block)
    rng = np.random.default_rng(53)
    bu = rng.normal(0, 0.5, 2 * w.ffn).astype(np.float32)
    bd = rng.normal(0, 0.5, w.N).astype(np.float32)
    y, gu, g = oracle.swiglu_mlp_forward(x, qgu, sgu, qd, sd, w.block, w.down_block,
                                         bias_gu=bu, bias_down=bd, out="f32",
                                         return_intermediates=True)
    gu_ref = oracle.linear_forward(x, qgu, sgu, w.block, bias=bu, out="bf16")
    assert np.array_equal(gu, gu_ref)
    assert np.array_equal(g, oracle.swiglu_bf16(gu_ref))
    y_ref = oracle.linear_forward(g, qd, sd, w.down_block, bias=bd, out="f32")
    assert np.array_equal(y, y_ref)
    # the second projection's own block matters: with b = 128 the codes differ
    qd2, sd2 = oracle.prepare_weights(w.weight("w2"), 128)
    assert not np.array_equal(y, oracle.linear_forward(g, qd2, sd2, 128, bias=bd, out="f32"))
