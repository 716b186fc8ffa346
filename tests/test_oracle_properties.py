"""Property tests of the oracle (hypothesis, CPU only): the same invariants
as the fixed-example pins, over generated shapes, blocks, rotation kinds and
values.  Each property follows from the mathematics, not from the oracle's
own code: the Hadamard blocks are involutions up to b, the quantiser commutes
with sign flips and powers of two, integer sums are exact, and rows are
independent.  Derandomized, so every run checks the same examples."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])

blocks = st.sampled_from([2, 4, 8, 16, 32, 64, 128, 256])
seeds = st.integers(0, 2**32 - 1)


@SETTINGS
@given(b=blocks, nblk=st.integers(1, 4), seed=seeds,
       rot=st.sampled_from(["sylvester", "regular"]))
def test_rotation_twice_is_b_times_identity(b, nblk, seed, rot):
    """H_b . H_b = b I for both kinds (Sylvester: symmetric with H H^T = b I;
    regular: H_4 = J - 2I is symmetric with H_4^2 = 4 I); exact on small
    integers."""
    if rot == "regular" and b not in (4, 16, 64, 256):
        return
    v = np.random.default_rng(seed).integers(-8, 9, (3, nblk * b)).astype(np.float32)
    w = oracle.fwht(oracle.fwht(v, b, rot), b, rot)
    assert np.array_equal(w, np.float32(b) * v)


@SETTINGS
@given(b=st.sampled_from([64, 128, 256]), k=st.integers(1, 6), j=st.integers(-20, 20),
       seed=seeds, spread=st.floats(0.0, 6.0))
def test_quantiser_sign_and_power_of_two(b, k, j, seed, spread):
    """q(-v) = -q(v) with the same scale; q(2^j v) = q(v), s(2^j v) = 2^j s(v);
    max |q| = 127 unless the row is zero; |v inv - q| <= 1/2."""
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal((4, k * b)) * np.exp2(rng.uniform(-spread, spread, (4, k * b))))
    v = v.astype(np.float32)
    q, s = oracle.rowquant(v, b)
    qn, sn = oracle.rowquant(-v, b)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    p = np.float32(2.0 ** j)
    q2, s2 = oracle.rowquant(v * p, b)
    assert np.array_equal(q2, q) and np.array_equal(s2, s * p)
    assert np.all(np.abs(q).max(axis=1) == 127) and q.min() >= -127
    inv = np.float32(127.0) / np.abs(v).max(axis=1, keepdims=True)
    assert np.all(np.abs((v * inv).astype(np.float64) - q) <= 0.5)


@SETTINGS
@given(M=st.integers(1, 9), N=st.integers(1, 9), K=st.integers(1, 300), seed=seeds)
def test_int32_contraction_is_exact(M, N, K, seed):
    """acc equals the int64 matrix product of the codes (|acc| stays far
    below 2^31 here), including the extreme codes +-127."""
    rng = np.random.default_rng(seed)
    qx = rng.integers(-127, 128, (M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, (N, K)).astype(np.int8)
    qx[0, :] = 127
    qw[0, :] = -127
    acc = oracle.gemm_i32(qx, qw)
    assert np.array_equal(acc.astype(np.int64), qx.astype(np.int64) @ qw.astype(np.int64).T)


@SETTINGS
@given(M=st.integers(2, 40), cut=st.integers(1, 39), b=st.sampled_from([64, 128]),
       out=st.sampled_from(["bf16", "f32"]), seed=seeds)
def test_forward_rows_are_independent(M, cut, b, out, seed):
    """Per-token scales make every output row a function of its input row
    only: forward(X)[a:] == forward(X[a:]) bit for bit."""
    cut = min(cut, M - 1)
    rng = np.random.default_rng(seed)
    K, N = 2 * b, 32
    x = oracle.f32_to_bf16(rng.standard_normal((M, K)).astype(np.float32) * 3)
    W = rng.normal(0, 0.05, (N, K)).astype(np.float32)
    qw, sw = oracle.prepare_weights(W, b)
    y = oracle.linear_forward(x, qw, sw, b, out=out)
    y2 = oracle.linear_forward(x[cut:], qw, sw, b, out=out)
    assert np.array_equal(y[cut:], y2)
