"""Helpers shared by the GPU parity tests: host <-> device marshalling of the
raw bf16 bits and the comparison rules.

Comparison rules (what "parity" means here):
  * INT8 codes, row scales and INT32 accumulators: bit for bit.
  * Outputs: normwise max|y_gpu - y_oracle| / max|y_oracle| <= 1e-3 for bf16
    and <= 1e-5 for fp32 (an elementwise relative error is unbounded near
    zeros).  Both sides run the same fp32 epilogue, so equality is expected and
    the mismatch count is reported.
"""
import numpy as np
import torch

BF16_TOL = 1e-3
F32_TOL = 1e-5


def dev():
    return torch.device("cuda", 0)


def to_dev_bf16(u16: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16))
    return t.view(torch.bfloat16).to(dev())


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def as_f64(y, kind):
    if kind == "bf16":
        return (np.asarray(y, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(y, np.float32).astype(np.float64)


def normwise_err(y_gpu, y_ref, kind):
    a, b = as_f64(y_gpu, kind), as_f64(y_ref, kind)
    denom = np.max(np.abs(b))
    if denom == 0:
        return float(np.max(np.abs(a - b)))
    return float(np.max(np.abs(a - b)) / denom)


def assert_output_parity(y_gpu, y_ref, kind, what=""):
    tol = BF16_TOL if kind == "bf16" else F32_TOL
    err = normwise_err(y_gpu, y_ref, kind)
    mism = int(np.count_nonzero(np.asarray(y_gpu) != np.asarray(y_ref)))
    print(f"[parity] {what}: normwise err {err:.3e} (tol {tol:g}), "
          f"{mism} of {np.asarray(y_ref).size} elements differ", flush=True)
    assert err <= tol, f"{what}: normwise error {err} > {tol}"
    return mism


def sample_rows(M, n, seed=0, tile=256):
    """First and last rows, rows on both sides of every 4th tile boundary, and
    a seeded random set."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1}
    for b in range(tile, M, tile * 4):
        rows.update({b - 1, b})
    rows.update(rng.choice(M, size=min(n, M), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < M), dtype=np.int64)


def announce(msg):
    print(f"[case] {msg}", flush=True)
