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


# The library's INT8 code matrices are K-tiled: code (m, k) at byte
#   ((m // 16) * (K // 64) + k // 64) * 1024 + (m % 16) * 64
#     + (((k // 16) % 4) ^ ((m // 4) % 4)) * 16 + k % 16
# of a buffer of Mp * K bytes, Mp = M rounded up to 16 (the public header's
# definition, restated here so the tests check the kernels against it).

def padded_rows(M: int) -> int:
    return (M + 15) // 16 * 16


def tiled_index(M: int, K: int) -> np.ndarray:
    m = np.arange(M, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    return (((m // 16) * (K // 64) + k // 64) * 1024 + (m % 16) * 64
            + (((k // 16) % 4) ^ ((m // 4) % 4)) * 16 + k % 16)


def _chunk_perm():
    # slot of chunk c in tile row r: c ^ ((r // 4) % 4)
    return np.array([[c ^ ((r // 4) % 4) for c in range(4)] for r in range(16)])


def untile(buf, M: int, K: int) -> np.ndarray:
    """Row-major [M, K] codes from a K-tiled buffer (device tensor or array).
    Same map as tiled_index, done on the (block, K-tile, row, slot, byte)
    view so that full-size matrices need no index array."""
    if isinstance(buf, torch.Tensor):
        buf = host(buf)
    Mp = padded_rows(M)
    b = np.asarray(buf).reshape(-1)[:Mp * K].reshape(Mp // 16, K // 64, 16, 4, 16)
    r = np.arange(16)[:, None]
    rows = b[:, :, r, _chunk_perm(), :]                # [block, ktile, row, chunk, byte]
    return rows.transpose(0, 2, 1, 3, 4).reshape(Mp, K)[:M]


def tile(q: np.ndarray) -> np.ndarray:
    """The K-tiled buffer (Mp, K) of row-major codes q [M, K]; padding rows 0."""
    M, K = q.shape
    Mp = padded_rows(M)
    full = np.zeros((Mp, K), dtype=np.int8)
    full[:M] = q
    rows = full.reshape(Mp // 16, 16, K // 64, 4, 16).transpose(0, 2, 1, 3, 4)
    out = np.empty_like(rows)                          # [block, ktile, row, slot, byte]
    out[:, :, np.arange(16)[:, None], _chunk_perm(), :] = rows
    return out.reshape(Mp, K)


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
