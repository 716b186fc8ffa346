"""Seeded synthetic inputs for the ConvRot W8A8 linear workloads.

This module only draws random numbers and narrows them to the storage types
the layer takes (bf16 activations by round-to-nearest-even, fp32 weights and
bias).  It holds none of the method's arithmetic and is shared by the tests,
the benchmark and the smoke check, so that the HIP path and the CPU oracle see
the same bytes.

Shapes follow the pages: hidden size K = 5376 (mmh3turbo README, "Why it is
fast, and where it is not": the K of the fast INT8 GEMM) and the packed
sequence of T = 38656 tokens at 768p (same section).  The heavy-tailed and
outlier-channel activations stand in for a residual stream whose magnitude
reaches ~2.4e5 (HyperFlow H3 Flash MLX card, "Where the weights come from").

Every tensor has its own PCG64 stream from ``SeedSequence(seed).spawn``.
"""
from __future__ import annotations

import dataclasses

import numpy as np

_STREAMS = ("x", "outliers", "w", "w2", "bias", "bias2")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Narrow fp32 to raw bf16 bits, round to nearest even (input recipe)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rngs(seed: int):
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(k)) for name, k in zip(_STREAMS, kids)}


@dataclasses.dataclass
class Workload:
    name: str
    kind: str                 # "linear" | "lowrank" | "mlp" | "swiglu"
    M: int
    K: int
    N: int
    block: int
    out: str                  # "bf16" | "f32"
    x_dist: str               # "normal" | "student_t4"
    outlier_frac: float = 0.0
    outlier_count: int = 0
    outlier_gain: float = 1.0
    w_std: float = 0.02
    bias_std: float | None = None
    rank: int = 0             # low-rank r
    ffn: int = 0              # MLP hidden width
    block2: int = 0           # block of the second projection (0: same as block)
    seed: int = 0
    description: str = ""

    def n_outliers(self) -> int:
        if self.outlier_count:
            return self.outlier_count
        return int(round(self.outlier_frac * self.K))

    # -------------------------------------------------------------- X ----
    def activations(self, rows: int | None = None, chunk: int = 4096) -> np.ndarray:
        """bf16 bits [M, K] (or the first ``rows`` rows)."""
        M = self.M if rows is None else min(rows, self.M)
        g = _rngs(self.seed)
        out = np.empty((M, self.K), dtype=np.uint16)
        n_out = self.n_outliers()
        cols = (np.sort(g["outliers"].choice(self.K, n_out, replace=False))
                if n_out else np.zeros(0, dtype=np.int64))
        for r0 in range(0, M, chunk):
            r1 = min(M, r0 + chunk)
            if self.x_dist == "normal":
                x = g["x"].standard_normal((r1 - r0, self.K), dtype=np.float32)
            elif self.x_dist == "student_t4":
                x = g["x"].standard_t(4.0, size=(r1 - r0, self.K)).astype(np.float32)
            else:
                raise ValueError(self.x_dist)
            if n_out:
                x[:, cols] *= np.float32(self.outlier_gain)
            out[r0:r1] = f32_to_bf16_bits(x)
        return out

    def outlier_channels(self) -> np.ndarray:
        g = _rngs(self.seed)
        n_out = self.n_outliers()
        if not n_out:
            return np.zeros(0, dtype=np.int64)
        return np.sort(g["outliers"].choice(self.K, n_out, replace=False))

    # -------------------------------------------------------- weights ----
    def weight(self, which: str = "w", shape=None) -> np.ndarray:
        """fp32 Gaussian weight, output-major [out, in]."""
        g = _rngs(self.seed)
        if shape is None:
            shape = self._weight_shape(which)
        return g[which].normal(0.0, self.w_std, size=shape).astype(np.float32)

    def _weight_shape(self, which):
        if self.kind == "linear":
            return (self.N, self.K)
        if self.kind == "lowrank":
            return (self.rank, self.K) if which == "w" else (self.N, self.rank)
        if self.kind == "mlp":
            return (self.ffn, self.K) if which == "w" else (self.N, self.ffn)
        if self.kind == "swiglu":
            # fc1 holds the gate (first ffn outputs) and the up projection
            return (2 * self.ffn, self.K) if which == "w" else (self.N, self.ffn)
        raise ValueError(self.kind)

    @property
    def down_block(self) -> int:
        return self.block2 or self.block

    def bias(self, which: str = "bias", n: int | None = None) -> np.ndarray | None:
        if self.bias_std is None:
            return None
        g = _rngs(self.seed)
        return g[which].normal(0.0, self.bias_std, size=(n or self.N,)).astype(np.float32)

    # ----------------------------------------------------------- cost ----
    def ops(self) -> int:
        """Algorithmic integer ops (2 per multiply-add) of one forward."""
        if self.kind == "linear":
            return 2 * self.M * self.N * self.K
        if self.kind == "lowrank":
            return 2 * self.M * self.rank * (self.K + self.N)
        if self.kind == "mlp":
            return 2 * self.M * self.ffn * (self.K + self.N)
        if self.kind == "swiglu":
            return 2 * self.M * self.ffn * (2 * self.K + self.N)
        raise ValueError(self.kind)


WORKLOADS = {
    "tiny": Workload(
        "tiny", "linear", M=256, K=512, N=512, block=128, out="f32",
        x_dist="normal", outlier_count=4, outlier_gain=20.0, w_std=0.02,
        description="tiny ConvRot linear M=256 K=512 N=512 b=128, fp32 out"),
    "linear_4096": Workload(
        "linear_4096", "linear", M=4096, K=5376, N=5376, block=128, out="bf16",
        x_dist="normal", outlier_frac=0.01, outlier_gain=30.0, w_std=0.02,
        bias_std=0.01,
        description="ConvRot linear M=4096 K=5376 N=5376 b=128, bf16 out + fp32 bias"),
    "qkv_38656": Workload(
        "qkv_38656", "linear", M=38656, K=5376, N=16128, block=128, out="bf16",
        x_dist="student_t4", w_std=0.02,
        description="fused QKV-shaped ConvRot linear M=38656 K=5376 N=16128 b=128, "
                    "Student-t(4) activations, bf16 out"),
    "mlp_16384": Workload(
        "mlp_16384", "mlp", M=16384, K=5376, N=5376, ffn=21504, block=128,
        out="bf16", x_dist="normal", w_std=0.02,
        description="MLP pair up M=16384 K=5376 N=21504, GELU, down K=21504 N=5376"),
    "swiglu_16384": Workload(
        "swiglu_16384", "swiglu", M=16384, K=5376, N=5376, ffn=21504, block=128, block2=64,
        out="bf16", x_dist="normal", w_std=0.02,
        description="SwiGLU MLP: fc1 M=16384 K=5376 N=2x21504 (gate | up) b=128, "
                    "g = silu(gate) * up, fc2 K=21504 N=5376 with ConvRot64 (b=64)"),
    "qk_38656": Workload(
        "qk_38656", "linear", M=38656, K=128, N=38656, block=128, out="bf16",
        x_dist="normal", w_std=0.02,
        description="small-K INT8 GEMM at the attention QK shape: T=38656 tokens, "
                    "head_dim K=128, b=128, bf16 out"),
    "lowrank_38656": Workload(
        "lowrank_38656", "lowrank", M=38656, K=5376, N=5376, rank=512, block=128,
        out="bf16", x_dist="normal", outlier_frac=0.02, outlier_gain=25.0,
        w_std=0.02,
        description="low-rank ConvRot linear M=38656 K=5376 r=512 N=5376"),
}


def scaled(name: str, **overrides) -> Workload:
    """A copy of a named workload with some fields replaced (smaller M, ...)."""
    return dataclasses.replace(WORKLOADS[name], **overrides)
