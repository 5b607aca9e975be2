"""Seeded synthetic inputs for the rotate->quantize->W4A4 linear path.

This module is shared by the CPU oracle side (tests, the bench's CPU leg) and
the HIP side (tests, bench). It holds none of the method's arithmetic: it only
draws random numbers and rounds them once to bfloat16, which is how every
input of the path is stored. Nothing here rotates, scales or quantizes.

Every tensor is drawn with NumPy's ``default_rng(SeedSequence([cfg, tensor]))``
where ``tensor`` is 0 for X, 1 for W, 2 for the outlier-channel choice and 3
for the per-channel scales. Samples are drawn in float32 and rounded to bf16
round-to-nearest-even, so the same bf16 bits feed both sides.

The workloads follow the shapes and value models of the MR-GPTQ FP4 inference
setting (activations with heavy tails and outlier channels, weights with a
small standard deviation):

=========  ==========================================================  =====
name       X (bf16)                                                     W
=========  ==========================================================  =====
tiny       16x256 N(0,1), 4 outlier channels x50                        256x256 N(0,0.02)
decode     M in {1,4,16} x 4096, Student-t(5), 1% channels x30           4096x4096 N(0,0.02)
           (decode_wide: the same X against W 14336x4096; decode_wide32/64/128: 32, 64
           and 128 rows, a batch of sequences decoding together; decode_nv_wide1/16/64/128:
           NVFP4 block 16 against W 14336x4096)
prefill    2048x4096, Student-t(5), 1% channels x30                      14336x4096 N(0,0.02)
           (NVFP4 block 16 as stated; also run in MXFP4 block 32, Y bf16)
large      8192x8192 N(0,1), 0.5% channels x100                          28672x8192 N(0,0.02)
stress     16384x8192 Student-t(3) x exp(N(0,1)) per channel            (none)
=========  ==========================================================  =====
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "draw_x",
    "draw_w",
    "draw_signs",
]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 samples to bfloat16 (round-to-nearest-even) -> uint16 bits.

    Inputs are finite by construction; no NaN handling is needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to float32 (exact), for display and generator checks."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    M: int
    K: int
    N: int  # 0: no weight (rotate+quantize only)
    block: int  # Hadamard block size along K
    fmt: str  # "mxfp4" | "nvfp4"
    x_dist: str  # "normal" | "t5" | "t3_lognormal"
    outlier_frac: float  # fraction of K channels that are outliers (or an absolute count if >= 1)
    outlier_mult: float
    w_std: float = 0.02
    out_dtype: str = "f32"  # GEMM output dtype

    def n_outliers(self) -> int:
        if self.outlier_frac >= 1:
            return int(self.outlier_frac)
        return int(round(self.outlier_frac * self.K))


WORKLOADS = {
    "tiny": Workload("tiny", 1, 16, 256, 256, 32, "mxfp4", "normal", 4, 50.0),
    "decode1": Workload("decode1", 2, 1, 4096, 4096, 32, "mxfp4", "t5", 0.01, 30.0),
    "decode4": Workload("decode4", 2, 4, 4096, 4096, 32, "mxfp4", "t5", 0.01, 30.0),
    "decode16": Workload("decode16", 2, 16, 4096, 4096, 32, "mxfp4", "t5", 0.01, 30.0),
    "prefill_nv": Workload("prefill_nv", 3, 2048, 4096, 14336, 16, "nvfp4", "t5", 0.01, 30.0,
                           out_dtype="bf16"),
    # The prefill shape (K=4096, N=14336) run in MXFP4 with Hadamard block 32, the same
    # activation model and the same output convention (float32 accumulation, bf16 Y):
    # the headline linear-layer workload.
    "prefill_mx": Workload("prefill_mx", 6, 2048, 4096, 14336, 32, "mxfp4", "t5", 0.01, 30.0,
                           out_dtype="bf16"),
    "prefill_mx_m4096": Workload("prefill_mx_m4096", 7, 4096, 4096, 14336, 32, "mxfp4", "t5",
                                 0.01, 30.0, out_dtype="bf16"),
    # decode against the wider projection of the prefill layer (W 14336 x 4096, 31 MB of MXFP4)
    "decode_wide1": Workload("decode_wide1", 8, 1, 4096, 14336, 32, "mxfp4", "t5", 0.01, 30.0),
    "decode_wide4": Workload("decode_wide4", 8, 4, 4096, 14336, 32, "mxfp4", "t5", 0.01, 30.0),
    "decode_wide16": Workload("decode_wide16", 8, 16, 4096, 14336, 32, "mxfp4", "t5", 0.01, 30.0),
    "decode_wide32": Workload("decode_wide32", 8, 32, 4096, 14336, 32, "mxfp4", "t5", 0.01, 30.0),
    "decode_wide64": Workload("decode_wide64", 8, 64, 4096, 14336, 32, "mxfp4", "t5", 0.01, 30.0),
    "decode_wide128": Workload("decode_wide128", 8, 128, 4096, 14336, 32, "mxfp4", "t5", 0.01, 30.0),
    "decode_nv_wide1": Workload("decode_nv_wide1", 8, 1, 4096, 14336, 16, "nvfp4", "t5", 0.01, 30.0),
    "decode_nv_wide16": Workload("decode_nv_wide16", 8, 16, 4096, 14336, 16, "nvfp4", "t5", 0.01, 30.0),
    "decode_nv_wide64": Workload("decode_nv_wide64", 8, 64, 4096, 14336, 16, "nvfp4", "t5", 0.01, 30.0),
    "decode_nv_wide128": Workload("decode_nv_wide128", 8, 128, 4096, 14336, 16, "nvfp4", "t5", 0.01, 30.0),
    "large": Workload("large", 4, 8192, 8192, 28672, 128, "mxfp4", "normal", 0.005, 100.0),
    "stress_mx32": Workload("stress_mx32", 5, 16384, 8192, 0, 32, "mxfp4", "t3_lognormal", 0, 1.0),
    "stress_mx128": Workload("stress_mx128", 5, 16384, 8192, 0, 128, "mxfp4", "t3_lognormal", 0, 1.0),
    "stress_nv32": Workload("stress_nv32", 5, 16384, 8192, 0, 32, "nvfp4", "t3_lognormal", 0, 1.0),
    "stress_nv128": Workload("stress_nv128", 5, 16384, 8192, 0, 128, "nvfp4", "t3_lognormal", 0, 1.0),
}


def _rng(cfg_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, tensor_id]))


def draw_x(w: Workload, M: int | None = None) -> np.ndarray:
    """Activations X [M, K] as bf16 bits (uint16), seeded by the workload's id.

    Outlier channels: ``n`` distinct channel indices drawn without replacement;
    every X[:, c] in them is multiplied by ``outlier_mult`` before rounding.
    Per-channel log-normal scales: X[:, c] *= exp(z_c), z_c ~ N(0, 1).
    """
    M = w.M if M is None else M
    K = w.K
    g = _rng(w.cfg_id, 0)
    if w.x_dist == "normal":
        x = g.standard_normal((M, K), dtype=np.float32)
    elif w.x_dist == "t5":
        x = g.standard_t(5.0, size=(M, K)).astype(np.float32)
    elif w.x_dist == "t3_lognormal":
        x = g.standard_t(3.0, size=(M, K)).astype(np.float32)
        z = _rng(w.cfg_id, 3).standard_normal(K).astype(np.float32)
        x *= np.exp(z)[None, :]
    else:
        raise ValueError(w.x_dist)
    n = w.n_outliers()
    if n > 0:
        ch = _rng(w.cfg_id, 2).choice(K, size=n, replace=False)
        x[:, ch] *= np.float32(w.outlier_mult)
    return bf16_bits_from_f32(x)


def draw_w(w: Workload) -> np.ndarray:
    """Weights W [N, K] as bf16 bits, N(0, w_std^2) (w_std is a standard deviation)."""
    if w.N <= 0:
        raise ValueError(f"workload {w.name} has no weight")
    g = _rng(w.cfg_id, 1)
    x = g.standard_normal((w.N, w.K), dtype=np.float32)
    x *= np.float32(w.w_std)
    return bf16_bits_from_f32(x)


def draw_signs(K: int, seed: int) -> np.ndarray:
    """A +-1 diagonal (int8) for the randomized block Hadamard variant."""
    g = _rng(seed, 4)
    return np.where(g.integers(0, 2, size=K) == 1, 1, -1).astype(np.int8)


def draw_normal_bf16(shape, std: float, seed: int) -> np.ndarray:
    """Plain N(0, std^2) bf16 bits for small test cases."""
    g = np.random.default_rng(np.random.SeedSequence([1000 + seed, 0]))
    return bf16_bits_from_f32(g.standard_normal(shape, dtype=np.float32) * np.float32(std))
