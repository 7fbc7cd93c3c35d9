"""Seeded synthetic inputs for the W4A4 + INT8-outlier linear layer.

This module only draws numbers: it holds none of the layer's arithmetic, so
both the HIP path's tests/benchmark and the CPU oracle can take their inputs
from it. No dataset or trained weight is used: the shapes stand in for the
Llama 7B-65B projections that the Atom summary page evaluates (Summary
paragraph 3), and the heavy outlier columns imitate the outlier activation
channels that page and the QUIK abstract describe.

Recipe (numpy PCG64 ``default_rng(seed)``), in this draw order:
  1. outlier channel indices: ``rng.choice(K, n_out, replace=False)``;
  2. X [M, K] in float32 from the config's distribution, outlier columns
     multiplied by the config's factor, then cast to fp16 (round to nearest);
  3. W [N, K] in float32 ~ N(0, w_std), cast to fp16.
For the producer fused with the preceding RMSNorm, X is the norm's input and
the norm weight gamma [K] ~ 1 + N(0, 0.1) in fp16 comes from a generator of
its own (``draw_norm_weight``).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    n_out: int
    group: int            # 0: one INT4 scale per row; else group size along K
    seed: int
    x_dist: str           # "normal" or "laplace", unit scale
    outlier_factor: float
    w_std: float
    note: str = ""

    @property
    def K_n(self) -> int:
        return self.K - self.n_out


# The five workloads: shapes, quantization granularity and value recipes.
TINY = Workload("tiny_w4a4_m16_k256_n256", 16, 256, 256, 16, 0, 1, "normal", 50.0, 0.02,
                "per-token INT4 activations, per-channel INT4 weights, 16 INT8 outliers")
QPROJ_7B = Workload("llama7b_qproj_prefill_m2048_k4096_n4096_g128", 2048, 4096, 4096, 128,
                    128, 2, "normal", 30.0, 0.02,
                    "group 128 INT4 activations and weights, 128 INT8 outliers")
UPPROJ_7B = Workload("llama7b_upproj_m4096_k4096_n11008", 4096, 11008, 4096, 256, 0, 3,
                     "laplace", 50.0, 0.02,
                     "per-token / per-channel INT4, 256 INT8 outliers, producer timed")
DECODE_65B = Workload("llama65b_decode_k8192_n8192_g128", 256, 8192, 8192, 128, 128, 4,
                      "normal", 30.0, 0.02,
                      "X drawn once with 256 rows; M in {1,8,32,128,256} are row prefixes")
DECODE_M = (1, 8, 32, 128, 256)
DOWNPROJ_65B = Workload("llama65b_downproj_m8192_k22016_n8192", 8192, 8192, 22016, 256, 0, 5,
                        "normal", 100.0, 0.01,
                        "per-token / per-channel INT4, 256 INT8 outliers")

ALL = (TINY, QPROJ_7B, UPPROJ_7B, DECODE_65B, DOWNPROJ_65B)


def draw(M: int, N: int, K: int, n_out: int, seed: int, x_dist: str = "normal",
         outlier_factor: float = 50.0, w_std: float = 0.02):
    """Return (X fp16 [M, K], W fp16 [N, K], outlier_idx int32 [n_out])."""
    rng = np.random.default_rng(seed)
    outliers = rng.choice(K, n_out, replace=False).astype(np.int32)
    if x_dist == "normal":
        X = rng.standard_normal((M, K), dtype=np.float32)
    elif x_dist == "laplace":
        X = rng.laplace(0.0, 1.0, (M, K)).astype(np.float32)
    else:
        raise ValueError(x_dist)
    if n_out:
        X[:, outliers] *= np.float32(outlier_factor)
    X = X.astype(np.float16)
    W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_std)).astype(np.float16)
    return X, W, outliers


def draw_norm_weight(K: int, seed: int, std: float = 0.1):
    """RMSNorm weight gamma fp16 [K] ~ 1 + N(0, std), from its own generator
    (seed sequence [seed, 1]) so that the draws above are unchanged."""
    rng = np.random.default_rng([seed, 1])
    return (1.0 + std * rng.standard_normal(K, dtype=np.float32)).astype(np.float16)


def draw_workload(w: Workload, M: int | None = None):
    """Inputs of a named workload; M (when given) takes a row prefix of X."""
    X, W, o = draw(w.M, w.N, w.K, w.n_out, w.seed, w.x_dist, w.outlier_factor, w.w_std)
    if M is not None:
        X = np.ascontiguousarray(X[:M])
    return X, W, o
