"""Seeded synthetic inputs for the decomposed int8 matmul.

This module only draws random numbers.  It holds none of the method's
arithmetic (no thresholds, scales, rounding or products), so that both the
CPU oracle's tests and the GPU path can take their inputs from here without
sharing any computation.

Shapes and value distributions follow the workloads the pages talk about:
LLaMA-7B / 13B projection shapes (7B q_proj 4096x4096, FFN 4096<->11008,
13B 5120x13824) and the activation picture of the LLM.int8() notes
("LLM.int8() notes", section 2.2 on outliers): normally distributed
activations with a few feature columns of much larger magnitude present in
every row, plus heavy-tailed columns for the threshold sweep.

Recipe (all configs):

* Two independent streams per config: ``default_rng([seed, 0])`` draws X,
  ``default_rng([seed, 1])`` draws W.  So X can be regenerated without W.
* X: ``standard_normal((M, K), float32)``; then ``choice(K, n_out,
  replace=False)`` picks the outlier columns; their entries are replaced by
  ``uniform(lo, hi, (M, n_out)) * (2*integers(0, 2, (M, n_out)) - 1)``
  (a random sign per entry).  For the sweep workload the chosen columns get
  ``standard_t(3, (M, n_out))`` instead.
* W: ``standard_normal((N, K), float32) * 0.02``, stored out-major [N][K]
  (the nn.Linear layout: one row per output channel).
* Everything is cast to float16 with round-to-nearest-even; every value is
  asserted finite.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "Case",
    "CONFIGS",
    "make_x",
    "make_w",
    "make_case",
    "config_case",
    "DEFAULT_THRESHOLD",
]

# Default outlier threshold used by the workloads (the value the bitsandbytes
# configuration on the pages uses).  Workload metadata only.
DEFAULT_THRESHOLD = 6.0


@dataclasses.dataclass
class Case:
    name: str
    M: int
    K: int
    N: int
    threshold: float
    X: np.ndarray  # float16 [M][K]
    W: Optional[np.ndarray]  # float16 [N][K] (None when only X was asked for)
    outlier_cols: np.ndarray  # int64, the planted columns (sorted)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def _to_fp16(a: np.ndarray) -> np.ndarray:
    h = a.astype(np.float16)
    if not np.isfinite(h).all():
        raise ValueError("generated a non-finite float16 value")
    return h


def make_x(M: int, K: int, seed: int, n_out: int = 0, lo: float = 8.0,
           hi: float = 60.0, kind: str = "uniform", scale: float = 1.0
           ) -> Tuple[np.ndarray, np.ndarray]:
    """Activation matrix X [M][K] float16 and the sorted planted columns.

    ``kind="uniform"``: planted entries are +-U(lo, hi).
    ``kind="t3"``: planted entries are Student-t(3) samples (unscaled).
    """
    rng = _rng(seed, 0)
    X = rng.standard_normal((M, K), dtype=np.float32) * np.float32(scale)
    n_out = min(n_out, K)
    cols = rng.choice(K, size=n_out, replace=False) if n_out > 0 else np.zeros(0, np.int64)
    if n_out > 0:
        if kind == "uniform":
            mag = rng.uniform(lo, hi, size=(M, n_out))
            sign = 2 * rng.integers(0, 2, size=(M, n_out)) - 1
            X[:, cols] = (mag * sign).astype(np.float32)
        elif kind == "t3":
            X[:, cols] = rng.standard_t(3, size=(M, n_out)).astype(np.float32)
        else:
            raise ValueError(kind)
    return _to_fp16(X), np.sort(cols.astype(np.int64))


def make_w(N: int, K: int, seed: int, std: float = 0.02) -> np.ndarray:
    """Weight W [N][K] float16 ~ N(0, std^2), one row per output channel."""
    rng = _rng(seed, 1)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    return _to_fp16(W)


def make_case(name: str, M: int, K: int, N: int, seed: int, n_out: int,
              lo: float = 8.0, hi: float = 60.0, kind: str = "uniform",
              threshold: float = DEFAULT_THRESHOLD, with_w: bool = True) -> Case:
    X, cols = make_x(M, K, seed, n_out, lo, hi, kind)
    W = make_w(N, K, seed) if with_w else None
    return Case(name, M, K, N, threshold, X, W, cols)


# The five workloads.  (M, K, N, seed, n_outlier_columns, lo, hi, kind)
CONFIGS: Dict[str, dict] = {
    # Tiny: 16x1024 by 1024x1024, 2 planted columns in [8, 20].
    "tiny": dict(M=16, K=1024, N=1024, seed=1001, n_out=2, lo=8.0, hi=20.0),
    # LLaMA-7B q_proj prefill: 4096 tokens, 4096 -> 4096, 6 columns in [8, 60].
    "q_proj": dict(M=4096, K=4096, N=4096, seed=1002, n_out=6, lo=8.0, hi=60.0),
    # LLaMA-7B FFN prefill, up projection: 2048 tokens, 4096 -> 11008,
    # 0.5% of 4096 columns (20) in [6, 40].
    "ffn_up": dict(M=2048, K=4096, N=11008, seed=1003, n_out=20, lo=6.0, hi=40.0),
    # ... and down projection 11008 -> 4096, 0.5% of 11008 columns (55).
    "ffn_down": dict(M=2048, K=11008, N=4096, seed=1004, n_out=55, lo=6.0, hi=40.0),
    # Decode: M in {1, 4, 16} rows, 8192 -> 28672, 8 columns in [8, 60].
    "decode1": dict(M=1, K=8192, N=28672, seed=1005, n_out=8, lo=8.0, hi=60.0),
    "decode4": dict(M=4, K=8192, N=28672, seed=1005, n_out=8, lo=8.0, hi=60.0),
    "decode16": dict(M=16, K=8192, N=28672, seed=1005, n_out=8, lo=8.0, hi=60.0),
    # LLaMA-13B-shaped threshold sweep: 4096 tokens, 5120 -> 13824,
    # 51 Student-t(3) columns (1% of K).
    "sweep13b": dict(M=4096, K=5120, N=13824, seed=1006, n_out=51, kind="t3"),
}

# Thresholds of the sweep workload.
SWEEP_THRESHOLDS: List[float] = [0.0, 5.0, 6.0, 7.0, math.inf]


def config_case(name: str, threshold: float = DEFAULT_THRESHOLD,
                with_w: bool = True) -> Case:
    c = dict(CONFIGS[name])
    return make_case(name, c.pop("M"), c.pop("K"), c.pop("N"), c.pop("seed"),
                     c.pop("n_out"), threshold=threshold, with_w=with_w, **c)
