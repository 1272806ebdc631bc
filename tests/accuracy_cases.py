"""The accuracy study of the decomposition on synthetic outlier inputs:
relative error against the exact product X.W^T (float64, the unquantized
float16 weight) for

* the decomposed matmul at a sweep of thresholds (t = +inf is the plain
  vector-wise int8 matmul: row scales for X, channel scales for W);
* per-tensor int8 (one absmax scale for all of X, one for all of W: the
  "per-tensor" scheme of "8-bit quantization in practice", section 2.1);
* the fp16 matmul of the unquantized operands (fp32 accumulation).

The pages' claims it checks: outlier columns wreck plain int8 and the
decomposition repairs it ("LLM.int8() notes", sections 2.2-2.3); per-channel
scales beat a per-tensor scale (section 2.1); lowering the threshold moves
work to fp16 and the error toward the fp16 level (section 2.3).  Shared by
the CPU study (oracle only) and the GPU study (the HIP path).
"""

from __future__ import annotations

import math

import numpy as np

from oracle import int8mm_ref as ref
import workloads

THRESHOLDS = (math.inf, 16.0, 8.0, 6.0, 4.0, 2.0, 0.0)


def study_inputs(M: int, K: int, N: int, seed: int):
    """X with 6 planted outlier columns (+-U(8, 60) in every row, as in the
    q_proj workload) and 1% heavy-tailed columns (Student-t(3), as in the
    13B sweep); W ~ N(0, 0.02)."""
    X, planted = workloads.make_x(M, K, seed, 6, 8.0, 60.0, "uniform")
    rng = np.random.default_rng(seed + 1)
    free = np.setdiff1d(np.arange(K), planted)
    heavy = rng.choice(free, max(1, K // 100), replace=False)
    X[:, heavy] = rng.standard_t(3, size=(M, heavy.size)).astype(np.float16)
    W = workloads.make_w(N, K, seed, 0.02)
    return X, W


def exact_product(X16, W16):
    return X16.astype(np.float64) @ W16.astype(np.float64).T


def rel_err(Y, Y_exact) -> float:
    return float(np.linalg.norm(Y.astype(np.float64) - Y_exact) / np.linalg.norm(Y_exact))


def per_tensor_int8(X16, W16):
    """One absmax scale per tensor, codes as the per-channel quantizer,
    exact integer product, fp32 rescale, one rounding to fp16."""
    a_x = np.float32(np.abs(X16).max())
    a_w = np.float32(np.abs(W16).max())
    Xq = ref.quantize_rows_ref(X16, np.full(X16.shape[0], a_x, np.float32))
    Wq = ref.quantize_rows_ref(W16, np.full(W16.shape[0], a_w, np.float32))
    C = ref.int8_gemm_ref(Xq, Wq)
    s = np.float32(a_x * a_w) / np.float32(127 * 127)
    return (C.astype(np.float32) * s).astype(np.float16)


def fp16_matmul(X16, W16):
    return (X16.astype(np.float32) @ W16.astype(np.float32).T).astype(np.float16)


def dequantized_weight_product(X16, Wq, a_w):
    """X . W_hat^T in float64 (W_hat = Wq*a_w/127): the limit of t = 0."""
    W_hat = Wq.astype(np.float64) * (a_w.astype(np.float64)[:, None] / 127.0)
    return X16.astype(np.float64) @ W_hat.T


def check_claims(errs: dict, per_tensor: float, fp16: float, t0_limit: float) -> None:
    """The pages' claims on one study (errs: threshold -> relative error)."""
    # outlier columns wreck plain vector-wise int8; the decomposition repairs it
    assert errs[math.inf] > 4.0 * errs[6.0], errs
    # a per-tensor scale is worse still than row / channel scales
    assert per_tensor > errs[math.inf], (per_tensor, errs[math.inf])
    # lowering the threshold never costs accuracy (10% slack for rounding noise)
    ts = sorted(errs, reverse=True)
    for hi, lo in zip(ts, ts[1:]):
        assert errs[lo] <= errs[hi] * 1.1, (hi, lo, errs)
    # t = 0: only the weight's quantization is left
    assert abs(errs[0.0] - t0_limit) <= 0.05 * t0_limit, (errs[0.0], t0_limit)
    assert fp16 < errs[0.0]


def format_table(errs: dict, per_tensor: float, fp16: float, n_out: dict) -> str:
    lines = ["| variant | \\|O\\| | relative error vs exact X.W^T |", "|---|---:|---:|"]
    for t in sorted(errs, reverse=True):
        name = "vector-wise int8 (t = inf)" if t == math.inf else f"decomposed, t = {t:g}"
        lines.append(f"| {name} | {n_out[t]} | {errs[t]:.3e} |")
    lines.append(f"| per-tensor int8 | 0 | {per_tensor:.3e} |")
    lines.append(f"| fp16 matmul (unquantized W) | - | {fp16:.3e} |")
    return "\n".join(lines)
