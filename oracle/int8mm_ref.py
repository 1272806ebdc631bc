"""Plain numpy oracle for the LLM.int8() mixed-precision decomposed matmul.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.

What is computed (notation: X float16 [M][K] activations, W float16 [N][K]
weight with one row per output channel, t the outlier threshold):

    Y = X_O . W_O  (fp16 operands, fp32 accumulation)
      + dequant( int8(X_R) . int8(W_R) )

* O is the set of input-feature columns whose largest |x| over the rows of
  this X exceeds t, R the rest ("LLM.int8() notes", section 2.3, the
  decomposition formula and its split-by-column sketch).
* W is quantized once, per output channel, with absmax/127 scales
  ("PyTorch 2.9 supports LLM.int8()", section 1, per-channel weight
  quantization); X is quantized per call ("dynamic" activation quantization,
  same page, section 2) with one absmax scale per row taken over the R
  columns ("vector-wise" quantization, "LLM.int8() notes" introduction).
  Values round half to even and clamp to [-127, 127].
* The int8 product accumulates exactly (int32 on the device), is rescaled by
  a_x[m] * a_w[n] / 127^2, and the fp16 outlier product is added (the two
  partial results are merged: "PyTorch 2.9 supports LLM.int8()", section 3).

Readings where the pages are silent or garbled:

* the outlier comparison is strict: a column is an outlier when its max |x|
  is > t (the comparison operator is lost in the page's extracted code);
* a scale of 0 (all-zero row or channel, or an empty R) quantizes to 0;
* W_O is the dequantized int8 weight, fp16(fp32(fp32(Wq)*a_w)/127): the
  prepared weight keeps only int8 values and fp32 scales, as with
  ``has_fp16_weights=False`` on the per-channel page;
* the dequant scale is fp32(a_x*a_w)/16129, the merge fp32(fp32(C)*s + Y_O),
  rounded once to fp16 (overflow to +-inf as IEEE does);
* a linear layer's bias (fp16 b [N]) is added in fp32 after the merge, before
  that one rounding.
"""

from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np

Q_MAX = 127  # symmetric int8 range [-127, 127]


def quantize_rows_ref(A16: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Absmax quantization of each row of ``A16`` with its own scale.

    q[i, j] = clamp(rint(fp32(127 * A[i, j]) / scale[i]), -127, 127), and 0 in
    rows whose scale is 0.  ``127 * a`` is exact in fp32 for fp16 ``a``; the
    division is IEEE fp32 and ``rint`` rounds half to even, as the "round"
    of the per-channel page is read.  ("PyTorch 2.9 supports LLM.int8()",
    sections 1 and 2.)
    """
    A32 = np.asarray(A16, dtype=np.float16).astype(np.float32)
    s = np.asarray(scale, dtype=np.float32).reshape(-1, 1)
    num = A32 * np.float32(Q_MAX)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(num / s)
    q = np.where(s == 0, np.float32(0), q)
    q = np.clip(q, -Q_MAX, Q_MAX)
    return q.astype(np.int8)


def prepare_weight_ref(W16: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-output-channel weight quantization, run once per weight.

    a_w[n] = max_k |W[n, k]| (a float16 value, kept as fp32) and
    Wq[n, :] = quantize(W[n, :], a_w[n])  -- "PyTorch 2.9 supports
    LLM.int8()", section 1 (one scale per output channel, absmax / 127).
    The scale covers all K input features, outlier columns included: it is
    fixed before any activation is seen.
    """
    W16 = np.asarray(W16, dtype=np.float16)
    N, K = W16.shape
    if K == 0:
        return np.zeros((N, 0), np.int8), np.zeros(N, np.float32)
    a_w = np.abs(W16).max(axis=1).astype(np.float32)
    return quantize_rows_ref(W16, a_w), a_w


def outlier_mask_ref(X16: np.ndarray, threshold: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Outlier feature columns of this X.

    colmax[k] = max over the M rows of |X[m, k]|; mask[k] = colmax[k] > t
    (strict); O = ascending column indices with mask set.  "LLM.int8()
    notes", section 2.3: the columns whose absolute activation exceeds the
    threshold, found over the batch dimension of the current input.
    Returns (mask bool[K], O int64[|O|], colmax float32[K]).
    """
    X16 = np.asarray(X16, dtype=np.float16)
    M, K = X16.shape
    if M == 0:
        colmax = np.zeros(K, np.float32)
    else:
        colmax = np.abs(X16).max(axis=0).astype(np.float32)
    mask = colmax > np.float32(threshold)
    O = np.flatnonzero(mask).astype(np.int64)
    return mask, O, colmax


def quantize_activation_ref(X16: np.ndarray, mask: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Dynamic per-row quantization of X over the regular columns R.

    a_x[m] = max over k in R of |X[m, k]| (0 when R is empty);
    Xq[m, k] = quantize(X[m, k], a_x[m]) for k in R and 0 for k in O.
    "PyTorch 2.9 supports LLM.int8()", section 2 (scale from the actual max
    of each input, no calibration), applied row-wise ("vector-wise").
    """
    X16 = np.asarray(X16, dtype=np.float16)
    M, K = X16.shape
    XR = np.where(mask[None, :], np.float16(0), X16)
    if K == 0:
        a_x = np.zeros(M, np.float32)
    else:
        a_x = np.abs(XR).max(axis=1).astype(np.float32) if M > 0 else np.zeros(0, np.float32)
    return quantize_rows_ref(XR, a_x), a_x


def outlier_slices_ref(X16: np.ndarray, Wq: np.ndarray, a_w: np.ndarray,
                       O: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """The fp16 operands of the outlier product.

    X_O[m, j] = X[m, O_j] (float16 [M][|O|]) and
    W_O[j, n] = fp16( fp32( fp32(Wq[n, O_j]) * a_w[n] ) / 127 )  (float16
    [|O|][N]), the dequantized int8 weight rows of the outlier features
    ("LLM.int8() notes", section 2.3: x[:, mask] and w[mask, :]).
    """
    X_O = np.asarray(X16, dtype=np.float16)[:, O]
    wq = Wq[:, O].astype(np.float32)  # [N][|O|]
    deq = (wq * a_w.astype(np.float32)[:, None]) / np.float32(Q_MAX)
    W_O = deq.astype(np.float16).T.copy()  # [|O|][N]
    return X_O, W_O


def int8_gemm_ref(Xq: np.ndarray, Wq: np.ndarray, chunk: int = 2048) -> np.ndarray:
    """C[m, n] = sum_k Xq[m, k] * Wq[n, k] as exact integers (int32).

    Computed with a float64 BLAS product in column chunks: every partial sum
    is an integer of magnitude <= 127^2 * K < 2^53, so it is exact in any
    summation order.  (The int8 term of the decomposition, "LLM.int8()
    notes", section 2.3; int32 accumulation as on INT8 matrix units.)
    """
    M, K = Xq.shape
    N = Wq.shape[0]
    C = np.empty((M, N), np.int32)
    if M == 0 or N == 0:
        return C
    A = Xq.astype(np.float64)
    for n0 in range(0, N, chunk):
        B = Wq[n0:n0 + chunk].astype(np.float64)
        C[:, n0:n0 + chunk] = (A @ B.T).astype(np.int64).astype(np.int32)
    return C


def outlier_gemm_ref(X_O: np.ndarray, W_O: np.ndarray, N: int) -> np.ndarray:
    """Y_O = X_O . W_O with fp16 operands and fp32 accumulation (float32 BLAS)."""
    M = X_O.shape[0]
    if X_O.shape[1] == 0 or M == 0 or N == 0:
        return np.zeros((M, N), np.float32)
    return X_O.astype(np.float32) @ W_O.astype(np.float32)


def epilogue_ref(C: np.ndarray, a_x: np.ndarray, a_w: np.ndarray, Y_O: np.ndarray,
                 bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Dequantize and merge: s = fp32(a_x[m]*a_w[n]) / 16129,
    Y = fp16( fp32( fp32( fp32(C)*s ) + Y_O ) + b[n] ), each step rounded in
    fp32, the bias term (fp16 b [N]) only when given.
    ("PyTorch 2.9 supports LLM.int8()", section 3: the two parts are merged;
    its ``Linear8bitLt`` example carries the layer's bias, added here after
    the merge and before the single rounding to fp16.)
    """
    s = (a_x.astype(np.float32)[:, None] * a_w.astype(np.float32)[None, :]) / np.float32(Q_MAX * Q_MAX)
    with np.errstate(over="ignore"):
        y = C.astype(np.float32) * s
        y = y + Y_O.astype(np.float32)
        if bias is not None:
            y = y + np.asarray(bias, np.float16).astype(np.float32)[None, :]
        return y.astype(np.float16)


def int8_matmul_ref(X16: np.ndarray, Wq: np.ndarray, a_w: np.ndarray,
                    threshold: float = 6.0, stages: bool = False,
                    bias: Optional[np.ndarray] = None):
    """The whole decomposed matmul, step by step.

    ``Wq`` [N][K] int8 and ``a_w`` [N] fp32 are the prepared weight.
    ``threshold`` is taken as an fp32 value (the boundary passes a float).
    ``bias`` (fp16 [N], optional) is the linear layer's bias.
    Returns Y float16 [M][N], or (Y, dict of every intermediate) if
    ``stages``.
    """
    X16 = np.asarray(X16, dtype=np.float16)
    t = np.float32(threshold)
    if np.isnan(t) or t < 0:
        raise ValueError("threshold must be a non-negative number")
    M, K = X16.shape
    N = Wq.shape[0]
    assert Wq.shape == (N, K), (Wq.shape, (N, K))
    if bias is not None:
        bias = np.asarray(bias, np.float16)
        assert bias.shape == (N,), (bias.shape, N)
    mask, O, colmax = outlier_mask_ref(X16, t)
    Xq, a_x = quantize_activation_ref(X16, mask)
    X_O, W_O = outlier_slices_ref(X16, Wq, a_w, O)
    C = int8_gemm_ref(Xq, Wq)
    Y_O = outlier_gemm_ref(X_O, W_O, N)
    Y = epilogue_ref(C, a_x, a_w, Y_O, bias)
    if not stages:
        return Y
    return Y, dict(mask=mask, O=O, colmax=colmax, Xq=Xq, a_x=a_x, X_O=X_O,
                   W_O=W_O, C=C, Y_O=Y_O)


def tolerance_bound(X16: np.ndarray, Wq: np.ndarray, a_w: np.ndarray,
                    rel: float = 1e-2, abs_: float = 1e-3,
                    bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-element bound on |Y_gpu - Y_oracle|: rel*(|X| |W_hat|^T)[m, n] + abs_,
    plus 2^-10 |b[n]| with a bias (two fp16 ulps at the bias' magnitude: the
    terms are summed in another order before the one rounding to fp16).

    W_hat = Wq * a_w / 127 is the dequantized weight; the product of absolute
    values is taken in float64.
    """
    W_hat = Wq.astype(np.float64) * (a_w.astype(np.float64)[:, None] / Q_MAX)
    tol = rel * (np.abs(X16.astype(np.float64)) @ np.abs(W_hat).T) + abs_
    if bias is not None:
        tol = tol + 2.0 ** -10 * np.abs(np.asarray(bias, np.float16).astype(np.float64))[None, :]
    return tol


def fp16_ulp(y: np.ndarray) -> np.ndarray:
    """Spacing of float16 numbers at |y| (the subnormal spacing near 0)."""
    a = np.abs(np.asarray(y, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return np.exp2(e - 10)


def summary(Y: np.ndarray) -> Dict[str, float]:
    y = Y.astype(np.float64)
    return dict(sum=float(y.sum()), abs_sum=float(np.abs(y).sum()),
                max=float(np.abs(y).max()) if y.size else 0.0)


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("annotations", "math", "np")]
