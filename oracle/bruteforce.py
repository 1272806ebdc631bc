"""Exact-rational brute force of the decomposed int8 matmul, for tiny shapes.

TEST INFRASTRUCTURE ONLY.  Pure Python: every value is a
``fractions.Fraction``; rounding to an integer is Python's round-half-even on
the exact rational; rounding to fp32 / fp16 is done from the exact rational by
``round_to_binary``.  Nothing here calls numpy arithmetic, so it pins the
numpy oracle (``int8mm_ref``) independently:

* Wq, a_w, mask, O, a_x, Xq and C must agree bit for bit;
* W_O is the exact dequantized value rounded to fp32, then to fp16;
* Y is the exact rational result of the merged decomposition, rounded once to
  fp16; the numpy oracle rounds its fp32 intermediates and may differ from it
  by at most one fp16 ulp.
"""

from __future__ import annotations

from fractions import Fraction
from typing import List, Optional, Sequence

Q_MAX = 127


def round_half_even(r: Fraction) -> int:
    return round(r)  # Fraction.__round__ rounds half to even


def _floor_log2(r: Fraction) -> int:
    """floor(log2(r)) for r > 0, exactly."""
    n, d = r.numerator, r.denominator
    e = n.bit_length() - d.bit_length()
    # 2^e <= n/d < 2^(e+1) ?
    if e >= 0:
        if n < (d << e):
            e -= 1
    else:
        if (n << -e) < d:
            e -= 1
    return e


def round_to_binary(r: Fraction, p: int, emin: int, emax: int) -> Fraction:
    """Round r to the nearest binary float with p significant bits
    (round half to even), subnormals below 2^emin; overflow gives +-inf
    (returned as a float)."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = -r if r < 0 else r
    e = max(_floor_log2(a), emin)
    ulp = Fraction(2) ** (e - p + 1)
    q = round_half_even(a / ulp)
    v = q * ulp
    largest = (Fraction(2) - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if v > largest:
        return float("inf") * sign  # type: ignore[return-value]
    return sign * v


def to_f32(r: Fraction) -> Fraction:
    return round_to_binary(r, 24, -126, 127)


def to_f16(r: Fraction) -> Fraction:
    return round_to_binary(r, 11, -14, 15)


def _q(x: Fraction, a: Fraction) -> int:
    if a == 0:
        return 0
    return max(-Q_MAX, min(Q_MAX, round_half_even(Q_MAX * x / a)))


def bf_prepare_weight(W: Sequence[Sequence[float]]):
    """a_w[n] = max |W[n, :]|, Wq[n, k] = round(127 W / a_w)."""
    Wf = [[Fraction(v) for v in row] for row in W]
    a_w = [max((abs(v) for v in row), default=Fraction(0)) for row in Wf]
    Wq = [[_q(v, a) for v in row] for row, a in zip(Wf, a_w)]
    return Wq, a_w


def bf_int8_matmul(X: Sequence[Sequence[float]], Wq: List[List[int]],
                   a_w: List[Fraction], t: float,
                   bias: Optional[Sequence[float]] = None):
    """Returns a dict with mask, O, a_x, Xq, W_O (fp16-rounded rationals,
    [|O|][N]), C (ints) and Y_exact (rationals) and Y16 (fp16-rounded).
    ``bias`` (fp16 values, [N]) is added exactly to Y_exact."""
    Xf = [[Fraction(v) for v in row] for row in X]
    M = len(Xf)
    K = len(Xf[0]) if M else len(Wq[0]) if Wq else 0
    N = len(Wq)
    colmax = [max((abs(Xf[m][k]) for m in range(M)), default=Fraction(0)) for k in range(K)]
    if t == float("inf"):
        mask = [False] * K  # nothing exceeds an infinite threshold
    else:
        T = Fraction(t)
        mask = [c > T for c in colmax]
    O = [k for k in range(K) if mask[k]]
    R = [k for k in range(K) if not mask[k]]
    a_x = [max((abs(Xf[m][k]) for k in R), default=Fraction(0)) for m in range(M)]
    Xq = [[0 if mask[k] else _q(Xf[m][k], a_x[m]) for k in range(K)] for m in range(M)]
    # W_O[j][n] = fp16(fp32(Wq * a_w / 127)); Wq * a_w is exact in fp32.
    W_O = [[to_f16(to_f32(Fraction(Wq[n][k]) * a_w[n] / Q_MAX)) for n in range(N)] for k in O]
    C = [[sum(Xq[m][k] * Wq[n][k] for k in range(K)) for n in range(N)] for m in range(M)]
    Y_exact = []
    for m in range(M):
        row = []
        for n in range(N):
            y = Fraction(C[m][n]) * a_x[m] * a_w[n] / (Q_MAX * Q_MAX)
            y += sum((Xf[m][k] * W_O[j][n] for j, k in enumerate(O)), Fraction(0))
            if bias is not None:
                y += Fraction(bias[n])
            row.append(y)
        Y_exact.append(row)
    Y16 = [[to_f16(y) for y in row] for row in Y_exact]
    return dict(colmax=colmax, mask=mask, O=O, a_x=a_x, Xq=Xq, W_O=W_O, C=C,
                Y_exact=Y_exact, Y16=Y16)
