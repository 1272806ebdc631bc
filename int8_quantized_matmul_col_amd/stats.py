"""Column statistics of an activation, for choosing the outlier threshold.

"8-bit quantization in practice" (section 5.1) sets the threshold from the
activations' statistics rather than by default: it looks at the largest
|activation| against its 99th percentile (a large ratio means outliers) and
lowers the threshold where outliers are large.  Its section 2.3 gives the
trade-off: too low a threshold sends many columns to fp16 (less speed-up),
too high a one quantizes the outliers (accuracy collapses).

What decides the split is the per-column maximum colmax[k] = max_m |X[m,k]|:
column k is an outlier column for every threshold t < colmax[k].  It comes
from the library's outlier-detection kernels (``int8_column_absmax``, exact),
and |O| at each candidate threshold is counted by the library as well
(``int8_outlier_counts``, the outlier test's own strict comparison).  The
maximum and the 99th percentile of the K column maxima are summaries for the
reader (torch reductions over K values), not a step of the matmul path.
"""

from __future__ import annotations

from typing import Dict, Iterable, Optional, Sequence

from . import binding

# thresholds reported by default: the pages' usual range (5-7) and around it
DEFAULT_THRESHOLDS = (0.0, 1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0, 10.0, 16.0, float("inf"))


def outlier_stats(X, thresholds: Iterable[float] = DEFAULT_THRESHOLDS,
                  colmax=None) -> Dict[str, object]:
    """Summary of the column maxima of X (float16 [M][K] on the GPU):

    * ``max`` -- the largest |x|; ``q99`` -- the 99th percentile of the
      column maxima; ``ratio`` = max / q99 (about 1 without outlier columns);
    * ``n_outliers[t]`` -- |O| at threshold t (columns with colmax > t);
    * ``fp16_fraction[t]`` -- |O| / K, the share of the multiply-adds that
      take the fp16 path at t;
    * ``histogram`` -- the column maxima binned at the thresholds, from the
      same counts: a list of (lo, hi, n), n = columns with lo < colmax <= hi,
      the first bin from lo = -inf (colmax <= the smallest threshold), the
      last up to hi = +inf (above the largest finite threshold).

    ``colmax`` may be passed if it was already computed.
    """
    import torch
    cm = binding.int8_column_absmax(X) if colmax is None else colmax
    M, K = X.shape
    out: Dict[str, object] = {"M": int(M), "K": int(K)}
    if K == 0:
        out.update(max=0.0, q99=0.0, ratio=float("nan"), n_outliers={}, fp16_fraction={},
                   histogram=[])
        return out
    c = cm.float()
    mx = float(c.max())
    q99 = float(torch.quantile(c, 0.99))
    ts = []
    for t in thresholds:
        t = float(t)
        if t != t or t < 0:
            raise ValueError("thresholds must be non-negative numbers")
        ts.append(t)
    counts = {}
    lim = binding.INT8MM_MAX_COUNT_THRESHOLDS
    for i in range(0, len(ts), lim):
        part = ts[i:i + lim]
        got = binding.int8_outlier_counts(cm, part).cpu().tolist()
        counts.update({t: int(n) for t, n in zip(part, got)})
    edges = sorted(counts)
    if not edges:
        edges = [float("inf")]
        counts_inf = {float("inf"): 0}
    else:
        counts_inf = counts
    hist = [(float("-inf"), edges[0], K - counts_inf[edges[0]])]
    hist += [(lo, hi, counts_inf[lo] - counts_inf[hi]) for lo, hi in zip(edges, edges[1:])]
    if edges[-1] != float("inf"):
        hist.append((edges[-1], float("inf"), counts_inf[edges[-1]]))
    out.update(max=mx, q99=q99, ratio=(mx / q99) if q99 > 0 else float("inf"),
               n_outliers=counts, fp16_fraction={t: n / K for t, n in counts.items()},
               histogram=hist)
    return out


def suggest_threshold(X=None, max_fp16_fraction: float = 0.01,
                      candidates: Sequence[float] = (4.0, 5.0, 6.0, 7.0, 8.0, 10.0, 16.0),
                      stats: Optional[Dict[str, object]] = None) -> float:
    """Smallest candidate threshold whose fp16 share |O|/K is at most
    ``max_fp16_fraction`` (so that the outlier columns are kept in fp16 while
    the int8 path keeps nearly all of the work); +inf when none qualifies.
    The candidates default to the pages' usual range and above it."""
    if stats is None:
        if X is None:
            raise ValueError("give X or stats")
        stats = outlier_stats(X, thresholds=candidates)
    K = int(stats["K"])
    counts = stats["n_outliers"]
    for t in sorted(float(t) for t in candidates):
        n = counts.get(t)
        if n is None:
            raise ValueError(f"stats hold no count for threshold {t}")
        if K == 0 or n <= max_fp16_fraction * K:
            return t
    return float("inf")


__all__ = ["DEFAULT_THRESHOLDS", "outlier_stats", "suggest_threshold"]
