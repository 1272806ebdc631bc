"""GPU parity of the column maxima (int8_column_absmax) and of the
threshold statistics built on them, against the CPU oracle."""

import math

import numpy as np
import pytest

import workloads
from gpu_cases import to_dev
from oracle import int8mm_ref as ref

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,n_out", [(1, 64, 1), (16, 1000, 2), (5, 3, 1), (17, 1024, 2),
                                       (300, 520, 5), (33, 37, 2), (4096, 257, 3), (0, 40, 0)])
def test_column_absmax_parity(lib, M, K, n_out):
    print(f"case colmax M={M} K={K}", flush=True)
    import torch
    if M == 0:
        X = np.zeros((0, K), np.float16)
    else:
        X, _ = workloads.make_x(M, K, M * 31 + K, n_out, 8.0, 60.0, "uniform")
        X[0, 0] = np.float16(-0.0)
    cm = lib.int8_column_absmax(to_dev(X))
    torch.cuda.synchronize()
    got = cm.cpu().numpy()
    if M == 0:
        assert not got.view(np.uint16).any()
        return
    _, _, colmax = ref.outlier_mask_ref(X, 6.0)
    assert np.array_equal(got.astype(np.float32), colmax)
    assert not (got.view(np.uint16) & 0x8000).any()  # maxima of |x|: no negative zero


@pytest.mark.parametrize("M,K", [(512, 2048), (7, 37), (3, 1), (64, 5000)])
def test_outlier_counts_parity(lib, M, K):
    """int8_outlier_counts against the oracle's |O| at each threshold,
    including thresholds equal to a column maximum (strict: not counted)."""
    print(f"case outlier_counts M={M} K={K}", flush=True)
    import torch
    X, _ = workloads.make_x(M, K, 3 * M + K, min(3, K), 8.0, 60.0, "uniform")
    rng = np.random.default_rng(K)
    cols = rng.choice(K, min(K, 9), replace=False)
    X[:, cols] = (rng.standard_t(3, size=(M, cols.size)) * 2).astype(np.float16)
    _, _, colmax = ref.outlier_mask_ref(X, 6.0)
    ties = [float(v) for v in np.unique(colmax)[-5:]]  # exact column maxima
    ts = [0.0, 0.5, 2.0, 5.0, 6.0, 7.0, 60.0, math.inf] + ties
    cm = lib.int8_column_absmax(to_dev(X))
    got = lib.int8_outlier_counts(cm, ts)
    torch.cuda.synchronize()
    assert got.dtype == torch.int32 and got.shape == (len(ts),)
    for t, n in zip(ts, got.cpu().tolist()):
        _, O, _ = ref.outlier_mask_ref(X, t)
        assert n == O.size, t


def test_outlier_counts_edge_cases(lib):
    import torch
    # K == 0: every count is zero
    empty = torch.empty((0,), dtype=torch.float16, device="cuda")
    z = lib.int8_outlier_counts(empty, [0.0, 6.0])
    # every threshold slot at the limit; an infinite column maximum counts
    # only below +inf
    cm = torch.tensor([0.0, 6.0, 6.00390625, float("inf"), 1.0], dtype=torch.float16,
                      device="cuda")
    lim = lib.binding.INT8MM_MAX_COUNT_THRESHOLDS
    ts = [0.0, 6.0, 1e30, math.inf] + [float(i) / 8 for i in range(lim - 4)]
    got = lib.int8_outlier_counts(cm, ts)
    torch.cuda.synchronize()
    assert z.cpu().tolist() == [0, 0]
    vals = [0.0, 6.0, 6.00390625, math.inf, 1.0]
    assert got.cpu().tolist() == [sum(v > t for v in vals) for t in ts]
    with pytest.raises(lib.Int8mmError):
        lib.int8_outlier_counts(cm, [6.0] * (lim + 1))


def test_outlier_stats_counts_match_oracle(lib):
    import torch
    X, _ = workloads.make_x(512, 2048, 77, 0, 8.0, 60.0, "uniform")
    rng = np.random.default_rng(5)
    cols = rng.choice(2048, 21, replace=False)
    X[:, cols] = (rng.standard_t(3, size=(512, 21)) * 2).astype(np.float16)  # heavy tails
    # more thresholds than one int8_outlier_counts call takes
    ts = (0.0, 1.0, 3.0, 5.0, 6.0, 7.0, 12.0, math.inf) + tuple(0.25 * i + 0.1 for i in range(70))
    st = lib.outlier_stats(to_dev(X), thresholds=ts)
    torch.cuda.synchronize()
    for t in ts:
        _, O, _ = ref.outlier_mask_ref(X, t)
        assert st["n_outliers"][t] == O.size, t
        assert st["fp16_fraction"][t] == O.size / 2048
    _, _, colmax = ref.outlier_mask_ref(X, 6.0)
    assert st["max"] == float(colmax.max())
    # the histogram bins the oracle's column maxima at the sorted thresholds
    hist = st["histogram"]
    assert sum(n for _, _, n in hist) == 2048
    edges = sorted(set(ts))
    assert [h[1] for h in hist] == edges and hist[0][0] == -math.inf
    for lo, hi, n in hist:
        assert n == int(np.sum((colmax > lo) & (colmax <= hi))), (lo, hi)
    # the percentile interpolates between two column maxima in fp32 on the GPU
    assert st["q99"] == pytest.approx(float(np.quantile(colmax.astype(np.float64), 0.99)), rel=1e-4)
    assert st["ratio"] > 1.5  # heavy-tailed columns stand out


def test_suggest_threshold_is_the_smallest_candidate_within_the_fp16_share(lib):
    import torch
    X, planted = workloads.make_x(1024, 4096, 123, 6, 8.0, 60.0, "uniform")
    cands = (4.0, 5.0, 6.0, 7.0, 8.0, 10.0, 16.0)
    t = lib.suggest_threshold(to_dev(X), max_fp16_fraction=0.01, candidates=cands)
    torch.cuda.synchronize()
    n = {c: ref.outlier_mask_ref(X, c)[1].size for c in cands}
    assert n[t] <= 0.01 * 4096
    assert all(n[c] > 0.01 * 4096 for c in cands if c < t)
    # the planted columns (|x| >= 8 in every row) are outliers there
    assert set(np.asarray(planted).tolist()) <= set(ref.outlier_mask_ref(X, t)[1].tolist())
