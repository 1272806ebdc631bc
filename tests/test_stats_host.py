"""Host-side logic of the threshold statistics (no GPU): the summaries that
outlier_stats and suggest_threshold build from the library's column maxima
and counts.  The two library calls are replaced by CPU stand-ins computed
from the oracle's column maxima, so that only the bookkeeping is tested
here; tests/test_gpu_stats.py runs the same functions on the GPU."""

import math

import numpy as np
import pytest
import torch

import workloads
from int8_quantized_matmul_col_amd import binding, stats
from oracle import int8mm_ref as ref


@pytest.fixture
def cpu_library(monkeypatch):
    calls = []

    def colmax_cpu(X):
        _, _, cm = ref.outlier_mask_ref(X.numpy(), 6.0)
        return torch.from_numpy(cm.astype(np.float16))

    def counts_cpu(cm, thresholds):
        calls.append(len(thresholds))
        assert 1 <= len(thresholds) <= binding.INT8MM_MAX_COUNT_THRESHOLDS
        c = cm.float().numpy()
        return torch.tensor([int(np.sum(c > t)) for t in thresholds], dtype=torch.int32)

    monkeypatch.setattr(binding, "int8_column_absmax", colmax_cpu)
    monkeypatch.setattr(binding, "int8_outlier_counts", counts_cpu)
    return calls


def _x():
    X, _ = workloads.make_x(64, 300, 11, 4, 8.0, 60.0, "uniform")
    return torch.from_numpy(X)


def test_histogram_partitions_the_columns(cpu_library):
    X = _x()
    ts = (7.0, 0.0, 2.0, 6.0, math.inf, 30.0)
    st = stats.outlier_stats(X, thresholds=ts)
    _, _, cm = ref.outlier_mask_ref(X.numpy(), 6.0)
    hist = st["histogram"]
    assert [h[1] for h in hist] == sorted(ts)
    assert [h[0] for h in hist] == [-math.inf] + sorted(ts)[:-1]
    assert sum(n for _, _, n in hist) == 300
    for lo, hi, n in hist:
        assert n == int(np.sum((cm > lo) & (cm <= hi)))
    for t in ts:
        assert st["n_outliers"][t] == int(np.sum(cm > t))
        assert st["fp16_fraction"][t] == st["n_outliers"][t] / 300


def test_histogram_has_an_open_last_bin_without_inf(cpu_library):
    st = stats.outlier_stats(_x(), thresholds=(6.0, 1.0))
    hist = st["histogram"]
    assert hist[-1][:2] == (6.0, math.inf)
    assert hist[-1][2] == st["n_outliers"][6.0]
    assert sum(n for _, _, n in hist) == 300


def test_more_thresholds_than_one_call_takes(cpu_library):
    ts = [0.125 * i for i in range(150)]
    st = stats.outlier_stats(_x(), thresholds=ts)
    lim = binding.INT8MM_MAX_COUNT_THRESHOLDS
    assert cpu_library == [lim, lim, 150 - 2 * lim]
    assert len(st["n_outliers"]) == 150 and len(st["histogram"]) == 151


def test_no_thresholds_and_empty_k(cpu_library):
    st = stats.outlier_stats(_x(), thresholds=())
    assert st["histogram"] == [(-math.inf, math.inf, 300)] and st["n_outliers"] == {}
    st0 = stats.outlier_stats(torch.zeros((5, 0), dtype=torch.float16), thresholds=(6.0,))
    assert st0["histogram"] == [] and st0["n_outliers"] == {}


def test_bad_thresholds_are_refused(cpu_library):
    for bad in (-1.0, math.nan):
        with pytest.raises(ValueError):
            stats.outlier_stats(_x(), thresholds=(6.0, bad))


def test_suggest_threshold_from_stats(cpu_library):
    X = _x()
    cands = (4.0, 6.0, 8.0, 16.0)
    t = stats.suggest_threshold(X, max_fp16_fraction=0.02, candidates=cands)
    _, _, cm = ref.outlier_mask_ref(X.numpy(), 6.0)
    assert np.sum(cm > t) <= 0.02 * 300
    assert all(np.sum(cm > c) > 0.02 * 300 for c in cands if c < t)
