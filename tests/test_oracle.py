"""CPU pins of the oracle against things other than itself.

Each test fixes a part of the oracle by an independent route: exact rational
brute force, the closed form of the quantizer, threshold limits that reduce
the method to textbook matmuls, invariants, the method's error bound and
exactly representable examples.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import int8mm_ref as ref
from oracle import bruteforce as bf
import workloads


def _fp16_all_nonneg_finite():
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    return bits.view(np.float16)


def _int_mant_exp(v16):
    """Exact (mantissa, exponent) integers with v = m * 2^e for fp16 values."""
    f, e = np.frexp(v16.astype(np.float64))
    m = np.rint(f * 2048.0).astype(np.int64)
    return m, e.astype(np.int64) - 11


def _exact_rne_quant(x16, a16):
    """round_half_even(127*x/a) computed with exact integer arithmetic."""
    mx, ex = _int_mant_exp(np.abs(x16))
    ma, ea = _int_mant_exp(np.full_like(x16, a16))
    d = ex - ea
    num = 127 * mx * np.where(d > 0, np.left_shift(np.int64(1), np.maximum(d, 0)), 1)
    den = ma * np.where(d < 0, np.left_shift(np.int64(1), np.maximum(-d, 0)), 1)
    q = num // den
    rem2 = 2 * (num - q * den)
    q = np.where(rem2 > den, q + 1, np.where(rem2 == den, q + (q & 1), q))
    q = np.minimum(q, 127)
    return np.where(x16 < 0, -q, q)


# ---------------------------------------------------------------- quantizer


QUANT_SCALES = [2.0 ** -24, 2.0 ** -14, 0.0999755859375, 1.0, 1.5, 3.0, 5.98828125,
                6.0, 100.0, 127.0, 1000.0, 65504.0]


@pytest.mark.parametrize("seed", [0])
def test_quantizer_closed_form_exhaustive(seed):
    """fp32 division + rint equals exact round-half-even of 127*x/a for every
    fp16 x with |x| <= a (closed form of the rounding reading)."""
    rng = np.random.default_rng(seed)
    pos = _fp16_all_nonneg_finite()
    scales = [np.float16(s) for s in QUANT_SCALES]
    scales += list(rng.choice(pos[pos > 0], size=24, replace=False))
    for a in scales:
        xs = pos[pos <= a]
        xs = np.concatenate([xs, -xs])
        q = ref.quantize_rows_ref(xs[None, :], np.array([np.float32(a)]))[0]
        exact = _exact_rne_quant(xs, np.float16(a))
        assert np.array_equal(q.astype(np.int64), exact), f"scale {a}"


def test_quantizer_ties_round_half_even():
    # a = 127 makes 127*x/a == x; x = k + 0.5 are exact ties.
    xs = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5, 127.0], np.float16)
    q = ref.quantize_rows_ref(xs[None, :], np.array([127.0], np.float32))[0]
    assert q.tolist() == [0, 2, 2, 0, -2, -2, 126, -126, 127]


def test_quantizer_invariants():
    rng = np.random.default_rng(7)
    A = (rng.standard_normal((64, 300)) * rng.uniform(0.01, 50, (64, 1))).astype(np.float16)
    a = np.abs(A).max(axis=1).astype(np.float32)
    q = ref.quantize_rows_ref(A, a).astype(np.int64)
    # |q| <= 127 and the absmax positions hold +-127
    assert np.abs(q).max() <= 127
    am = np.abs(A).astype(np.float32) == a[:, None]
    assert np.all(np.abs(q[am]) == 127)
    assert np.all(np.sign(q[am]) == np.sign(A.astype(np.float32)[am]))
    # error <= scale/2, i.e. |254 x - 2 q a| <= a (exact in float64)
    err = np.abs(254.0 * A.astype(np.float64) - 2.0 * q * a[:, None].astype(np.float64))
    assert np.all(err <= a[:, None].astype(np.float64))
    # odd symmetry
    qn = ref.quantize_rows_ref(-A, a).astype(np.int64)
    assert np.array_equal(qn, -q)
    # scaling a row and its scale by 2^k leaves the codes unchanged
    for k in (-3, 2):
        A2 = (A.astype(np.float32) * 2.0 ** k).astype(np.float16)
        ok = np.all(A2.astype(np.float32) == A.astype(np.float32) * 2.0 ** k, axis=1)
        q2 = ref.quantize_rows_ref(A2, a * np.float32(2.0 ** k)).astype(np.int64)
        assert np.array_equal(q2[ok], q[ok])
    # zero scale -> zero codes
    z = ref.quantize_rows_ref(np.zeros((2, 5), np.float16), np.zeros(2, np.float32))
    assert not z.any()


def test_prepare_weight_per_channel():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((9, 33)) * 0.02).astype(np.float16)
    W[4] = 0
    Wq, a_w = ref.prepare_weight_ref(W)
    assert Wq.dtype == np.int8 and a_w.dtype == np.float32
    assert np.array_equal(a_w, np.abs(W).max(axis=1).astype(np.float32))
    assert not Wq[4].any() and a_w[4] == 0
    for n in range(9):
        if a_w[n] > 0:
            assert 127 in np.abs(Wq[n].astype(np.int64))


# ---------------------------------------------------------------- brute force


def _compare_with_bruteforce(X, W, t, bias=None):
    Wq, a_w = ref.prepare_weight_ref(W)
    bwq, baw = bf.bf_prepare_weight(W.astype(np.float64).tolist())
    assert np.array_equal(Wq.astype(np.int64), np.array(bwq, np.int64).reshape(Wq.shape))
    assert [Fraction(float(v)) for v in a_w] == baw
    Y, st = ref.int8_matmul_ref(X, Wq, a_w, t, stages=True, bias=bias)
    b = bf.bf_int8_matmul(X.astype(np.float64).tolist(), [list(map(int, r)) for r in Wq],
                          [Fraction(float(v)) for v in a_w], t,
                          None if bias is None else bias.astype(np.float64).tolist())
    M, K = X.shape
    N = W.shape[0]
    assert st["mask"].tolist() == b["mask"]
    assert st["O"].tolist() == b["O"]
    assert [Fraction(float(v)) for v in st["a_x"]] == b["a_x"]
    assert st["Xq"].astype(np.int64).tolist() == b["Xq"]
    assert st["C"].astype(np.int64).tolist() == b["C"]
    assert [[Fraction(float(v)) for v in row] for row in st["W_O"]] == b["W_O"]
    # Y: exact rational rounded once to fp16 vs the oracle's fp32 chain
    y16 = np.array([[float(v) for v in row] for row in b["Y16"]], np.float64).reshape(M, N)
    yo = Y.astype(np.float64)
    assert np.all(np.abs(yo - y16) <= ref.fp16_ulp(y16) + 1e-300), (yo, y16)
    return st


def test_bruteforce_4x8x4_with_outlier_and_ties():
    # 4x8 activations: column 2 carries outliers, column 5 has |x| == 6 exactly
    # (stays regular under the strict comparison), row 3 has exact ties.
    X = np.array([
        [0.5, -1.25, 9.0, 0.75, 2.0, 6.0, -0.125, 1.0],
        [1.0, 2.0, -0.5, -3.0, 0.25, 1.5, 0.0, -2.5],
        [0.0, 0.0, 7.5, 0.0, 0.0, 0.0, 0.0, 0.0],
        # row absmax over R is 127/32, so 127*x/a == 32*x: x = odd/64 are ties
        [3.96875, 0.078125, 1.0, -0.046875, 0.015625, 1.5, -0.078125, 2.0],
    ], np.float16)
    W = np.array([
        [0.02, -0.01, 0.03, 0.0, 0.015, -0.025, 0.005, 0.01],
        [-0.04, 0.02, 0.01, 0.03, -0.02, 0.0, 0.01, -0.005],
        [0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0],
        [0.1, -0.1, 0.05, -0.05, 0.025, -0.025, 0.0125, -0.0125],
    ], np.float16)
    st = _compare_with_bruteforce(X, W, 6.0)
    assert st["O"].tolist() == [2]
    # row 2 has only zeros in R: scale 0, codes 0
    assert st["a_x"][2] == 0 and not st["Xq"][2].any()
    # ties round half to even: 2.5 -> 2, -1.5 -> -2, 0.5 -> 0, -2.5 -> -2
    assert st["Xq"][3].tolist() == [127, 2, 0, -2, 0, 48, -2, 64]


@pytest.mark.parametrize("seed", range(12))
def test_bruteforce_random_small(seed):
    rng = np.random.default_rng(100 + seed)
    M, K, N = rng.integers(1, 9), rng.integers(1, 17), rng.integers(1, 9)
    X = rng.standard_normal((M, K)).astype(np.float32)
    nout = rng.integers(0, min(3, K) + 1)
    cols = rng.choice(K, nout, replace=False)
    X[:, cols] *= rng.uniform(4, 20)
    X = X.astype(np.float16)
    W = (rng.standard_normal((N, K)) * rng.choice([0.02, 1.0, 30.0])).astype(np.float16)
    t = [0.0, 2.0, 6.0, math.inf][seed % 4]
    _compare_with_bruteforce(X, W, t)


def test_bruteforce_4x8x4_with_bias():
    # the 4x8x4 case above with a bias per output channel: magnitudes both
    # below and far above the matmul term, one negative, one exact zero
    X = np.array([
        [0.5, -1.25, 9.0, 0.75, 2.0, 6.0, -0.125, 1.0],
        [1.0, 2.0, -0.5, -3.0, 0.25, 1.5, 0.0, -2.5],
        [0.0, 0.0, 7.5, 0.0, 0.0, 0.0, 0.0, 0.0],
        [3.96875, 0.078125, 1.0, -0.046875, 0.015625, 1.5, -0.078125, 2.0],
    ], np.float16)
    W = np.array([
        [0.02, -0.01, 0.03, 0.0, 0.015, -0.025, 0.005, 0.01],
        [-0.04, 0.02, 0.01, 0.03, -0.02, 0.0, 0.01, -0.005],
        [0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0],
        [0.1, -0.1, 0.05, -0.05, 0.025, -0.025, 0.0125, -0.0125],
    ], np.float16)
    bias = np.array([0.125, -3.5, 0.0, 40.0], np.float16)
    _compare_with_bruteforce(X, W, 6.0, bias)
    # channel 2 has an all-zero weight: Y there is the bias itself
    Wq, a_w = ref.prepare_weight_ref(W)
    Y = ref.int8_matmul_ref(X, Wq, a_w, 6.0, bias=bias)
    assert np.all(Y[:, 2] == 0)
    Y1 = ref.int8_matmul_ref(X, Wq, a_w, 6.0, bias=np.array([0, 0, 2.5, 0], np.float16))
    assert np.all(Y1[:, 2] == np.float16(2.5))


@pytest.mark.parametrize("seed", range(8))
def test_bruteforce_random_small_with_bias(seed):
    rng = np.random.default_rng(300 + seed)
    M, K, N = rng.integers(1, 9), rng.integers(1, 17), rng.integers(1, 9)
    X = rng.standard_normal((M, K)).astype(np.float32)
    cols = rng.choice(K, rng.integers(0, min(3, K) + 1), replace=False)
    X[:, cols] *= rng.uniform(4, 20)
    X = X.astype(np.float16)
    W = (rng.standard_normal((N, K)) * rng.choice([0.02, 1.0, 30.0])).astype(np.float16)
    bias = (rng.standard_normal(N) * rng.choice([1e-3, 0.5, 50.0])).astype(np.float16)
    t = [0.0, 2.0, 6.0, math.inf][seed % 4]
    _compare_with_bruteforce(X, W, t, bias)


def test_zero_bias_is_no_bias():
    rng = np.random.default_rng(7)
    X = rng.standard_normal((5, 40)).astype(np.float16)
    W = (rng.standard_normal((6, 40)) * 0.1).astype(np.float16)
    Wq, a_w = ref.prepare_weight_ref(W)
    Y0 = ref.int8_matmul_ref(X, Wq, a_w, 1.5)
    Y1 = ref.int8_matmul_ref(X, Wq, a_w, 1.5, bias=np.zeros(6, np.float16))
    assert np.array_equal(Y0, Y1)


def test_dequantized_outlier_weight_exhaustive():
    # W_O = the exact q * a_w / 127 rounded to fp32, then to fp16, for every
    # code q and every positive normal fp16 scale a_w.  The exact quotient is
    # formed in float64 (q*a_w has at most 19 significant bits, and p/127 is
    # never closer than 2^-31 relative to an fp32 rounding tie, far beyond
    # float64's 2^-53), so one rounding to fp32 here is the correct rounding.
    a = np.arange(0x0400, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    q = np.arange(-127, 128, dtype=np.int8)
    Wq = np.repeat(q[None, :], a.size, axis=0)  # [N = #scales][K = 255 codes]
    O = np.arange(255)
    X = np.zeros((1, 255), np.float16)
    _, W_O = ref.outlier_slices_ref(X, Wq, a, O)  # [|O|][N]
    exact = (q.astype(np.float64)[:, None] * a.astype(np.float64)[None, :]) / 127.0
    want = exact.astype(np.float32).astype(np.float16)
    assert np.array_equal(W_O.view(np.uint16), want.view(np.uint16))


def test_round_to_binary_matches_hardware_casts():
    rng = np.random.default_rng(11)
    vals = rng.standard_normal(2000) * np.exp2(rng.integers(-20, 20, 2000))
    with np.errstate(over="ignore"):
        for v in vals:
            assert float(bf.to_f32(Fraction(float(v)))) == float(np.float32(v))
            assert float(bf.to_f16(Fraction(float(v)))) == float(np.float16(v))


# ---------------------------------------------------------------- special thresholds


def _plain_vectorwise_int8(X, W):
    """Vector-wise int8 matmul written independently (float64 division, torch
    round-half-even): absmax per row of X and per row of W over all K."""
    x = torch.from_numpy(X.astype(np.float64))
    w = torch.from_numpy(W.astype(np.float64))
    ax = x.abs().amax(dim=1, keepdim=True)
    aw = w.abs().amax(dim=1, keepdim=True)
    xq = torch.where(ax > 0, torch.round(127.0 * x / ax), torch.zeros_like(x))
    wq = torch.where(aw > 0, torch.round(127.0 * w / aw), torch.zeros_like(w))
    c = xq @ wq.T
    return xq.numpy(), wq.numpy(), c.numpy(), (c * ax * aw.T / 127.0 ** 2).numpy()


def test_threshold_inf_is_pure_int8():
    c = workloads.make_case("t", 48, 200, 40, seed=5, n_out=3, lo=8, hi=60)
    Wq, a_w = ref.prepare_weight_ref(c.W)
    Y, st = ref.int8_matmul_ref(c.X, Wq, a_w, math.inf, stages=True)
    xq, wq, cc, y = _plain_vectorwise_int8(c.X, c.W)
    assert st["O"].size == 0
    assert np.array_equal(st["Xq"].astype(np.float64), xq)
    assert np.array_equal(Wq.astype(np.float64), wq)
    assert np.array_equal(st["C"].astype(np.float64), cc)
    assert np.all(np.abs(Y.astype(np.float64) - y) <= ref.fp16_ulp(y) + 1e-6 * np.abs(y))


def test_threshold_zero_is_fp16_matmul():
    c = workloads.make_case("t", 40, 150, 56, seed=6, n_out=2)
    X = c.X.copy()
    X[:, 7] = 0  # an all-zero column stays regular (0 is not > 0) and adds 0
    Wq, a_w = ref.prepare_weight_ref(c.W)
    Y, st = ref.int8_matmul_ref(X, Wq, a_w, 0.0, stages=True)
    assert not st["C"].any()
    assert st["O"].size == X.shape[1] - 1 and 7 not in st["O"]
    W_hat = ((Wq.astype(np.float32) * a_w[:, None]) / np.float32(127)).astype(np.float16)
    Z = X.astype(np.float64) @ W_hat.astype(np.float64).T
    slack = X.shape[1] * 2.0 ** -23 * (np.abs(X.astype(np.float64)) @ np.abs(W_hat.astype(np.float64)).T)
    assert np.all(np.abs(Y.astype(np.float64) - Z) <= ref.fp16_ulp(Z) + slack)


def test_outlier_count_monotone_in_threshold():
    X, _ = workloads.make_x(256, 512, seed=9, n_out=12, kind="t3")
    prev = None
    for t in [0.0, 0.5, 1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0, 20.0, math.inf]:
        mask, O, _ = ref.outlier_mask_ref(X, t)
        if prev is not None:
            assert np.all(prev | ~mask)  # mask(t_high) is a subset of mask(t_low)
        prev = mask


def test_strict_threshold_comparison():
    X = np.array([[6.0, 6.00390625, -6.0], [1.0, 1.0, 1.0]], np.float16)
    mask, O, _ = ref.outlier_mask_ref(X, 6.0)
    assert O.tolist() == [1]


# ---------------------------------------------------------------- whole-method properties


def test_error_bound_against_exact_product():
    """|Y - X W^T| is within the quantization error the method allows."""
    c = workloads.make_case("t", 64, 256, 48, seed=12, n_out=4, lo=8, hi=60)
    Wq, a_w = ref.prepare_weight_ref(c.W)
    Y, st = ref.int8_matmul_ref(c.X, Wq, a_w, 6.0, stages=True)
    X = c.X.astype(np.float64)
    W = c.W.astype(np.float64)
    exact = X @ W.T
    R = ~st["mask"]
    W_hat = Wq.astype(np.float64) * a_w.astype(np.float64)[:, None] / 127.0
    bound = (np.abs(X[:, R]) @ np.full((R.sum(), W.shape[0]), 1.0) * (a_w.astype(np.float64)[None, :] / 254.0)
             + (st["a_x"].astype(np.float64)[:, None] / 254.0) * (np.ones((X.shape[0], R.sum())) @ np.abs(W_hat[:, R]).T))
    O = st["O"]
    W_O = st["W_O"].astype(np.float64)  # [|O|][N]
    bound += np.abs(X[:, O]) @ np.abs(W[:, O].T - W_O)
    absprod = np.abs(X) @ np.abs(W_hat).T
    bound += 2.0 ** -11 * np.abs(exact) + 2.0 ** -11 * bound + 64 * 2.0 ** -24 * absprod + 1e-6
    assert np.all(np.abs(Y.astype(np.float64) - exact) <= bound)
    # and the decomposition beats plain int8 on these outlier inputs
    _, _, _, y_plain = _plain_vectorwise_int8(c.X, c.W)
    assert np.abs(Y.astype(np.float64) - exact).mean() < np.abs(y_plain - exact).mean()


def test_permutation_equivariance():
    c = workloads.make_case("t", 32, 96, 24, seed=13, n_out=3)
    Wq, a_w = ref.prepare_weight_ref(c.W)
    Y, st = ref.int8_matmul_ref(c.X, Wq, a_w, 6.0, stages=True)
    rng = np.random.default_rng(0)
    pk = rng.permutation(c.K)
    Y2, st2 = ref.int8_matmul_ref(c.X[:, pk], Wq[:, pk], a_w, 6.0, stages=True)
    assert np.array_equal(st2["C"], st["C"])
    assert np.array_equal(st2["mask"], st["mask"][pk])
    assert np.array_equal(st2["a_x"], st["a_x"])
    pm = rng.permutation(c.M)
    Y3, st3 = ref.int8_matmul_ref(c.X[pm], Wq, a_w, 6.0, stages=True)
    assert np.array_equal(Y3, Y[pm])
    assert np.array_equal(st3["Xq"], st["Xq"][pm])


def test_exact_integer_example():
    """With every regular row absmax equal to 127 and integer entries, the
    codes are the entries themselves, every scale product is 127*127, and Y
    is the plain integer matmul (exact in fp16 below 2048)."""
    rng = np.random.default_rng(21)
    M, K, N = 6, 10, 5
    X = rng.integers(-9, 10, (M, K)).astype(np.float64)
    X[:, 0] = 127 * rng.choice([-1, 1], M)  # row absmax over R = 127
    X[:, 4] = rng.integers(130, 200, M) * rng.choice([-1, 1], M)  # outlier column
    W = rng.integers(-3, 4, (N, K)).astype(np.float64)
    W[:, 9] = 127
    t = 128.0
    Wq, a_w = ref.prepare_weight_ref(W.astype(np.float16))
    assert np.array_equal(Wq, W.astype(np.int8)) and np.all(a_w == 127)
    Y, st = ref.int8_matmul_ref(X.astype(np.float16), Wq, a_w, t, stages=True)
    assert st["O"].tolist() == [4]
    Xr = X.copy()
    Xr[:, 4] = 0
    assert np.array_equal(st["Xq"], Xr.astype(np.int8))
    expect = X @ W.T
    assert np.abs(expect).max() < 2048
    assert np.array_equal(Y.astype(np.float64), expect)


# ---------------------------------------------------------------- workloads


@pytest.mark.parametrize("name,count", [("tiny", 2), ("q_proj", 6), ("ffn_up", 20),
                                        ("ffn_down", 55), ("decode1", 8), ("decode16", 8)])
def test_workload_outlier_columns_are_the_planted_ones(name, count):
    case = workloads.config_case(name, with_w=False)
    mask, O, _ = ref.outlier_mask_ref(case.X, 6.0)
    assert O.tolist() == case.outlier_cols.tolist()
    assert O.size == count


def test_sweep_workload_outlier_counts():
    case = workloads.config_case("sweep13b", with_w=False)
    counts = {}
    for t in workloads.SWEEP_THRESHOLDS:
        mask, O, _ = ref.outlier_mask_ref(case.X, t)
        counts[t] = O.size
    assert counts[math.inf] == 0
    assert counts[0.0] == case.K
    assert set(case.outlier_cols.tolist()) <= set(np.flatnonzero(ref.outlier_mask_ref(case.X, 7.0)[0]).tolist())
    assert counts[5.0] >= counts[6.0] >= counts[7.0] >= 51
