"""GPU parity of the HIP path (through the C ABI) against the CPU oracle,
element by element, on seeded inputs at sizes the oracle finishes in
seconds: several tiles, ragged tails, both kernels (decode M <= 16 and the
prefill tile GEMM), and the method's degenerate cases."""

import math

import numpy as np
import pytest

import workloads
from gpu_cases import run_case, check_prepare, to_dev

pytestmark = pytest.mark.gpu


def _case(M, K, N, seed, n_out=3, lo=8.0, hi=60.0, kind="uniform", wstd=0.02):
    X, _ = workloads.make_x(M, K, seed, n_out, lo, hi, kind)
    W = workloads.make_w(N, K, seed, wstd)
    return X, W


SHAPES = [
    # (M, K, N, n_out, t)          decode path: M <= 16
    (1, 64, 16, 1, 6.0),
    (1, 1, 1, 0, 6.0),
    (4, 1000, 300, 2, 6.0),
    (16, 1024, 1024, 2, 6.0),
    (5, 3, 7, 1, 6.0),
    (16, 520, 100, 4, 0.0),
    (9, 200, 33, 3, math.inf),
    # the few-rows activation launch at each of its widths: 256 threads up to
    # K = 2048, 1024 threads up to 8192, two chunks per thread up to 16384;
    # past that the general mask and row passes
    (1, 2056, 64, 2, 6.0),
    (16, 8192, 48, 3, 6.0),
    (16, 8200, 64, 3, 6.0),
    (1, 16384, 40, 2, 6.0),
    (16, 16384, 48, 4, 6.0),
    (3, 16392, 40, 2, 6.0),
    # decode grids that cover more 16-row groups than the prepared weight's
    # padded rows hold (8704 rows: 546 groups launched for 544), and G = 3
    # groups per workgroup not dividing the group count (11008 rows)
    (1, 1024, 8704, 3, 6.0),
    (16, 1024, 8704, 3, 6.0),
    (16, 4096, 11008, 4, 6.0),
    # one row: the decode kernel codes X itself up to ldk = 16384 -- many
    # outlier steps (its static schedule), t = 0 (a_x = 0), t = inf, 2049
    # groups of 16 rows (8 per workgroup); past 16384 the activation launch.
    # The same cases at two to four rows (activation launch, then decode).
    (1, 2048, 300, 40, 6.0),
    (1, 520, 100, 4, 0.0),
    (1, 200, 33, 3, math.inf),
    (1, 512, 32784, 3, 6.0),
    (1, 16392, 40, 2, 6.0),
    (2, 8192, 300, 40, 6.0),
    (4, 520, 100, 4, 0.0),
    (2, 200, 33, 3, math.inf),
    (4, 512, 32784, 3, 6.0),
    (3, 8200, 64, 3, 6.0),
    # two to four rows coded inside the decode kernel (ldk <= 8192, up to 7
    # weight groups per workgroup): three rows (the fourth repeats the
    # third), two rows over 3 groups per workgroup, four rows at ldk = 8192
    (3, 4096, 700, 5, 6.0),
    (2, 1024, 8704, 3, 6.0),
    (4, 8192, 96, 6, 6.0),
    # prefill path: M > 16
    (17, 1024, 1024, 2, 6.0),
    (300, 520, 300, 5, 6.0),
    (257, 257, 257, 3, 6.0),
    (33, 37, 29, 2, 6.0),          # K % 8 != 0: unaligned rows of X
    (512, 1024, 768, 6, 6.0),
    (256, 4096, 256, 20, 6.0),
    (64, 130, 40, 2, 0.0),         # every non-zero column is an outlier
    (96, 320, 96, 4, math.inf),    # pure int8
    (40, 96, 520, 90, 0.5),        # |O| close to K
    (300, 2112, 520, 7, 6.0),      # few tiles: each as two 256x128 halves, odd step count
    (260, 2048, 300, 2, 0.0),      # half-tile grid with every column an outlier
    (300, 9000, 64, 5, 6.0),       # rows too long for one wave: a block per row
    (300, 4700, 64, 5, 6.0),       # row pass held in 10 chunks per lane (4 waves per SIMD)
    (280, 2600, 64, 3, 6.0),       # ... 6 chunks per lane
    (40, 10000, 64, 3, 6.0),       # a block per row, 6 chunks per lane
    # rows of exactly the form's chunks (no per-chunk tests): a wave per row
    # with 6, 12 and 16 chunks per lane, a block per row with 4, 6 and 8
    (300, 3072, 64, 3, 6.0),
    (264, 6144, 40, 2, 6.0),
    (272, 8192, 64, 3, 6.0),
    (100, 8192, 64, 3, 6.0),
    (40, 12288, 64, 3, 6.0),
    (20, 16384, 64, 2, 6.0),
    # more tiles than CUs with a short last round: its 14 tiles run as
    # 256x128 halves (one group of 8 pairs, 6 adjacent pairs), ragged in M
    # and N; then the same with more than three fp16 outlier steps (the
    # first half of each pair computes the whole tile)
    (2200, 96, 7600, 3, 6.0),
    (2200, 256, 7600, 100, 6.0),
    # more rows than one pass of the row-pass blocks covers: a wave per row
    # beyond 4 * 2048 rows (two and three passes), a block per row beyond
    # 2048 rows, and the streamed form (unaligned rows) beyond 8192 rows
    (8300, 256, 72, 3, 6.0),
    (20000, 128, 40, 2, 6.0),
    (2100, 9000, 64, 5, 6.0),
    (8250, 100, 40, 2, 6.0),
]


@pytest.mark.parametrize("M,K,N,n_out,t", SHAPES)
def test_parity_shapes(lib, M, K, N, n_out, t):
    print(f"case M={M} K={K} N={N} n_out={n_out} t={t}", flush=True)
    X, W = _case(M, K, N, seed=M * 7919 + K * 31 + N, n_out=n_out)
    run_case(lib, X, W, t)


def test_threshold_equal_to_column_max_is_not_outlier(lib):
    X, W = _case(40, 256, 64, seed=3, n_out=0)
    X[:, 10] = np.float16(0.5)
    X[7, 10] = np.float16(6.0)   # column max exactly t: stays regular
    X[3, 20] = np.float16(6.00390625)  # next fp16 above t: outlier
    X[:, 30] = np.float16(-6.0)
    for M in (40, 8):
        Y, _ = run_case(lib, X[:M].copy(), W, 6.0)
    for r in (7, 3):  # one row holding the column max (M = 1)
        run_case(lib, X[r:r + 1].copy(), W, 6.0)


def test_zero_rows_and_columns(lib):
    X, W = _case(48, 200, 80, seed=4, n_out=3)
    X[5] = 0            # all-zero row: scale 0, codes 0
    X[:, 17] = 0        # all-zero column
    W[9] = 0            # all-zero weight channel: a_w = 0
    run_case(lib, X, W, 6.0)
    run_case(lib, X[:12].copy(), W, 6.0)
    # a row whose only non-zero entries are outliers: empty R-range -> a_x = 0
    X2 = X.copy()
    X2[6] = 0
    X2[6, 3] = 50.0
    run_case(lib, X2, W, 6.0)
    # the same rows alone (coded inside the decode kernel) and among four
    run_case(lib, X[5:6].copy(), W, 6.0)
    run_case(lib, X2[6:7].copy(), W, 6.0)
    run_case(lib, X2[4:8].copy(), W, 6.0)


def test_exact_ties_round_half_even(lib):
    rng = np.random.default_rng(8)
    M, K, N = 32, 128, 48
    # rows with R-absmax 127/32 and entries odd/64: 127*x/a = 32*x is an exact .5 tie
    X = (rng.integers(-127, 128, (M, K)) * 2 + 1).astype(np.float32) / 64.0
    X = np.clip(X, -3.96875, 3.96875)
    X[:, 0] = 3.96875
    X = X.astype(np.float16)
    W = (rng.integers(-127, 128, (N, K)) * 2 + 1).astype(np.float32) / 64.0
    W = np.clip(W, -3.96875, 3.96875)
    W[:, 1] = -3.96875
    W = W.astype(np.float16)
    for m in (M, 7, 1):
        run_case(lib, X[:m].copy(), W, 6.0)


def test_heavy_tailed_sweep_small(lib):
    X, W = _case(128, 320, 200, seed=12, n_out=8, kind="t3")
    for t in workloads.SWEEP_THRESHOLDS:
        run_case(lib, X, W, t)


def test_prepare_weight_ties_and_odd_shapes(lib):
    rng = np.random.default_rng(2)
    W = (rng.integers(-127, 128, (37, 257)) * 2 + 1).astype(np.float32) / 64.0
    W = np.clip(W, -3.96875, 3.96875)
    W[:, 5] = 3.96875
    check_prepare(lib, W.astype(np.float16))
    check_prepare(lib, workloads.make_w(3, 1, 5))
    check_prepare(lib, np.zeros((4, 70), np.float16))


@pytest.mark.parametrize("N,K", [(6, 32768), (5, 32769), (3, 40000), (9, 1001), (4, 2048)])
def test_prepare_weight_row_lengths(lib, N, K):
    # rows held in registers up to 32768 columns (load rounds 1 .. 16), the
    # two-pass form beyond; K % 8 != 0 takes the element-wise loads
    print(f"case prepare N={N} K={K}", flush=True)
    W = workloads.make_w(N, K, N * 100003 + K, 0.02)
    W[:, K // 3] = np.float16(-0.5)  # the absmax at a negative entry
    check_prepare(lib, W)


def test_empty_and_degenerate_shapes(lib):
    import torch
    mm = lib
    W = workloads.make_w(8, 64, 1)
    Wq, s = mm.int8_prepare_weight(to_dev(W))
    # M == 0: empty output, no work
    Y = mm.int8_matmul(torch.empty((0, 64), dtype=torch.float16, device="cuda"), Wq, s)
    assert Y.shape == (0, 8)
    # K == 0: empty contraction -> Y == 0
    W0 = torch.empty((8, 0), dtype=torch.float16, device="cuda")
    Wq0, s0 = mm.int8_prepare_weight(W0)
    X0 = torch.empty((5, 0), dtype=torch.float16, device="cuda")
    Y0 = mm.int8_matmul(X0, Wq0, s0)
    torch.cuda.synchronize()
    assert Y0.shape == (5, 8) and not Y0.float().abs().sum().item()
    assert not s0.abs().sum().item()


def test_workspace_reuse_across_shapes(lib):
    """One workspace sized for the largest call, reused by smaller ones in a row
    (its contents on entry must not matter)."""
    import torch
    mm = lib
    ws = mm.workspace_for(300, 520, 300, "cuda")
    ws.fill_(0xAB)
    from oracle import int8mm_ref as ref
    from gpu_cases import check_y
    for (M, K, N, t) in [(300, 520, 300, 6.0), (40, 520, 300, 0.0), (3, 520, 300, 6.0),
                         (300, 520, 300, math.inf)]:
        X, W = _case(M, K, N, seed=M + N, n_out=4)
        Wq, s = mm.int8_prepare_weight(to_dev(W))
        Y = mm.int8_matmul(to_dev(X), Wq, s, threshold=t, workspace=ws)
        torch.cuda.synchronize()
        Wq_r, s_r = ref.prepare_weight_ref(W)
        Y_r, st = ref.int8_matmul_ref(X, Wq_r, s_r, t, stages=True)
        check_y(Y.cpu().numpy(), Y_r, X, Wq_r, s_r, st["O"].size)


def test_output_overflow_gives_inf(lib):
    # |Y| beyond the fp16 range becomes +-inf in both paths
    M, K, N = 20, 64, 16
    X = np.full((M, K), 100.0, np.float16)
    W = np.full((N, K), 60.0, np.float16)
    W[1] = -60.0
    Y, Y_ref = run_case(lib, X, W, 1000.0)
    assert np.isinf(Y_ref).all()


@pytest.mark.parametrize("M,t", [(3, math.inf), (20, math.inf), (3, 6.0), (20, 6.0)])
def test_maximum_k_at_the_int32_bound(lib, M, t):
    # K = the largest accepted: every code is +-127, so |C| reaches
    # 127^2 * K = 2147479576 (just below 2^31) with no outlier column, on
    # both kernels (decode M <= 16, prefill in 256x128 half tiles); with t = 6
    # three planted columns leave the int8 part
    K, N = 133144, 64
    print(f"case max K M={M} K={K} N={N} t={t}", flush=True)
    X = np.ones((M, K), np.float16)
    X[1::2] = np.float16(-1.0)
    if t != math.inf:
        X[:, [7, 70000, K - 1]] = np.float16(30.0)
    W = np.full((N, K), 0.25, np.float16)
    W[::3] = np.float16(-0.25)
    Y, Y_ref = run_case(lib, X, W, t)
    if t == math.inf:  # |C| = 127^2 K exactly (checked bit for bit by run_case): Y = fp16(K/4)
        assert np.all(np.abs(Y_ref) == np.float16(0.25 * K))


def test_wrong_shaped_outputs_are_refused(lib):
    import torch
    X, W = _case(32, 128, 64, seed=21, n_out=2)
    Xd, Wd = to_dev(X), to_dev(W)
    Wq, s = lib.int8_prepare_weight(Wd)
    with pytest.raises(ValueError, match="shape"):
        lib.int8_matmul(Xd, Wq, s, out=torch.empty((32, 63), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError, match="shape"):
        lib.int8_linear(Xd, Wq, s, out=torch.empty((31, 64), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError, match="shape"):
        lib.int8_prepare_weight(Wd, out=(torch.empty((64, 128), dtype=torch.int8, device="cuda"), s))
    with pytest.raises(ValueError, match="shape"):
        lib.int8_prepare_weight(Wd, out=(torch.empty_like(Wq), torch.empty((63,), device="cuda")))
    # the right shapes are accepted
    Y = lib.int8_matmul(Xd, Wq, s, out=torch.empty((32, 64), dtype=torch.float16, device="cuda"))
    assert Y.shape == (32, 64)
