"""Shared driver of the GPU parity tests: run the HIP path through the C ABI
(via the binding) and the oracle on the same seeded inputs, and compare.

Bar: bit-exact for the mask, |O|, O, the int8 codes, both scales, the
compacted fp16 slices and the int32 accumulators; for Y the tolerance
|dY| <= 1e-2 (|X| |W_hat|^T) + 1e-3, plus a tighter check of one fp16 ulp
plus fp32 slack that catches any real arithmetic difference.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import int8mm_ref as ref


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_prepare(mm, W16: np.ndarray):
    N, K = W16.shape
    Wq_d, s_d = mm.int8_prepare_weight(to_dev(W16))
    torch.cuda.synchronize()
    Wq = mm.untile(Wq_d, Wq_d.shape[0]).cpu().numpy()  # [Np][ldk] row-major
    s = s_d.cpu().numpy()
    Wq_r, s_r = ref.prepare_weight_ref(W16)
    assert np.array_equal(s, s_r), "w_scale"
    assert np.array_equal(Wq[:N, :K], Wq_r), "Wq"
    assert not Wq[:N, K:].any(), "Wq padding columns"
    assert not Wq[N:].any(), "Wq padding rows"
    return Wq_d, s_d, Wq_r, s_r


def y_bounds(X16, Wq_r, s_r, Y_ref, n_out, bias=None):
    """(method tolerance, tight bound).  The tight bound allows one fp16
    ulp of the result plus the fp32 rounding that different summation orders
    of the |O| outlier products, the rescaled int32 term and the bias (when
    there is one) can produce."""
    loose = ref.tolerance_bound(X16, Wq_r, s_r, bias=bias)
    absprod = ref.tolerance_bound(X16, Wq_r, s_r, rel=1.0, abs_=0.0)
    mag = absprod
    if bias is not None:
        mag = mag + np.abs(np.asarray(bias, np.float16).astype(np.float64))[None, :]
    tight = ref.fp16_ulp(Y_ref.astype(np.float64)) + (n_out + 16) * 2.0 ** -23 * mag
    return loose, tight


def check_y(Y: np.ndarray, Y_ref: np.ndarray, X16, Wq_r, s_r, n_out, what="Y", bias=None):
    loose, tight = y_bounds(X16, Wq_r, s_r, Y_ref, n_out, bias)
    y = Y.astype(np.float64)
    yr = Y_ref.astype(np.float64)
    fin = np.isfinite(yr)
    assert np.array_equal(np.isfinite(y), fin), f"{what}: non-finite pattern"
    assert np.array_equal(y[~fin], yr[~fin]), f"{what}: infinities"
    d = np.abs(y[fin] - yr[fin])
    assert np.all(d <= loose[fin]), f"{what}: max excess {np.max(d - loose[fin])}"
    bad = d > tight[fin]
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond 1 ulp, worst {np.max(d - tight[fin])}"


def run_stages(mm, X16, Wq_d, s_d, t, Wq_r, s_r):
    """Stage-by-stage comparison; returns the oracle result dict."""
    M, K = X16.shape
    X_d = to_dev(X16)
    o = mm.int8_matmul_stages(X_d, Wq_d, s_d, threshold=t, want_c=True)
    torch.cuda.synchronize()
    Y_ref, st = ref.int8_matmul_ref(X16, Wq_r, s_r, t, stages=True)
    nO = int(o["n_outliers"].item())
    O = st["O"]
    assert nO == O.size, f"|O| {nO} vs {O.size}"
    assert np.array_equal(o["mask"].cpu().numpy().astype(bool), st["mask"]), "mask"
    assert np.array_equal(o["outlier_idx"].cpu().numpy()[:nO], O), "O"
    assert np.array_equal(o["x_scale"].cpu().numpy(), st["a_x"]), "x_scale"
    Xq = o["Xq"].cpu().numpy()
    assert np.array_equal(Xq[:, :K], st["Xq"]), "Xq"
    assert not Xq[:, K:].any(), "Xq padding"
    opad = (nO + 63) // 64 * 64
    XO = o["X_O"].cpu().numpy()
    assert np.array_equal(XO[:, :nO].view(np.uint16), st["X_O"].view(np.uint16)), "X_O"
    assert not XO[:, nO:opad].view(np.uint16).any(), "X_O padding"
    WO = o["W_O"].cpu().numpy()
    assert np.array_equal(WO[:, :nO].view(np.uint16), st["W_O"].T.view(np.uint16)), "W_O"
    assert not WO[:, nO:opad].view(np.uint16).any(), "W_O padding"
    C = o["C"].cpu().numpy()
    assert np.array_equal(C, st["C"]), f"C: {np.count_nonzero(C != st['C'])} mismatches"
    return Y_ref, st, X_d


def run_case(mm, X16, W16, t, stages=True, repeat=2):
    Wq_d, s_d, Wq_r, s_r = check_prepare(mm, W16)
    if stages:
        Y_ref, st, X_d = run_stages(mm, X16, Wq_d, s_d, t, Wq_r, s_r)
    else:
        X_d = to_dev(X16)
        Y_ref, st = ref.int8_matmul_ref(X16, Wq_r, s_r, t, stages=True)
    Ys = []
    for _ in range(repeat):
        Ys.append(mm.int8_matmul(X_d, Wq_d, s_d, threshold=t))
    torch.cuda.synchronize()
    Y = Ys[0].cpu().numpy()
    check_y(Y, Y_ref, X16, Wq_r, s_r, st["O"].size)
    for Y2 in Ys[1:]:
        assert np.array_equal(Y2.cpu().numpy().view(np.uint16), Y.view(np.uint16)), "nondeterministic Y"
    if X16.shape[0] == 1:
        # one row: int8_matmul codes X inside the decode kernel; the stage
        # call takes the activation launch, whose codes were checked above
        Ys = mm.int8_matmul_stages(X_d, Wq_d, s_d, threshold=t, want_c=False)["Y"]
        torch.cuda.synchronize()
        assert np.array_equal(Ys.cpu().numpy().view(np.uint16), Y.view(np.uint16)), "one-row Y"
    return Y, Y_ref
