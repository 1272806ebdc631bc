"""The accuracy study through the HIP path (see accuracy_cases): on
synthetic outlier inputs at a prefill shape, the decomposed matmul's error
against the exact product, per threshold, matches the oracle's, and the
pages' claims about outliers, scales and the threshold hold for it."""

import math

import numpy as np
import pytest

import accuracy_cases as ac
from gpu_cases import check_prepare, check_y, to_dev
from oracle import int8mm_ref as ref

pytestmark = pytest.mark.gpu


def test_accuracy_study_on_the_gpu(lib):
    import torch
    M, K, N = 1024, 4096, 1024
    print(f"case accuracy study M={M} K={K} N={N}", flush=True)
    X, W = ac.study_inputs(M, K, N, seed=2025)
    Wq_d, s_d, Wq_r, s_r = check_prepare(lib, W)
    X_d = to_dev(X)
    Ye = ac.exact_product(X, W)
    errs, errs_ref, n_out = {}, {}, {}
    for t in ac.THRESHOLDS:
        Y = lib.int8_matmul(X_d, Wq_d, s_d, threshold=t)
        torch.cuda.synchronize()
        Y = Y.cpu().numpy()
        Y_ref, st = ref.int8_matmul_ref(X, Wq_r, s_r, t, stages=True)
        check_y(Y, Y_ref, X, Wq_r, s_r, st["O"].size)
        errs[t] = ac.rel_err(Y, Ye)
        errs_ref[t] = ac.rel_err(Y_ref, Ye)
        n_out[t] = st["O"].size
        assert abs(errs[t] - errs_ref[t]) <= 0.01 * errs_ref[t], (t, errs[t], errs_ref[t])
    pt = ac.rel_err(ac.per_tensor_int8(X, W), Ye)
    f16 = ac.rel_err(ac.fp16_matmul(X, W), Ye)
    t0 = ac.rel_err(ac.dequantized_weight_product(X, Wq_r, s_r), Ye)
    print(ac.format_table(errs, pt, f16, n_out), flush=True)
    ac.check_claims(errs, pt, f16, t0)
