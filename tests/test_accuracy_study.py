"""The accuracy study on the CPU oracle (see accuracy_cases): the pages'
claims about outliers, scales and the threshold hold for the oracle's
decomposition on synthetic outlier inputs."""

import math

import numpy as np

import accuracy_cases as ac
from oracle import int8mm_ref as ref


def test_accuracy_claims_on_the_oracle():
    X, W = ac.study_inputs(256, 1024, 256, seed=2024)
    Wq, a_w = ref.prepare_weight_ref(W)
    Ye = ac.exact_product(X, W)
    errs, n_out = {}, {}
    for t in ac.THRESHOLDS:
        Y, st = ref.int8_matmul_ref(X, Wq, a_w, t, stages=True)
        errs[t] = ac.rel_err(Y, Ye)
        n_out[t] = st["O"].size
    pt = ac.rel_err(ac.per_tensor_int8(X, W), Ye)
    f16 = ac.rel_err(ac.fp16_matmul(X, W), Ye)
    t0 = ac.rel_err(ac.dequantized_weight_product(X, Wq, a_w), Ye)
    print(ac.format_table(errs, pt, f16, n_out))
    ac.check_claims(errs, pt, f16, t0)
    assert n_out[math.inf] == 0 and n_out[0.0] == np.count_nonzero(np.abs(X).max(axis=0))
