"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's arithmetic (on the
CPU, by monkeypatching the oracle module) and checks that at least one of
the independent pins in ``test_oracle`` then fails.  This is what makes the
pins a check of the oracle rather than a restatement of it.
"""

import math

import numpy as np
import pytest

from oracle import int8mm_ref as ref
import test_oracle as pins
import test_accuracy_study as study

_orig = {n: getattr(ref, n) for n in ("quantize_rows_ref", "outlier_mask_ref",
                                      "quantize_activation_ref", "outlier_slices_ref",
                                      "outlier_gemm_ref", "epilogue_ref", "int8_gemm_ref",
                                      "prepare_weight_ref")}


def _round_half_away(A16, scale):
    A32 = np.asarray(A16, np.float16).astype(np.float32)
    s = np.asarray(scale, np.float32).reshape(-1, 1)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = A32 * np.float32(127) / s
        q = np.sign(r) * np.floor(np.abs(r) + np.float32(0.5))
    q = np.where(s == 0, 0, q)
    return np.clip(q, -127, 127).astype(np.int8)


def _reciprocal_multiply(A16, scale):
    A32 = np.asarray(A16, np.float16).astype(np.float32)
    s = np.asarray(scale, np.float32).reshape(-1, 1)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(A32 * (np.float32(127) / s))
    q = np.where(s == 0, 0, q)
    return np.clip(q, -127, 127).astype(np.int8)


def _mask_ge(X16, t):
    X16 = np.asarray(X16, np.float16)
    colmax = np.abs(X16).max(axis=0).astype(np.float32)
    mask = colmax >= np.float32(t)
    return mask, np.flatnonzero(mask), colmax


def _scale_over_all_columns(X16, mask):
    X16 = np.asarray(X16, np.float16)
    a_x = np.abs(X16).max(axis=1).astype(np.float32)
    XR = np.where(mask[None, :], np.float16(0), X16)
    return _orig["quantize_rows_ref"](XR, a_x), a_x


def _per_tensor_scale(X16, mask):
    XR = np.where(mask[None, :], np.float16(0), np.asarray(X16, np.float16))
    a = np.float32(np.abs(XR).max()) if XR.size else np.float32(0)
    a_x = np.full(XR.shape[0], a, np.float32)
    return _orig["quantize_rows_ref"](XR, a_x), a_x


def _drop_outlier_term(X_O, W_O, N):
    return np.zeros((X_O.shape[0], N), np.float32)


def _outlier_weight_not_dequantized(X16, Wq, a_w, O):
    X_O = np.asarray(X16, np.float16)[:, O]
    return X_O, Wq[:, O].astype(np.float16).T.copy()


def _b32(bias):
    return 0 if bias is None else np.asarray(bias, np.float16).astype(np.float32)[None, :]


def _epilogue_single_127(C, a_x, a_w, Y_O, bias=None):
    s = (a_x[:, None] * a_w[None, :]).astype(np.float32) / np.float32(127)
    with np.errstate(over="ignore"):
        return (C.astype(np.float32) * s + Y_O + _b32(bias)).astype(np.float16)


def _epilogue_wrong_sign(C, a_x, a_w, Y_O, bias=None):
    s = (a_x[:, None] * a_w[None, :]).astype(np.float32) / np.float32(16129)
    with np.errstate(over="ignore"):
        return (C.astype(np.float32) * s - Y_O + _b32(bias)).astype(np.float16)


def _bias_dropped(C, a_x, a_w, Y_O, bias=None):
    return _orig["epilogue_ref"](C, a_x, a_w, Y_O, None)


def _bias_sign(C, a_x, a_w, Y_O, bias=None):
    nb = None if bias is None else -np.asarray(bias, np.float16)
    return _orig["epilogue_ref"](C, a_x, a_w, Y_O, nb)


def _bias_reversed_index(C, a_x, a_w, Y_O, bias=None):
    rb = None if bias is None else np.asarray(bias, np.float16)[::-1].copy()
    return _orig["epilogue_ref"](C, a_x, a_w, Y_O, rb)


# (Forming W_O as fp16(fp32(Wq/127) * a_w) is not among the mistakes: the two
# fp32 roundings can move the value by one fp32 ulp, but the exact quotient
# q*a_w/127 is never within about 2^-19 (relative) of an fp16 rounding tie, so the
# fp16 result is the same for every code and scale.)


def _outlier_columns_shifted(X16, Wq, a_w, O):
    # the slices taken one feature to the right of the outlier columns
    K = np.asarray(X16).shape[1]
    return _orig["outlier_slices_ref"](X16, Wq, a_w, (np.asarray(O) + 1) % max(K, 1))


def _weight_scale_per_tensor(W16):
    W16 = np.asarray(W16, np.float16)
    N, K = W16.shape
    if K == 0:
        return np.zeros((N, 0), np.int8), np.zeros(N, np.float32)
    a = np.float32(np.abs(W16).max())
    a_w = np.full(N, a, np.float32)
    return _orig["quantize_rows_ref"](W16, a_w), a_w


def _gemm_transposed_k(Xq, Wq, chunk=2048):
    # contracts against the reversed feature axis of W
    return _orig["int8_gemm_ref"](Xq, Wq[:, ::-1].copy(), chunk)


MUTATIONS = {
    "round_half_away_from_zero": ("quantize_rows_ref", _round_half_away),
    "reciprocal_multiply": ("quantize_rows_ref", _reciprocal_multiply),
    "non_strict_threshold": ("outlier_mask_ref", _mask_ge),
    "row_scale_over_all_columns": ("quantize_activation_ref", _scale_over_all_columns),
    "per_tensor_activation_scale": ("quantize_activation_ref", _per_tensor_scale),
    "dropped_outlier_term": ("outlier_gemm_ref", _drop_outlier_term),
    "outlier_weight_not_dequantized": ("outlier_slices_ref", _outlier_weight_not_dequantized),
    "dequant_by_127_not_127sq": ("epilogue_ref", _epilogue_single_127),
    "outlier_term_sign": ("epilogue_ref", _epilogue_wrong_sign),
    "gemm_wrong_k_index": ("int8_gemm_ref", _gemm_transposed_k),
    "outlier_columns_shifted": ("outlier_slices_ref", _outlier_columns_shifted),
    "weight_scale_per_tensor": ("prepare_weight_ref", _weight_scale_per_tensor),
    "bias_dropped": ("epilogue_ref", _bias_dropped),
    "bias_wrong_sign": ("epilogue_ref", _bias_sign),
    "bias_wrong_index": ("epilogue_ref", _bias_reversed_index),
}


def _run_pins():
    """Returns the names of the pins that fail."""
    failed = []
    checks = [
        ("closed_form", pins.test_quantizer_closed_form_exhaustive, (0,)),
        ("ties", pins.test_quantizer_ties_round_half_even, ()),
        ("invariants", pins.test_quantizer_invariants, ()),
        ("bf_4x8x4", pins.test_bruteforce_4x8x4_with_outlier_and_ties, ()),
        ("t_inf", pins.test_threshold_inf_is_pure_int8, ()),
        ("t_zero", pins.test_threshold_zero_is_fp16_matmul, ()),
        ("error_bound", pins.test_error_bound_against_exact_product, ()),
        ("exact_integer", pins.test_exact_integer_example, ()),
        ("strict", pins.test_strict_threshold_comparison, ()),
        ("bf_bias_4x8x4", pins.test_bruteforce_4x8x4_with_bias, ()),
        ("accuracy_claims", study.test_accuracy_claims_on_the_oracle, ()),
        ("w_o_exhaustive", pins.test_dequantized_outlier_weight_exhaustive, ()),
    ] + [(f"bf_random_{s}", pins.test_bruteforce_random_small, (s,)) for s in range(6)] + [
        (f"bf_bias_random_{s}", pins.test_bruteforce_random_small_with_bias, (s,))
        for s in range(4)]
    for name, fn, args in checks:
        try:
            with np.errstate(all="ignore"):
                fn(*args)
        except (AssertionError, ValueError, IndexError):
            failed.append(name)
    return failed


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, monkeypatch):
    name, fn = MUTATIONS[mutation]
    monkeypatch.setattr(ref, name, fn)
    failed = _run_pins()
    assert failed, f"planted mistake '{mutation}' passed every pin"


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins() == []
