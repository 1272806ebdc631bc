"""Fixtures under tests/golden: constants the pages fix, and a frozen record
of the oracle on the tiny workload (written by tests/golden/make_golden.py)."""

import inspect
import json
import math
import os

import numpy as np

from oracle import int8mm_ref as ref
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_pages_constants():
    facts = _load("pages_facts.json")["facts"]
    assert ref.Q_MAX == facts["scale_divisor"]["value"]
    lo, hi = facts["clamp_range"]["value"]
    q = ref.quantize_rows_ref(np.array([[-65504.0, 65504.0, 1.0]], np.float16),
                              np.array([1.0], np.float32))
    assert q.min() == lo and q.max() == hi
    assert workloads.DEFAULT_THRESHOLD == facts["default_outlier_threshold"]["value"]
    # the Python binding's default threshold (read without loading the library)
    import int8_quantized_matmul_col_amd.binding as b
    assert inspect.signature(b.int8_matmul).parameters["threshold"].default == \
        facts["default_outlier_threshold"]["value"]
    # threshold 0: every non-zero column takes the fp16 path
    X = np.array([[0.5, -0.25, 0.0]], np.float16)
    assert ref.outlier_mask_ref(X, 0.0)[1].tolist() == [0, 1]
    assert facts["threshold_zero_means_all_fp16"]["value"]


def test_tiny_oracle_record():
    import hashlib
    g = _load("tiny_oracle.json")
    case = workloads.config_case("tiny")
    Wq, a_w = ref.prepare_weight_ref(case.W)
    Y, st = ref.int8_matmul_ref(case.X, Wq, a_w, g["threshold"], stages=True)
    d = lambda a: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
    assert st["O"].tolist() == g["O"]
    assert [float(v).hex() for v in st["a_x"]] == g["a_x_f32_hex"]
    for k, v in [("Wq", Wq), ("a_w", a_w), ("Xq", st["Xq"]), ("X_O", st["X_O"]),
                 ("W_O", st["W_O"]), ("C", st["C"]), ("Y", Y)]:
        assert d(v) == g["sha256"][k], k
    assert int(st["C"].astype(np.int64).sum()) == g["C_sum"]
    assert math.isclose(float(Y.astype(np.float64).sum()), g["Y_sum"])
