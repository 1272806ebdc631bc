"""Writes the oracle regression fixtures in this folder.

Calls only ``oracle`` (arithmetic) and ``workloads`` (seeded inputs).  Run
from the repository root:  python tests/golden/make_golden.py
"""

import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import int8mm_ref as ref  # noqa: E402
import workloads  # noqa: E402


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def tiny_fixture() -> dict:
    case = workloads.config_case("tiny")
    Wq, a_w = ref.prepare_weight_ref(case.W)
    Y, st = ref.int8_matmul_ref(case.X, Wq, a_w, case.threshold, stages=True)
    return {
        "what": "oracle stages for the tiny workload (16x1024 by 1024x1024, threshold 6.0)",
        "written_by": "tests/golden/make_golden.py (oracle + workloads only)",
        "M": case.M, "K": case.K, "N": case.N, "threshold": case.threshold,
        "O": st["O"].tolist(),
        "a_x_f32_hex": [float(v).hex() for v in st["a_x"]],
        "sha256": {
            "Wq": digest(Wq), "a_w": digest(a_w), "Xq": digest(st["Xq"]),
            "X_O": digest(st["X_O"]), "W_O": digest(st["W_O"]), "C": digest(st["C"]),
            "Y": digest(Y),
        },
        "C_sum": int(st["C"].astype(np.int64).sum()),
        "C_abs_sum": int(np.abs(st["C"].astype(np.int64)).sum()),
        "Y_sum": float(Y.astype(np.float64).sum()),
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(tiny_fixture(), f, indent=1)
        f.write("\n")
    print("wrote tiny_oracle.json")
