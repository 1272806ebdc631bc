"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the plain int8_matmul entry point with a default
workspace), plus the stage outputs.  Every element is compared: the oracle
computes these shapes in seconds (float64 BLAS for the exact int32
accumulators)."""

import math

import numpy as np
import pytest

import workloads
from gpu_cases import run_case

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.parametrize("name", ["tiny", "q_proj", "ffn_up", "ffn_down"])
def test_full_config(lib, name):
    case = workloads.config_case(name)
    print(f"config {name} M={case.M} K={case.K} N={case.N}", flush=True)
    run_case(lib, case.X, case.W, case.threshold)


def test_full_decode(lib):
    # one 28672x8192 weight, shared by the three decode shapes
    W = workloads.make_w(28672, 8192, workloads.CONFIGS["decode1"]["seed"])
    for name in ("decode1", "decode4", "decode16"):
        case = workloads.config_case(name, with_w=False)
        print(f"config {name} M={case.M}", flush=True)
        run_case(lib, case.X, W, case.threshold, repeat=2)


@pytest.mark.parametrize("t", workloads.SWEEP_THRESHOLDS)
def test_full_sweep(lib, t):
    case = workloads.config_case("sweep13b")
    print(f"sweep13b t={t}", flush=True)
    run_case(lib, case.X, case.W, t, stages=(t != 0.0), repeat=1)
