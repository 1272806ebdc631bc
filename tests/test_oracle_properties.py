"""Property-based pins of the oracle (hypothesis, derandomized so that every
run draws the same examples): on small random problems the numpy oracle
agrees with the exact-rational brute force -- every integer stage bit for
bit, Y within one fp16 ulp of the exactly rounded value -- for values drawn
from binary16 (ties, zeros, negative zeros and outlier magnitudes included)
and thresholds around them."""

import math

import numpy as np
from hypothesis import HealthCheck, given, settings, strategies as st

from test_oracle import _compare_with_bruteforce

# binary16 values the quantizer finds interesting: small integers and halves
# (ties once scaled), signed zeros, ordinary values and outlier magnitudes
_VALUES = st.one_of(
    st.sampled_from([0.0, -0.0, 0.5, -0.5, 1.0, -1.5, 2.5, 3.96875, 6.0, -6.0, 7.5, 60.0]),
    st.floats(min_value=-4.0, max_value=4.0, width=16),
    st.floats(min_value=-64.0, max_value=64.0, width=16),
)


@st.composite
def _problem(draw):
    M = draw(st.integers(1, 6))
    K = draw(st.integers(1, 12))
    N = draw(st.integers(1, 6))
    X = np.array(draw(st.lists(_VALUES, min_size=M * K, max_size=M * K)), np.float16).reshape(M, K)
    W = np.array(draw(st.lists(_VALUES, min_size=N * K, max_size=N * K)), np.float16)
    W = (W.astype(np.float32) / np.float32(draw(st.sampled_from([1.0, 16.0, 256.0])))).astype(np.float16)
    W = W.reshape(N, K)
    t = draw(st.sampled_from([0.0, 1.0, 2.5, 6.0, 7.5, math.inf]))
    bias = None
    if draw(st.booleans()):
        bias = np.array(draw(st.lists(_VALUES, min_size=N, max_size=N)), np.float16)
    return X, W, t, bias


@settings(max_examples=60, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(_problem())
def test_oracle_matches_bruteforce_on_random_problems(p):
    X, W, t, bias = p
    _compare_with_bruteforce(X, W, t, bias)
