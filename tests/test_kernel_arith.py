"""Host checks of arithmetic shortcuts taken by the HIP kernels.

The activation kernel quantizes a row with r = RN(127/a) and t = the exact
product x*r rounded half-even to an integer (one fma adding 1.5*2^23), and
falls back to the IEEE division fp32(127*x)/a wherever |x*r - t| (one fused
multiply-add, rounded once to fp32) exceeds 1/2 - 2^-14.  The test below
runs that rule, in numpy float32 / float64, over every binary16 pair
0 <= x <= a (a > 0 finite, about 5e8 pairs) and checks that where the kernel
keeps t it equals rint(fp32(fp32(127*x)/a)), the quantizer that defines the
codes ("PyTorch 2.9 supports LLM.int8()", section 2: round(127*x/absmax)).
Negative x follow by symmetry of rint and of the rule.  This does not use the
oracle: it pins the kernel's shortcut against the defining formula.
"""

import numpy as np

GUARD = np.float32(0.5) - np.float32(2.0 ** -14)


def test_fast_quantizer_matches_ieee_division_on_all_binary16_pairs():
    allf = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    bad = 0
    deferred = 0
    total = 0
    for ia in range(1, 0x7C00):
        a = allf[ia]
        x = allf[: ia + 1]
        r = np.float32(127.0) / a                       # correctly rounded fp32 division
        # exact product (24 + 11 significant bits fit float64), half-even integer
        t = np.rint(x.astype(np.float64) * np.float64(r))
        # fma(x, r, -t): exact in float64 (24 + 11 significant bits), then one fp32 rounding
        dev = np.abs((x.astype(np.float64) * np.float64(r) - t).astype(np.float32))
        keep = dev <= GUARD
        ref = np.rint((np.float32(127.0) * x) / a)      # the defining quantizer
        bad += int(np.count_nonzero(keep & (t != ref)))
        deferred += int(np.count_nonzero(~keep))
        total += x.size
    assert total == 503856639
    assert bad == 0
    # the division fallback is rare (it costs ~10x the fast path)
    assert deferred / total < 1e-3
