"""The scale quotient the encoders compute (kvq_device.hpp div_by): absmax /
qmax as q1 = absmax * fp32(1/qmax) followed by one fused correction
fma(fma(-q1, qmax, a), fp32(1/qmax), q1).  The scale must be fp16 of the
IEEE fp32 quotient (the oracle's reading DP), so the method must return
exactly that quotient.  Checked here over every fp32 value of the subnormal
range and of two whole binades, for qmax = 7 (int4) and 127 (int8): the
residual and the correction scale exactly with a between binades, so these
cover every normal a whose quotient is normal.

The fused multiply-adds are emulated in x87 extended precision (64-bit
significands), where both the residual and the corrected sum are exact
before the final rounding to fp32."""

import numpy as np
import pytest


def _method(a: np.ndarray, q: float) -> np.ndarray:
    c = np.float32(1.0) / np.float32(q)
    q1 = (a * c).astype(np.float32)
    r = a.astype(np.longdouble) - q1.astype(np.longdouble) * np.longdouble(q)
    return (q1.astype(np.longdouble) + r * np.longdouble(c)).astype(np.float32)


@pytest.mark.skipif(np.finfo(np.longdouble).nmant < 63, reason="needs x87 extended precision")
@pytest.mark.parametrize("q", [7.0, 127.0])
@pytest.mark.parametrize("lo,hi", [(1, 1 << 23), (0x3F800000, 0x40000000), (0x46800000, 0x47000000)])
def test_division_matches_ieee_quotient(q, lo, hi):
    chunk = 1 << 23
    for s in range(lo, hi, chunk):
        a = np.arange(s, min(s + chunk, hi), dtype=np.uint32).view(np.float32)
        got = _method(a, q)
        want = a / np.float32(q)          # IEEE fp32 division, round to nearest even
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
