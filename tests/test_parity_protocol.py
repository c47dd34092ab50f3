"""The parity protocol itself (tests/parity.py), on the CPU: the oracle's own
codes pass, and planted mistakes in a result fail -- among them the scale
taken as absmax * fp32(1/7) instead of the quotient absmax / 7, which the
no-rotation rule must reject."""

import numpy as np
import pytest

import oracle as O
from tests import parity as P


def _inputs(n, D, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((n, D)) * np.exp(0.5 * rng.standard_normal(D))).astype(np.float16)
    lam = np.exp(0.3 * rng.standard_normal((n, D))).astype(np.float32)
    return x, lam


@pytest.mark.parametrize("rot", [O.SRFT, O.SRHT, O.IDENTITY])
@pytest.mark.parametrize("bits,G", [(4, 32), (4, 16), (8, 32)])
def test_oracle_codes_pass(rot, bits, G):
    x, lam = _inputs(600, 128, 1)
    s = O.plan_signs(128, rot, 9)
    codes, scales, _ = O.encode(x, lam, rot, s, G, bits)
    n0 = len(P.RECORDS)
    rep = P.compare_codes(codes, scales, x, lam, rot, s, G, bits)
    assert rep["code_mismatch"] == 0 and rep["scale_mismatch"] == 0
    assert len(P.RECORDS) == n0 + 1 and P.RECORDS[-1]["elements"] == 600 * 128


def _reciprocal_scale_result(x, lam, G, bits):
    """Codes and scales of an unrotated encode whose scale is fp16(absmax *
    fp32(1/qmax)) and whose codes use that scale."""
    qmax = O.code_range(bits)[1]
    w32 = (lam.astype(np.float64) * x.astype(np.float64)).astype(np.float32)
    a = np.max(np.abs(w32.reshape(w32.shape[0], -1, G)), axis=-1)
    scales = (a * np.float32(1.0 / qmax)).astype(np.float16)
    q = P.requantize(w32.astype(np.float64), scales, G, bits)
    return O.pack_codes(q, bits), scales


def test_identity_rejects_reciprocal_scale():
    """The mistake behind a mixed-radix failure at D=80, groups of 16: a few
    scales sit within 1e-7 of an fp16 midpoint, where absmax * fp32(1/7)
    rounds the other way.  Those are boundary cases by the rotated rule, but
    with no rotation the scales must match exactly."""
    x, lam = _inputs(20000, 80, 3)
    codes, scales = _reciprocal_scale_result(x, lam, 16, 4)
    ref_codes, ref_scales, _ = O.encode(x, lam, O.IDENTITY, O.plan_signs(80, O.IDENTITY, 0), 16, 4)
    n_diff = int((scales.view(np.uint16) != ref_scales.view(np.uint16)).sum())
    assert n_diff > 0
    with pytest.raises(AssertionError, match="no rotation"):
        P.compare_codes(codes, scales, x, lam, O.IDENTITY, O.plan_signs(80, O.IDENTITY, 0), 16, 4)


def _flip_codes(codes, w, scales, n, bits=4):
    """Flip the n codes nearest a rounding boundary to the other side."""
    dist, _ = O.boundary_distances(w, scales, O.GROUP, bits)
    q = O.unpack_codes(codes, bits).astype(np.int16)
    flat = np.argsort(dist, axis=None)[:n]
    idx = np.unravel_index(flat, dist.shape)
    s = np.repeat(scales.astype(np.float64), O.GROUP, axis=-1)
    r = w / s
    q[idx] = np.where(np.rint(r[idx]) > r[idx], np.floor(r[idx]), np.ceil(r[idx]))
    return O.pack_codes(q, bits)


def test_small_sample_count_rule():
    """30,240 elements (the size of the D=80 case above at 378 vectors): two
    boundary flips pass, three fail; a flip far from a boundary always
    fails."""
    x, lam = _inputs(236, 128, 5)      # 30,208 elements
    s = O.plan_signs(128, O.SRFT, 4)
    codes, scales, w = O.encode(x, lam, O.SRFT, s)
    assert P.poisson_quantile(P.FRACTION * 30240) == 2
    P.compare_codes(_flip_codes(codes, w, scales, 2), scales, x, lam, O.SRFT, s)
    with pytest.raises(AssertionError, match="allowed 2"):
        P.compare_codes(_flip_codes(codes, w, scales, 3), scales, x, lam, O.SRFT, s)
    q = O.unpack_codes(codes).astype(np.int16)
    q[0, 5] += 1 if q[0, 5] < 7 else -1
    with pytest.raises(AssertionError, match="boundary distance"):
        P.compare_codes(O.pack_codes(q), scales, x, lam, O.SRFT, s)


def test_identity_band_is_tight():
    """The no-rotation code band covers a reciprocal within 1 ulp and no
    more: 2^-22 (qmax + 1) code units."""
    assert P.identity_band(4) == pytest.approx(8 * 2.0 ** -22)
    assert P.identity_band(8) == pytest.approx(128 * 2.0 ** -22)
    assert P.identity_band(4) < P.BOUNDARY / 50
