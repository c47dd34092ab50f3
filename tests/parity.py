"""Comparison of GPU results with the CPU oracle, by the parity protocol.

Codes and scales must be bit-exact except where the oracle's float64 value
sits within 1e-4 of a rounding boundary:
  * a scale may differ only where a/qmax (qmax = 7 for int4, 127 for int8)
    lies within 1e-4 (relative) of an fp16 rounding midpoint;
  * a code may differ only where w/scale lies within 1e-4 (in code units) of
    a half-integer; in a group whose scale differs, the GPU codes are checked
    against the oracle's w re-quantized with the GPU's scale.
With no rotation (KVQ_IDENTITY) both sides hold the same float32 w = lambda
* x and the same float32 abs-max, and both take the scale as fp16 of the
IEEE float32 quotient, so every scale must match bit for bit; a code may
differ only where the kernel's multiply by a reciprocal (1 ulp) instead of a
division can move w/scale across a half-integer, i.e. within (qmax + 1) *
2^-22 code units of one.
The mismatch fraction (codes + scales, per element) is reported and must stay
below 1e-5 on every sample of at least 10^6 elements (int4 codes).  For int8
codes the bar is 1e-4: the same float32 rotation error, measured in code
units, is about 127/7 times larger on the int8 grid, and so is the expected
rate of boundary flips (2 E|w/scale| times the relative error), which puts
the int4 bar at 1.8e-4 for int8; 1e-4 is kept.  Smaller samples cannot
resolve a rate of 1e-5 (the expected count is below 10); there every
mismatch must still be a boundary case, and the count may not exceed the
99% quantile of a Poisson count whose mean is the bar times the number of
elements (flips are rare independent events, so their count in n elements
is Poisson).
The decisions are compared twice: against the oracle's float32 decisions
(its reading DP, the kernel's precision; the bars above apply), and against
the plain definition with each exact quotient rounded once (decide="fp64");
there every mismatch must also be a boundary case and the fraction must stay
below the bar on samples of at least 10^6 elements.  Every comparison is
recorded in RECORDS (written out by the test session when KVQ_PARITY_REPORT
names a file).
"""

from __future__ import annotations

import os

import numpy as np

import oracle as O

BOUNDARY = 1e-4
FRACTION = 1e-5          # int4 codes
FRACTION8 = 1e-4         # int8 codes (see above)
SMALL_SAMPLE_P = 0.99    # quantile of the small-sample count rule
ROT_NAMES = {O.SRFT: "srft", O.SRHT: "srht", O.IDENTITY: "identity"}

RECORDS: list = []


def identity_band(bits: int) -> float:
    """Code units within which the kernel's reciprocal multiply may flip an
    unrotated code: |w/scale| <= qmax + 1/2, and the reciprocal (1 ulp), the
    product and the oracle's division (half an ulp each) together move the
    quotient by at most 2^-22 relative."""
    return (O.code_range(bits)[1] + 1) * 2.0 ** -22


def poisson_quantile(mu: float, p: float = SMALL_SAMPLE_P) -> int:
    """Smallest k with P(Poisson(mu) <= k) >= p."""
    term = cdf = np.exp(-mu)
    k = 0
    while cdf < p:
        k += 1
        term *= mu / k
        cdf += term
    return k


def _mismatches(qg, sg16, w, scales_ref, codes_ref, G, bits, decide):
    """Scale and code mismatches of the GPU's codes qg and scales sg16 (fp16
    bits) against the oracle's (scales_ref, codes_ref), with the boundary
    distance of each and, in groups whose scale differs, the codes expected
    with the GPU's scale."""
    sr = scales_ref.view(np.uint16)
    code_dist, scale_dist = O.boundary_distances(w, scales_ref, G, bits)
    scale_bad = sg16 != sr
    qr = O.unpack_codes(codes_ref, bits)
    q_expect = qr
    if scale_bad.any():
        sg = sg16.view(np.float16)
        q_alt = _requantize(w, sg, G, bits, decide)
        bad_full = np.repeat(scale_bad, G, axis=-1)
        q_expect = np.where(bad_full, q_alt, qr)
        cd_alt, _ = O.boundary_distances(w, sg, G, bits)
        code_dist = np.where(bad_full, cd_alt, code_dist)
    code_bad = qg != q_expect
    return scale_bad, scale_dist, code_bad, code_dist


def _requantize(w64, scales16, G, bits, decide):
    """Oracle codes of w with the given fp16 scales, decided in float32
    (reading DP) or from the float64 values."""
    qmin, qmax = O.code_range(bits)
    s16 = np.repeat(np.asarray(scales16, dtype=np.float16), G, axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        if decide == "fp64":
            s = s16.astype(np.float64)
            r = O.rint_of_quotient(np.asarray(w64, dtype=np.float64), np.where(s > 0, s, 1.0))
        else:
            s = s16.astype(np.float32)
            r = np.rint(np.asarray(w64, dtype=np.float64).astype(np.float32) / s)
    q = np.where(s == 0, 0, np.clip(r, qmin, qmax))
    return q.astype(np.int16)


def requantize(w64: np.ndarray, scales16: np.ndarray, G: int = O.GROUP, bits: int = 4) -> np.ndarray:
    """Oracle codes of w with the given fp16 scales (the same float32 decision
    as the oracle's quantizer)."""
    return _requantize(w64, scales16, G, bits, "fp32")


def _test_id() -> str:
    return os.environ.get("PYTEST_CURRENT_TEST", "").rsplit(" (", 1)[0]


def compare_codes(codes_gpu, scales_gpu, x16, lam, rotation, signs, G: int = O.GROUP, bits: int = 4):
    """Check GPU codes/scales of vectors x16 [N, D] against the oracle.

    Returns a report dict; raises AssertionError on any mismatch that is not a
    boundary case or when the mismatch fraction is too large."""
    codes_ref, scales_ref, w = O.encode(x16, lam, rotation, signs, G, bits)
    codes_gpu = np.asarray(codes_gpu).reshape(codes_ref.shape)
    scales_gpu = np.asarray(scales_gpu).reshape(scales_ref.shape)
    N, D = w.shape[0], w.shape[-1]
    n_el = N * D
    sg = scales_gpu.view(np.uint16)
    qg = O.unpack_codes(codes_gpu, bits)
    bar = FRACTION if bits == 4 else FRACTION8

    # the oracle's float32 decisions (reading DP): the parity bar
    scale_bad, scale_dist, code_bad, code_dist = _mismatches(qg, sg, w, scales_ref, codes_ref, G, bits, "fp32")
    n_scale_bad, n_code_bad = int(scale_bad.sum()), int(code_bad.sum())
    # the plain definition, each exact quotient rounded once
    q64, scales64 = O.quantize_groups(w, G, bits, decide="fp64")
    codes64 = O.pack_codes(q64, bits)
    scale_bad64, scale_dist64, code_bad64, code_dist64 = _mismatches(qg, sg, w, scales64, codes64, G, bits, "fp64")
    n_scale_bad64, n_code_bad64 = int(scale_bad64.sum()), int(code_bad64.sum())
    frac = (n_code_bad + n_scale_bad) / max(n_el, 1)
    frac64 = (n_code_bad64 + n_scale_bad64) / max(n_el, 1)
    rec = {
        "test": _test_id(), "rotation": ROT_NAMES.get(rotation, str(rotation)), "D": D, "G": G, "bits": bits,
        "vectors": N, "elements": n_el, "groups": N * (D // G),
        "code_mismatch": n_code_bad, "scale_mismatch": n_scale_bad, "mismatch_frac": frac,
        "code_mismatch_fp64": n_code_bad64, "scale_mismatch_fp64": n_scale_bad64, "mismatch_frac_fp64": frac64,
    }
    RECORDS.append(rec)

    if rotation == O.IDENTITY:
        if n_scale_bad:
            amax = np.abs(w.reshape(N, D // G, G)).max(-1).astype(np.float32)
            sr = scales_ref.reshape(N, D // G).view(np.uint16)
            cases = [f"(vector {i}, group {j}: absmax {amax[i, j]!r} = 0x{amax[i, j].view(np.uint32):08x}, "
                     f"gpu 0x{sg.reshape(N, -1)[i, j]:04x}, oracle 0x{sr[i, j]:04x})"
                     for i, j in np.argwhere(scale_bad.reshape(N, -1))[:4]]
            raise AssertionError(f"{n_scale_bad} scale mismatches with no rotation (must be bit-exact): "
                                 + ", ".join(cases))
        band = identity_band(bits)
        if n_code_bad:
            assert np.all(code_dist[code_bad] <= band), (
                f"{n_code_bad} code mismatches with no rotation, max boundary distance "
                f"{code_dist[code_bad].max():.3e} > {band:.3e}")
    if n_scale_bad:
        assert np.all(scale_dist[scale_bad] <= BOUNDARY), (
            f"{n_scale_bad} scale mismatches, max boundary distance {scale_dist[scale_bad].max():.3e}")
    if n_code_bad:
        assert np.all(code_dist[code_bad] <= BOUNDARY), (
            f"{n_code_bad} code mismatches, max boundary distance {code_dist[code_bad].max():.3e}")
    if n_scale_bad64:
        assert np.all(scale_dist64[scale_bad64] <= BOUNDARY), (
            f"{n_scale_bad64} scale mismatches against the float64 decisions, max boundary distance "
            f"{scale_dist64[scale_bad64].max():.3e}")
    if n_code_bad64:
        assert np.all(code_dist64[code_bad64] <= BOUNDARY), (
            f"{n_code_bad64} code mismatches against the float64 decisions, max boundary distance "
            f"{code_dist64[code_bad64].max():.3e}")
    if n_el >= 1_000_000:
        assert frac < bar, f"mismatch fraction {frac:.3e} >= {bar}"
        assert frac64 < bar, f"mismatch fraction against the float64 decisions {frac64:.3e} >= {bar}"
    else:
        allowed = poisson_quantile(bar * n_el)
        assert n_code_bad + n_scale_bad <= allowed, (
            f"{n_code_bad + n_scale_bad} boundary mismatches in {n_el} elements (allowed {allowed})")
    return dict(rec, code_mismatch_frac=n_code_bad / max(n_el, 1),
                scale_mismatch_frac_per_group=n_scale_bad / max(N * (D // G), 1), w=w)


def compare_rotation(w_gpu, x16, lam, rotation, signs, rel: float = 1e-5):
    """Rotated fp32 values: per vector max|w_gpu - w_ref| <= rel * max|w_ref|."""
    w_ref = O.rotate(x16, lam, rotation, signs)
    w_gpu = np.asarray(w_gpu, dtype=np.float64).reshape(w_ref.shape)
    err = np.max(np.abs(w_gpu - w_ref), axis=-1)
    scale = np.max(np.abs(w_ref), axis=-1)
    worst = float(np.max(err / np.maximum(scale, 1e-30)))
    assert np.all(err <= rel * scale), f"rotation relative error {worst:.3e} > {rel}"
    return worst


def ulp16(x: np.ndarray) -> np.ndarray:
    """Spacing of fp16 numbers at |x| (subnormal spacing near zero)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def compare_decode(y_gpu, codes, scales, lam, rotation, signs, G: int = O.GROUP, atol: float = 1e-3,
                   bits: int = 4):
    """Decoded values of the same codes: fp32 within atol absolute; fp16
    within half an fp16 ulp of the oracle value plus atol."""
    ref = O.decode(codes, scales, lam, rotation, signs, G, bits)
    y = np.asarray(y_gpu)
    yg = y.astype(np.float64).reshape(ref.shape)
    err = np.abs(yg - ref)
    if y.dtype == np.float16:
        bound = 0.5 * ulp16(ref) + atol
        assert np.all(err <= bound), f"fp16 decode error {np.max(err - bound):.3e} over bound"
        not_rne = int(np.sum(y.reshape(ref.shape) != ref.astype(np.float16)))
        return {"max_err": float(err.max()), "not_rne": not_rne}
    assert np.all(err <= atol), f"decode max error {err.max():.3e} > {atol}"
    return {"max_err": float(err.max())}


def compare_attention(o_gpu, o_ref, rel: float = 2e-3):
    """Per (b, h): ||o_gpu - o_ref||_inf <= rel * ||o_ref||_inf."""
    o = np.asarray(o_gpu, dtype=np.float64).reshape(o_ref.shape)
    err = np.max(np.abs(o - o_ref), axis=-1)
    scale = np.max(np.abs(o_ref), axis=-1)
    worst = float(np.max(err / np.maximum(scale, 1e-30)))
    assert np.all(err <= rel * scale), f"attention relative error {worst:.3e} > {rel}"
    return worst
