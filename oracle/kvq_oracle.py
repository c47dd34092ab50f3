"""Plain CPU oracle: SRFT/SRHT rotation, per-channel lambda, group-32 abs-max
scaling, int4 nibble packing, the inverse read path, and decode-step
attention over the int4 cache.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg use it.

What the method computes, and where it is stated
-------------------------------------------------
* Rotation.  The gist.science explainer ("Methodik", item 1) defines the
  sign-randomized Fourier transform as pack(F . diag(s) . x) with F the
  unitary DFT and s a fixed random sign vector; the paper's abstract names
  the Walsh-Hadamard alternative (SRHT) and reports no measurable quality
  difference between the two.
* Order of the fused pipeline (explainer, "Methodik", item 2): sign multiply
  on load, FFT over log2(d/2) radix-2 passes (so the transform length is
  d/2 complex points), pack to a real representation, per-channel lambda
  rescale, per-group abs-max reduction, rounding to signed int4, and packing
  two int4 values per byte.
* Per-channel plus per-group scaling (explainer, "Methodik", item 3).
* Compression 3.0x-3.56x (explainer, "Speichereffizienz"): 16 bits against
  4 + 16/32 bits per channel, i.e. groups of 32 with fp16 scales.

Readings where the pages are silent:
  R1  s has one sign per complex pair (length D/2) for SRFT and one per real
      channel (length D) for SRHT.
  R2  "pack" pairs adjacent channels: z_k = x_{2k} + i x_{2k+1}; unpacking
      the transform output uses the same interleave (no Hermitian post-step).
  R4  forward DFT kernel exp(-2 pi i k m / M), scale M^{-1/2} (unitary).
  R5  lambda multiplies after the rotation; the read side divides by it.
  R6  groups are 32 consecutive *output* channels.
  R7  scale = fp16(absmax / 7), round-to-nearest-even, subnormals kept.
  R8  codes round half to even.
  R10 an all-zero group stores scale +0 and code 0 (nibble 8).
  R12 nibble = q + 8 (offset binary); the even channel sits in the low nibble.
  B8  the int8 variant (explainer, "Methodik" 2: rounding to signed int4 or
      int8) takes scale = fp16(absmax / 127), codes clamped to [-128, 127]
      and stored as two's-complement bytes, one per channel.  Groups of 16
      (explainer, "Methodik" 3) are the G = 16 case of the same quantizer.
  DP  where a floating-point value decides an integer (the fp16 scale, the
      int4 code) the decision is taken in float32, the precision the GPU
      kernel computes in: w is the float64 rotation rounded to float32, the
      quotients absmax/7 and w/scale are IEEE float32 divisions (correctly
      rounded), then rounded to fp16 / rounded half-to-even to an integer.
      The plain definition (each exact quotient rounded once, from the
      float64 values) is kept beside it as decide="fp64", for reporting.

Signs come from SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014), written here from
its published definition.
"""

from __future__ import annotations

import cmath
import math

import numpy as np

__all__ = [
    "SRFT", "SRHT", "IDENTITY", "HERMITIAN", "ROTATIONS", "GROUP",
    "splitmix64", "plan_signs",
    "rotate_forward", "rotate_inverse",
    "quantize_groups", "fp16_of_quotient", "rint_of_quotient",
    "pack_nibbles", "unpack_nibbles", "pack_codes", "unpack_codes",
    "code_range",
    "encode", "decode", "rotate",
    "boundary_distances",
    "attention_int4", "attention_f16",
    "srft_matrix_bruteforce", "srht_matrix_bruteforce", "hermitian_matrix_bruteforce",
    "rotation_matrix",
    "compression_ratio",
]

SRFT = 0
SRHT = 1
IDENTITY = 2
HERMITIAN = 3          # real-input DFT variant (quality study only; no kernel)
ROTATIONS = (SRFT, SRHT, IDENTITY)
GROUP = 32

_U64 = (1 << 64) - 1


# ---------------------------------------------------------------------------
# Signs
# ---------------------------------------------------------------------------

def splitmix64(seed: int, n: int) -> list[int]:
    """First ``n`` outputs of SplitMix64 seeded with ``seed``.

    Published definition (Steele, Lea & Flood 2014): the state advances by
    the golden-ratio increment 0x9E3779B97F4A7C15; each output is the state
    passed through the 64-bit finaliser (xor-shift 30, multiply
    0xBF58476D1CE4E5B9, xor-shift 27, multiply 0x94D049BB133111EB,
    xor-shift 31), all arithmetic modulo 2^64.
    """
    out = []
    state = seed & _U64
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & _U64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _U64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _U64
        out.append(z ^ (z >> 31))
    return out


def plan_signs(D: int, rotation: int, seed: int) -> np.ndarray:
    """The fixed random sign vector s of the rotation (explainer, Methodik 1).

    Bit i of the stream is bit (i mod 64) of output floor(i/64); the sign is
    1 - 2*bit.  SRFT uses D/2 signs (one per complex pair, reading R1), SRHT
    and the HERMITIAN variant D signs, IDENTITY none.
    """
    if rotation == IDENTITY:
        return np.zeros(0, dtype=np.int8)
    n = D // 2 if rotation == SRFT else D
    words = splitmix64(seed, (n + 63) // 64)
    bits = [(words[i // 64] >> (i % 64)) & 1 for i in range(n)]
    return np.array([1 - 2 * b for b in bits], dtype=np.int8)


# ---------------------------------------------------------------------------
# Rotations (float64)
# ---------------------------------------------------------------------------

def _sylvester(D: int) -> np.ndarray:
    """Sylvester Hadamard matrix: H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    H = np.ones((1, 1))
    while H.shape[0] < D:
        H = np.block([[H, H], [H, -H]])
    assert H.shape[0] == D, "SRHT needs a power-of-two D"
    return H


def rotate_forward(x: np.ndarray, rotation: int, signs: np.ndarray) -> np.ndarray:
    """y = R x over the last axis, float64.

    SRFT (explainer, Methodik 1; readings R1, R2, R4): pair adjacent channels
    into M = D/2 complex values, multiply by the signs, take the unitary
    M-point DFT, and unpair real/imaginary parts back into adjacent channels.
    SRHT (abstract): y = D^{-1/2} H_D (s * x), H_D Sylvester-ordered.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if rotation == IDENTITY:
        return x.copy()
    if rotation == SRFT:
        M = D // 2
        z = signs.astype(np.float64) * (x[..., 0::2] + 1j * x[..., 1::2])
        Z = np.fft.fft(z, n=M, axis=-1, norm="ortho")
        y = np.empty_like(x)
        y[..., 0::2] = Z.real
        y[..., 1::2] = Z.imag
        return y
    if rotation == SRHT:
        H = _sylvester(D)
        return ((signs.astype(np.float64) * x) @ H.T) / math.sqrt(D)
    if rotation == HERMITIAN:
        # real-input DFT of the signed D-vector, unitary; the Hermitian half
        # spectrum unpacked into D reals: X_0 and X_{D/2} (real), then
        # sqrt(2) (Re X_m, Im X_m) for 0 < m < D/2
        X = np.fft.rfft(signs.astype(np.float64) * x, axis=-1, norm="ortho")
        y = np.empty_like(x)
        y[..., 0] = X[..., 0].real
        y[..., 1] = X[..., D // 2].real
        y[..., 2::2] = math.sqrt(2.0) * X[..., 1:D // 2].real
        y[..., 3::2] = math.sqrt(2.0) * X[..., 1:D // 2].imag
        return y
    raise ValueError("unknown rotation")


def rotate_inverse(y: np.ndarray, rotation: int, signs: np.ndarray) -> np.ndarray:
    """x = R^T y over the last axis, float64 (R is orthogonal, so R^-1 = R^T).

    SRFT: re-pair, unitary inverse DFT (kernel exp(+2 pi i k m / M)), multiply
    by the signs, unpair.  SRHT: x = s * (D^{-1/2} H_D y).
    """
    y = np.asarray(y, dtype=np.float64)
    D = y.shape[-1]
    if rotation == IDENTITY:
        return y.copy()
    if rotation == SRFT:
        M = D // 2
        Z = y[..., 0::2] + 1j * y[..., 1::2]
        z = np.fft.ifft(Z, n=M, axis=-1, norm="ortho") * signs.astype(np.float64)
        x = np.empty_like(y)
        x[..., 0::2] = z.real
        x[..., 1::2] = z.imag
        return x
    if rotation == SRHT:
        H = _sylvester(D)
        return signs.astype(np.float64) * ((y @ H.T) / math.sqrt(D))
    if rotation == HERMITIAN:
        X = np.empty(y.shape[:-1] + (D // 2 + 1,), dtype=np.complex128)
        X[..., 0] = y[..., 0]
        X[..., D // 2] = y[..., 1]
        X[..., 1:D // 2] = (y[..., 2::2] + 1j * y[..., 3::2]) / math.sqrt(2.0)
        return signs.astype(np.float64) * np.fft.irfft(X, n=D, axis=-1, norm="ortho")
    raise ValueError("unknown rotation")


def rotation_matrix(D: int, rotation: int, signs: np.ndarray) -> np.ndarray:
    """The D x D real matrix R, column j = R e_j (float64)."""
    return rotate_forward(np.eye(D), rotation, signs).T


# ---------------------------------------------------------------------------
# Brute-force cross-checks (pure Python, tiny D only)
# ---------------------------------------------------------------------------

def srft_matrix_bruteforce(D: int, signs) -> list[list[float]]:
    """SRFT as a D x D list-of-rows matrix, each column built from the
    definition with explicit complex-exponential sums (no FFT routine)."""
    M = D // 2
    R = [[0.0] * D for _ in range(D)]
    for col in range(D):
        x = [0.0] * D
        x[col] = 1.0
        z = [signs[k] * complex(x[2 * k], x[2 * k + 1]) for k in range(M)]
        for m in range(M):
            acc = 0j
            for k in range(M):
                acc += z[k] * cmath.exp(-2j * math.pi * k * m / M)
            acc /= math.sqrt(M)
            R[2 * m][col] = acc.real
            R[2 * m + 1][col] = acc.imag
    return R


def hermitian_matrix_bruteforce(D: int, signs) -> list[list[float]]:
    """The real-DFT variant as a D x D matrix from its cosine / sine basis:
    row 0 = 1/sqrt(D), row 1 = (-1)^j / sqrt(D), rows 2m and 2m+1 =
    sqrt(2/D) cos(2 pi m j / D) and -sqrt(2/D) sin(2 pi m j / D), times the
    sign of column j."""
    R = [[0.0] * D for _ in range(D)]
    for j in range(D):
        R[0][j] = signs[j] / math.sqrt(D)
        R[1][j] = signs[j] * (-1) ** j / math.sqrt(D)
        for m in range(1, D // 2):
            R[2 * m][j] = signs[j] * math.sqrt(2.0 / D) * math.cos(2 * math.pi * m * j / D)
            R[2 * m + 1][j] = -signs[j] * math.sqrt(2.0 / D) * math.sin(2 * math.pi * m * j / D)
    return R


def srht_matrix_bruteforce(D: int, signs) -> list[list[float]]:
    """SRHT as a D x D matrix from the closed form of the Sylvester Hadamard
    entries, H[i][j] = (-1)^popcount(i & j)."""
    R = [[0.0] * D for _ in range(D)]
    for i in range(D):
        for j in range(D):
            h = -1.0 if bin(i & j).count("1") % 2 else 1.0
            R[i][j] = h * signs[j] / math.sqrt(D)
    return R


# ---------------------------------------------------------------------------
# Quantizer (explainer, Methodik 2 and 3)
# ---------------------------------------------------------------------------

def code_range(bits: int):
    """(qmin, qmax) of signed codes of the given width: (-8, 7) for int4,
    (-128, 127) for int8.  The scale divides the group abs-max by qmax."""
    if bits not in (4, 8):
        raise ValueError(f"code width {bits} is not 4 or 8")
    return -(1 << (bits - 1)), (1 << (bits - 1)) - 1


def _fp16_midpoints(t: np.ndarray):
    """The fp16 neighbours lo <= t < hi of non-negative float64 values t and
    their midpoint, all as float64 (lo = hi = t where t is an fp16 value)."""
    lo = t.astype(np.float16)
    lo = np.where(lo.astype(np.float64) > t, np.nextafter(lo, np.float16(0)), lo)
    hi = np.nextafter(lo, np.float16(np.inf))
    return lo, hi, (lo.astype(np.float64) + hi.astype(np.float64)) / 2


def fp16_of_quotient(a: np.ndarray, d: int) -> np.ndarray:
    """fp16 of the exact quotient a / d (a >= 0 float64, d = 7 or 127),
    rounded once to nearest, ties to even, subnormals kept.

    numpy rounds the float64 quotient to fp16; that is one rounding of the
    exact quotient because the float64 quotient of a float64 by a small
    integer lands on an fp16 rounding midpoint only when the exact quotient
    does (the midpoint m has at most 12 significant bits, so m * d is a
    float64 value and the float64 neighbours of a / d sit at least 4/d of a
    float64 ulp of m away)."""
    a = np.asarray(a, dtype=np.float64)
    q = a / float(d)
    assert np.all(q <= 65504.0), "scale overflows fp16 (reading R11)"
    return q.astype(np.float16)


def rint_of_quotient(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """rint_half_even of the exact quotient w / s (float64 w, s > 0 an fp16
    value): the float64 quotient is a half-integer only when the exact one
    is (k + 1/2 times an fp16 value is a float64 value, and a float64 w next
    to it gives a quotient at least a float64 ulp away), so rounding it is
    one rounding of the exact quotient."""
    return np.rint(w / s)


def quantize_groups(w: np.ndarray, G: int = GROUP, bits: int = 4, decide: str = "fp32"):
    """Per-group abs-max scale and signed codes of the lambda-scaled rotation.

    Takes w (float64, last axis D) and returns
      q      int8  [..., D]     codes in [qmin, qmax] (code_range(bits))
      scale  float16 [..., D/G] one scale per group of G consecutive channels
    Decision precision, decide = "fp32" (reading DP): w is rounded to
    float32; the group abs-max a is exact in float32; scale =
    fp16_RNE(fp32(a / qmax)); the code is rint_half_even(fp32(w / scale))
    clamped to [qmin, qmax], and 0 where the scale is zero (reading R10).
    decide = "fp64" takes the same decisions on the float64 values with one
    rounding of each exact quotient: scale = fp16_RNE(a / qmax) and code =
    rint_half_even(w / scale), the plain definition with no float32 step.
    """
    qmin, qmax = code_range(bits)
    if decide == "fp64":
        w64 = np.asarray(w, dtype=np.float64)
        D = w64.shape[-1]
        assert D % G == 0
        wg = w64.reshape(w64.shape[:-1] + (D // G, G))
        a = np.max(np.abs(wg), axis=-1)
        scale = fp16_of_quotient(a, qmax)
        s64 = scale.astype(np.float64)[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            k = rint_of_quotient(wg, np.where(s64 > 0, s64, 1.0))
        q = np.where(s64 == 0, 0.0, np.clip(k, qmin, qmax))
        return q.reshape(w64.shape).astype(np.int8), scale
    assert decide == "fp32", f"unknown decision precision {decide!r}"
    w32 = np.asarray(w, dtype=np.float64).astype(np.float32)
    D = w32.shape[-1]
    assert D % G == 0
    wg = w32.reshape(w32.shape[:-1] + (D // G, G))
    a = np.max(np.abs(wg), axis=-1)                       # float32, exact
    with np.errstate(over="raise"):
        scale = (a / np.float32(qmax)).astype(np.float16)  # fp32 quotient -> fp16 RNE
    s32 = scale.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = wg / s32                                  # IEEE float32 division
    q = np.where(s32 == 0, np.float32(0), np.clip(np.rint(ratio), qmin, qmax))
    return q.reshape(w32.shape).astype(np.int8), scale


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Two int4 codes per byte (explainer, Methodik 2): nibble = q + 8, the
    even channel in the low nibble (reading R12)."""
    q = np.asarray(q, dtype=np.int16)
    lo = q[..., 0::2] + 8
    hi = q[..., 1::2] + 8
    assert lo.min(initial=0) >= 0 and hi.max(initial=0) <= 15
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles: bytes [..., D/2] -> codes int8 [..., D]."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int16)
    q = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int16)
    q[..., 0::2] = (b & 0xF) - 8
    q[..., 1::2] = (b >> 4) - 8
    return q.astype(np.int8)


def pack_codes(q: np.ndarray, bits: int = 4) -> np.ndarray:
    """Code bytes of one vector: int4 as nibbles (pack_nibbles), int8 as
    two's-complement bytes, one per channel (reading B8)."""
    if bits == 4:
        return pack_nibbles(q)
    qmin, qmax = code_range(bits)
    q = np.asarray(q, dtype=np.int16)
    assert q.min(initial=0) >= qmin and q.max(initial=0) <= qmax
    return (q & 0xFF).astype(np.uint8)


def unpack_codes(b: np.ndarray, bits: int = 4) -> np.ndarray:
    """Inverse of pack_codes: code bytes -> signed codes int16 [..., D]."""
    if bits == 4:
        return unpack_nibbles(b).astype(np.int16)
    code_range(bits)
    b = np.asarray(b, dtype=np.uint8).astype(np.int16)
    return np.where(b >= 128, b - 256, b).astype(np.int16)


# ---------------------------------------------------------------------------
# Encode / decode
# ---------------------------------------------------------------------------

def rotate(x16: np.ndarray, lam: np.ndarray, rotation: int, signs: np.ndarray) -> np.ndarray:
    """w = lambda * (R x) in float64 for fp16 input x (explainer, Methodik 2:
    the per-channel rescale follows the transform)."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    return np.asarray(lam, dtype=np.float64) * rotate_forward(x, rotation, signs)


def encode(x16, lam, rotation: int, signs: np.ndarray, G: int = GROUP, bits: int = 4, decide: str = "fp32"):
    """The full write path: x (fp16, [..., D]) and lambda ([..., D], broadcast
    like numpy) -> (codes uint8 [..., D*bits/8], scales fp16 [..., D/G],
    w float64).  ``decide`` selects the decision precision of the quantizer
    (quantize_groups)."""
    w = rotate(x16, lam, rotation, signs)
    q, scale = quantize_groups(w, G, bits, decide)
    return pack_codes(q, bits), scale, w


def decode(codes, scales, lam, rotation: int, signs: np.ndarray, G: int = GROUP, bits: int = 4) -> np.ndarray:
    """The read path: unpack, rescale by the group scale, divide by lambda,
    inverse rotation (R^T).  Returns float64 [..., D]."""
    q = unpack_codes(codes, bits).astype(np.float64)
    D = q.shape[-1]
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    s_full = np.repeat(s, G, axis=-1)
    assert s_full.shape[-1] == D
    y = q * s_full / np.asarray(lam, dtype=np.float64)
    return rotate_inverse(y, rotation, signs)


def boundary_distances(w: np.ndarray, scale_used: np.ndarray, G: int = GROUP, bits: int = 4):
    """How close each decision was to a rounding boundary, in float64.

    Returns (code_dist [..., D], scale_rel_dist [..., D/G]):
      code_dist  = | w/scale - (k + 1/2) | for the nearest half-integer, in
                   code units, computed with the scale actually used;
      scale_rel_dist = | a/qmax - m | / (a/qmax) for the midpoint m of the
                   fp16 values lo <= a/qmax < hi, the one that decides
                   between them (inf where a = 0).
    """
    qmax = code_range(bits)[1]
    w = np.asarray(w, dtype=np.float64)
    D = w.shape[-1]
    s = np.repeat(np.asarray(scale_used, dtype=np.float16).astype(np.float64), G, axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s > 0, w / s, 0.0)
    code_dist = np.abs(r - (np.floor(r) + 0.5))
    code_dist = np.where(s > 0, code_dist, np.inf)
    a = np.max(np.abs(w.reshape(w.shape[:-1] + (D // G, G))), axis=-1)
    t = a / float(qmax)
    # fp16 neighbours of t and their midpoint
    _, _, mid = _fp16_midpoints(t)
    with np.errstate(divide="ignore", invalid="ignore"):
        scale_dist = np.where(t > 0, np.abs(t - mid) / t, np.inf)
    return code_dist, scale_dist


# ---------------------------------------------------------------------------
# Decode-step attention
# ---------------------------------------------------------------------------

def _softmax_weighted(q, K, V, sm_scale):
    """Textbook attention for one query vector: softmax(sm_scale q.K^T) V,
    with max subtraction, float64."""
    e = sm_scale * (K @ q)
    e = e - e.max()
    p = np.exp(e)
    p /= p.sum()
    return p @ V


def attention_int4(q16, k_codes, k_scales, lam_k, v_codes, v_scales, lam_v,
                   seq_len: int, sm_scale: float, rotation: int, signs, G: int = GROUP, bits: int = 4):
    """Decode-step attention over the quantized cache (int4 codes, or int8
    with bits = 8).

    Shapes: q [B, Hq, D] fp16; codes [B, Hkv, Tcap, D*bits/8]; scales
    [B, Hkv, Tcap, D/G]; lambda [Hkv, D].  Tokens 0..seq_len-1 of each
    (b, kv head) are decoded with ``decode`` and query head h reads kv head
    h // (Hq / Hkv).  Returns float64 [B, Hq, D].
    """
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    B, Hq, D = q.shape
    Hkv = k_codes.shape[1]
    rep = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for g in range(Hkv):
            K = decode(k_codes[b, g, :seq_len], k_scales[b, g, :seq_len], lam_k[g], rotation, signs, G, bits)
            V = decode(v_codes[b, g, :seq_len], v_scales[b, g, :seq_len], lam_v[g], rotation, signs, G, bits)
            for h in range(g * rep, (g + 1) * rep):
                out[b, h] = _softmax_weighted(q[b, h], K, V, sm_scale)
    return out


def attention_f16(q16, k16, v16, seq_len: int, sm_scale: float):
    """The same attention over an unquantized fp16 cache [B, Hkv, Tcap, D]."""
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    B, Hq, D = q.shape
    Hkv = k16.shape[1]
    rep = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for g in range(Hkv):
            K = np.asarray(k16[b, g, :seq_len], dtype=np.float16).astype(np.float64)
            V = np.asarray(v16[b, g, :seq_len], dtype=np.float16).astype(np.float64)
            for h in range(g * rep, (g + 1) * rep):
                out[b, h] = _softmax_weighted(q[b, h], K, V, sm_scale)
    return out


# ---------------------------------------------------------------------------
# Storage
# ---------------------------------------------------------------------------

def compression_ratio(D: int, G: int = GROUP, code_bits: int = 4, scale_bits: int = 16) -> float:
    """fp16 bytes over int4-code-plus-scale bytes for one D-vector."""
    return (16 * D) / (code_bits * D + scale_bits * (D // G))
