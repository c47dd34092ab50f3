"""Pins that tie the CPU oracle to what the pages and the mathematics fix.

None of these re-types the oracle's own formula or re-calls the routine it
uses; each compares it with something independent: a brute-force matrix
built from the definition, a different library routine, a closed form, an
invariant, a hand-constructed quantizer case, an exhaustive enumeration, a
statistic, or a value the pages print.  ``tests/test_oracle_mutants.py``
plants plausible mistakes in the oracle and checks that these pins catch
them.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _random_signs(n, seed):
    return (1 - 2 * _rng(seed).integers(0, 2, n)).astype(np.int8)


# ---------------------------------------------------------------- signs ----

def check_splitmix64():
    with open(os.path.join(GOLDEN, "splitmix64_seed1234567.txt")) as f:
        lines = [l.strip() for l in f if l.strip() and not l.startswith("#")]
    seed = int(lines[0].split()[1])
    want = [int(v) for v in lines[1:]]
    assert O.splitmix64(seed, len(want)) == want


def test_splitmix64_published_outputs():
    check_splitmix64()


def test_sign_vector_lengths_and_values():
    for D in (2, 4, 128, 256):
        s = O.plan_signs(D, O.SRFT, 7)
        assert s.shape == (D // 2,) and set(np.unique(s)) <= {-1, 1}
        s = O.plan_signs(D, O.SRHT, 7)
        assert s.shape == (D,)
    # bit i of word i // 64 -> sign 1 - 2 bit: word 0 of seed 1234567 is odd
    # (6457827717110365317 ends in binary ...101), so the first sign is -1,
    # the second +1, the third -1.
    s = O.plan_signs(256, O.SRHT, 1234567)
    assert list(s[:3]) == [-1, 1, -1]
    # bit 64 comes from word 1 = 3203168211198807973 (odd) -> -1
    assert s[64] == -1


# ------------------------------------------------------------ rotations ----

def check_srft_bruteforce(Ds=(2, 4, 8, 16)):
    for D in Ds:
        s = _random_signs(D // 2, D)
        R = O.rotation_matrix(D, O.SRFT, s)
        Rb = np.array(O.srft_matrix_bruteforce(D, [int(v) for v in s]))
        assert np.max(np.abs(R - Rb)) < 1e-12, D


def check_srht_bruteforce(Ds=(2, 4, 8, 16)):
    for D in Ds:
        s = _random_signs(D, D + 1)
        R = O.rotation_matrix(D, O.SRHT, s)
        Rb = np.array(O.srht_matrix_bruteforce(D, [int(v) for v in s]))
        assert np.max(np.abs(R - Rb)) < 1e-12, D
        # scipy's Sylvester Hadamard, scaled to be orthogonal
        Rs = scipy.linalg.hadamard(D) / math.sqrt(D) * s[None, :]
        assert np.max(np.abs(R - Rs)) < 1e-12, D


def check_srft_against_dft_matrix(Ds=(8, 128, 256)):
    """pack(F diag(s) x) with F = scipy's explicit unitary DFT matrix."""
    for D in Ds:
        M = D // 2
        s = _random_signs(M, 3 * D)
        F = scipy.linalg.dft(M, scale="sqrtn")
        x = _rng(D).standard_normal((5, D))
        z = x[:, 0::2] + 1j * x[:, 1::2]
        Z = (F @ (s[:, None] * z.T)).T
        want = np.empty_like(x)
        want[:, 0::2] = Z.real
        want[:, 1::2] = Z.imag
        got = O.rotate_forward(x, O.SRFT, s)
        assert np.max(np.abs(got - want)) < 1e-12, D


def check_srft_one_hot(D=128):
    """Closed-form columns: e_{2k} and e_{2k+1} through the unitary DFT."""
    M = D // 2
    s = _random_signs(M, 99)
    c = 1 / math.sqrt(M)
    for k in (0, 1, 5, M - 1):
        m = np.arange(M)
        ang = 2 * math.pi * k * m / M
        x = np.zeros(D)
        x[2 * k] = 1
        y = O.rotate_forward(x, O.SRFT, s)
        assert np.allclose(y[0::2], s[k] * np.cos(ang) * c, atol=1e-14)
        assert np.allclose(y[1::2], -s[k] * np.sin(ang) * c, atol=1e-14)
        x = np.zeros(D)
        x[2 * k + 1] = 1
        y = O.rotate_forward(x, O.SRFT, s)
        assert np.allclose(y[0::2], s[k] * np.sin(ang) * c, atol=1e-14)
        assert np.allclose(y[1::2], s[k] * np.cos(ang) * c, atol=1e-14)
    # e_0 -> half the channels equal s_0 / sqrt(M), the rest zero
    y = O.rotate_forward(np.eye(D)[0], O.SRFT, s)
    assert np.allclose(y[0::2], s[0] * c) and np.allclose(y[1::2], 0)


def check_orthogonal_and_inverse(Ds=(16, 128, 256)):
    for D in Ds:
        for rot in (O.SRFT, O.SRHT):
            s = O.plan_signs(D, rot, 5 + D)
            R = O.rotation_matrix(D, rot, s)
            assert np.max(np.abs(R @ R.T - np.eye(D))) < 1e-12
            x = _rng(D).standard_normal((7, D)) * 3
            y = O.rotate_forward(x, rot, s)
            assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
            assert np.max(np.abs(O.rotate_inverse(y, rot, s) - x)) < 1e-12
            # row i of the inverse applied to I is R^T e_i = row i of R
            assert np.max(np.abs(O.rotate_inverse(np.eye(D), rot, s) - R)) < 1e-12


def test_srft_equals_bruteforce_matrix():
    check_srft_bruteforce()


def test_srht_equals_closed_form_and_scipy():
    check_srht_bruteforce()


def test_srft_equals_explicit_dft_matrix():
    check_srft_against_dft_matrix()


# Mixed-radix SRFT (non-power-of-two D: the pages pick SRFT over SRHT for
# its mixed-radix sizes, abstract): the same definition at D = 6, 10, 12
# (M = 3, 5, 6) by brute force, and at D = 80, 96 (M = 40, 48) against
# scipy's explicit DFT matrix, the closed-form columns and orthogonality.

def check_srft_mixed_radix():
    check_srft_bruteforce(Ds=(6, 10, 12, 20))
    check_srft_against_dft_matrix(Ds=(80, 96))
    check_srft_one_hot(80)
    check_srft_one_hot(96)
    for D in (80, 96):
        s = O.plan_signs(D, O.SRFT, 17 + D)
        assert s.size == D // 2
        R = O.rotation_matrix(D, O.SRFT, s)
        assert np.max(np.abs(R @ R.T - np.eye(D))) < 1e-12
        x = _rng(D).standard_normal((7, D))
        assert np.max(np.abs(O.rotate_inverse(O.rotate_forward(x, O.SRFT, s), O.SRFT, s) - x)) < 1e-12


def test_srft_mixed_radix_sizes():
    check_srft_mixed_radix()


def test_quantizer_on_mixed_radix_sizes():
    """Groups of 32 at D = 96 (3 groups) and of 16 at D = 80 (5 groups): the
    sigma/2 bound in the w domain and through orthogonality."""
    rng = _rng(21)
    for D, G in ((96, 32), (96, 16), (80, 16)):
        x = (rng.standard_normal((500, D)) * 2).astype(np.float16)
        lam = np.exp(0.3 * rng.standard_normal(D)).astype(np.float32)
        s = O.plan_signs(D, O.SRFT, 3)
        for bits in (4, 8):
            codes, scales, w = O.encode(x, lam, O.SRFT, s, G, bits)
            assert codes.shape == (500, D * bits // 8) and scales.shape == (500, D // G)
            q = O.unpack_codes(codes, bits).astype(np.float64)
            sig = np.repeat(scales.astype(np.float64), G, axis=-1)
            normal = sig >= 2.0 ** -14
            assert np.all((np.abs(w - q * sig) <= sig / 2 + np.abs(w) * 2.0 ** -23)[normal])
            xh = O.decode(codes, scales, lam, O.SRFT, s, G, bits)
            lhs = np.linalg.norm(x.astype(np.float64) - xh, axis=-1)
            rhs = np.linalg.norm(sig / (2 * lam.astype(np.float64)), axis=-1)
            assert np.all(lhs <= rhs * (1 + 1e-6) + 1e-9)


def test_srft_one_hot_closed_form():
    check_srft_one_hot(128)
    check_srft_one_hot(256)


def test_rotations_orthogonal_inverse_exact():
    check_orthogonal_and_inverse()


def test_identity_rotation():
    x = _rng(1).standard_normal((3, 64))
    assert np.array_equal(O.rotate_forward(x, O.IDENTITY, O.plan_signs(64, O.IDENTITY, 0)), x)


# ------------------------------------------------------------ quantizer ----

def _ident_encode(x_vals, lam_vals, G=O.GROUP, bits=4):
    """Encode one vector with the identity rotation: w = lambda * x."""
    x = np.asarray(x_vals, dtype=np.float16)[None, :]
    lam = np.asarray(lam_vals, dtype=np.float32)[None, :]
    codes, scales, w = O.encode(x, lam, O.IDENTITY, O.plan_signs(x.shape[-1], O.IDENTITY, 0), G, bits)
    return codes[0], scales[0], w[0]


def check_exact_construction():
    """w_j = k_j * sigma with max |k_j| = 7 gives sigma and k back exactly."""
    rng = _rng(11)
    D = 64
    for sigma in (np.float16(0.0137), np.float16(1.0), np.float16(3.75), np.float16(611.5)):
        k = rng.integers(-7, 8, D)
        k[3] = 7
        k[40] = -7
        codes, scales, _ = _ident_encode(k.astype(np.float16), np.full(D, np.float32(sigma)))
        assert np.all(scales == sigma), (sigma, scales)
        assert np.array_equal(O.unpack_nibbles(codes[None])[0], k.astype(np.int8))


def check_half_even_ties():
    D = 32
    x = np.zeros(D, dtype=np.float16)
    x[:8] = [7, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5]   # a = 7 -> sigma = 1
    codes, scales, _ = _ident_encode(x, np.ones(D))
    assert scales[0] == 1
    q = O.unpack_nibbles(codes[None])[0]
    assert list(q[:8]) == [7, 0, 2, 2, 0, -2, -2, 4]


def check_zero_group():
    D = 64
    x = np.zeros(D, dtype=np.float16)
    x[32:] = np.linspace(-3, 3, 32).astype(np.float16)
    codes, scales, _ = _ident_encode(x, np.ones(D))
    assert scales[0] == 0 and not np.signbit(scales[0])
    assert np.all(codes[:16] == 0x88)


def check_subnormal_scale():
    """a / 7 below the fp16 normal range: the scale rounds to a subnormal and
    the clamp to [-8, 7] engages; expected values by exact rational
    arithmetic."""
    D = 32
    ulp = Fraction(1, 2 ** 24)                 # fp16 subnormal spacing
    mult = [10, -10, 3, -3, 1, 0, 7, -6] + [0] * 24
    x = np.array([float(m * ulp) for m in mult], dtype=np.float16)
    codes, scales, _ = _ident_encode(x, np.ones(D))
    a = max(abs(m) for m in mult) * ulp
    t = a / 7                                   # 10/7 ulp -> rounds to 1 ulp
    sig = Fraction(round(t / ulp)) * ulp        # nearest multiple (no tie here)
    assert Fraction(float(scales[0])) == sig
    want = []
    for m in mult:
        r = Fraction(m) * ulp / sig
        k = math.floor(r + Fraction(1, 2))
        want.append(max(-8, min(7, k)))
    assert list(O.unpack_nibbles(codes[None])[0]) == want
    assert -8 in want and 7 in want


def check_error_bound(n=4000, D=128, seed=3):
    rng = _rng(seed)
    x = (rng.standard_normal((n, D)) * np.exp(0.5 * rng.standard_normal(D))).astype(np.float16)
    lam = np.exp(0.3 * rng.standard_normal(D)).astype(np.float32)
    for rot in (O.SRFT, O.SRHT):
        s = O.plan_signs(D, rot, 42)
        codes, scales, w = O.encode(x, lam, rot, s)
        q = O.unpack_nibbles(codes).astype(np.float64)
        sig = np.repeat(scales.astype(np.float64), O.GROUP, axis=-1)
        normal = sig >= 2.0 ** -14
        err = np.abs(w - q * sig)
        slack = np.abs(w) * 2.0 ** -23               # float32 rounding of w
        assert np.all((err <= sig / 2 + slack)[normal])
        # x-domain bound through orthogonality: ||x - x^||_2 <= ||sigma/(2 lambda)||_2
        xh = O.decode(codes, scales, lam, rot, s)
        lhs = np.linalg.norm(x.astype(np.float64) - xh, axis=-1)
        rhs = np.linalg.norm(sig / (2 * lam.astype(np.float64)), axis=-1)
        assert np.all(lhs <= rhs * (1 + 1e-6) + 1e-9)


def check_nibbles_exhaustive():
    pairs = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)], dtype=np.int8)
    packed = O.pack_nibbles(pairs)
    assert sorted(packed[:, 0].tolist()) == list(range(256))
    assert np.array_equal(O.unpack_nibbles(packed), pairs)
    allb = np.arange(256, dtype=np.uint8)[:, None]
    assert np.array_equal(O.pack_nibbles(O.unpack_nibbles(allb)), allb)
    # layout: even channel low nibble, offset binary
    assert O.pack_nibbles(np.array([[-8, 7]]))[0, 0] == 0xF0
    assert O.pack_nibbles(np.array([[7, -8]]))[0, 0] == 0x0F
    assert O.pack_nibbles(np.array([[0, 0]]))[0, 0] == 0x88
    assert O.pack_nibbles(np.array([[1, -1]]))[0, 0] == 0x79


def test_exact_quantizer_construction():
    check_exact_construction()


def test_round_half_to_even():
    check_half_even_ties()


def test_all_zero_group():
    check_zero_group()


def test_subnormal_scale_exact_codes():
    check_subnormal_scale()


def test_error_bound_scale_over_two():
    check_error_bound()


def test_nibble_layout_exhaustive():
    check_nibbles_exhaustive()


# ------------------------------------------ int8 codes and groups of 16 --
# The explainer ("Methodik" 2) rounds to signed int4 or int8, and its scaling
# section ("Methodik" 3) uses groups of 16: scale = fp16(absmax / 127) for
# int8, codes clamped to [-128, 127] and stored as two's-complement bytes.

def check_exact_construction_int8():
    """w_j = k_j * sigma with max |k_j| = qmax gives sigma and k back exactly,
    for int8 (groups of 32 and 16) and int4 in groups of 16."""
    rng = _rng(13)
    D = 64
    for bits, G in ((8, 32), (8, 16), (4, 16)):
        qmax = 127 if bits == 8 else 7
        for sigma in (np.float16(0.0137), np.float16(1.0), np.float16(3.75), np.float16(61.5)):
            k = rng.integers(-qmax, qmax + 1, D)
            for g in range(D // G):           # every group reaches +-qmax
                k[g * G + 1] = qmax if g % 2 == 0 else -qmax
            codes, scales, _ = _ident_encode(k.astype(np.float16), np.full(D, np.float32(sigma)), G, bits)
            assert scales.shape == (D // G,) and np.all(scales == sigma), (bits, G, sigma, scales)
            assert codes.shape == (D * bits // 8,)
            assert np.array_equal(O.unpack_codes(codes[None], bits)[0], k), (bits, G)


def check_half_even_ties_int8():
    D = 32
    x = np.zeros(D, dtype=np.float16)
    x[:8] = [127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5]   # a = 127 -> sigma = 1
    x[16:24] = [126.5, -126.5, 125.5, 64.5, -64.5, 0, 1, -1]
    codes, scales, _ = _ident_encode(x, np.ones(D), 16, 8)
    assert scales[0] == 1 and scales[1] == np.float16(126.5 / 127)
    q = O.unpack_codes(codes[None], 8)[0]
    assert list(q[:8]) == [127, 0, 2, 2, 0, -2, -2, 4]
    # second group: sigma = fp16(126.5/127); each code against exact rationals
    sig = Fraction(float(scales[1]))
    for j in range(16, 24):
        r = Fraction(float(x[j])) / sig
        fl = math.floor(r)
        k = fl + (1 if (r - fl > Fraction(1, 2) or (r - fl == Fraction(1, 2) and fl % 2 == 1)) else 0)
        assert q[j] == max(-128, min(127, k)), (j, q[j], k)


def check_subnormal_scale_int8():
    """a / 127 below the fp16 normal range: the scale rounds to a subnormal
    and both ends of the int8 clamp engage; expected values by exact
    rational arithmetic."""
    D = 32
    ulp = Fraction(1, 2 ** 24)                 # fp16 subnormal spacing
    mult = [190, -190, 3, -3, 1, 0, 127, -128, -129, 128, 5] + [0] * 21
    x = np.array([float(m * ulp) for m in mult], dtype=np.float16)
    codes, scales, _ = _ident_encode(x, np.ones(D), 32, 8)
    a = max(abs(m) for m in mult) * ulp
    t = a / 127                                 # 190/127 ulp -> rounds to 1 ulp
    sig = Fraction(round(t / ulp)) * ulp
    assert Fraction(float(scales[0])) == sig
    want = []
    for m in mult:
        r = Fraction(m) * ulp / sig
        k = math.floor(r + Fraction(1, 2))
        want.append(max(-128, min(127, k)))
    assert list(O.unpack_codes(codes[None], 8)[0]) == want
    assert -128 in want and 127 in want


def check_error_bound_variants(n=2000, D=128, seed=4):
    """|w - q sigma| <= sigma / 2 on every normal-scale group, and the
    x-domain bound through orthogonality, for int4/G16, int8/G32, int8/G16."""
    rng = _rng(seed)
    x = (rng.standard_normal((n, D)) * np.exp(0.5 * rng.standard_normal(D))).astype(np.float16)
    lam = np.exp(0.3 * rng.standard_normal(D)).astype(np.float32)
    for bits, G in ((4, 16), (8, 32), (8, 16)):
        for rot in (O.SRFT, O.SRHT):
            s = O.plan_signs(D, rot, 42)
            codes, scales, w = O.encode(x, lam, rot, s, G, bits)
            q = O.unpack_codes(codes, bits).astype(np.float64)
            sig = np.repeat(scales.astype(np.float64), G, axis=-1)
            normal = sig >= 2.0 ** -14
            err = np.abs(w - q * sig)
            slack = np.abs(w) * 2.0 ** -23
            assert np.all((err <= sig / 2 + slack)[normal]), (bits, G, rot)
            xh = O.decode(codes, scales, lam, rot, s, G, bits)
            lhs = np.linalg.norm(x.astype(np.float64) - xh, axis=-1)
            rhs = np.linalg.norm(sig / (2 * lam.astype(np.float64)), axis=-1)
            assert np.all(lhs <= rhs * (1 + 1e-6) + 1e-9)


def check_codes_int8_exhaustive():
    q = np.arange(-128, 128, dtype=np.int16)[None, :]
    b = O.pack_codes(q, 8)
    assert sorted(b[0].tolist()) == list(range(256))
    assert np.array_equal(O.unpack_codes(b, 8), q)
    allb = np.arange(256, dtype=np.uint8)[None, :]
    assert np.array_equal(O.pack_codes(O.unpack_codes(allb, 8), 8), allb)
    # two's complement, one byte per channel in channel order
    assert O.pack_codes(np.array([[-1, -128, 127, 0, 1]]), 8).tolist() == [[0xFF, 0x80, 0x7F, 0x00, 0x01]]


def check_compression_variants():
    """bytes(fp16) / bytes(codes + fp16 scales) = 16 / (bits + 16 / G), and the
    oracle's buffers have exactly those sizes."""
    for bits, G, ratio in ((4, 32, Fraction(32, 9)), (4, 16, Fraction(16, 5)),
                           (8, 32, Fraction(32, 17)), (8, 16, Fraction(16, 9))):
        for D in (128, 256):
            assert abs(O.compression_ratio(D, G, bits) - float(ratio)) < 1e-15
            x = np.zeros((1, D), dtype=np.float16)
            codes, scales, _ = O.encode(x, np.ones(D), O.SRFT, O.plan_signs(D, O.SRFT, 0), G, bits)
            assert Fraction(x.nbytes, codes.nbytes + scales.nbytes) == ratio


def test_int8_and_group16_exact_construction():
    check_exact_construction_int8()


def test_int8_round_half_to_even():
    check_half_even_ties_int8()


def test_int8_subnormal_scale_exact_codes():
    check_subnormal_scale_int8()


def test_int8_and_group16_error_bound():
    check_error_bound_variants()


def test_int8_code_layout_exhaustive():
    check_codes_int8_exhaustive()


def test_compression_variants_closed_form():
    check_compression_variants()


def test_uniform_noise_statistic_int8_group16():
    """The same uniform-noise statistic for int8 in groups of 16."""
    rng = _rng(6)
    n, D, G = 8000, 128, 16
    x = (rng.standard_normal((n, D))).astype(np.float16)
    s = O.plan_signs(D, O.SRHT, 2)
    codes, scales, w = O.encode(x, np.ones(D), O.SRHT, s, G, 8)
    q = O.unpack_codes(codes, 8).astype(np.float64)
    sig = np.repeat(scales.astype(np.float64), G, axis=-1)
    wg = np.abs(w).reshape(n, D // G, G)
    is_max = (wg == wg.max(axis=-1, keepdims=True)).reshape(n, D)
    ratio = ((w - q * sig) ** 2 / (sig ** 2 / 12))[~is_max]
    assert ratio.size > 900_000
    assert abs(ratio.mean() - 1) < 0.05, ratio.mean()


def check_uniform_noise_statistic(n=12000, D=128, seed=5):
    """Away from the group maximum the rounding error behaves like uniform
    noise of width sigma: E[(w - q sigma)^2] / (sigma^2 / 12) ~ 1 (the
    bounded-noise model behind the rank-reduction paper's perturbation
    argument).  Sanity check within 5% on ~1.5e6 samples."""
    rng = _rng(seed)
    x = (rng.standard_normal((n, D))).astype(np.float16)
    lam = np.ones(D, dtype=np.float32)
    s = O.plan_signs(D, O.SRFT, 1)
    codes, scales, w = O.encode(x, lam, O.SRFT, s)
    q = O.unpack_nibbles(codes).astype(np.float64)
    sig = np.repeat(scales.astype(np.float64), O.GROUP, axis=-1)
    wg = np.abs(w).reshape(n, D // O.GROUP, O.GROUP)
    is_max = (wg == wg.max(axis=-1, keepdims=True)).reshape(n, D)
    ratio = ((w - q * sig) ** 2 / (sig ** 2 / 12))[~is_max]
    assert ratio.size > 1_000_000
    assert abs(ratio.mean() - 1) < 0.05, ratio.mean()


def test_uniform_noise_statistic():
    check_uniform_noise_statistic()


def check_compression_figure():
    vals = {}
    with open(os.path.join(GOLDEN, "compression.txt")) as f:
        for l in f:
            if l.strip() and not l.startswith("#"):
                k, v = l.split()
                vals[k] = float(v)
    G = int(vals["group"])
    for D in (128, 256):
        r = O.compression_ratio(D, G)
        assert round(r, 2) == vals["explainer_max"]
        assert r >= vals["abstract_min"]
    # the oracle's actual buffers have exactly that many bytes
    x = np.zeros((1, 128), dtype=np.float16)
    codes, scales, _ = O.encode(x, np.ones(128), O.SRFT, O.plan_signs(128, O.SRFT, 0))
    assert x.nbytes / (codes.nbytes + scales.nbytes) == O.compression_ratio(128, G)


def test_compression_matches_printed_figure():
    check_compression_figure()


# ------------------------------------- decisions in float64 (one rounding) --
# The plain definition of the quantizer rounds each exact quotient once:
# scale = fp16_RNE(a / qmax), code = rint_half_even(w / scale).  The pins
# below compute those roundings in exact rational arithmetic on the fp16
# grid and on the integers, and construct the inputs where a float64 or
# float32 intermediate would round twice.

def _fp16_round_exact(fr: Fraction) -> Fraction:
    """The fp16 value nearest a non-negative rational, ties to even
    (subnormal spacing 2^-24 below 2^-14)."""
    if fr == 0:
        return Fraction(0)
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1
    e = max(e, -14)
    ulp = Fraction(2) ** (e - 10)
    k = fr / ulp
    n = math.floor(k)
    rem = k - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n * ulp


def _rint_exact(fr: Fraction) -> int:
    n = math.floor(fr)
    rem = fr - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def _fp16_midpoint_cases():
    """Abs-max values a whose quotient a / qmax sits exactly on, or within
    2^-30 (relative) of, an fp16 rounding midpoint: below, on and above it,
    at both parities of the lower neighbour, normal and subnormal."""
    out = []
    for lo_bits in (0x3C00, 0x3C01, 0x4A3F, 0x4A40, 0x0200, 0x0201, 0x1C00, 0x1C01):
        lo = Fraction(float(np.array(lo_bits, dtype=np.uint16).view(np.float16)))
        hi = Fraction(float(np.array(lo_bits + 1, dtype=np.uint16).view(np.float16)))
        mid = (lo + hi) / 2
        for qmax in (7, 127):
            for rel in (Fraction(-1, 2 ** 30), Fraction(0), Fraction(1, 2 ** 30)):
                a = float(mid * qmax * (1 + rel))        # rounded to float64
                out.append((a, qmax))
    return out


def check_fp16_quotient_exact():
    rng = _rng(17)
    cases = _fp16_midpoint_cases()
    for a in np.abs(rng.standard_normal(3000) * np.exp(3 * rng.standard_normal(3000))):
        a = min(float(a), 60000.0)
        cases.append((float(a), 7))
        cases.append((float(a), 127))
    n_double = 0
    for a, qmax in cases:
        want = _fp16_round_exact(Fraction(a) / qmax)
        got = O.fp16_of_quotient(np.array([a]), qmax)[0]
        assert Fraction(float(got)) == want, (a, qmax, float(got), float(want))
        # the float32 route rounds twice: it differs on some constructed case
        via32 = (np.float32(a) / np.float32(qmax)).astype(np.float16)
        n_double += Fraction(float(via32)) != want
    assert n_double > 0


def check_rint_quotient_exact():
    """Ties, values 2^-45 either side of them, and the float64 neighbours of
    exact ties."""
    cases = []
    for s in (1.0, 0.0137, 0.3, 3.75, 5.9, 2.0 ** -20):
        s16 = float(np.float16(s))
        for k in range(-9, 9):
            t = (k + 0.5) * s16                       # exact in float64
            for rel in (-(2.0 ** -45), 0.0, 2.0 ** -45):
                cases.append((t * (1 + rel), s16))
            cases.append((float(np.nextafter(t, np.inf)), s16))
            cases.append((float(np.nextafter(t, -np.inf)), s16))
            cases.append((k * s16, s16))
    for w, s in cases:
        want = _rint_exact(Fraction(w) / Fraction(s))
        got = O.rint_of_quotient(np.array([w]), np.array([s]))[0]
        assert got == want, (w, s, got, want)


def check_float64_quotients_never_land_on_boundaries():
    """The fact behind the float64 decisions: near every fp16 rounding
    midpoint m (within 40 float64 steps of m d) the float64 quotient a / d
    equals m only when a = m d; near every half-integer multiple of every
    fp16 value the quotient w / s is that half-integer only when w is the
    multiple."""
    b = np.arange(1, 0x7BFF, dtype=np.uint16)
    lo = b.view(np.float16).astype(np.float64)
    hi = (b + 1).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2
    for d in (7.0, 127.0):
        t = mid * d
        for k in range(-40, 41):
            a = t + k * np.spacing(t)
            assert not np.any((a / d == mid) & (a != t))
    for h in np.arange(-8, 8) + 0.5:
        t = h * lo
        for k in range(-4, 5):
            w = t + k * np.spacing(t)
            assert not np.any((w / lo == h) & (w != t))


def check_fp64_decisions_construction():
    """quantize_groups(decide="fp64"): exact-grid groups give the scale and
    codes back; a group whose abs-max quotient is 2^-30 above an fp16
    midpoint rounds up where the float32 decision (DP) rounds to even."""
    rng = _rng(5)
    D, G = 64, 32
    k = rng.integers(-7, 8, D)
    k[0], k[40] = 7, -7
    sigma = np.float16(0.8125)
    w = k * float(sigma)
    q64, s64 = O.quantize_groups(w[None], G, 4, decide="fp64")
    assert np.all(s64 == sigma) and np.array_equal(q64[0], k.astype(np.int8))
    # abs-max 7 m (1 + 2^-30), m the midpoint of 1 and 1 + 2^-10 (1 is even)
    m = 1 + 2.0 ** -11
    w2 = np.zeros(G)
    w2[0] = 7 * m * (1 + 2.0 ** -30)
    w2[1] = 2.5 * (1 + 2.0 ** -10)                   # a code exactly at a tie with the upper scale
    _, s_dp = O.quantize_groups(w2[None], G, 4)
    q_64, s_64 = O.quantize_groups(w2[None], G, 4, decide="fp64")
    assert float(s_dp[0, 0]) == 1.0
    assert Fraction(float(s_64[0, 0])) == 1 + Fraction(1, 2 ** 10)
    assert q_64[0, 0] == 7 and q_64[0, 1] == 2       # 2.5 -> 2 (even)


def test_fp16_of_quotient_single_rounding():
    check_fp16_quotient_exact()


def test_rint_of_quotient_half_even_exact():
    check_rint_quotient_exact()


def test_fp64_decision_quantizer_construction():
    check_fp64_decisions_construction()


def test_float64_quotients_never_land_on_boundaries():
    check_float64_quotients_never_land_on_boundaries()


# ------------------------------------------------------------ boundaries ---

def test_boundary_distances_on_constructed_values():
    D = 32
    w = np.zeros((1, D))
    w[0, :4] = [7.0, 0.5, 2.25, -3.4999]
    code_d, scale_d = O.boundary_distances(w, np.array([[1.0]], dtype=np.float16))
    assert code_d[0, 1] == 0 and abs(code_d[0, 2] - 0.25) < 1e-15
    assert abs(code_d[0, 3] - 1e-4) < 1e-12
    # a / 7 exactly at an fp16 midpoint: 1 + 2^-11 lies between 1 and 1 + 2^-10
    w2 = np.zeros((1, D))
    w2[0, 0] = 7 * (1 + 2.0 ** -11)
    _, sd = O.boundary_distances(w2, np.array([[1.0]], dtype=np.float16))
    assert sd[0, 0] == 0


def test_boundary_distances_against_brute_force():
    """Code distances against a search over every half-integer in reach, and
    scale distances against the fp16 neighbours found in a table of every
    positive finite fp16 value, on random groups of both widths and group
    sizes (including values at fp16 binade edges and subnormal scales)."""
    pos = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)   # sorted
    halves = np.arange(-300, 300) + 0.5
    rng = _rng(11)
    for bits, G in ((4, 32), (4, 16), (8, 32), (8, 16)):
        qmax = O.code_range(bits)[1]
        D = 64
        w = rng.standard_normal((6, D)) * np.exp(rng.uniform(-12, 3, (6, 1)))
        w[0, 0] = qmax * 2.0 ** -3            # a / qmax on a binade edge
        w[1, :] *= 1e-6                       # subnormal fp16 scales
        a = np.abs(w.reshape(6, D // G, G)).max(-1)
        sc = O.fp16_of_quotient(a, qmax)
        code_d, scale_d = O.boundary_distances(w, sc, G, bits)
        assert np.any((sc > 0) & (sc < np.float16(2.0 ** -14)))    # subnormal scales are covered
        s = np.repeat(sc.astype(np.float64), G, axis=-1)
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(s > 0, w / s, 0.0)
        want_code = np.where(s > 0, np.abs(r[..., None] - halves).min(-1), np.inf)
        assert np.array_equal(code_d, want_code)
        t = a / qmax
        i = np.searchsorted(pos, t, side="right")      # pos[i-1] <= t < pos[i]
        lo = np.where(i > 0, pos[np.maximum(i - 1, 0)], 0.0)
        mid = (lo + pos[i]) / 2
        assert np.array_equal(scale_d, np.abs(t - mid) / t)


# ------------------------------------------------------------- decode -----

def test_decode_of_exact_construction():
    D = 64
    k = _rng(2).integers(-8, 8, D).astype(np.int8)
    sig = np.array([0.75, 0.03125], dtype=np.float16)
    lam = np.exp(0.3 * _rng(3).standard_normal(D))
    codes = O.pack_nibbles(k[None])
    got = O.decode(codes, sig[None], lam, O.IDENTITY, O.plan_signs(D, O.IDENTITY, 0))[0]
    want = k * np.repeat(sig.astype(np.float64), 32) / lam
    assert np.max(np.abs(got - want)) < 1e-15


def test_decode_inverts_rotation_on_grid_values():
    """If lambda*Rx already sits on the code grid, decode returns x."""
    D = 128
    for rot in (O.SRFT, O.SRHT):
        s = O.plan_signs(D, rot, 9)
        k = _rng(rot).integers(-7, 8, (3, D)).astype(np.int8)
        k[:, ::32] = 7
        sig = np.float16(0.5)
        lam = np.ones(D)
        y = k * float(sig)
        x = O.rotate_inverse(y, rot, s)
        codes = O.pack_nibbles(k)
        got = O.decode(codes, np.full((3, D // 32), sig), lam, rot, s)
        assert np.max(np.abs(got - x)) < 1e-12


# ------------------------------------------------------------ attention ---

def _tiny_cache(B, Hkv, T, D, rot, seed, G=O.GROUP, bits=4):
    rng = _rng(seed)
    s = O.plan_signs(D, rot, seed)
    x = (rng.standard_normal((B, Hkv, T, D)) * 2).astype(np.float16)
    lam = np.exp(0.3 * rng.standard_normal((Hkv, D))).astype(np.float32)
    codes, scales, _ = O.encode(x, lam[None, :, None, :], rot, s, G, bits)
    return codes, scales, lam, s


def _brute_attention(q16, kc, ks, lk, vc, vs, lv, L, sm_scale, D, signs, G=32, bits=4):
    """Pure-Python loops: unpack by hand, rescale, apply the brute-force
    SRFT matrix transposed, exponentiate and average."""
    R = O.srft_matrix_bruteforce(D, [int(v) for v in signs])
    def dec(code_row, scale_row, lam):
        y = []
        for j in range(D):
            if bits == 4:
                byte = int(code_row[j // 2])
                c = ((byte & 0xF) if j % 2 == 0 else (byte >> 4)) - 8
            else:
                byte = int(code_row[j])
                c = byte - 256 if byte >= 128 else byte
            y.append(c * float(scale_row[j // G]) / float(lam[j]))
        return [sum(R[i][c] * y[i] for i in range(D)) for c in range(D)]
    B, Hq, _ = q16.shape
    Hkv = kc.shape[1]
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            Ks = [dec(kc[b, g, t], ks[b, g, t], lk[g]) for t in range(L)]
            Vs = [dec(vc[b, g, t], vs[b, g, t], lv[g]) for t in range(L)]
            qv = [float(v) for v in q16[b, h]]
            e = [sm_scale * sum(qv[i] * Kt[i] for i in range(D)) for Kt in Ks]
            mx = max(e)
            p = [math.exp(v - mx) for v in e]
            tot = sum(p)
            for c in range(D):
                out[b, h, c] = sum(p[t] * Vs[t][c] for t in range(L)) / tot
    return out


def check_attention_bruteforce():
    D, B, Hkv, Hq, T = 32, 2, 2, 4, 6
    kc, ks, lk, s = _tiny_cache(B, Hkv, T, D, O.SRFT, 21)
    vc, vs, lv, _ = _tiny_cache(B, Hkv, T, D, O.SRFT, 21)
    vc, vs, lv = vc[:, :, ::-1].copy(), vs[:, :, ::-1].copy(), lv[::-1].copy()
    q = (_rng(4).standard_normal((B, Hq, D))).astype(np.float16)
    for L in (1, 3, T):
        sm = 1 / math.sqrt(D)
        got = O.attention_int4(q, kc, ks, lk, vc, vs, lv, L, sm, O.SRFT, s)
        want = _brute_attention(q, kc, ks, lk, vc, vs, lv, L, sm, D, s)
        assert np.max(np.abs(got - want)) < 1e-12


def test_attention_bruteforce_loops():
    check_attention_bruteforce()


def check_attention_bruteforce_int8():
    """Brute-force loops over int8 caches in groups of 16 and 32, and an int4
    cache in groups of 16."""
    D, B, Hkv, Hq, T = 32, 1, 2, 4, 5
    q = (_rng(7).standard_normal((B, Hq, D))).astype(np.float16)
    for bits, G in ((8, 16), (8, 32), (4, 16)):
        kc, ks, lk, s = _tiny_cache(B, Hkv, T, D, O.SRFT, 23, G, bits)
        vc, vs, lv, _ = _tiny_cache(B, Hkv, T, D, O.SRFT, 24, G, bits)
        vs = vs.copy()
        sm = 1 / math.sqrt(D)
        got = O.attention_int4(q, kc, ks, lk, vc, vs, lv, T, sm, O.SRFT, s, G, bits)
        want = _brute_attention(q, kc, ks, lk, vc, vs, lv, T, sm, D, s, G, bits)
        assert np.max(np.abs(got - want)) < 1e-12, (bits, G)


def test_attention_bruteforce_int8_group16():
    check_attention_bruteforce_int8()


def test_attention_special_cases():
    D, B, Hkv, Hq, T = 128, 1, 2, 8, 16
    kc, ks, lk, s = _tiny_cache(B, Hkv, T, D, O.SRFT, 5)
    vc, vs, lv, _ = _tiny_cache(B, Hkv, T, D, O.SRFT, 6)
    q = (_rng(8).standard_normal((B, Hq, D))).astype(np.float16)
    V = np.stack([O.decode(vc[0, g], vs[0, g], lv[g], O.SRFT, s) for g in range(Hkv)])
    # seq_len = 1: the output is the single decoded value vector
    o = O.attention_int4(q, kc, ks, lk, vc, vs, lv, 1, 0.1, O.SRFT, s)
    for h in range(Hq):
        assert np.max(np.abs(o[0, h] - V[h // 4, 0])) < 1e-12
    # q = 0: uniform weights, the mean of the decoded values
    o = O.attention_int4(np.zeros_like(q), kc, ks, lk, vc, vs, lv, T, 0.1, O.SRFT, s)
    for h in range(Hq):
        assert np.max(np.abs(o[0, h] - V[h // 4].mean(0))) < 1e-12
    # all keys equal: uniform weights again
    kc2 = np.repeat(kc[:, :, :1], T, axis=2)
    ks2 = np.repeat(ks[:, :, :1], T, axis=2)
    o = O.attention_int4(q, kc2, ks2, lk, vc, vs, lv, T, 0.1, O.SRFT, s)
    for h in range(Hq):
        assert np.max(np.abs(o[0, h] - V[h // 4].mean(0))) < 1e-12
    # a dominant key picks its value
    k16 = np.zeros((B, Hkv, T, D), dtype=np.float16)
    v16 = (_rng(9).standard_normal((B, Hkv, T, D))).astype(np.float16)
    k16[0, :, 5, :] = 4.0
    qq = np.full((B, Hq, D), 4.0, dtype=np.float16)
    o = O.attention_f16(qq, k16, v16, T, 1.0)
    assert np.max(np.abs(o[0, 0] - v16[0, 0, 5].astype(np.float64))) < 1e-12


def test_attention_f16_matches_scipy_softmax():
    import scipy.special
    rng = _rng(12)
    B, Hkv, Hq, T, D = 2, 2, 4, 40, 64
    k = rng.standard_normal((B, Hkv, T, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, D)).astype(np.float16)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    got = O.attention_f16(q, k, v, 33, 0.125)
    for b in range(B):
        for h in range(Hq):
            g = h // 2
            e = 0.125 * (k[b, g, :33].astype(np.float64) @ q[b, h].astype(np.float64))
            p = scipy.special.softmax(e)
            assert np.max(np.abs(got[b, h] - p @ v[b, g, :33].astype(np.float64))) < 1e-12
