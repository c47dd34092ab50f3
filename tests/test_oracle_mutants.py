"""Plant plausible mistakes in the CPU oracle and check that the pins catch
every one of them.

Each mutant replaces one oracle function (on the CPU only) with a copy that
carries a single slip -- a dropped term, a wrong sign, a swapped index or
operand -- and then runs the pin checks from ``test_oracle_pins``.  A mutant
that passes every pin would mean the pins could not tell that mistake from
the method, so the test fails.
"""

import math

import numpy as np
import pytest

import oracle as O
import oracle.kvq_oracle as K
from tests import test_oracle_pins as P

_orig = {name: getattr(K, name) for name in K.__all__ if callable(getattr(K, name))}


def _srft_fwd(x, signs, pair_swap=False, unpair_swap=False, norm="ortho", conj=False, use_signs=True):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    M = D // 2
    a, b = (x[..., 1::2], x[..., 0::2]) if pair_swap else (x[..., 0::2], x[..., 1::2])
    z = a + 1j * b
    if use_signs:
        z = signs.astype(np.float64) * z
    Z = (np.fft.ifft(z, axis=-1, norm="ortho") if conj else np.fft.fft(z, axis=-1, norm=norm))
    y = np.empty_like(x)
    if unpair_swap:
        y[..., 0::2], y[..., 1::2] = Z.imag, Z.real
    else:
        y[..., 0::2], y[..., 1::2] = Z.real, Z.imag
    return y


def _rot_fwd_factory(**kw):
    def f(x, rotation, signs):
        if rotation == K.SRFT:
            return _srft_fwd(x, signs, **kw)
        return _orig["rotate_forward"](x, rotation, signs)
    return f


def _srht_no_norm(x, rotation, signs):
    if rotation == K.SRHT:
        return _orig["rotate_forward"](x, rotation, signs) * math.sqrt(np.shape(x)[-1])
    return _orig["rotate_forward"](x, rotation, signs)


def _srht_sign_after(x, rotation, signs):
    if rotation == K.SRHT:
        H = K._sylvester(np.shape(x)[-1])
        return signs * ((np.asarray(x, dtype=np.float64) @ H.T) / math.sqrt(np.shape(x)[-1]))
    return _orig["rotate_forward"](x, rotation, signs)


def _inv_no_signs(y, rotation, signs):
    return _orig["rotate_inverse"](y, rotation, np.ones_like(signs))


def _quant_factory(div=7.0, half_away=False, lo=-8, hi=7, strided=False, div8=127.0, lo8=-128, hi8=127,
                   half_away8=False, g16_as_32=False):
    def q(w, G=K.GROUP, bits=4, decide="fp32"):
        if decide != "fp32":
            return _orig["quantize_groups"](w, G, bits, decide)
        if bits == 8:
            d, l, h, away = div8, lo8, hi8, half_away8
        else:
            d, l, h, away = div, lo, hi, half_away
        if g16_as_32 and G == 16:
            G = 32
        w32 = np.asarray(w, dtype=np.float64).astype(np.float32)
        D = w32.shape[-1]
        if strided:   # groups of every (D/G)-th channel instead of consecutive ones
            wg = np.swapaxes(w32.reshape(w32.shape[:-1] + (G, D // G)), -1, -2)
        else:
            wg = w32.reshape(w32.shape[:-1] + (D // G, G))
        a = np.max(np.abs(wg), axis=-1)
        scale = (a / np.float32(d)).astype(np.float16)
        s32 = scale.astype(np.float32)[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            r = wg / s32
        rr = np.sign(r) * np.floor(np.abs(r) + 0.5) if away else np.rint(r)
        qq = np.where(s32 == 0, 0, np.clip(rr, l, h))
        if strided:
            qq = np.swapaxes(qq, -1, -2)
        return qq.reshape(w32.shape).astype(np.int8), scale
    return q


def _fp16_quotient_via_fp32(a, d):
    """The quotient taken in float32 first (the DP decision) instead of once."""
    return (np.asarray(a, dtype=np.float64).astype(np.float32) / np.float32(d)).astype(np.float16)


def _rint_quotient_half_up(w, s):
    """floor(w / s + 1/2): ties rounded up instead of to even."""
    return np.floor(w / s + 0.5)


def _pack_codes_offset8(q, bits=4):
    if bits == 8:   # offset binary q + 128 instead of two's complement
        return (np.asarray(q, dtype=np.int16) + 128).astype(np.uint8)
    return _orig["pack_codes"](q, bits)


def _unpack_codes_unsigned8(b, bits=4):
    if bits == 8:   # bytes read as unsigned
        return np.asarray(b, dtype=np.uint8).astype(np.int16)
    return _orig["unpack_codes"](b, bits)


def _pack_swapped(q):
    q = np.asarray(q, dtype=np.int16)
    return ((q[..., 1::2] + 8) | ((q[..., 0::2] + 8) << 4)).astype(np.uint8)


def _unpack_swapped(b):
    b = np.asarray(b, dtype=np.uint8).astype(np.int16)
    q = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int16)
    q[..., 1::2] = (b & 0xF) - 8
    q[..., 0::2] = (b >> 4) - 8
    return q.astype(np.int8)


def _pack_twos(q):
    q = np.asarray(q, dtype=np.int16)
    return ((q[..., 0::2] & 0xF) | ((q[..., 1::2] & 0xF) << 4)).astype(np.uint8)


def _decode_mul_lambda(codes, scales, lam, rotation, signs, G=K.GROUP, bits=4):
    return _orig["decode"](codes, scales, 1.0 / np.asarray(lam, dtype=np.float64), rotation, signs, G, bits)


def _attn_bad_gqa(q16, kc, ks, lk, vc, vs, lv, seq_len, sm_scale, rotation, signs, G=K.GROUP, bits=4):
    out = _orig["attention_int4"](q16, kc, ks, lk, vc, vs, lv, seq_len, sm_scale, rotation, signs, G, bits)
    # interleaved head -> kv-head map (h % Hkv) instead of blocks (h // rep)
    B, Hq, D = out.shape
    Hkv = kc.shape[1]
    rep = Hq // Hkv
    perm = [(h % Hkv) * rep + h // Hkv for h in range(Hq)]
    return out[:, perm]


def _attn_double_scale(q16, kc, ks, lk, vc, vs, lv, seq_len, sm_scale, rotation, signs, G=K.GROUP, bits=4):
    return _orig["attention_int4"](q16, kc, ks, lk, vc, vs, lv, seq_len, sm_scale * sm_scale,
                                   rotation, signs, G, bits)


def _splitmix_bad(seed, n):
    out, state, U = [], seed, (1 << 64) - 1
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & U
        z = state
        z = ((z ^ (z >> 31)) * 0xBF58476D1CE4E5B9) & U
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & U
        out.append(z ^ (z >> 31))
    return out


def _signs_msb_first(D, rotation, seed):
    s = _orig["plan_signs"](D, rotation, seed)
    if s.size >= 64:
        s = s.copy()
        s[:64] = s[:64][::-1]
    return s


MUTANTS = {
    "srft-no-signs": ("rotate_forward", _rot_fwd_factory(use_signs=False)),
    "srft-not-unitary": ("rotate_forward", _rot_fwd_factory(norm="backward")),
    "srft-pair-swapped": ("rotate_forward", _rot_fwd_factory(pair_swap=True)),
    "srft-unpair-swapped": ("rotate_forward", _rot_fwd_factory(unpair_swap=True)),
    "srft-conjugate-kernel": ("rotate_forward", _rot_fwd_factory(conj=True)),
    "srht-no-normalisation": ("rotate_forward", _srht_no_norm),
    "srht-signs-after-transform": ("rotate_forward", _srht_sign_after),
    "inverse-drops-signs": ("rotate_inverse", _inv_no_signs),
    "scale-absmax-over-8": ("quantize_groups", _quant_factory(div=8.0)),
    "round-half-away": ("quantize_groups", _quant_factory(half_away=True)),
    "clamp-symmetric-7": ("quantize_groups", _quant_factory(lo=-7)),
    "groups-strided": ("quantize_groups", _quant_factory(strided=True)),
    "nibbles-swapped": ("pack_nibbles", _pack_swapped),
    "unpack-swapped": ("unpack_nibbles", _unpack_swapped),
    "nibbles-twos-complement": ("pack_nibbles", _pack_twos),
    "decode-multiplies-lambda": ("decode", _decode_mul_lambda),
    "attention-gqa-interleaved": ("attention_int4", _attn_bad_gqa),
    "attention-double-scale": ("attention_int4", _attn_double_scale),
    "splitmix-wrong-shift": ("splitmix64", _splitmix_bad),
    "int8-scale-absmax-over-128": ("quantize_groups", _quant_factory(div8=128.0)),
    "int8-clamp-symmetric-127": ("quantize_groups", _quant_factory(lo8=-127)),
    "int8-round-half-away": ("quantize_groups", _quant_factory(half_away8=True)),
    "g16-grouped-as-32": ("quantize_groups", _quant_factory(g16_as_32=True)),
    "int8-offset-binary": ("pack_codes", _pack_codes_offset8),
    "int8-unpack-unsigned": ("unpack_codes", _unpack_codes_unsigned8),
    "signs-bit-order": ("plan_signs", _signs_msb_first),
    "fp64-scale-via-fp32": ("fp16_of_quotient", _fp16_quotient_via_fp32),
    "fp64-code-half-up": ("rint_of_quotient", _rint_quotient_half_up),
}

CHECKS = [
    P.check_splitmix64,
    P.test_sign_vector_lengths_and_values,
    P.check_srft_bruteforce,
    P.check_srht_bruteforce,
    P.check_srft_against_dft_matrix,
    P.check_srft_one_hot,
    P.check_orthogonal_and_inverse,
    P.check_exact_construction,
    P.check_half_even_ties,
    P.check_zero_group,
    P.check_subnormal_scale,
    lambda: P.check_error_bound(n=500),
    P.check_nibbles_exhaustive,
    P.check_compression_figure,
    P.test_decode_of_exact_construction,
    P.test_decode_inverts_rotation_on_grid_values,
    P.check_attention_bruteforce,
    P.test_attention_special_cases,
    P.check_exact_construction_int8,
    P.check_half_even_ties_int8,
    P.check_subnormal_scale_int8,
    lambda: P.check_error_bound_variants(n=300),
    P.check_codes_int8_exhaustive,
    P.check_compression_variants,
    P.check_attention_bruteforce_int8,
    P.check_srft_mixed_radix,
    P.check_fp16_quotient_exact,
    P.check_rint_quotient_exact,
    P.check_fp64_decisions_construction,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    fn_name, bad = MUTANTS[name]
    monkeypatch.setattr(K, fn_name, bad)
    monkeypatch.setattr(O, fn_name, bad)
    caught = []
    for chk in CHECKS:
        try:
            chk()
        except Exception as e:  # noqa: BLE001 -- any failure counts as caught
            caught.append((getattr(chk, "__name__", "check"), type(e).__name__))
    assert caught, f"mutant {name} passed every pin"
