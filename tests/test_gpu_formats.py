"""GPU parity of the code-format variants: int4 codes in groups of 16, int8
codes (scale = fp16(absmax / 127), two's-complement bytes) in groups of 32
and 16, through the same encode / decode / attention entry points and
kernels as the int4 group-32 cache, against the CPU oracle on the same
seeded inputs.

The bars are those of the int4 cache: codes and scales bit-exact except
within 1e-4 of a rounding boundary (mismatch fraction below 1e-5 for int4,
1e-4 for int8 codes), decoded values within 1e-3 absolute (fp32) or half an
fp16 ulp plus 1e-3 (fp16), attention within 2e-3 relative per (batch, head).
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import kv_cache_int4_amd as K
from kv_cache_int4_amd import workloads as W
from tests import parity as P
from tests.test_gpu_parity import batch_for, ROTS, check_encode, lam_per_vector, np16, run_attn, say

pytestmark = pytest.mark.gpu

FORMATS = {"int4-g16": (4, 16), "int8-g32": (8, 32), "int8-g16": (8, 16)}


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.library()


def decode_both(plan, rot, codes_d, scales_d, c, s, lam, B, H, T, t0=0):
    """Decode the written tokens into a strided fp16 output (canaries around
    it) and into fp32; both against the oracle's decode of the same codes."""
    D = plan.D
    signs = O.plan_signs(D, ROTS[rot], plan.seed)
    lv = lam_per_vector(lam, B, H, T)
    out = torch.full((B, H, T + 3, D + 8), 7.0, dtype=torch.float16, device="cuda")
    y = out[:, :, 1:1 + T, :D]
    K.decode(plan, codes_d, scales_d, lam.cuda(), y, t0=t0)
    torch.cuda.synchronize()
    o = out.cpu()
    assert bool((o[:, :, 0] == 7.0).all()) and bool((o[:, :, 1 + T:] == 7.0).all())
    assert bool((o[:, :, :, D:] == 7.0).all())
    cf = c.reshape(-1, plan.code_bytes)
    sf = s.reshape(-1, D // plan.G)
    r16 = P.compare_decode(np16(y).reshape(-1, D), cf, sf, lv, ROTS[rot], signs, plan.G, bits=plan.bits)
    y32 = torch.empty((B, H, T, D), dtype=torch.float32, device="cuda")
    K.decode(plan, codes_d, scales_d, lam.cuda(), y32, t0=t0)
    torch.cuda.synchronize()
    r32 = P.compare_decode(np16(y32).reshape(-1, D), cf, sf, lv, ROTS[rot], signs, plan.G, bits=plan.bits)
    return r16, r32


@pytest.mark.parametrize("fmt", sorted(FORMATS))
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("rot", ["srft", "srht", "identity"])
@pytest.mark.parametrize("T,path", [(63, "lanes"), (130, "lanes"), (130, "tiles")])
def test_format_ragged_offsets_strides(fmt, D, rot, T, path):
    """Ragged tails, a write offset inside a larger cache, strided input rows
    and a lambda table shared across the batch; on the one-wave-per-vector
    path (small calls) and on the tile path."""
    bits, G = FORMATS[fmt]
    g = W.gen("cpu", 91, D, T)
    H = 2
    B = batch_for(path, H, T)
    base = torch.randn((B, H, T + 5, D + 24), generator=g).to(torch.float16) * 3
    x = base[:, :, 2:2 + T, 8:8 + D]
    lam = torch.exp(0.3 * torch.randn((H, D), generator=g))
    plan = K.Plan(D, G, rot, 5151, bits=bits)
    codes_d, scales_d, c, s, _ = check_encode(fmt, plan, rot, x, lam, Tcap=T + 40, t0=17)
    r16, r32 = decode_both(plan, rot, codes_d, scales_d, c, s, lam, B, H, T, t0=17)
    say(f"   decode fp16 {r16}, fp32 {r32}")


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_format_qwen_prefix_full_srft(fmt):
    """Qwen2.5-1.5B-shaped prefix (458,752 vectors, D=128), SRFT: every
    vector's codes and scales checked, decode included."""
    bits, G = FORMATS[fmt]
    cfg = W.CONFIGS["qwen"]
    x, lam = W.prefix_inputs(cfg)
    plan = K.Plan(cfg.D, G, "srft", cfg.sign_seed, bits=bits)
    codes_d, scales_d, c, s, rep = check_encode(f"qwen-{fmt}", plan, "srft", x, lam)
    assert rep["elements"] == cfg.vectors * cfg.D
    B, H, T, D = x.shape
    y = torch.empty((B, H, T, D), dtype=torch.float16, device="cuda")
    K.decode(plan, codes_d, scales_d, lam.cuda(), y)
    torch.cuda.synchronize()
    signs = O.plan_signs(D, O.SRFT, plan.seed)
    r = P.compare_decode(np16(y).reshape(-1, D), c.reshape(-1, plan.code_bytes), s.reshape(-1, D // G),
                         lam_per_vector(lam, B, H, T), O.SRFT, signs, G, bits=bits)
    say(f"   decode fp16: {r}")


@pytest.mark.parametrize("fmt", sorted(FORMATS))
@pytest.mark.parametrize("rot", ["srft", "srht"])
def test_format_gemma_prefix_full(fmt, rot):
    """Gemma-3-1B-shaped prefix (212,992 vectors, D=256), SRFT and SRHT:
    every vector checked, decode included."""
    bits, G = FORMATS[fmt]
    cfg = W.CONFIGS["gemma"]
    x, lam = W.prefix_inputs(cfg)
    plan = K.Plan(cfg.D, G, rot, cfg.sign_seed, bits=bits)
    codes_d, scales_d, c, s, rep = check_encode(f"gemma-{fmt}", plan, rot, x, lam)
    B, H, T, D = x.shape
    y = torch.empty((B, H, T, D), dtype=torch.float16, device="cuda")
    K.decode(plan, codes_d, scales_d, lam.cuda(), y)
    torch.cuda.synchronize()
    signs = O.plan_signs(D, ROTS[rot], plan.seed)
    r = P.compare_decode(np16(y).reshape(-1, D), c.reshape(-1, plan.code_bytes), s.reshape(-1, D // G),
                         lam_per_vector(lam, B, H, T), ROTS[rot], signs, G, bits=bits)
    say(f"   decode fp16: {r}")


@pytest.mark.parametrize("fmt", sorted(FORMATS))
@pytest.mark.parametrize("D", [128, 256])
def test_format_special_groups(fmt, D):
    """Identity rotation: exact grid values, half-even ties with
    power-of-two scales, all-zero groups and subnormal-scale groups (the
    clamp reaching the lowest code)."""
    bits, G = FORMATS[fmt]
    qmin, qmax = O.code_range(bits)
    rng = np.random.default_rng(8)
    N = 64
    x = np.zeros((N, D), dtype=np.float16)
    for n in range(N):
        for g in range(D // G):
            kind = (n + g) % 4
            sl = slice(G * g, G * g + G)
            if kind == 0:       # exact grid with sigma = 0.5
                k = rng.integers(-qmax, qmax + 1, G)
                k[0] = qmax
                x[n, sl] = (k * 0.5).astype(np.float16)
            elif kind == 1:     # ties with sigma = 1
                t = np.array([qmax, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5] * (G // 8), dtype=np.float64)
                x[n, sl] = t.astype(np.float16)
            elif kind == 2:     # all zero
                pass
            else:               # subnormal scale: multiples of 2^-24
                m = rng.integers(-(qmax + qmax // 2), qmax + qmax // 2 + 1, G)
                m[0] = qmax + qmax // 2
                x[n, sl] = (m * 2.0 ** -24).astype(np.float16)
    xt = torch.from_numpy(x).reshape(1, 1, N, D)
    lt = torch.ones((1, D), dtype=torch.float32)
    plan = K.Plan(D, G, "identity", 0, bits=bits)
    _, _, c, s, rep = check_encode(f"special-{fmt}", plan, "identity", xt, lt)
    codes_ref, scales_ref, _ = O.encode(x, np.ones((N, D), dtype=np.float32), O.IDENTITY,
                                        O.plan_signs(D, O.IDENTITY, 0), G, bits)
    assert np.array_equal(s.reshape(N, -1).view(np.uint16), scales_ref.view(np.uint16))
    assert np.array_equal(c.reshape(N, -1), codes_ref)
    assert (O.unpack_codes(codes_ref, bits) == qmin).any()


# -------------------------------------------------------------- attention --

def format_cache(plan, B, Hkv, Hq, T, Tcap, seed, plant=()):
    """Decode-step inputs and their caches in the plan's format (tokens
    0..T-1 encoded with kvq_encode).  plant: (b, query head, token) spots
    whose key is made to dominate that head's scores."""
    D = plan.D
    k16, v16, lam_k, lam_v, q = W.decode_inputs(B, Hkv, Hq, Tcap, D, seed, "cuda")
    rep = Hq // Hkv
    for b, h, t in plant:
        qv = q[b, h].float()
        k16[b, h // rep, t] = (1200.0 / float((qv * qv).sum()) * qv).to(torch.float16)
    kc = torch.empty((B, Hkv, Tcap, plan.code_bytes), dtype=torch.uint8, device="cuda")
    ksc = torch.empty((B, Hkv, Tcap, D // plan.G), dtype=torch.float16, device="cuda")
    vc, vsc = torch.empty_like(kc), torch.empty_like(ksc)
    K.encode(plan, k16[:, :, :T], lam_k, kc, ksc, 0)
    K.encode(plan, v16[:, :, :T], lam_v, vc, vsc, 0)
    return q, kc, ksc, vc, vsc, lam_k, lam_v


def oracle_attention(plan, rot, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm):
    signs = O.plan_signs(plan.D, ROTS[rot], plan.seed)
    return O.attention_int4(np16(q), kc.cpu().numpy(), ksc.cpu().numpy(), lam_k.cpu().numpy(),
                            vc.cpu().numpy(), vsc.cpu().numpy(), lam_v.cpu().numpy(), L, sm, ROTS[rot], signs,
                            plan.G, plan.bits)


@pytest.mark.parametrize("fmt", sorted(FORMATS))
@pytest.mark.parametrize("rot", ["srft", "srht", "identity"])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (2, 1)])
@pytest.mark.parametrize("L", [17, 2051])
def test_format_attention(fmt, rot, Hq, Hkv, L):
    bits, G = FORMATS[fmt]
    D, B = 128, 2
    plan = K.Plan(D, G, rot, 33, bits=bits)
    say(f"[attn] {fmt} rot={rot} Hq={Hq} Hkv={Hkv} L={L}")
    q, kc, ksc, vc, vsc, lam_k, lam_v = format_cache(plan, B, Hkv, Hq, L, L + 9, 13)
    sm = 1 / math.sqrt(D)
    ref = oracle_attention(plan, rot, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm)
    for dt in (torch.float32, torch.float16):
        out = run_attn(plan, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm, dt)
        worst = P.compare_attention(np16(out), ref)
        say(f"   {dt}: rel err {worst:.2e}")


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_format_attention_dominant_token(fmt):
    """Planted dominant tokens (rows 1-3 of a block, the tail block, a later
    split) in every format: the softmax maximum must cover every row."""
    bits, G = FORMATS[fmt]
    D, B, Hq, Hkv, L = 128, 2, 8, 2, 2051
    plan = K.Plan(D, G, "srft", 59, bits=bits)
    spots = [(0, 0, 5), (0, 3, 1047), (1, 5, L - 1), (1, 6, 324), (1, 1, 1601)]
    q, kc, ksc, vc, vsc, lam_k, lam_v = format_cache(plan, B, Hkv, Hq, L, L + 5, 27, spots)
    sm = 1 / math.sqrt(D)
    ref = oracle_attention(plan, "srft", q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm)
    out = run_attn(plan, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm, torch.float32)
    worst = P.compare_attention(np16(out), ref)
    say(f"   {fmt} dominant tokens: rel err {worst:.2e}")


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_format_attention_decode_step_full_size(fmt):
    """The decode step at full size in every format: batch 64, Hq 8 / Hkv 2,
    32768 cached tokens plus one appended (T=1, t0=32768); 4 seeded (b, kv
    head) pairs checked against the oracle."""
    bits, G = FORMATS[fmt]
    cfg = W.CONFIGS["decode"]
    B, Hkv, Hq, D = cfg.B, cfg.H, 8, cfg.D
    T0 = cfg.T
    L, Tcap = T0 + 1, T0 + 256
    plan = K.Plan(D, G, "srft", cfg.sign_seed, bits=bits)
    say(f"[attn-full] {fmt}: building caches")
    k16, v16, lam_k, lam_v, q = W.decode_inputs(B, Hkv, Hq, Tcap, D, cfg.data_seed, "cuda")
    kc = torch.empty((B, Hkv, Tcap, plan.code_bytes), dtype=torch.uint8, device="cuda")
    ksc = torch.empty((B, Hkv, Tcap, D // G), dtype=torch.float16, device="cuda")
    vc, vsc = torch.empty_like(kc), torch.empty_like(ksc)
    K.encode(plan, k16[:, :, :T0], lam_k, kc, ksc, 0)
    K.encode(plan, v16[:, :, :T0], lam_v, vc, vsc, 0)
    K.encode(plan, k16[:, :, T0:T0 + 1], lam_k, kc, ksc, T0)
    K.encode(plan, v16[:, :, T0:T0 + 1], lam_v, vc, vsc, T0)
    sm = 1 / math.sqrt(D)
    out = run_attn(plan, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm, torch.float16)
    rng = np.random.default_rng(6)
    rep = Hq // Hkv
    for b, g in [(int(b), int(g)) for b, g in zip(rng.choice(B, 4, replace=False), rng.integers(0, Hkv, 4))]:
        sl = slice(b, b + 1)
        signs = O.plan_signs(D, O.SRFT, plan.seed)
        ref = O.attention_int4(np16(q[sl, g * rep:(g + 1) * rep]), kc[sl, g:g + 1, :L].cpu().numpy(),
                               ksc[sl, g:g + 1, :L].cpu().numpy(), lam_k[g:g + 1].cpu().numpy(),
                               vc[sl, g:g + 1, :L].cpu().numpy(), vsc[sl, g:g + 1, :L].cpu().numpy(),
                               lam_v[g:g + 1].cpu().numpy(), L, sm, O.SRFT, signs, G, bits)
        w = P.compare_attention(np16(out[sl, g * rep:(g + 1) * rep]).astype(np.float64), ref)
        say(f"   (b={b}, g={g}): rel {w:.2e}")
