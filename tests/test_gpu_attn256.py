"""GPU parity of decode-step attention at head size 256 (Gemma-3 1B has four
query heads over one KV head of 256 channels; the abstract reports its decode
latency against fp16).  Every rotation and code format, GQA ratios 1 to 8,
sequence lengths with ragged tails, a dominant token, more than 16 splits,
both output types and the fp16-cache comparator, each within 2e-3 relative
per (batch, head) of the oracle run on the GPU-written cache; the full-size
decode step is sampled.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
import kv_cache_int4_amd as K
from kv_cache_int4_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu

ROTS = {"srft": O.SRFT, "srht": O.SRHT, "identity": O.IDENTITY}
D = 256


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.library()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np16(t):
    return t.detach().cpu().numpy()


def cache(plan, k16, v16, lam_k, lam_v, T):
    """Quantized K and V caches [B, Hkv, Tcap, ...] with tokens 0..T-1
    written by kvq_encode."""
    B, Hkv, Tcap, _ = k16.shape
    cb, ng = plan.code_bytes, plan.D // plan.G
    kc = torch.empty((B, Hkv, Tcap, cb), dtype=torch.uint8, device="cuda")
    ks = torch.empty((B, Hkv, Tcap, ng), dtype=torch.float16, device="cuda")
    vc, vs = torch.empty_like(kc), torch.empty_like(ks)
    K.encode(plan, k16[:, :, :T], lam_k, kc, ks, 0)
    K.encode(plan, v16[:, :, :T], lam_v, vc, vs, 0)
    return kc, ks, vc, vs


def attn(plan, q, kc, ks, lk, vc, vs, lv, L, sm, dt):
    B, Hq, _ = q.shape
    ws = torch.empty(K.attn_workspace_size(D, B, Hq, L), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), dtype=dt, device="cuda")
    K.attn_decode(plan, q, kc, ks, lk, vc, vs, lv, L, sm, out, ws)
    torch.cuda.synchronize()
    return out


def oracle(plan, rot, q, kc, ks, lk, vc, vs, lv, L, sm):
    signs = O.plan_signs(D, ROTS[rot], plan.seed)
    return O.attention_int4(np16(q), np16(kc), np16(ks), np16(lk), np16(vc), np16(vs), np16(lv), L, sm,
                            ROTS[rot], signs, plan.G, plan.bits)


def f16_check(q, k16, v16, L, sm):
    B, Hq, _ = q.shape
    ws = torch.empty(K.attn_workspace_size(D, B, Hq, L), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    K.attn_decode_f16(q, k16, v16, L, sm, out, ws)
    torch.cuda.synchronize()
    ref = O.attention_f16(np16(q), np16(k16), np16(v16), L, sm)
    return P.compare_attention(np16(out), ref)


@pytest.mark.parametrize("rot", ["srft", "srht", "identity"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (8, 2), (2, 2), (16, 2)])
@pytest.mark.parametrize("L", [1, 17, 300, 2051])
def test_attention256_small(rot, Hq, Hkv, L):
    B = 2
    plan = K.Plan(D, 32, rot, 31)
    say(f"[attn256] rot={rot} Hq={Hq} Hkv={Hkv} L={L}")
    k16, v16, lk, lv, q = W.decode_inputs(B, Hkv, Hq, L + 9, D, 11, "cuda")
    kc, ks, vc, vs = cache(plan, k16, v16, lk, lv, L)
    sm = 1 / math.sqrt(D)
    ref = oracle(plan, rot, q, kc, ks, lk, vc, vs, lv, L, sm)
    for dt in (torch.float32, torch.float16):
        out = attn(plan, q, kc, ks, lk, vc, vs, lv, L, sm, dt)
        say(f"   int4 {dt}: rel err {P.compare_attention(np16(out), ref):.2e}")
    say(f"   fp16 comparator: rel err {f16_check(q, k16, v16, L, sm):.2e}")


@pytest.mark.parametrize("bits,G", [(4, 16), (8, 32), (8, 16)])
@pytest.mark.parametrize("rot", ["srft", "srht"])
@pytest.mark.parametrize("Hq,Hkv,L", [(4, 1, 1111), (8, 2, 45)])
def test_attention256_formats(bits, G, rot, Hq, Hkv, L):
    B = 2
    plan = K.Plan(D, G, rot, 19, bits=bits)
    say(f"[attn256-fmt] int{bits} G={G} rot={rot} Hq={Hq} Hkv={Hkv} L={L}")
    k16, v16, lk, lv, q = W.decode_inputs(B, Hkv, Hq, L + 3, D, 13, "cuda")
    kc, ks, vc, vs = cache(plan, k16, v16, lk, lv, L)
    sm = 1 / math.sqrt(D)
    ref = oracle(plan, rot, q, kc, ks, lk, vc, vs, lv, L, sm)
    for dt in (torch.float32, torch.float16):
        out = attn(plan, q, kc, ks, lk, vc, vs, lv, L, sm, dt)
        say(f"   {dt}: rel err {P.compare_attention(np16(out), ref):.2e}")


@pytest.mark.parametrize("rot", ["srft", "srht"])
def test_attention256_dominant_token(rot):
    """A token whose score exceeds every other by far more than exp2's range:
    the running maximum must cover every row of a block and every split.
    Dominant tokens sit inside blocks, in the tail block and in later
    splits; the output is then (nearly) that token's value vector."""
    B, Hq, Hkv, L = 2, 4, 1, 2051
    plan = K.Plan(D, 32, rot, 57)
    say(f"[attn256-dominant] rot={rot}")
    k16, v16, lk, lv, q = W.decode_inputs(B, Hkv, Hq, L + 5, D, 23, "cuda")
    spots = [(0, 0, 5), (0, 3, 1000 + 32 + 12 + 3), (1, 2, L - 1), (1, 1, 300 + 16 + 8)]
    for b, h, t in spots:
        qv = q[b, h].float()
        c = 1200.0 / float((qv * qv).sum())
        k16[b, 0, t] = (c * qv).to(torch.float16)
    kc, ks, vc, vs = cache(plan, k16, v16, lk, lv, L)
    sm = 1 / math.sqrt(D)
    ref = oracle(plan, rot, q, kc, ks, lk, vc, vs, lv, L, sm)
    signs = O.plan_signs(D, ROTS[rot], plan.seed)
    for b, h, t in spots:
        vhat = O.decode(np16(vc[b, 0, t]), np16(vs[b, 0, t]), np16(lv[0]), ROTS[rot], signs)
        assert np.max(np.abs(ref[b, h] - vhat)) <= 1e-6 * np.max(np.abs(vhat)) + 1e-9
    for dt in (torch.float32, torch.float16):
        out = attn(plan, q, kc, ks, lk, vc, vs, lv, L, sm, dt)
        say(f"   {dt}: rel err {P.compare_attention(np16(out), ref):.2e}")


@pytest.mark.parametrize("Hq,Hkv,L", [(4, 1, 9000), (6, 1, 5000), (2, 2, 4500)])
def test_attention256_many_splits(Hq, Hkv, L):
    """Batch 1: few (batch, kv head, head chunk) units, each cut into more
    than 16 splits (the general merge path); Hq = 6 leaves a second chunk of
    two heads.  int4 (SRFT) and the fp16 comparator against the oracle."""
    B = 1
    plan = K.Plan(D, 32, "srft", 71)
    say(f"[attn256-splits] Hq={Hq} Hkv={Hkv} L={L}")
    k16, v16, lk, lv, q = W.decode_inputs(B, Hkv, Hq, L + 3, D, 29, "cuda")
    kc, ks, vc, vs = cache(plan, k16, v16, lk, lv, L)
    sm = 1 / math.sqrt(D)
    ref = oracle(plan, "srft", q, kc, ks, lk, vc, vs, lv, L, sm)
    out = attn(plan, q, kc, ks, lk, vc, vs, lv, L, sm, torch.float32)
    say(f"   int4: rel err {P.compare_attention(np16(out), ref):.2e}")
    say(f"   fp16 comparator: rel err {f16_check(q, k16, v16, L, sm):.2e}")


def test_attention256_decode_step_full_size():
    """The Gemma-3-1B-shaped decode step at full size: batch 64, 4 query
    heads over 1 KV head, D=256, 32768 cached tokens plus one appended with
    kvq_encode (T=1, t0=32768), attention over 32769 tokens; 6 seeded
    sequences checked against the oracle, and the fp16 comparator."""
    cfg = W.CONFIGS["decode256"]
    B, Hkv, Hq = cfg.B, cfg.H, cfg.Hq
    T0 = cfg.T
    L = T0 + 1
    Tcap = T0 + 256
    plan = K.Plan(D, 32, "srft", cfg.sign_seed)
    say("[attn256-full] building caches")
    k16, v16, lk, lv, q = W.decode_inputs(B, Hkv, Hq, Tcap, D, cfg.data_seed, "cuda")
    kc, ks, vc, vs = cache(plan, k16, v16, lk, lv, T0)
    K.encode(plan, k16[:, :, T0:T0 + 1], lk, kc, ks, T0)
    K.encode(plan, v16[:, :, T0:T0 + 1], lv, vc, vs, T0)
    sm = 1 / math.sqrt(D)
    out = attn(plan, q, kc, ks, lk, vc, vs, lv, L, sm, torch.float16)
    ws = torch.empty(K.attn_workspace_size(D, B, Hq, L), dtype=torch.uint8, device="cuda")
    out16 = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
    K.attn_decode_f16(q, k16, v16, L, sm, out16, ws)
    torch.cuda.synchronize()
    signs = O.plan_signs(D, O.SRFT, plan.seed)
    for b in np.random.default_rng(4).choice(B, 6, replace=False):
        sl = slice(int(b), int(b) + 1)
        ref = O.attention_int4(np16(q[sl]), np16(kc[sl, :, :L]), np16(ks[sl, :, :L]), np16(lk), np16(vc[sl, :, :L]),
                               np16(vs[sl, :, :L]), np16(lv), L, sm, O.SRFT, signs)
        w1 = P.compare_attention(np16(out[sl]).astype(np.float64), ref)
        ref16 = O.attention_f16(np16(q[sl]), np16(k16[sl]), np16(v16[sl]), L, sm)
        w2 = P.compare_attention(np16(out16[sl]).astype(np.float64), ref16)
        say(f"   b={int(b)}: int4 rel {w1:.2e}, fp16 rel {w2:.2e}")
