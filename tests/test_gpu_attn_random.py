"""GPU parity of decode-step attention on seeded random call shapes: every
rotation and code format, batch 1-3, 1-3 kv heads with 1-8 query heads
each (so that a wave's chunk of four heads is full, partial, or one of two),
sequence lengths from one token to a few thousand with caches longer than
the sequence, fp32 or fp16 output; the fp16-cache comparator on the same
shape.  Each case against the oracle at the 2e-3 relative bar.
"""

import math

import numpy as np
import pytest
import torch

import kv_cache_int4_amd as K
from tests import parity as P
from tests.test_gpu_formats import FORMATS as OTHER_FORMATS, format_cache, oracle_attention
from tests.test_gpu_parity import np16, run_attn, say
import oracle as O

pytestmark = pytest.mark.gpu

N_CASES = 24
FORMATS = dict(OTHER_FORMATS, **{"int4-g32": (4, 32)})


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.library()


def draw_case(i: int):
    rng = np.random.default_rng(5000 + i)
    rot = str(rng.choice(["srft", "srht", "identity"]))
    fmt = str(rng.choice(sorted(FORMATS)))
    B = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 4))
    rep = int(rng.integers(1, 9))
    L = int(rng.choice([1, 2, 31, 32, 33])) if i % 4 == 0 else int(rng.integers(34, 3000))
    Tcap = L + int(rng.integers(0, 40))
    out_dt = torch.float16 if rng.integers(2) else torch.float32
    return dict(rot=rot, fmt=fmt, B=B, Hkv=Hkv, Hq=Hkv * rep, L=L, Tcap=Tcap, out_dt=out_dt, seed=6000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_attention_random_shape(i):
    c = draw_case(i)
    say(f"[attn-random {i}] {c}")
    bits, G = FORMATS[c["fmt"]]
    D, B, Hq, Hkv, L = 128, c["B"], c["Hq"], c["Hkv"], c["L"]
    plan = K.Plan(D, G, c["rot"], c["seed"], bits=bits)
    q, kc, ksc, vc, vsc, lam_k, lam_v = format_cache(plan, B, Hkv, Hq, L, c["Tcap"], c["seed"])
    sm = 1 / math.sqrt(D)
    ref = oracle_attention(plan, c["rot"], q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm)
    out = run_attn(plan, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm, c["out_dt"])
    worst = P.compare_attention(np16(out), ref)
    say(f"   int4/int8 cache: rel err {worst:.2e}")
    # the fp16-cache comparator over the same shape
    g = torch.Generator(device="cuda").manual_seed(c["seed"])
    k16 = torch.randn((B, Hkv, c["Tcap"], D), generator=g, device="cuda").to(torch.float16)
    v16 = torch.randn((B, Hkv, c["Tcap"], D), generator=g, device="cuda").to(torch.float16)
    ws = torch.empty(K.attn_workspace_size(D, B, Hq, L), dtype=torch.uint8, device="cuda")
    o16 = torch.empty((B, Hq, D), dtype=c["out_dt"], device="cuda")
    K.attn_decode_f16(q, k16, v16, L, sm, o16, ws)
    torch.cuda.synchronize()
    ref16 = O.attention_f16(np16(q), np16(k16), np16(v16), L, sm)
    worst16 = P.compare_attention(np16(o16), ref16)
    say(f"   fp16 cache: rel err {worst16:.2e}")
