"""GPU parity on seeded random call shapes: every head size (80, 96, 128,
256), rotation and code format the plans accept, with random batch, head
and token counts, write offsets inside larger caches, padded input rows and
lambda tables shared or per batch.  Encode (codes and scales), the rotation
alone, and the fp16 and fp32 decodes are checked against the CPU oracle at
the bars of tests/parity.py.
"""

import numpy as np
import pytest
import torch

import oracle as O
import kv_cache_int4_amd as K
from tests import parity as P
from tests.test_gpu_formats import decode_both
from tests.test_gpu_parity import ROTS, check_encode, lam_per_vector, np16, say

pytestmark = pytest.mark.gpu

N_CASES = 40


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.library()


def draw_case(i: int):
    """Shape and plan of case i (seeded by i)."""
    rng = np.random.default_rng(1000 + i)
    D = int(rng.choice([80, 96, 128, 256]))
    rots = ["srft", "identity"] + (["srht"] if D in (128, 256) else [])
    rot = str(rng.choice(rots))
    fmts = [(b, g) for b in (4, 8) for g in (32, 16) if D % g == 0]
    bits, G = fmts[int(rng.integers(len(fmts)))]
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    T = int(rng.integers(1, 200))
    t0 = int(rng.integers(0, 21))
    Tcap = t0 + T + int(rng.integers(0, 9))
    pad = 8 * int(rng.integers(0, 3))        # extra fp16 per input row (16-byte rows)
    shared_lam = bool(rng.integers(2))
    scale = float(rng.choice([0.01, 1.0, 30.0]))
    return dict(D=D, rot=rot, bits=bits, G=G, B=B, H=H, T=T, t0=t0, Tcap=Tcap, pad=pad,
                shared_lam=shared_lam, scale=scale, seed=2000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    c = draw_case(i)
    say(f"[case {i}] {c}")
    g = torch.Generator().manual_seed(c["seed"])
    D, B, H, T = c["D"], c["B"], c["H"], c["T"]
    base = (torch.randn((B, H, T + 2, D + c["pad"]), generator=g) * c["scale"]).to(torch.float16)
    x = base[:, :, 1:1 + T, :D]
    lam_shape = (H, D) if c["shared_lam"] else (B, H, D)
    lam = torch.exp(0.3 * torch.randn(lam_shape, generator=g))
    plan = K.Plan(D, c["G"], c["rot"], c["seed"], bits=c["bits"])
    name = f"case{i}-D{D}-{c['rot']}-int{c['bits']}-g{c['G']}"
    codes_d, scales_d, cc, ss, _ = check_encode(name, plan, c["rot"], x, lam, Tcap=c["Tcap"], t0=c["t0"])
    r16, r32 = decode_both(plan, c["rot"], codes_d, scales_d, cc, ss, lam, B, H, T, t0=c["t0"])
    say(f"   decode fp16 {r16}, fp32 {r32}")
    w = torch.empty((B, H, T, D), dtype=torch.float32, device="cuda")
    K.rotate(plan, x.cuda(), lam.cuda(), w)
    torch.cuda.synchronize()
    signs = O.plan_signs(D, ROTS[c["rot"]], plan.seed)
    worst = P.compare_rotation(np16(w).reshape(-1, D), np16(x).reshape(-1, D), lam_per_vector(lam, B, H, T),
                               ROTS[c["rot"]], signs)
    say(f"   rotation rel err {worst:.2e}")
