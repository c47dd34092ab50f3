"""GPU parity at head sizes that are not powers of two: D = 96 (M = 48 =
4*4*3) and D = 80 (M = 40 = 4*2*5), the SRFT over the mixed-radix DFT and the
unrotated codec, in every code format whose group size divides D (D = 80:
groups of 16 only).

The bars are those of the power-of-two sizes: rotated fp32 within 1e-5
relative; codes and scales bit-exact except within 1e-4 of a rounding
boundary (mismatch fraction below 1e-5 for int4, 1e-4 for int8 codes);
decoded values within 1e-3 absolute (fp32) or half an fp16 ulp plus 1e-3
(fp16).
"""

import numpy as np
import pytest
import torch

import oracle as O
import kv_cache_int4_amd as K
from kv_cache_int4_amd import workloads as W
from tests import parity as P
from tests.test_gpu_formats import decode_both
from tests.test_gpu_parity import ROTS, check_encode, lam_per_vector, np16, say

pytestmark = pytest.mark.gpu

FORMATS = {"int4-g32": (4, 32), "int4-g16": (4, 16), "int8-g32": (8, 32), "int8-g16": (8, 16)}
CASES = [(D, f) for D in (96, 80) for f in sorted(FORMATS) if D % FORMATS[f][1] == 0]


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.library()


@pytest.mark.parametrize("D,fmt", CASES)
@pytest.mark.parametrize("rot", ["srft", "identity"])
@pytest.mark.parametrize("T", [1, 63, 130])
def test_mixed_ragged_offsets_strides(D, fmt, rot, T):
    """Ragged tails (one token, a partial tile, two tiles and a tail), a
    write offset inside a larger cache, strided input rows, lambda shared
    across the batch; rotation, fp16 and fp32 decode."""
    bits, G = FORMATS[fmt]
    g = W.gen("cpu", 93, D, T)
    B, H = 3, 2
    base = torch.randn((B, H, T + 5, D + 24), generator=g).to(torch.float16) * 3
    x = base[:, :, 2:2 + T, 8:8 + D]
    lam = torch.exp(0.3 * torch.randn((H, D), generator=g))
    plan = K.Plan(D, G, rot, 6161, bits=bits)
    codes_d, scales_d, c, s, _ = check_encode(f"mixed-{fmt}", plan, rot, x, lam, Tcap=T + 40, t0=17)
    r16, r32 = decode_both(plan, rot, codes_d, scales_d, c, s, lam, B, H, T, t0=17)
    say(f"   decode fp16 {r16}, fp32 {r32}")
    w = torch.empty((B, H, T, D), dtype=torch.float32, device="cuda")
    K.rotate(plan, x.cuda(), lam.cuda(), w)
    torch.cuda.synchronize()
    signs = O.plan_signs(D, ROTS[rot], plan.seed)
    worst = P.compare_rotation(np16(w).reshape(-1, D), np16(x).reshape(-1, D), lam_per_vector(lam, B, H, T),
                               ROTS[rot], signs)
    say(f"   rotation rel err {worst:.2e}")


@pytest.mark.parametrize("key", ["d96", "d80"])
def test_mixed_prefix_full_int4(key):
    """The 28-layer prefix shape (458,752 vectors) at D=96 / D=80, SRFT, int4
    codes in groups of 16: every vector's codes and scales, and its fp16
    decode, checked; the decode error within the quantization bound."""
    cfg = W.CONFIGS[key]
    x, lam = W.prefix_inputs(cfg)
    plan = K.Plan(cfg.D, 16, "srft", cfg.sign_seed)
    codes_d, scales_d, c, s, rep = check_encode(f"{key}-int4-g16", plan, "srft", x, lam)
    assert rep["elements"] == cfg.vectors * cfg.D
    B, H, T, D = x.shape
    y = torch.empty((B, H, T, D), dtype=torch.float16, device="cuda")
    K.decode(plan, codes_d, scales_d, lam.cuda(), y)
    torch.cuda.synchronize()
    signs = O.plan_signs(D, O.SRFT, plan.seed)
    lv = lam_per_vector(lam, B, H, T)
    yh = np16(y).reshape(-1, D)
    r = P.compare_decode(yh, c.reshape(-1, plan.code_bytes), s.reshape(-1, D // 16), lv, O.SRFT, signs, 16)
    say(f"   decode fp16: {r}")
    # |x - decode|_2 <= |sigma / (2 lambda)|_2 (orthogonal rotation), plus
    # the fp16 rounding of the output
    sig = np.repeat(s.reshape(-1, D // 16).astype(np.float64), 16, axis=-1)
    bound = np.linalg.norm(sig / (2 * lv.astype(np.float64)), axis=-1)
    xh = np16(x).reshape(-1, D).astype(np.float64)
    err = np.linalg.norm(yh.astype(np.float64) - xh, axis=-1)
    slack = np.linalg.norm(P.ulp16(xh) / 2, axis=-1) + 1e-3
    assert np.all(err <= bound * (1 + 1e-4) + slack)


@pytest.mark.parametrize("D,fmt", [c for c in CASES if c[1] != "int4-g16"])
def test_mixed_prefix_formats(D, fmt):
    """The other formats on 8 layers of the prefix shape (131,072 vectors),
    SRFT: every vector checked, fp16 decode included."""
    bits, G = FORMATS[fmt]
    cfg = W.CONFIGS["d96" if D == 96 else "d80"]
    x, lam = W.prefix_inputs(cfg)
    x, lam = x[:16], lam[:16]
    plan = K.Plan(D, G, "srft", cfg.sign_seed, bits=bits)
    codes_d, scales_d, c, s, _ = check_encode(f"D{D}-{fmt}", plan, "srft", x, lam)
    B, H, T, _ = x.shape
    y = torch.empty((B, H, T, D), dtype=torch.float16, device="cuda")
    K.decode(plan, codes_d, scales_d, lam.cuda(), y)
    torch.cuda.synchronize()
    signs = O.plan_signs(D, O.SRFT, plan.seed)
    r = P.compare_decode(np16(y).reshape(-1, D), c.reshape(-1, plan.code_bytes), s.reshape(-1, D // G),
                         lam_per_vector(lam, B, H, T), O.SRFT, signs, G, bits=bits)
    say(f"   decode fp16: {r}")


@pytest.mark.parametrize("D,fmt", CASES)
def test_mixed_special_groups(D, fmt):
    """Identity rotation: exact grid values, half-even ties with
    power-of-two scales, all-zero groups and subnormal-scale groups."""
    bits, G = FORMATS[fmt]
    qmin, qmax = O.code_range(bits)
    rng = np.random.default_rng(18)
    N = 70
    x = np.zeros((N, D), dtype=np.float16)
    for n in range(N):
        for g in range(D // G):
            kind = (n + g) % 4
            sl = slice(G * g, G * g + G)
            if kind == 0:
                k = rng.integers(-qmax, qmax + 1, G)
                k[0] = qmax
                x[n, sl] = (k * 0.5).astype(np.float16)
            elif kind == 1:
                t = np.array([qmax, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5] * (G // 8), dtype=np.float64)
                x[n, sl] = t.astype(np.float16)
            elif kind == 3:
                m = rng.integers(-(qmax + qmax // 2), qmax + qmax // 2 + 1, G)
                m[0] = qmax + qmax // 2
                x[n, sl] = (m * 2.0 ** -24).astype(np.float16)
    xt = torch.from_numpy(x).reshape(1, 1, N, D)
    lt = torch.ones((1, D), dtype=torch.float32)
    plan = K.Plan(D, G, "identity", 0, bits=bits)
    _, _, c, s, _ = check_encode(f"special-D{D}-{fmt}", plan, "identity", xt, lt)
    codes_ref, scales_ref, _ = O.encode(x, np.ones((N, D), dtype=np.float32), O.IDENTITY,
                                        O.plan_signs(D, O.IDENTITY, 0), G, bits)
    assert np.array_equal(s.reshape(N, -1).view(np.uint16), scales_ref.view(np.uint16))
    assert np.array_equal(c.reshape(N, -1), codes_ref)
    assert (O.unpack_codes(codes_ref, bits) == qmin).any()


def test_mixed_rejections_and_empty():
    """SRHT and groups that do not divide D are refused at plan creation;
    empty calls are no-ops."""
    for D, G, rot in [(96, 32, "srht"), (80, 32, "srft"), (80, 16, "srht")]:
        with pytest.raises(K.KvqError):
            K.Plan(D, G, rot, 0)
    plan = K.Plan(96, 32, "srft", 1)
    x = torch.empty((2, 3, 0, 96), dtype=torch.float16, device="cuda")
    lam = torch.ones((3, 96), dtype=torch.float32, device="cuda")
    codes = torch.full((2, 3, 4, plan.code_bytes), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((2, 3, 4, 3), 1234.0, dtype=torch.float16, device="cuda")
    K.encode(plan, x, lam, codes, scales, 2)
    torch.cuda.synchronize()
    assert bool((codes == 0x5A).all()) and bool((scales == 1234.0).all())


@pytest.mark.parametrize("D,G", [(96, 32), (80, 16)])
def test_mixed_multi_tile_waves_sampled(D, G):
    """A call with more tiles than the grid holds (B=4, H=8, T=20000: 10,016
    tiles, over 32 waves per CU), so waves take several tiles and stream the
    next one in while computing: 16384 seeded sample vectors checked against
    the oracle, encode and fp16 decode."""
    B, H, T = 4, 8, 20000
    g = W.gen("cuda", 77, D, T)
    std = torch.exp(0.5 * torch.randn((H, D), generator=g, device="cuda"))
    x = (torch.randn((B, H, T, D), generator=g, device="cuda") * std[None, :, None, :]).to(torch.float16)
    lam = torch.exp(0.3 * torch.randn((B, H, D), generator=g, device="cuda"))
    plan = K.Plan(D, G, "srft", 4242)
    codes = torch.empty((B, H, T, plan.code_bytes), dtype=torch.uint8, device="cuda")
    scales = torch.empty((B, H, T, D // G), dtype=torch.float16, device="cuda")
    K.encode(plan, x, lam, codes, scales)
    y = torch.empty_like(x)
    K.decode(plan, codes, scales, lam, y)
    torch.cuda.synchronize()
    idx = torch.from_numpy(np.random.default_rng(5).choice(B * H * T, 16384, replace=False)).cuda()
    xs = x.reshape(-1, D)[idx].cpu().numpy()
    cs = codes.reshape(-1, plan.code_bytes)[idx].cpu().numpy()
    ss = scales.reshape(-1, D // G)[idx].cpu().numpy()
    ys = y.reshape(-1, D)[idx].cpu().numpy()
    lv = lam.reshape(B * H, D)[(idx // T)].cpu().numpy()
    signs = O.plan_signs(D, O.SRFT, plan.seed)
    rep = P.compare_codes(cs, ss, xs, lv, O.SRFT, signs, G)
    say(f"   D={D} sampled codes: {rep['code_mismatch']} / {rep['scale_mismatch']} mismatches")
    P.compare_decode(ys, cs, ss, lv, O.SRFT, signs, G)
