"""GPU parity of the D=128 SRFT encoder with the DFT on the matrix cores
(plan option KVQ_OPT_MFMA_ROTATION: the 64-point DFT factored as two 8-point
stages, fp16 MFMA against the exact fp16 input with a hi/lo-split matrix,
then fp32 MFMA with the twiddles folded in).  Same bars as the VALU encoder:
the rotated fp32 within 1e-5 relative per vector, codes and scales bit-exact
except at rounding boundaries (fraction < 1e-5 for int4, 1e-4 for int8), and
the codes decode through the ordinary decoder."""

import numpy as np
import pytest
import torch

import oracle as O
import kv_cache_int4_amd as K
from kv_cache_int4_amd import workloads as W
from tests import parity as P
from tests.test_gpu_formats import decode_both
from tests.test_gpu_parity import check_encode, lam_per_vector, np16, say

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.library()


def _x(B, H, T, D, seed, scale=1.0, pad=0):
    g = torch.Generator().manual_seed(seed)
    std = torch.exp(0.5 * torch.randn((H, D + pad), generator=g))
    base = (torch.randn((B, H, T + 2, D + pad), generator=g) * std[None, :, None, :] * scale).to(torch.float16)
    return base[:, :, 1:1 + T, :D]


@pytest.mark.parametrize("T", [1, 5, 16, 63, 64, 200])
@pytest.mark.parametrize("shared_lam", [True, False])
def test_mfma_rotation_small(T, shared_lam):
    """The rotated values w = lambda R x (rotate mode of the same kernel)
    within 1e-5 relative, on ragged tiles (T = 1 .. 200: partial groups of
    16 vectors and partial tiles) with padded input rows."""
    B, H, D = 2, 3, 128
    x = _x(B, H, T, D, 10 + T, pad=8)
    lam = torch.exp(0.3 * torch.randn((H, D) if shared_lam else (B, H, D), generator=torch.Generator().manual_seed(3)))
    plan = K.Plan(D, 32, "srft", 1234, mfma=True)
    w = torch.empty((B, H, T, D), dtype=torch.float32, device="cuda")
    K.rotate(plan, x.cuda(), lam.cuda(), w)
    torch.cuda.synchronize()
    signs = O.plan_signs(D, O.SRFT, plan.seed)
    worst = P.compare_rotation(np16(w).reshape(-1, D), np16(x).reshape(-1, D), lam_per_vector(lam, B, H, T), O.SRFT,
                               signs)
    say(f"[mfma rotate] T={T}: rel err {worst:.2e}")


@pytest.mark.parametrize("bits,G", [(4, 32), (4, 16), (8, 32), (8, 16)])
@pytest.mark.parametrize("scale", [0.01, 1.0, 30.0])
def test_mfma_encode_ragged_offsets(bits, G, scale):
    """Codes and scales of every format, written at an offset t0 inside a
    larger cache (canaries around the written tokens), then decoded by the
    ordinary decoder."""
    B, H, T, D = 2, 2, 131, 128
    x = _x(B, H, T, D, 77, scale=scale, pad=16)
    lam = torch.exp(0.3 * torch.randn((B, H, D), generator=torch.Generator().manual_seed(5)))
    plan = K.Plan(D, G, "srft", 99, bits=bits, mfma=True)
    codes_d, scales_d, c, s, rep = check_encode(f"mfma-int{bits}-g{G}", plan, "srft", x, lam, Tcap=T + 40, t0=17)
    r16, r32 = decode_both(plan, "srft", codes_d, scales_d, c, s, lam, B, H, T, t0=17)
    say(f"   decode fp16 {r16}, fp32 {r32}")


def test_mfma_qwen_prefix_full():
    """The Qwen2.5-1.5B-shaped prefix (458,752 vectors): every vector, with
    the rotation alone against the oracle on a sample."""
    cfg = W.CONFIGS["qwen"]
    x, lam = W.prefix_inputs(cfg)
    plan = K.Plan(cfg.D, 32, "srft", cfg.sign_seed, mfma=True)
    _, _, _, _, rep = check_encode("qwen-mfma", plan, "srft", x, lam)
    assert rep["elements"] == cfg.vectors * cfg.D
    B, H, T, D = x.shape
    w = torch.empty((B, H, T, D), dtype=torch.float32, device="cuda")
    K.rotate(plan, x.cuda(), lam.cuda(), w)
    torch.cuda.synchronize()
    idx = np.random.default_rng(1).choice(B * H * T, 20000, replace=False)
    lv = lam.numpy()[(idx // T) // H, (idx // T) % H]
    worst = P.compare_rotation(np16(w).reshape(-1, D)[idx], np16(x).reshape(-1, D)[idx], lv, O.SRFT,
                               O.plan_signs(D, O.SRFT, plan.seed))
    say(f"   rotation rel err {worst:.2e}")


def test_mfma_multi_tile_waves_sampled():
    """More tiles than the grid holds (B=2, H=8, T=80000: 20,000 tiles, over
    64 waves per CU), so waves take several tiles: 16384 seeded sample
    vectors checked."""
    B, H, T, D = 2, 8, 80000, 128
    g = W.gen("cuda", 55, D, T)
    std = torch.exp(0.5 * torch.randn((H, D), generator=g, device="cuda"))
    x = (torch.randn((B, H, T, D), generator=g, device="cuda") * std[None, :, None, :]).to(torch.float16)
    lam = torch.exp(0.3 * torch.randn((B, H, D), generator=g, device="cuda"))
    plan = K.Plan(D, 32, "srft", 4242, mfma=True)
    codes = torch.empty((B, H, T, D // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((B, H, T, D // 32), dtype=torch.float16, device="cuda")
    K.encode(plan, x, lam, codes, scales)
    torch.cuda.synchronize()
    idx = torch.from_numpy(np.random.default_rng(5).choice(B * H * T, 16384, replace=False)).cuda()
    xs = x.reshape(-1, D)[idx].cpu().numpy()
    cs = codes.reshape(-1, D // 2)[idx].cpu().numpy()
    ss = scales.reshape(-1, D // 32)[idx].cpu().numpy()
    lv = lam.reshape(B * H, D)[(idx // T)].cpu().numpy()
    rep = P.compare_codes(cs, ss, xs, lv, O.SRFT, O.plan_signs(D, O.SRFT, plan.seed))
    say(f"   sampled codes: {rep['code_mismatch']} / {rep['scale_mismatch']} mismatches")


def test_mfma_matches_valu_encoder_where_decisive():
    """Both encoders on the same input: every code and scale that differs
    between them lies at a rounding boundary of the oracle (the two
    transforms round differently), and they differ rarely."""
    cfg = W.CONFIGS["qwen"]
    x, lam = W.prefix_inputs(W.Config(cfg.name, cfg.D, 4, cfg.H, cfg.T, cfg.law, cfg.index))
    out = []
    for mfma in (False, True):
        plan = K.Plan(cfg.D, 32, "srft", cfg.sign_seed, mfma=mfma)
        B, H, T, D = x.shape
        codes = torch.empty((B, H, T, D // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((B, H, T, D // 32), dtype=torch.float16, device="cuda")
        K.encode(plan, x.cuda(), lam.cuda(), codes, scales)
        torch.cuda.synchronize()
        out.append((codes.cpu().numpy(), scales.cpu().numpy()))
    dc = int((out[0][0] != out[1][0]).sum())
    ds = int((out[0][1].view(np.uint16) != out[1][1].view(np.uint16)).sum())
    say(f"   VALU vs MFMA encoder: {dc} code bytes, {ds} scales differ of {out[0][0].size}, {out[0][1].size}")
    assert dc <= 1e-4 * out[0][0].size and ds <= 1e-3 * out[0][1].size
