"""GPU parity: libkvq (through the C ABI) against the CPU oracle on the same
seeded inputs.

Bars: rotated fp32 within 1e-5 relative per vector; codes and scales
bit-exact except within 1e-4 of a rounding boundary with the mismatch
fraction below 1e-5; decoded values within 1e-3 absolute (fp32) or half an
fp16 ulp plus 1e-3 (fp16); attention within 2e-3 relative per (batch,
head).  Output buffers carry canary bytes around the written
region to catch stray writes.
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


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.library()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np16(t):
    return t.detach().cpu().numpy()


def lam_per_vector(lam, B, H, T):
    """lambda [B,H,D] or [H,D] -> [B*H*T, D] for the oracle."""
    l = lam.detach().cpu().numpy().astype(np.float32)
    if l.ndim == 2:
        l = np.broadcast_to(l[None], (B,) + l.shape)
    return np.repeat(l[:, :, None, :], T, axis=2).reshape(-1, l.shape[-1])


def gpu_encode(plan, x, lam, Tcap=None, t0=0):
    """Encode on the GPU into a cache pre-filled with canary values; return
    the device buffers and the written slice, and assert that every token
    outside [t0, t0 + T) still holds its canary."""
    B, H, T, D = x.shape
    Tcap = T + t0 if Tcap is None else Tcap
    codes = torch.full((B, H, Tcap, plan.code_bytes), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((B, H, Tcap, D // plan.G), 1234.0, dtype=torch.float16, device="cuda")
    K.encode(plan, x, lam, codes, scales, t0)
    torch.cuda.synchronize()
    c, s = codes.cpu(), scales.cpu()
    if t0 > 0:
        assert bool((c[:, :, :t0] == 0x5A).all()) and bool((s[:, :, :t0] == 1234.0).all())
    if t0 + T < Tcap:
        assert bool((c[:, :, t0 + T:] == 0x5A).all()) and bool((s[:, :, t0 + T:] == 1234.0).all())
    return codes, scales, c[:, :, t0:t0 + T].numpy(), s[:, :, t0:t0 + T].numpy()


def check_encode(name, plan, rot, x, lam, Tcap=None, t0=0):
    B, H, T, D = x.shape
    say(f"[encode] {name} D={D} rot={rot} bits={plan.bits} G={plan.G} B={B} H={H} T={T} t0={t0}")
    xd = x.cuda() if not x.is_cuda else x
    codes_d, scales_d, c, s = gpu_encode(plan, xd, lam.cuda(), Tcap, t0)
    signs = O.plan_signs(D, ROTS[rot], plan.seed)
    xs = np16(x).reshape(-1, D)
    lv = lam_per_vector(lam, B, H, T)
    rep = P.compare_codes(c.reshape(-1, plan.code_bytes), s.reshape(-1, D // plan.G), xs, lv, ROTS[rot], signs,
                          plan.G, plan.bits)
    say(f"   codes ok: code mismatches {rep['code_mismatch']}, scale mismatches {rep['scale_mismatch']}, "
        f"fraction {rep['mismatch_frac']:.2e}")
    return codes_d, scales_d, c, s, rep


# ----------------------------------------------------------------- encode --

@pytest.mark.parametrize("rot", ["srft", "srht", "identity"])
def test_small_roundtrip_all_rotations(rot):
    cfg = W.CONFIGS["small"]
    x, lam = W.prefix_inputs(cfg)
    plan = K.Plan(cfg.D, 32, rot, cfg.sign_seed)
    codes_d, scales_d, c, s, rep = check_encode("small", plan, rot, x, lam)
    signs = O.plan_signs(cfg.D, ROTS[rot], plan.seed)
    B, H, T, D = x.shape
    lv = lam_per_vector(lam, B, H, T)
    # rotation alone
    w = torch.empty((B, H, T, D), dtype=torch.float32, device="cuda")
    K.rotate(plan, x.cuda(), lam.cuda(), w)
    worst = P.compare_rotation(np16(w).reshape(-1, D), np16(x).reshape(-1, D), lv, ROTS[rot], signs)
    say(f"   rotation rel err {worst:.2e}")
    # decode fp32 and fp16 of the same codes
    for dt in (torch.float32, torch.float16):
        y = torch.empty((B, H, T, D), dtype=dt, device="cuda")
        K.decode(plan, codes_d, scales_d, lam.cuda(), y)
        torch.cuda.synchronize()
        r = P.compare_decode(np16(y).reshape(-1, D), c.reshape(-1, D // 2), s.reshape(-1, D // 32), lv,
                             ROTS[rot], signs)
        say(f"   decode {dt}: {r}")
    # round trip within the quantization bound (orthogonality)
    y = torch.empty((B, H, T, D), dtype=torch.float32, device="cuda")
    K.decode(plan, codes_d, scales_d, lam.cuda(), y)
    sig = np.repeat(s.reshape(-1, D // 32).astype(np.float64), 32, axis=-1)
    bound = np.linalg.norm(sig / (2 * lv.astype(np.float64)), axis=-1)
    err = np.linalg.norm(np16(y).reshape(-1, D).astype(np.float64) - np16(x).reshape(-1, D), axis=-1)
    normal = (sig >= 2.0 ** -14).all(axis=-1)
    assert np.all((err <= bound * (1 + 1e-4) + 1e-4)[normal])


def test_qwen_prefix_full_srft():
    """Qwen2.5-1.5B-shaped prefix (28 layers x {K,V} x 2 heads x 4096 tokens,
    D=128): every vector checked."""
    cfg = W.CONFIGS["qwen"]
    x, lam = W.prefix_inputs(cfg)
    plan = K.Plan(cfg.D, 32, "srft", cfg.sign_seed)
    _, _, _, _, rep = check_encode("qwen-full", plan, "srft", x, lam)
    assert rep["elements"] == cfg.vectors * cfg.D


@pytest.mark.parametrize("rot", ["srft", "srht"])
def test_gemma_prefix_full(rot):
    """Gemma-3-1B-shaped prefix (26 layers x {K,V} x 1 head x 4096 tokens,
    D=256), SRFT and SRHT: every vector checked, decode included."""
    cfg = W.CONFIGS["gemma"]
    x, lam = W.prefix_inputs(cfg)
    plan = K.Plan(cfg.D, 32, rot, cfg.sign_seed)
    codes_d, scales_d, c, s, rep = check_encode("gemma-full", plan, rot, x, lam)
    B, H, T, D = x.shape
    signs = O.plan_signs(D, ROTS[rot], plan.seed)
    lv = lam_per_vector(lam, B, H, T)
    y = torch.empty((B, H, T, D), dtype=torch.float16, device="cuda")
    K.decode(plan, codes_d, scales_d, lam.cuda(), y)
    torch.cuda.synchronize()
    r = P.compare_decode(np16(y).reshape(-1, D), c.reshape(-1, D // 2), s.reshape(-1, D // 32), lv,
                         ROTS[rot], signs)
    say(f"   decode fp16: {r}")


# Calls of a few thousand vectors or fewer run one wave per vector, larger
# ones the tile kernels: batch sizes that put a call on either path.
PATH_VECTORS = 8200


def batch_for(path: str, H: int, T: int) -> int:
    return 3 if path == "lanes" else PATH_VECTORS // (H * T) + 1


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("rot", ["srft", "srht", "identity"])
@pytest.mark.parametrize("T,path", [(1, "lanes"), (63, "lanes"), (65, "lanes"), (130, "lanes"), (1, "tiles"),
                                    (63, "tiles"), (130, "tiles")])
def test_ragged_tokens_offsets_strides(D, rot, T, path):
    """Ragged tails, a write offset inside a larger cache, strided input rows
    and a lambda table shared across the batch; on the one-wave-per-vector
    path (small calls) and on the tile path."""
    g = W.gen("cpu", 77, D, T)
    H = 2
    B = batch_for(path, H, T)
    base = torch.randn((B, H, T + 5, D + 24), generator=g).to(torch.float16) * 3
    x = base[:, :, 2:2 + T, 8:8 + D]            # strides (H*(T+5)*(D+24), ...), row stride D+24
    lam = torch.exp(0.3 * torch.randn((H, D), generator=g))
    plan = K.Plan(D, 32, rot, 4242)
    codes_d, scales_d, c, s, _ = check_encode("ragged", plan, rot, x, lam, Tcap=T + 40, t0=17)
    signs = O.plan_signs(D, ROTS[rot], plan.seed)
    lv = lam_per_vector(lam, B, H, T)
    # decode the written tokens into a strided fp16 output and fp32
    out = torch.full((B, H, T + 3, D + 8), 7.0, dtype=torch.float16, device="cuda")
    y = out[:, :, 1:1 + T, :D]
    K.decode(plan, codes_d, scales_d, lam.cuda(), y, t0=17)
    torch.cuda.synchronize()
    o = out.cpu()
    assert bool((o[:, :, 0] == 7.0).all()) and bool((o[:, :, 1 + T:] == 7.0).all())
    assert bool((o[:, :, :, D:] == 7.0).all())
    P.compare_decode(np16(y).reshape(-1, D), c.reshape(-1, D // 2), s.reshape(-1, D // 32), lv,
                     ROTS[rot], signs)
    y32 = torch.empty((B, H, T, D), dtype=torch.float32, device="cuda")
    K.decode(plan, codes_d, scales_d, lam.cuda(), y32, t0=17)
    torch.cuda.synchronize()
    P.compare_decode(np16(y32).reshape(-1, D), c.reshape(-1, D // 2), s.reshape(-1, D // 32), lv,
                     ROTS[rot], signs)


@pytest.mark.parametrize("D", [128, 256])
def test_quantizer_special_groups(D):
    """Identity rotation: exact grid values, half-even ties with power-of-two
    scales, all-zero groups and subnormal-scale groups (clamp to -8)."""
    rng = np.random.default_rng(5)
    N = 64
    x = np.zeros((N, D), dtype=np.float16)
    lam = np.ones((N, D), dtype=np.float32)
    for n in range(N):
        for g in range(D // 32):
            kind = (n + g) % 4
            sl = slice(32 * g, 32 * g + 32)
            if kind == 0:       # exact grid with sigma = 0.5
                k = rng.integers(-7, 8, 32)
                k[0] = 7
                x[n, sl] = (k * 0.5).astype(np.float16)
            elif kind == 1:     # ties with sigma = 1
                x[n, sl] = np.array([7, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5] * 4, dtype=np.float16)
            elif kind == 2:     # all zero
                pass
            else:               # subnormal scale: multiples of 2^-24
                m = rng.integers(-10, 11, 32)
                m[0] = 10
                x[n, sl] = (m * 2.0 ** -24).astype(np.float16)
    xt = torch.from_numpy(x).reshape(1, 1, N, D)
    lt = torch.ones((1, D), dtype=torch.float32)
    plan = K.Plan(D, 32, "identity", 0)
    _, _, c, s, rep = check_encode("special", plan, "identity", xt, lt)
    codes_ref, scales_ref, _ = O.encode(x, lam, O.IDENTITY, O.plan_signs(D, O.IDENTITY, 0))
    assert np.array_equal(s.reshape(N, -1).view(np.uint16), scales_ref.view(np.uint16))
    assert np.array_equal(c.reshape(N, -1), codes_ref)
    assert (O.unpack_nibbles(codes_ref) == -8).any()


def test_empty_calls_are_noops():
    plan = K.Plan(128, 32, "srft", 1)
    x = torch.zeros((2, 2, 0, 128), dtype=torch.float16, device="cuda")
    lam = torch.ones((2, 128), device="cuda")
    codes = torch.full((2, 2, 8, 64), 3, dtype=torch.uint8, device="cuda")
    scales = torch.zeros((2, 2, 8, 4), dtype=torch.float16, device="cuda")
    K.encode(plan, x, lam, codes, scales, 4)
    torch.cuda.synchronize()
    assert bool((codes == 3).all())


def test_mistral_bulk_sampled():
    """Mistral-7B-shaped bulk calls at full per-call size (B=16, H=8,
    T=8192, D=128, Student-t(3) values): two calls (layer 0 K and V) encoded
    and decoded on the GPU, 32768 seeded sample vectors checked against the
    oracle."""
    cfg = W.CONFIGS["mistral"]
    plan = K.Plan(cfg.D, 32, "srft", cfg.sign_seed)
    signs = O.plan_signs(cfg.D, O.SRFT, plan.seed)
    rng = np.random.default_rng(0)
    for kv in (0, 1):
        say(f"[mistral] call layer 0 kv {kv}")
        x = W.student_t3(cfg.H, cfg.T, cfg.D, cfg.data_seed, "cuda", 0, kv).unsqueeze(0).expand(
            cfg.B, -1, -1, -1).contiguous()
        # batch rows differ: perturb deterministically per batch row
        x = (x.float() * (1.0 + 0.01 * torch.arange(cfg.B, device="cuda").view(-1, 1, 1, 1))).half()
        lam = W.lognormal_lambda((cfg.H, cfg.D), cfg.lambda_seed, "cuda", 0.3, 0, kv)
        codes = torch.empty((cfg.B, cfg.H, cfg.T, cfg.D // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((cfg.B, cfg.H, cfg.T, cfg.D // 32), dtype=torch.float16, device="cuda")
        K.encode(plan, x, lam, codes, scales)
        y = torch.empty_like(x)
        K.decode(plan, codes, scales, lam, y)
        torch.cuda.synchronize()
        idx = rng.choice(cfg.B * cfg.H * cfg.T, 32768, replace=False)
        xs = x.reshape(-1, cfg.D)[torch.from_numpy(idx).cuda()].cpu().numpy()
        cs = codes.reshape(-1, cfg.D // 2)[torch.from_numpy(idx).cuda()].cpu().numpy()
        ss = scales.reshape(-1, cfg.D // 32)[torch.from_numpy(idx).cuda()].cpu().numpy()
        ys = y.reshape(-1, cfg.D)[torch.from_numpy(idx).cuda()].cpu().numpy()
        heads = (idx // cfg.T) % cfg.H
        lv = lam.cpu().numpy()[heads]
        rep = P.compare_codes(cs, ss, xs, lv, O.SRFT, signs)
        say(f"   codes: {rep['code_mismatch']} / {rep['scale_mismatch']} mismatches")
        P.compare_decode(ys, cs, ss, lv, O.SRFT, signs)


@pytest.mark.parametrize("rot", ["srft", "srht"])
def test_d256_multi_tile_waves_sampled(rot):
    """D=256 with more tiles than the grid holds (B=2, H=8, T=40000: 20,000
    tiles of 32 vectors: more than 64 waves per CU, past which the encoder's
    grid, like the decoder's, stops at 32 per CU), so waves take several
    tiles: 16384 seeded sample vectors checked, encode and fp16 decode."""
    B, H, T, D = 2, 8, 40000, 256
    g = W.gen("cuda", 78, D, T)
    std = torch.exp(0.5 * torch.randn((H, D), generator=g, device="cuda"))
    x = (torch.randn((B, H, T, D), generator=g, device="cuda") * std[None, :, None, :]).to(torch.float16)
    lam = torch.exp(0.3 * torch.randn((H, D), generator=g, device="cuda"))
    plan = K.Plan(D, 32, rot, 4343)
    codes = torch.empty((B, H, T, D // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((B, H, T, D // 32), dtype=torch.float16, device="cuda")
    K.encode(plan, x, lam, codes, scales)
    y = torch.empty_like(x)
    K.decode(plan, codes, scales, lam, y)
    torch.cuda.synchronize()
    idx = torch.from_numpy(np.random.default_rng(6).choice(B * H * T, 16384, replace=False)).cuda()
    xs = x.reshape(-1, D)[idx].cpu().numpy()
    cs = codes.reshape(-1, D // 2)[idx].cpu().numpy()
    ss = scales.reshape(-1, D // 32)[idx].cpu().numpy()
    ys = y.reshape(-1, D)[idx].cpu().numpy()
    lv = lam.cpu().numpy()[((idx // T) % H).cpu().numpy()]
    signs = O.plan_signs(D, ROTS[rot], plan.seed)
    rep = P.compare_codes(cs, ss, xs, lv, ROTS[rot], signs)
    say(f"   D=256 {rot} sampled codes: {rep['code_mismatch']} / {rep['scale_mismatch']} mismatches")
    P.compare_decode(ys, cs, ss, lv, ROTS[rot], signs)


# -------------------------------------------------------------- attention --

def build_cache(plan, B, Hkv, Hq, T, Tcap, D, seed):
    """Decode-step inputs on the GPU and their int4 caches (tokens 0..T-1
    encoded with kvq_encode)."""
    k16, v16, lam_k, lam_v, q = W.decode_inputs(B, Hkv, Hq, Tcap, D, seed, "cuda")
    kc = torch.empty((B, Hkv, Tcap, D // 2), dtype=torch.uint8, device="cuda")
    ksc = torch.empty((B, Hkv, Tcap, D // 32), dtype=torch.float16, device="cuda")
    vc = torch.empty_like(kc)
    vsc = torch.empty_like(ksc)
    K.encode(plan, k16[:, :, :T], lam_k, kc, ksc, 0)
    K.encode(plan, v16[:, :, :T], lam_v, vc, vsc, 0)
    return k16, v16, lam_k, lam_v, q, kc, ksc, vc, vsc


def run_attn(plan, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm, out_dtype=torch.float32):
    B, Hq, D = q.shape
    ws = torch.empty(K.attn_workspace_size(D, B, Hq, L), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), dtype=out_dtype, device="cuda")
    K.attn_decode(plan, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm, out, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("rot", ["srft", "srht", "identity"])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (2, 1), (16, 2)])
@pytest.mark.parametrize("L", [1, 17, 300, 2051])
def test_attention_small(rot, Hq, Hkv, L):
    D, B = 128, 2
    plan = K.Plan(D, 32, rot, 31)
    Tcap = L + 9
    say(f"[attn] rot={rot} Hq={Hq} Hkv={Hkv} L={L}")
    k16, v16, lam_k, lam_v, q, kc, ksc, vc, vsc = build_cache(plan, B, Hkv, Hq, L, Tcap, D, 11)
    sm = 1 / math.sqrt(D)
    signs = O.plan_signs(D, ROTS[rot], plan.seed)
    ref = O.attention_int4(np16(q), kc.cpu().numpy(), ksc.cpu().numpy(), lam_k.cpu().numpy(),
                           vc.cpu().numpy(), vsc.cpu().numpy(), lam_v.cpu().numpy(), L, sm, ROTS[rot], signs)
    for dt in (torch.float32, torch.float16):
        out = run_attn(plan, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm, dt)
        worst = P.compare_attention(np16(out), ref)
        say(f"   int4 {dt}: rel err {worst:.2e}")
    # fp16 comparator over the unquantized cache
    ws = torch.empty(K.attn_workspace_size(D, B, Hq, L), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    K.attn_decode_f16(q, k16, v16, L, sm, out, ws)
    torch.cuda.synchronize()
    ref16 = O.attention_f16(np16(q), k16.cpu().numpy(), v16.cpu().numpy(), L, sm)
    worst = P.compare_attention(np16(out), ref16)
    say(f"   fp16 comparator: rel err {worst:.2e}")


@pytest.mark.parametrize("rot", ["srft", "srht"])
def test_attention_dominant_token(rot):
    """A token whose score exceeds every other by far more than exp2's range
    (about 150 in log2 units): the softmax must take its maximum over every
    row of the block and every split, else exp2 overflows.  The dominant
    tokens sit in rows 1, 2 and 3 of a block, in the tail block and in a
    later split; the output is then (nearly) that token's value vector."""
    D, B, Hq, Hkv = 128, 2, 8, 2
    L = 2051
    Tcap = L + 5
    plan = K.Plan(D, 32, rot, 57)
    say(f"[attn-dominant] rot={rot} L={L}")
    k16, v16, lam_k, lam_v, q = W.decode_inputs(B, Hkv, Hq, Tcap, D, 23, "cuda")
    rep = Hq // Hkv
    # (b, query head, dominant token)
    spots = [(0, 0, 5), (0, 3, 1000 + 32 + 12 + 3), (1, 5, L - 1), (1, 6, 300 + 16 + 8), (1, 1, 1601)]
    for b, h, t in spots:
        qv = q[b, h].float()
        c = 1200.0 / float((qv * qv).sum())
        k16[b, h // rep, t] = (c * qv).to(torch.float16)
    kc = torch.empty((B, Hkv, Tcap, D // 2), dtype=torch.uint8, device="cuda")
    ksc = torch.empty((B, Hkv, Tcap, D // 32), dtype=torch.float16, device="cuda")
    vc, vsc = torch.empty_like(kc), torch.empty_like(ksc)
    K.encode(plan, k16[:, :, :L], lam_k, kc, ksc, 0)
    K.encode(plan, v16[:, :, :L], lam_v, vc, vsc, 0)
    sm = 1 / math.sqrt(D)
    signs = O.plan_signs(D, ROTS[rot], plan.seed)
    ref = O.attention_int4(np16(q), kc.cpu().numpy(), ksc.cpu().numpy(), lam_k.cpu().numpy(),
                           vc.cpu().numpy(), vsc.cpu().numpy(), lam_v.cpu().numpy(), L, sm, ROTS[rot], signs)
    # the reference itself is dominated by the planted token
    for b, h, t in spots:
        vhat = O.decode(vc[b, h // rep, t].cpu().numpy(), vsc[b, h // rep, t].cpu().numpy(),
                        lam_v[h // rep].cpu().numpy(), ROTS[rot], signs)
        assert np.max(np.abs(ref[b, h] - vhat)) <= 1e-6 * np.max(np.abs(vhat)) + 1e-9
    for dt in (torch.float32, torch.float16):
        out = run_attn(plan, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm, dt)
        worst = P.compare_attention(np16(out), ref)
        say(f"   int4 {dt}: rel err {worst:.2e}")


def test_attention_decode_step_full_size():
    """The decode step at full size: batch 64, Hq 8 / Hkv 2, D=128, 32768
    cached tokens plus one appended with kvq_encode (T=1, t0=32768), then
    attention over 32769 tokens; 8 seeded (b, kv head) pairs checked against
    the oracle (all their query heads)."""
    cfg = W.CONFIGS["decode"]
    B, Hkv, Hq, D = cfg.B, cfg.H, 8, cfg.D
    T0 = cfg.T
    L = T0 + 1
    Tcap = T0 + 256
    plan = K.Plan(D, 32, "srft", cfg.sign_seed)
    say("[attn-full] building caches")
    k16, v16, lam_k, lam_v, q, kc, ksc, vc, vsc = build_cache(plan, B, Hkv, Hq, T0, Tcap, D, cfg.data_seed)
    # append one token per sequence
    K.encode(plan, k16[:, :, T0:T0 + 1], lam_k, kc, ksc, T0)
    K.encode(plan, v16[:, :, T0:T0 + 1], lam_v, vc, vsc, T0)
    sm = 1 / math.sqrt(D)
    say("[attn-full] int4 attention")
    out = run_attn(plan, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm, torch.float16)
    ws = torch.empty(K.attn_workspace_size(D, B, Hq, L), dtype=torch.uint8, device="cuda")
    out16 = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
    say("[attn-full] fp16 comparator")
    K.attn_decode_f16(q, k16, v16, L, sm, out16, ws)
    torch.cuda.synchronize()
    signs = O.plan_signs(D, O.SRFT, plan.seed)
    rng = np.random.default_rng(4)
    pairs = [(int(b), int(g)) for b, g in zip(rng.choice(B, 8, replace=False), rng.integers(0, Hkv, 8))]
    rep = Hq // Hkv
    for b, g in pairs:
        sl = slice(b, b + 1)
        kcs = kc[sl, g:g + 1, :L].cpu().numpy()
        kss = ksc[sl, g:g + 1, :L].cpu().numpy()
        vcs = vc[sl, g:g + 1, :L].cpu().numpy()
        vss = vsc[sl, g:g + 1, :L].cpu().numpy()
        qs = np16(q[sl, g * rep:(g + 1) * rep])
        ref = O.attention_int4(qs, kcs, kss, lam_k[g:g + 1].cpu().numpy(), vcs, vss,
                               lam_v[g:g + 1].cpu().numpy(), L, sm, O.SRFT, signs)
        w1 = P.compare_attention(np16(out[sl, g * rep:(g + 1) * rep]).astype(np.float64), ref)
        ref16 = O.attention_f16(qs, k16[sl, g:g + 1].cpu().numpy(), v16[sl, g:g + 1].cpu().numpy(), L, sm)
        w2 = P.compare_attention(np16(out16[sl, g * rep:(g + 1) * rep]).astype(np.float64), ref16)
        say(f"   (b={b}, g={g}): int4 rel {w1:.2e}, fp16 rel {w2:.2e}")


@pytest.mark.parametrize("Hq,Hkv,L", [(4, 1, 9000), (6, 1, 5000), (2, 2, 4500)])
def test_attention_many_splits(Hq, Hkv, L):
    """Batch 1 with one or two kv heads: few (batch, kv head, head chunk)
    units, so each is cut into more than 16 splits (the general merge path);
    Hq = 6 leaves a second chunk of two heads.  int4 (SRFT) and the fp16
    comparator against the oracle."""
    D, B = 128, 1
    Tcap = L + 3
    plan = K.Plan(D, 32, "srft", 71)
    say(f"[attn-splits] Hq={Hq} Hkv={Hkv} L={L}")
    k16, v16, lam_k, lam_v, q, kc, ksc, vc, vsc = build_cache(plan, B, Hkv, Hq, L, Tcap, D, 29)
    sm = 1 / math.sqrt(D)
    signs = O.plan_signs(D, O.SRFT, plan.seed)
    ref = O.attention_int4(np16(q), kc.cpu().numpy(), ksc.cpu().numpy(), lam_k.cpu().numpy(),
                           vc.cpu().numpy(), vsc.cpu().numpy(), lam_v.cpu().numpy(), L, sm, O.SRFT, signs)
    out = run_attn(plan, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm, torch.float32)
    say(f"   int4: rel err {P.compare_attention(np16(out), ref):.2e}")
    ws = torch.empty(K.attn_workspace_size(D, B, Hq, L), dtype=torch.uint8, device="cuda")
    out16 = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    K.attn_decode_f16(q, k16, v16, L, sm, out16, ws)
    torch.cuda.synchronize()
    ref16 = O.attention_f16(np16(q), k16.cpu().numpy(), v16.cpu().numpy(), L, sm)
    say(f"   fp16 comparator: rel err {P.compare_attention(np16(out16), ref16):.2e}")


def test_attention_workspace_reuse():
    """One workspace, sized for the largest call, serves a run of calls of
    different shapes, split counts and caches in stream order; repeating a
    call reproduces its output bit for bit (the merge takes the splits in a
    fixed order)."""
    D = 128
    plan = K.Plan(D, 32, "srft", 5)
    sm = 1 / math.sqrt(D)
    shapes = [(8, 8, 2, 3000), (1, 4, 1, 9000), (2, 2, 1, 40), (8, 8, 2, 3000)]
    ws = torch.empty(K.attn_workspace_size(D, 8, 8, 9000), dtype=torch.uint8, device="cuda")
    caches = {}
    first = {}
    for i, (B, Hq, Hkv, L) in enumerate(shapes):
        say(f"[attn-reuse] call {i}: B={B} Hq={Hq} Hkv={Hkv} L={L}")
        key = (B, Hq, Hkv, L)
        if key not in caches:
            caches[key] = build_cache(plan, B, Hkv, Hq, L, L + 1, D, 40 + i)
        k16, v16, lam_k, lam_v, q, kc, ksc, vc, vsc = caches[key]
        for rep in range(2):
            out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
            K.attn_decode(plan, q, kc, ksc, lam_k, vc, vsc, lam_v, L, sm, out, ws)
            out16 = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
            K.attn_decode_f16(q, k16, v16, L, sm, out16, ws)
            torch.cuda.synchronize()
            if key in first:
                assert torch.equal(out, first[key][0]) and torch.equal(out16, first[key][1])
            else:
                first[key] = (out, out16)
        if i == 1:
            signs = O.plan_signs(D, O.SRFT, plan.seed)
            ref = O.attention_int4(np16(q), kc.cpu().numpy(), ksc.cpu().numpy(), lam_k.cpu().numpy(),
                                   vc.cpu().numpy(), vsc.cpu().numpy(), lam_v.cpu().numpy(), L, sm, O.SRFT,
                                   signs)
            say(f"   int4: rel err {P.compare_attention(np16(first[key][0]), ref):.2e}")
