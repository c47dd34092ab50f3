"""GPU parity at sizes whose byte offsets pass 2^31 (and, for the codec
input, 2^32): the codec on one head of 33.6M D=128 vectors (8.6 GB of fp16
rows, 2.1 GB of codes), of 16.8M D=256 vectors and of 33.6M D=96 vectors,
and the decode-step attention over a 33.6M-token int4 cache.  Every address
past the 32-bit range is exercised.

The codec is checked on sampled vectors on both sides of those offsets and
at the end, against the oracle (codes, scales and the fp16 decode).  The
attention over a cache that size is beyond the oracle, so four tokens are
planted, one per query head, on both sides of the 2^31-byte code offset, at
the start and in the final partial block: the query heads have disjoint
channel supports (orthogonal, in the rotated basis too), and each planted
key is a large multiple of its head's query, so its score leads every other
by about 100 (natural log units) for that head alone.  Each head's output is
then its planted token's value row, decoded by the oracle from the GPU's
codes, to far below the 2e-3 bar.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import kv_cache_int4_amd as K
from tests import parity as P
from tests.test_gpu_parity import np16, say

pytestmark = pytest.mark.gpu

D = 128
T_BIG = (1 << 25) + 100          # 33,554,532 vectors / tokens: codes pass 2^31 bytes


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.library()


def fill_normal(t, std, seed):
    """t[..., D] = N(0, 1) * std, generated in chunks of 2^20 rows."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    flat = t.view(-1, t.shape[-1])
    n, step = flat.shape[0], 1 << 20
    for i in range(0, n, step):
        j = min(n, i + step)
        flat[i:j] = (torch.randn((j - i, t.shape[-1]), generator=g, device="cuda") * std).to(t.dtype)


@pytest.mark.parametrize("Dc,G,T", [(128, 32, T_BIG), (256, 32, (1 << 24) + 100), (96, 16, T_BIG)])
def test_codec_past_32bit_offsets_sampled(Dc, G, T):
    """SRFT encode and fp16 decode of one head of T vectors of size Dc: the
    input passes 2^32 bytes, the codes 2^31 (D=128, 256) or 2^30 (D=96)."""
    say(f"[large] codec: 1 x 1 x {T} x {Dc}, G={G}")
    g = torch.Generator(device="cuda").manual_seed(3)
    std = torch.exp(0.5 * torch.randn(Dc, generator=g, device="cuda"))
    lam = torch.exp(0.3 * torch.randn((1, Dc), generator=g, device="cuda"))
    x = torch.empty((1, 1, T, Dc), dtype=torch.float16, device="cuda")
    fill_normal(x, std, 11)
    plan = K.Plan(Dc, G, "srft", 99)
    codes = torch.empty((1, 1, T, Dc // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((1, 1, T, Dc // G), dtype=torch.float16, device="cuda")
    K.encode(plan, x, lam, codes, scales)
    y = torch.empty_like(x)
    K.decode(plan, codes, scales, lam, y)
    torch.cuda.synchronize()
    say("[large] codec: encoded and decoded; sampling")
    rng = np.random.default_rng(17)
    # vectors where the input passes 2^31 and 2^32 bytes and the codes 2^30
    # and 2^31 bytes
    marks = [c for c in ((1 << 31) // (2 * Dc), (1 << 32) // (2 * Dc), (1 << 30) // (Dc // 2),
                         (1 << 31) // (Dc // 2)) if c + 64 <= T]
    near = [np.arange(c - 64, c + 64) for c in marks]
    idx = np.unique(np.concatenate(near + [np.arange(T - 256, T), rng.choice(T, 4096, replace=False)]))
    it = torch.from_numpy(idx).cuda()
    xs = np16(x.view(-1, Dc)[it])
    cs = np16(codes.view(-1, Dc // 2)[it])
    ss = np16(scales.view(-1, Dc // G)[it])
    ys = np16(y.view(-1, Dc)[it])
    lv = np.broadcast_to(np16(lam).astype(np.float32), (len(idx), Dc))
    signs = O.plan_signs(Dc, O.SRFT, plan.seed)
    rep = P.compare_codes(cs, ss, xs, lv, O.SRFT, signs, G)
    say(f"   {len(idx)} sampled vectors ({len(marks)} offset marks): {rep['code_mismatch']} code / "
        f"{rep['scale_mismatch']} scale mismatches")
    r = P.compare_decode(ys, cs, ss, lv, O.SRFT, signs, G)
    say(f"   fp16 decode: {r}")


def test_attention_past_32bit_offsets_planted():
    L = T_BIG
    Tcap = L + 28
    B, Hkv, Hq = 1, 1, 4
    say(f"[large] attention: B={B} Hkv={Hkv} Hq={Hq} L={L}")
    g = torch.Generator(device="cuda").manual_seed(5)
    std = torch.exp(0.5 * torch.randn(D, generator=g, device="cuda"))
    lam_k = torch.exp(0.3 * torch.randn((Hkv, D), generator=g, device="cuda"))
    lam_v = torch.exp(0.3 * torch.randn((Hkv, D), generator=g, device="cuda"))
    # query heads on disjoint 32-channel supports
    q = torch.zeros((B, Hq, D), dtype=torch.float16, device="cuda")
    for h in range(Hq):
        q[0, h, 32 * h:32 * h + 32] = torch.randn(32, generator=g, device="cuda").to(torch.float16)
    k16 = torch.empty((B, Hkv, Tcap, D), dtype=torch.float16, device="cuda")
    v16 = torch.empty_like(k16)
    fill_normal(k16, std, 21)
    fill_normal(v16, std, 22)
    # planted tokens: both sides of 2^25 tokens (2^31 bytes of codes), the
    # start, and the last token (in the partial final block)
    spots = [(0, (1 << 25) - 1), (1, (1 << 25) + 3), (2, 5), (3, L - 1)]
    for h, t in spots:
        qv = q[0, h].float()
        c = 1200.0 / float((qv * qv).sum())
        k16[0, 0, t] = (c * qv).to(torch.float16)
    plan = K.Plan(D, 32, "srft", 77)
    kc = torch.empty((B, Hkv, Tcap, D // 2), dtype=torch.uint8, device="cuda")
    ks = torch.empty((B, Hkv, Tcap, D // 32), dtype=torch.float16, device="cuda")
    vc, vs = torch.empty_like(kc), torch.empty_like(ks)
    K.encode(plan, k16[:, :, :L], lam_k, kc, ks, 0)
    K.encode(plan, v16[:, :, :L], lam_v, vc, vs, 0)
    del k16, v16
    ws = torch.empty(K.attn_workspace_size(D, B, Hq, L), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    sm = 1 / math.sqrt(D)
    K.attn_decode(plan, q, kc, ks, lam_k, vc, vs, lam_v, L, sm, out, ws)
    torch.cuda.synchronize()
    say("[large] attention: done; checking planted tokens")
    signs = O.plan_signs(D, O.SRFT, plan.seed)
    lv = np16(lam_v).astype(np.float32)[0]
    ref = np.zeros((B, Hq, D))
    for h, t in spots:
        ref[0, h] = O.decode(np16(vc[0, 0, t]), np16(vs[0, 0, t]), lv, O.SRFT, signs)
        # the planted key still leads its head by far after quantization
        khat = O.decode(np16(kc[0, 0, t]), np16(ks[0, 0, t]), np16(lam_k).astype(np.float32)[0], O.SRFT, signs)
        assert sm * float(np.dot(np16(q[0, h]).astype(np.float64), khat)) > 90.0
    worst = P.compare_attention(np16(out), ref)
    say(f"   planted-token heads: rel err {worst:.2e}")
