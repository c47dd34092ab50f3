"""A decode step captured in a HIP graph: append K and V (kvq_encode, T=1)
then attention over the cache (kvq_attn_decode), all on the capturing
stream.  The library allocates, frees and synchronizes nothing inside these
calls and records no memset, so a serving loop can capture them.  The graph
is replayed several times, each with a new query and new appended token
written into its static inputs and with eager work and synchronizations in
between; every replay must equal the eager step on the same inputs bit for
bit (the kernels are deterministic), and the eager step matches the oracle.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import kv_cache_int4_amd as K
from kv_cache_int4_amd import workloads as W
from tests import parity as P
from tests.test_gpu_parity import np16, say

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.library()


def test_decode_step_graph_replays():
    D, B, Hkv, Hq, T0 = 128, 4, 2, 8, 3000
    Tcap = T0 + 8
    L = T0 + 1
    plan = K.Plan(D, 32, "srft", 2024)
    k16, v16, lam_k, lam_v, q = W.decode_inputs(B, Hkv, Hq, Tcap, D, 9, "cuda")
    kc = torch.empty((B, Hkv, Tcap, D // 2), dtype=torch.uint8, device="cuda")
    ks = torch.empty((B, Hkv, Tcap, D // 32), dtype=torch.float16, device="cuda")
    vc, vs = torch.empty_like(kc), torch.empty_like(ks)
    K.encode(plan, k16[:, :, :T0], lam_k, kc, ks, 0)
    K.encode(plan, v16[:, :, :T0], lam_v, vc, vs, 0)
    # static inputs and outputs of the captured step
    k_new = torch.empty((B, Hkv, 1, D), dtype=torch.float16, device="cuda")
    v_new = torch.empty_like(k_new)
    q_in = torch.empty_like(q)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(K.attn_workspace_size(D, B, Hq, L), dtype=torch.uint8, device="cuda")
    sm = 1 / math.sqrt(D)

    def step():
        K.encode(plan, k_new, lam_k, kc, ks, T0)
        K.encode(plan, v_new, lam_v, vc, vs, T0)
        K.attn_decode(plan, q_in, kc, ks, lam_k, vc, vs, lam_v, L, sm, out, ws)

    g = torch.Generator(device="cuda").manual_seed(31)

    def fresh_inputs():
        k_new.copy_(torch.randn(k_new.shape, generator=g, device="cuda").to(torch.float16))
        v_new.copy_(torch.randn(v_new.shape, generator=g, device="cuda").to(torch.float16))
        q_in.copy_(torch.randn(q.shape, generator=g, device="cuda").to(torch.float16))

    fresh_inputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    signs = O.plan_signs(D, O.SRFT, plan.seed)
    for r in range(4):
        say(f"[graph] replay {r}")
        fresh_inputs()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        kc_g, vc_g = kc[:, :, T0].clone(), vc[:, :, T0].clone()
        # eager work between replays, then the eager step on the same inputs
        out.zero_()
        kc[:, :, T0].zero_()
        vc[:, :, T0].zero_()
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        assert torch.equal(got, out), "replay differs from the eager step"
        assert torch.equal(kc_g, kc[:, :, T0]) and torch.equal(vc_g, vc[:, :, T0])
        if r == 0:
            ref = O.attention_int4(np16(q_in), kc.cpu().numpy(), ks.cpu().numpy(), lam_k.cpu().numpy(),
                                   vc.cpu().numpy(), vs.cpu().numpy(), lam_v.cpu().numpy(), L, sm, O.SRFT, signs)
            say(f"   eager step vs oracle: rel err {P.compare_attention(np16(out), ref):.2e}")


def test_stacked_kv_append_matches_two_calls():
    """K and V caches held as one [2B, Hkv, Tcap, ...] allocation (K rows
    first) take the new token's K and V in one kvq_encode call over 2B rows,
    with lambda_K / lambda_V given per row: the bytes written equal those of
    two separate calls."""
    D, B, Hkv, T0 = 128, 64, 2, 500
    Tcap = T0 + 4
    plan = K.Plan(D, 32, "srft", 11)
    k16, v16, lam_k, lam_v, _ = W.decode_inputs(B, Hkv, 8, Tcap, D, 3, "cuda")
    kvc = torch.full((2 * B, Hkv, Tcap, D // 2), 0x5A, dtype=torch.uint8, device="cuda")
    kvs = torch.full((2 * B, Hkv, Tcap, D // 32), 7.0, dtype=torch.float16, device="cuda")
    kc, ks = kvc[:B].clone(), kvs[:B].clone()
    vc, vs = kvc[B:].clone(), kvs[B:].clone()
    kv_new = torch.cat([k16[:, :, T0:T0 + 1], v16[:, :, T0:T0 + 1]]).contiguous()
    lam_kv = torch.cat([lam_k.expand(B, Hkv, D), lam_v.expand(B, Hkv, D)]).contiguous()
    K.encode(plan, kv_new, lam_kv, kvc, kvs, T0)
    K.encode(plan, k16[:, :, T0:T0 + 1], lam_k, kc, ks, T0)
    K.encode(plan, v16[:, :, T0:T0 + 1], lam_v, vc, vs, T0)
    torch.cuda.synchronize()
    assert torch.equal(kvc[:B], kc) and torch.equal(kvs[:B], ks)
    assert torch.equal(kvc[B:], vc) and torch.equal(kvs[B:], vs)
