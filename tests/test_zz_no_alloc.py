"""kvq_attn_decode_noalloc through the C ABI: the same results as
kvq_attn_decode with a caller-owned workspace, bit for bit, on two calls in a
row (the second smaller, so the per-GPU buffer holds the first call's
partials when it starts), and within the attention bar of the oracle.

Named to be collected last: it must pass alone in a fresh process and after
every other GPU test."""

import ctypes
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


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.library()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _cache(plan, B, Hkv, Hq, L, seed):
    D = plan.D
    k16, v16, lam_k, lam_v, q = W.decode_inputs(B, Hkv, Hq, L + 7, D, seed, "cuda")
    cb, ng = plan.code_bytes, D // plan.G
    kc = torch.empty((B, Hkv, L + 7, cb), dtype=torch.uint8, device="cuda")
    ks = torch.empty((B, Hkv, L + 7, ng), dtype=torch.float16, device="cuda")
    vc, vs = torch.empty_like(kc), torch.empty_like(ks)
    K.encode(plan, k16[:, :, :L], lam_k, kc, ks, 0)
    K.encode(plan, v16[:, :, :L], lam_v, vc, vs, 0)
    return q, kc, ks, lam_k, vc, vs, lam_v


def _call_noalloc(plan, q, kc, ks, lk, vc, vs, lv, L, sm, out):
    L_ = K.library()
    B, Hq, _ = q.shape
    Hkv, Tcap = kc.shape[1], kc.shape[2]
    dt = 1 if out.dtype == torch.float32 else 0
    st = L_.kvq_attn_decode_noalloc(plan.handle, q.data_ptr(), kc.data_ptr(), ks.data_ptr(), lk.data_ptr(),
                                    vc.data_ptr(), vs.data_ptr(), lv.data_ptr(), B, Hq, Hkv, Tcap, L,
                                    ctypes.c_float(sm), out.data_ptr(), dt,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == 0, L_.kvq_last_error()


def _call_ws(plan, q, kc, ks, lk, vc, vs, lv, L, sm, out):
    L_ = K.library()
    B, Hq, D = q.shape
    Hkv, Tcap = kc.shape[1], kc.shape[2]
    n = K.attn_workspace_size(D, B, Hq, L)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    dt = 1 if out.dtype == torch.float32 else 0
    st = L_.kvq_attn_decode(plan.handle, q.data_ptr(), kc.data_ptr(), ks.data_ptr(), lk.data_ptr(),
                            vc.data_ptr(), vs.data_ptr(), lv.data_ptr(), B, Hq, Hkv, Tcap, L,
                            ctypes.c_float(sm), out.data_ptr(), dt, ws.data_ptr(), n,
                            torch.cuda.current_stream().cuda_stream)
    assert st == 0, L_.kvq_last_error()


@pytest.mark.parametrize("rot,bits,G", [("srft", 4, 32), ("srht", 8, 16)])
def test_noalloc_matches_workspace_call(rot, bits, G):
    D = 128
    plan = K.Plan(D, G, rot, 71, bits=bits)
    sm = 1 / math.sqrt(D)
    shapes = [(16, 2, 8, 20000, 5), (2, 1, 4, 257, 6)]      # B, Hkv, Hq, L, seed: the second smaller
    for B, Hkv, Hq, L, seed in shapes:
        say(f"[noalloc] rot={rot} bits={bits} G={G} B={B} Hkv={Hkv} Hq={Hq} L={L}")
        q, kc, ks, lk, vc, vs, lv = _cache(plan, B, Hkv, Hq, L, seed)
        for dtype in (torch.float32, torch.float16):
            o_ws = torch.full((B, Hq, D), 7.0, dtype=dtype, device="cuda")
            o_na = torch.full((B, Hq, D), -7.0, dtype=dtype, device="cuda")
            _call_ws(plan, q, kc, ks, lk, vc, vs, lv, L, sm, o_ws)
            _call_noalloc(plan, q, kc, ks, lk, vc, vs, lv, L, sm, o_na)
            torch.cuda.synchronize()
            assert torch.equal(o_ws, o_na), f"noalloc differs from the workspace call ({dtype})"
        if L < 1000:
            signs = O.plan_signs(D, {"srft": O.SRFT, "srht": O.SRHT}[rot], plan.seed)
            ref = O.attention_int4(q.cpu().numpy(), kc.cpu().numpy(), ks.cpu().numpy(), lk.cpu().numpy(),
                                   vc.cpu().numpy(), vs.cpu().numpy(), lv.cpu().numpy(), L, sm,
                                   {"srft": O.SRFT, "srht": O.SRHT}[rot], signs, G, bits)
            worst = P.compare_attention(o_ws.float().cpu().numpy(), ref)
            say(f"   oracle rel err {worst:.2e}")


def test_noalloc_refuses_oversized_call():
    """A call whose partials exceed the per-GPU buffer is refused on the host
    (fake, never dereferenced pointers: nothing is launched)."""
    L_ = K.library()
    plan = K.Plan(128, 32, "srft", 1)
    A = 0x10000
    st = L_.kvq_attn_decode_noalloc(plan.handle, A, A, A, A, A, A, A, 4096, 32, 8, 300, 256,
                                    ctypes.c_float(0.1), A, 0, None)
    assert st == 4 and b"per-GPU buffer" in L_.kvq_last_error()
