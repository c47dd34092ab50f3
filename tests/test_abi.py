"""Host-side checks of the C ABI (no GPU needed).

The library is loaded on the CPU: every symbol the header declares must be
exported, plans must reproduce the oracle's sign vectors, and every argument
check must fail on the host, with its documented status and no GPU call
(nothing here ever reaches a kernel launch).
"""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle as O
import kv_cache_int4_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, HIP = range(6)
A = 0x10000        # a 16-byte aligned fake device address (never dereferenced)


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    L = K.library()
    syms = declared_symbols()
    assert len(syms) >= 13
    for s in syms:
        assert hasattr(L, s), f"{s} declared in kvq.h but not exported"


def test_library_is_built_for_gfx950():
    with open(K.library_path(), "rb") as f:
        blob = f.read()
    assert b"gfx950" in blob


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("rot", [O.SRFT, O.SRHT, O.IDENTITY])
@pytest.mark.parametrize("seed", [0, 1, 1004, 2**63 + 12345])
def test_plan_signs_match_oracle(D, rot, seed):
    p = K.Plan(D, 32, rot, seed)
    assert np.array_equal(p.signs(), O.plan_signs(D, rot, seed))
    assert p.info() == (D, 32, rot)


def test_plan_create_rejects():
    L = K.library()
    h = ctypes.c_void_p()
    assert L.kvq_plan_create(100, 32, 0, 0, ctypes.byref(h)) == UNSUPPORTED
    assert b"D=100" in L.kvq_last_error()
    assert L.kvq_plan_create(128, 8, 0, 0, ctypes.byref(h)) == UNSUPPORTED
    assert L.kvq_plan_create_ex(128, 32, 6, 0, 0, ctypes.byref(h)) == UNSUPPORTED
    assert b"bits=6" in L.kvq_last_error()
    assert L.kvq_plan_create_ex(128, 64, 8, 0, 0, ctypes.byref(h)) == UNSUPPORTED
    assert L.kvq_plan_create(128, 32, 7, 0, ctypes.byref(h)) == INVALID
    assert L.kvq_plan_create(128, 32, 0, 0, None) == INVALID
    assert L.kvq_plan_signs(None, None, 0) == INVALID
    assert L.kvq_strerror(WORKSPACE) == b"workspace missing or too small"
    L.kvq_plan_destroy(None)


@pytest.mark.parametrize("bits,G", [(4, 32), (4, 16), (8, 32), (8, 16)])
@pytest.mark.parametrize("D", [128, 256])
def test_plan_formats(bits, G, D):
    """Plans of every code width and group size: info reports them, signs are
    the oracle's, and kvq_plan_create is the 4-bit case."""
    p = K.Plan(D, G, "srht", 77, bits=bits)
    assert p.info_ex() == (D, G, bits, O.SRHT)
    assert p.info() == (D, G, O.SRHT)
    assert p.code_bytes == D * bits // 8
    assert np.array_equal(p.signs(), O.plan_signs(D, O.SRHT, 77))
    assert K.cache_shapes(2, 3, 5, D, G, bits) == ((2, 3, 5, D * bits // 8), (2, 3, 5, D // G))
    L = K.library()
    h = ctypes.c_void_p()
    assert L.kvq_plan_create(D, G, 0, 1, ctypes.byref(h)) == OK
    b = ctypes.c_int32()
    assert L.kvq_plan_info_ex(h, None, None, ctypes.byref(b), None) == OK and b.value == 4
    L.kvq_plan_destroy(h)


def test_plan_options():
    """KVQ_OPT_MFMA_ROTATION is accepted for D=128 SRFT plans of every format
    and refused elsewhere; unknown option bits are invalid."""
    L = K.library()
    h = ctypes.c_void_p()
    for bits, G in ((4, 32), (4, 16), (8, 32), (8, 16)):
        assert L.kvq_plan_create_opt(128, G, bits, O.SRFT, 7, 1, ctypes.byref(h)) == OK
        o = ctypes.c_uint32()
        assert L.kvq_plan_options(h, ctypes.byref(o)) == OK and o.value == 1
        L.kvq_plan_destroy(h)
    assert L.kvq_plan_create_opt(256, 32, 4, O.SRFT, 7, 1, ctypes.byref(h)) == UNSUPPORTED
    assert L.kvq_plan_create_opt(128, 32, 4, O.SRHT, 7, 1, ctypes.byref(h)) == UNSUPPORTED
    assert L.kvq_plan_create_opt(96, 32, 4, O.SRFT, 7, 1, ctypes.byref(h)) == UNSUPPORTED
    assert L.kvq_plan_create_opt(128, 32, 4, O.SRFT, 7, 2, ctypes.byref(h)) == INVALID
    assert L.kvq_plan_create_opt(128, 32, 4, O.SRFT, 7, 0, None) == INVALID
    p = K.Plan(128, 32, "srft", 7, mfma=True)
    assert np.array_equal(p.signs(), O.plan_signs(128, O.SRFT, 7))
    o = ctypes.c_uint32()
    assert L.kvq_plan_options(K.Plan(128, 32, "srft", 7).handle, ctypes.byref(o)) == OK and o.value == 0


@pytest.mark.parametrize("D,G", [(96, 32), (96, 16), (80, 16)])
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("rot", [O.SRFT, O.IDENTITY])
def test_plan_mixed_radix_sizes(D, G, bits, rot):
    """D = 96 and 80 take the SRFT (D/2 pair signs, the oracle's) and the
    identity, with groups that divide D."""
    p = K.Plan(D, G, rot, 91, bits=bits)
    assert p.info_ex() == (D, G, bits, rot)
    assert p.code_bytes == D * bits // 8
    assert np.array_equal(p.signs(), O.plan_signs(D, rot, 91))


def test_plan_mixed_radix_rejects():
    """SRHT needs a power-of-two D; G must divide D; attention is built for D = 128 and 256 only."""
    L = K.library()
    h = ctypes.c_void_p()
    assert L.kvq_plan_create(96, 32, O.SRHT, 0, ctypes.byref(h)) == UNSUPPORTED
    assert b"SRHT" in L.kvq_last_error()
    assert L.kvq_plan_create(80, 32, O.SRFT, 0, ctypes.byref(h)) == UNSUPPORTED
    assert b"does not divide" in L.kvq_last_error()
    assert L.kvq_plan_create(112, 16, O.SRFT, 0, ctypes.byref(h)) == UNSUPPORTED
    n = ctypes.c_size_t()
    assert L.kvq_attn_workspace_size(96, 1, 8, 100, ctypes.byref(n)) == UNSUPPORTED


def _encode(plan, x=A, B=1, H=2, T=4, sb=1024, sh=512, st=128, lam=A, lsb=0, codes=A, scales=A,
            Tcap=8, t0=0):
    return K.library().kvq_encode(plan.handle if plan else None, x, B, H, T, sb, sh, st, lam, lsb,
                                  codes, scales, Tcap, t0, None)


def test_encode_validation():
    p = K.Plan(128, 32, "srft", 1)
    assert _encode(None) == INVALID
    assert _encode(p, Tcap=3) == INVALID                 # t0 + T > Tcap
    assert _encode(p, t0=5) == INVALID
    assert _encode(p, B=-1) == INVALID
    assert _encode(p, x=None) == INVALID
    assert _encode(p, lam=None) == INVALID
    assert _encode(p, codes=None) == INVALID
    assert _encode(p, x=A + 2) == ALIGN
    assert _encode(p, st=130) == ALIGN                   # rows not 16-byte aligned
    assert _encode(p, st=-128) == INVALID
    assert _encode(p, codes=A + 8) == ALIGN
    assert _encode(p, scales=A + 2) == ALIGN
    assert _encode(p, lam=A + 1) == ALIGN
    assert _encode(p, lsb=-1) == INVALID
    assert _encode(p, B=1 << 40, H=1 << 20) == INVALID  # overflowing shape
    assert _encode(p, B=2, sb=1 << 62) == INVALID        # strides reaching past 2^62 elements
    assert b"reach" in K.library().kvq_last_error()
    assert _encode(p, st=1 << 28) == INVALID              # lane offsets are 32-bit
    assert b"2^28" in K.library().kvq_last_error()
    assert _encode(p, st=(1 << 28) - 8, codes=A + 8) == ALIGN   # below the limit: the next check decides
    # zero work is a no-op that touches nothing (NULL pointers allowed)
    assert _encode(p, T=0, x=None, lam=None, codes=None, scales=None) == OK
    assert K.library().kvq_last_error() == b""


def test_decode_and_rotate_validation():
    L = K.library()
    p = K.Plan(256, 32, "srht", 2)
    h = p.handle
    # codes, scales, B, H, Tcap, t0, T, lam, lsb, y, dtype, y strides
    assert L.kvq_decode(h, A, A, 1, 1, 8, 6, 4, A, 0, A, 0, 2048, 2048, 256, None) == INVALID
    assert L.kvq_decode(h, A, A, 1, 1, 8, 0, 4, A, 0, A, 2, 2048, 2048, 256, None) == INVALID
    assert L.kvq_decode(h, A, A, 1, 1, 8, 0, 4, A, 0, A + 8, 0, 2048, 2048, 256, None) == ALIGN
    assert L.kvq_decode(h, A, A, 1, 1, 8, 0, 4, A, 0, A, 0, 2048, 2048, 260, None) == ALIGN
    assert L.kvq_decode(h, A, A, 1, 1, 8, 0, 4, A, 0, A, 1, 2048, 2048, 257, None) == ALIGN
    assert L.kvq_decode(h, None, A, 1, 1, 8, 0, 4, A, 0, A, 0, 2048, 2048, 256, None) == INVALID
    assert L.kvq_decode(h, A, A, 1, 1, 8, 0, 0, A, 0, A, 0, 2048, 2048, 256, None) == OK
    assert L.kvq_decode(h, A, A, 2, 1, 8, 0, 4, A, 0, A, 0, 1 << 62, 2048, 256, None) == INVALID
    assert L.kvq_decode(h, A, A, 1, 1, 8, 0, 4, A, 0, A, 0, 2048, 2048, 1 << 28, None) == INVALID
    assert b"2^28" in L.kvq_last_error()
    assert L.kvq_rotate(h, A, 1, 1, 4, 1024, 1024, 256, A, 0, None, None) == INVALID
    assert L.kvq_rotate(h, A, 1, 1, 4, 1024, 1024, 256, A, 0, A + 4, None) == ALIGN
    assert L.kvq_rotate(None, A, 1, 1, 4, 1024, 1024, 256, A, 0, A, None) == INVALID


def test_decode_alignment_of_direct_loaded_rows():
    """The D=128/256 decoders move lambda rows (and scale rows of 16 bytes
    or more) with 16-byte direct loads: misaligned ones are refused on the
    host, before anything is enqueued.  (No call here passes every check:
    none reaches a launch.)"""
    L = K.library()

    def dec(plan, scales=A, lam=A, lsb=0):
        # codes, scales, B, H, Tcap, t0, T, lam, lsb, y, dtype, y strides
        return L.kvq_decode(plan.handle, A, scales, 2, 1, 8, 0, 4, lam, lsb, A, 0, 8 * plan.D, 8 * plan.D,
                            plan.D, None)

    for D, G in ((128, 32), (128, 16), (256, 32), (256, 16)):
        p = K.Plan(D, G, "srft", 5)
        assert dec(p, lam=A + 4) == ALIGN
        assert b"lambda" in L.kvq_last_error()
        assert dec(p, lsb=130) == ALIGN
        assert b"lambda_sb" in L.kvq_last_error()
        assert dec(p, scales=A + 2) == ALIGN
    # 16-byte scale rows: an 8-byte offset is refused for decode and encode
    for D, G in ((128, 16), (256, 32), (256, 16)):
        p = K.Plan(D, G, "srft", 5)
        assert dec(p, scales=A + 8) == ALIGN
        assert b"scales" in L.kvq_last_error()
        assert _encode(p, sb=4 * D, sh=2 * D, st=D, scales=A + 8) == ALIGN
        assert b"scales" in K.library().kvq_last_error()


def test_attention_validation():
    L = K.library()
    p = K.Plan(128, 32, "srft", 3)
    h = p.handle
    need = K.attn_workspace_size(128, 64, 8, 32769)
    assert need > 64 * 8 * 128 * 4
    args = dict(q=A, kc=A, ks=A, lk=A, vc=A, vs=A, lv=A, B=64, Hq=8, Hkv=2, Tcap=33024, L=32769,
                sm=0.088, out=A, dt=0, ws=A, wsb=need)

    def call(**kw):
        a = dict(args, **kw)
        return L.kvq_attn_decode(h, a["q"], a["kc"], a["ks"], a["lk"], a["vc"], a["vs"], a["lv"], a["B"],
                                 a["Hq"], a["Hkv"], a["Tcap"], a["L"], a["sm"], a["out"], a["dt"], a["ws"],
                                 a["wsb"], None)

    assert call(Hq=6, Hkv=4) == INVALID               # Hq % Hkv
    assert call(L=0) == INVALID
    assert call(L=40000) == INVALID                   # seq_len > Tcap
    assert call(wsb=need - 1) == WORKSPACE
    assert call(ws=None) == WORKSPACE
    assert call(kc=A + 4) == ALIGN
    assert call(ks=A + 2) == ALIGN
    assert call(q=None) == INVALID
    assert call(vc=None) == INVALID
    assert call(dt=5) == INVALID
    assert call(B=0) == OK                            # nothing to do
    assert call(Tcap=1 << 31) == INVALID              # tokens are counted in 32 bits
    assert b"2^31" in L.kvq_last_error()
    # head sizes with attention kernels: 128 and 256 (the mixed-radix sizes have none)
    p256 = K.Plan(256, 32, "srft", 3)
    assert L.kvq_attn_decode(p256.handle, A, A, A, A, A, A, A, 1, 2, 1, 8, 4, 0.1, A, 0, A, 0,
                             None) == WORKSPACE
    p96 = K.Plan(96, 32, "srft", 3)
    assert L.kvq_attn_decode(p96.handle, A, A, A, A, A, A, A, 1, 2, 1, 8, 4, 0.1, A, 0, A, need,
                             None) == UNSUPPORTED
    assert L.kvq_attn_decode_f16(96, A, A, A, 1, 2, 1, 8, 4, 0.1, A, 0, A, need, None) == UNSUPPORTED
    assert L.kvq_attn_decode_f16(256, A, A, A, 1, 2, 1, 8, 4, 0.1, A, 0, A, 0, None) == WORKSPACE
    assert L.kvq_attn_decode_f16(128, A, A, A, 1, 3, 2, 8, 4, 0.1, A, 0, A, need, None) == INVALID
    assert L.kvq_attn_decode_f16(128, A, None, A, 1, 2, 1, 8, 4, 0.1, A, 0, A, need, None) == INVALID
    # fp16 rows are addressed with 32-bit byte offsets: Tcap * 2D up to 4 GiB
    big = K.attn_workspace_size(256, 1, 2, 4)
    assert L.kvq_attn_decode_f16(256, A, A, A, 1, 2, 1, (1 << 23) + 1, 4, 0.1, A, 0, A, big, None) == INVALID
    assert b"4 GiB" in L.kvq_last_error()


def test_noalloc_attention_validation():
    """kvq_attn_decode_noalloc runs the checks of kvq_attn_decode, and refuses
    a call whose partials exceed its per-GPU buffer, on the host (fake
    pointers: nothing here reaches a launch)."""
    L = K.library()
    p = K.Plan(128, 32, "srft", 3)

    def call(B=64, Hq=8, Hkv=2, Tcap=33024, L_=32769, kc=A, q=A):
        return L.kvq_attn_decode_noalloc(p.handle, q, kc, A, A, A, A, A, B, Hq, Hkv, Tcap, L_, 0.088, A, 0, None)

    assert call(Hq=6, Hkv=4) == INVALID
    assert call(L_=0) == INVALID
    assert call(kc=A + 4) == ALIGN
    assert call(q=None) == INVALID
    assert call(B=0) == OK
    assert L.kvq_attn_decode_noalloc(None, A, A, A, A, A, A, A, 1, 1, 1, 8, 4, 0.1, A, 0, None) == INVALID
    assert call(B=4096, Hq=32, Hkv=8, Tcap=300, L_=256) == WORKSPACE
    assert b"per-GPU buffer" in L.kvq_last_error()


def test_diag_shader_clock_validation():
    """The clock probe's argument checks run on the host (fake pointers:
    nothing here reaches a launch)."""
    L = K.library()
    assert L.kvq_diag_shader_clock(None, 2000, None) == INVALID
    assert L.kvq_diag_shader_clock(A + 4, 2000, None) == ALIGN
    assert L.kvq_diag_shader_clock(A, 0, None) == INVALID
    assert L.kvq_diag_shader_clock(A, (1 << 24) + 1, None) == INVALID
    assert b"iters" in L.kvq_last_error()
    assert L.kvq_diag_wall_clock_khz(None) == INVALID
    with pytest.raises(ValueError):
        K.diag_shader_clock(torch.zeros(2, dtype=torch.int64))


def test_workspace_size_monotone():
    a = K.attn_workspace_size(128, 2, 8, 100)
    b = K.attn_workspace_size(128, 2, 8, 100000)
    assert 0 < a < b
    # D=256 partials are twice as wide
    assert K.attn_workspace_size(256, 2, 8, 100000) > b
    with pytest.raises(K.KvqError):
        K.attn_workspace_size(64, 2, 8, 100)
    with pytest.raises(K.KvqError):
        K.attn_workspace_size(96, 2, 8, 100)


def test_binding_refuses_host_tensors():
    """The Python binding hands raw pointers to the GPU: host tensors are
    refused before any library call (checked here on the CPU)."""
    p = K.Plan(128, 32, "srft", 1)
    x = torch.zeros((1, 2, 4, 128), dtype=torch.float16)
    lam = torch.ones((2, 128), dtype=torch.float32)
    codes = torch.zeros((1, 2, 8, 64), dtype=torch.uint8)
    scales = torch.zeros((1, 2, 8, 4), dtype=torch.float16)
    with pytest.raises(ValueError, match="host tensor"):
        K.encode(p, x, lam, codes, scales)
    with pytest.raises(ValueError, match="host tensor"):
        K.decode(p, codes, scales, lam, torch.zeros((1, 2, 8, 128), dtype=torch.float16))
    with pytest.raises(ValueError, match="host tensor"):
        K.rotate(p, x, lam, torch.zeros((1, 2, 4, 128), dtype=torch.float32))
    q = torch.zeros((1, 4, 128), dtype=torch.float16)
    out = torch.zeros((1, 4, 128), dtype=torch.float32)
    ws = torch.zeros(K.attn_workspace_size(128, 1, 4, 8), dtype=torch.uint8)
    with pytest.raises(ValueError, match="host tensor"):
        K.attn_decode(p, q, codes, scales, lam, codes, scales, lam, 8, 0.1, out, ws)
    kv = torch.zeros((1, 2, 8, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="host tensor"):
        K.attn_decode_f16(q, kv, kv, 8, 0.1, out, ws)
    # a batched lambda must have 1 or B rows (others would be read past its end)
    x3 = torch.zeros((3, 2, 4, 128), dtype=torch.float16)
    c3 = torch.zeros((3, 2, 8, 64), dtype=torch.uint8)
    s3 = torch.zeros((3, 2, 8, 4), dtype=torch.float16)
    lam2 = torch.ones((2, 2, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="lambda must be"):
        K.encode(p, x3, lam2, c3, s3)
    with pytest.raises(ValueError, match="lambda must be"):
        K.decode(p, c3, s3, lam2, torch.zeros((3, 2, 8, 128), dtype=torch.float16))
    with pytest.raises(ValueError, match="lambda must be"):
        K.rotate(p, x3, lam2, torch.zeros((3, 2, 4, 128), dtype=torch.float32))
    # shapes that do not match the plan are refused first
    with pytest.raises(ValueError, match="codes must be"):
        K.attn_decode(p, q, codes[..., :32], scales, lam, codes, scales, lam, 8, 0.1, out, ws)


def test_binding_shape_checks_are_not_asserts():
    """The binding's shape and dtype checks raise ValueError (they stay in
    force under python -O, where asserts vanish): a codes or output tensor
    too small for the call is refused before its pointer reaches a kernel."""
    p = K.Plan(128, 32, "srft", 1)
    x = torch.zeros((1, 2, 4, 128), dtype=torch.float16)
    lam = torch.ones((2, 128), dtype=torch.float32)
    codes = torch.zeros((1, 2, 8, 64), dtype=torch.uint8)
    scales = torch.zeros((1, 2, 8, 4), dtype=torch.float16)
    with pytest.raises(ValueError, match="codes must be"):
        K.encode(p, x, lam, codes[:, :1], scales)
    with pytest.raises(ValueError, match="scales must be"):
        K.encode(p, x, lam, codes, scales[..., :2])
    with pytest.raises(ValueError, match="x must be fp16"):
        K.encode(p, x.float(), lam, codes, scales)
    with pytest.raises(ValueError, match="y must be"):
        K.decode(p, codes, scales, lam, torch.zeros((1, 1, 8, 128), dtype=torch.float16))
    with pytest.raises(ValueError, match="y must be fp16 or fp32"):
        K.decode(p, codes, scales, lam, torch.zeros((1, 2, 8, 128), dtype=torch.float64))
    with pytest.raises(ValueError, match="w must be"):
        K.rotate(p, x, lam, torch.zeros((1, 2, 3, 128), dtype=torch.float32))
    q = torch.zeros((1, 4, 128), dtype=torch.float16)
    ws = torch.zeros(K.attn_workspace_size(128, 1, 4, 8), dtype=torch.uint8)
    with pytest.raises(ValueError, match="out must be fp16 or fp32"):
        K.attn_decode(p, q, codes, scales, lam, codes, scales, lam, 8, 0.1,
                      torch.zeros((1, 4, 128), dtype=torch.float64), ws)
    src = open(K.__file__).read()
    assert "\n    assert " not in src and "\n        assert " not in src
