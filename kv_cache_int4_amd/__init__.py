"""Python binding of libkvq, the MI355X int4 KV-cache quantizer.

Argument marshalling only: every step of encode, decode and attention runs in
the HIP kernels of ``libkvq.so`` (built in-tree by ``kv_cache_int4_amd.build``).
PyTorch supplies device memory and the current stream.  If the library is
missing the import of the entry points raises; there is no fallback.

Method: "When Quantization Is Free: An int4 KV Cache That Outruns fp16 on
Apple Silicon" (arXiv 2605.05699) -- sign-randomized FFT (or Walsh-Hadamard)
rotation, per-channel lambda, group-32 abs-max fp16 scale, int4 nibbles; int8
codes and groups of 16 as plan variants.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "KvqError", "Plan", "OPT_MFMA_ROTATION", "SRFT", "SRHT", "IDENTITY", "GROUP",
    "library", "library_path", "encode", "decode", "rotate",
    "attn_workspace_size", "attn_decode", "attn_decode_noalloc", "attn_decode_f16",
    "cache_shapes", "diag_shader_clock", "diag_wall_clock_khz",
]

SRFT, SRHT, IDENTITY = 0, 1, 2
GROUP = 32
_ROT_NAMES = {"srft": SRFT, "srht": SRHT, "identity": IDENTITY}
_F16, _F32 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libkvq.so")


class KvqError(RuntimeError):
    """A libkvq call returned an error status."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"kvq status {status}: {detail}")


_lib = None

_i32, _i64, _u64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
_vp, _sz = ctypes.c_void_p, ctypes.c_size_t


def library() -> ctypes.CDLL:
    """Load libkvq.so (once); raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m kv_cache_int4_amd.build`")
    L = ctypes.CDLL(path)
    sig = {
        "kvq_version": (ctypes.c_char_p, []),
        "kvq_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "kvq_last_error": (ctypes.c_char_p, []),
        "kvq_plan_create": (ctypes.c_int, [_i32, _i32, ctypes.c_int, _u64, ctypes.POINTER(_vp)]),
        "kvq_plan_create_ex": (ctypes.c_int, [_i32, _i32, _i32, ctypes.c_int, _u64, ctypes.POINTER(_vp)]),
        "kvq_plan_create_opt": (ctypes.c_int, [_i32, _i32, _i32, ctypes.c_int, _u64, ctypes.c_uint32,
                                               ctypes.POINTER(_vp)]),
        "kvq_plan_options": (ctypes.c_int, [_vp, ctypes.POINTER(ctypes.c_uint32)]),
        "kvq_plan_destroy": (None, [_vp]),
        "kvq_plan_signs": (ctypes.c_int, [_vp, _vp, _i64]),
        "kvq_plan_info": (ctypes.c_int, [_vp, ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
        "kvq_plan_info_ex": (ctypes.c_int, [_vp, ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                                            ctypes.POINTER(_i32)]),
        "kvq_encode": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _i64,
                                      _vp, _vp, _i64, _i64, _vp]),
        "kvq_decode": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _i64,
                                      _vp, ctypes.c_int, _i64, _i64, _i64, _vp]),
        "kvq_rotate": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _vp]),
        "kvq_attn_workspace_size": (ctypes.c_int, [_i32, _i64, _i64, _i64, ctypes.POINTER(_sz)]),
        "kvq_attn_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                           _i64, _i64, _i64, _i64, _i64, _f32, _vp, ctypes.c_int,
                                           _vp, _sz, _vp]),
        "kvq_attn_decode_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                   _i64, _i64, _i64, _i64, _i64, _f32, _vp, ctypes.c_int, _vp]),
        "kvq_attn_decode_f16": (ctypes.c_int, [_i32, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32,
                                               _vp, ctypes.c_int, _vp, _sz, _vp]),
        "kvq_diag_shader_clock": (ctypes.c_int, [_vp, _i32, _vp]),
        "kvq_diag_wall_clock_khz": (ctypes.c_int, [ctypes.POINTER(_i32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise KvqError(status, library().kvq_last_error().decode())


def _stream(idx: int) -> int:
    """The current HIP stream of device idx (torch's raw-handle getter where
    it has one: a call costs a fraction of building a Stream object, which
    matters for calls of a few microseconds)."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(idx)
    return torch.cuda.current_stream(idx).cuda_stream


def _on(idx: int, fn, *args):
    """fn(*args) with device idx current: the library launches on the
    current device."""
    import torch
    if idx == torch.cuda.current_device():
        return fn(*args)
    with torch.cuda.device(idx):
        return fn(*args)


def _ptr(t) -> int:
    return t.data_ptr() if t is not None else 0


def _req(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _device(*ts) -> int:
    """The one CUDA device every tensor lives on: the kernels take raw device
    pointers, so a host tensor or a tensor on another GPU is refused here
    rather than handed to the GPU."""
    idx = ts[0].get_device()
    for t in ts:
        d = t.get_device()
        _req(d >= 0, "every tensor must be on a GPU (got a host tensor)")
        _req(d == idx, f"tensors on different devices: cuda:{idx} and cuda:{d}")
    return idx


OPT_MFMA_ROTATION = 1


class Plan:
    """Head dimension D, group G, rotation ("srft" | "srht" | "identity"),
    the seed of the sign vector, the code width (4: int4 nibbles, 8: int8
    bytes) and, for D=128 SRFT plans, mfma=True to run the encoder's DFT on
    the matrix cores."""

    def __init__(self, D: int = 128, G: int = GROUP, rotation="srft", seed: int = 0, bits: int = 4,
                 mfma: bool = False):
        L = library()
        rot = _ROT_NAMES[rotation] if isinstance(rotation, str) else int(rotation)
        h = _vp()
        opts = OPT_MFMA_ROTATION if mfma else 0
        _check(L.kvq_plan_create_opt(D, G, bits, rot, seed & ((1 << 64) - 1), opts, ctypes.byref(h)))
        self._h = h
        self.D, self.G, self.rotation, self.seed, self.bits, self.mfma = D, G, rot, seed, bits, mfma

    @property
    def code_bytes(self) -> int:
        """Code bytes per token."""
        return self.D * self.bits // 8

    @property
    def handle(self):
        return self._h

    def signs(self):
        import numpy as np
        n = {SRFT: self.D // 2, SRHT: self.D, IDENTITY: 0}[self.rotation]
        out = np.zeros(n, dtype=np.int8)
        _check(library().kvq_plan_signs(self._h, out.ctypes.data if n else None, n))
        return out

    def info(self):
        D, G, R = _i32(), _i32(), _i32()
        _check(library().kvq_plan_info(self._h, ctypes.byref(D), ctypes.byref(G), ctypes.byref(R)))
        return D.value, G.value, R.value

    def info_ex(self):
        D, G, b, R = _i32(), _i32(), _i32(), _i32()
        _check(library().kvq_plan_info_ex(self._h, ctypes.byref(D), ctypes.byref(G), ctypes.byref(b),
                                          ctypes.byref(R)))
        return D.value, G.value, b.value, R.value

    def close(self):
        if getattr(self, "_h", None):
            library().kvq_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 -- interpreter shutdown
            pass


def cache_shapes(B: int, H: int, Tcap: int, D: int, G: int = GROUP, bits: int = 4):
    """(codes shape, scales shape) of a dense cache."""
    return (B, H, Tcap, D * bits // 8), (B, H, Tcap, D // G)


def _lam_args(lam, B, H, D):
    """lambda_sb of a [H, D] table (shared across the batch) or a [1 or B,
    H, D] one; any other leading size would make the kernels read rows past
    the tensor, so it is refused here."""
    if lam.dim() == 2:
        _req(tuple(lam.shape) == (H, D), f"lambda must be [{H}, {D}] or [1 or {B}, {H}, {D}]")
        return 0
    _req(lam.dim() == 3 and tuple(lam.shape[1:]) == (H, D) and lam.shape[0] in (1, B),
         f"lambda must be [{H}, {D}] or [1 or {B}, {H}, {D}] (got {tuple(lam.shape)})")
    _req(lam.stride(2) == 1 and lam.stride(1) == D, "lambda must be dense in (H, D)")
    return 0 if lam.shape[0] == 1 else lam.stride(0)


def _x_args(x, D):
    _req(x.dim() == 4 and x.shape[3] == D and x.stride(3) == 1, f"x must be [B, H, T, {D}] with unit D stride")
    return x.shape[0], x.shape[1], x.shape[2], x.stride(0), x.stride(1), x.stride(2)


def encode(plan: Plan, x, lam, codes, scales, t0: int = 0):
    """Quantize x [B, H, T, D] (fp16) into tokens t0..t0+T-1 of codes
    [B, H, Tcap, D*bits/8] (uint8) and scales [B, H, Tcap, D/G] (fp16)."""
    import torch
    _req(x.dtype == torch.float16 and codes.dtype == torch.uint8 and scales.dtype == torch.float16,
         "x must be fp16, codes uint8, scales fp16")
    _req(lam.dtype == torch.float32 and lam.is_contiguous(), "lambda must be contiguous fp32")
    _req(codes.is_contiguous() and scales.is_contiguous(), "codes and scales must be contiguous")
    B, H, T, sb, sh, st = _x_args(x, plan.D)
    _req(codes.dim() == 4, "codes must be [B, H, Tcap, D*bits/8]")
    Tcap = codes.shape[2]
    _req(tuple(codes.shape) == (B, H, Tcap, plan.code_bytes), f"codes must be {(B, H, Tcap, plan.code_bytes)}")
    _req(tuple(scales.shape) == (B, H, Tcap, plan.D // plan.G), f"scales must be {(B, H, Tcap, plan.D // plan.G)}")
    lsb = _lam_args(lam, B, H, plan.D)
    idx = _device(x, lam, codes, scales)
    _check(_on(idx, library().kvq_encode, plan.handle, _ptr(x), B, H, T, sb, sh, st, _ptr(lam),
               lsb, _ptr(codes), _ptr(scales), Tcap, t0, _stream(idx)))


def decode(plan: Plan, codes, scales, lam, y, t0: int = 0):
    """Dequantize tokens t0..t0+T-1 into y [B, H, T, D] (fp16 or fp32)."""
    import torch
    _req(codes.is_contiguous() and scales.is_contiguous() and lam.is_contiguous(),
         "codes, scales and lambda must be contiguous")
    _req(codes.dtype == torch.uint8 and scales.dtype == torch.float16 and lam.dtype == torch.float32,
         "codes must be uint8, scales fp16, lambda fp32")
    _req(codes.dim() == 4 and codes.shape[3] == plan.code_bytes, "codes must be [B, H, Tcap, D*bits/8]")
    B, H, Tcap = codes.shape[0], codes.shape[1], codes.shape[2]
    _req(tuple(scales.shape) == (B, H, Tcap, plan.D // plan.G), f"scales must be {(B, H, Tcap, plan.D // plan.G)}")
    _req(y.dim() == 4 and tuple(y.shape[:2]) == (B, H) and y.shape[3] == plan.D and y.stride(3) == 1,
         f"y must be [{B}, {H}, T, {plan.D}] with unit D stride")
    _req(y.dtype in (torch.float16, torch.float32), "y must be fp16 or fp32")
    dt = {torch.float16: _F16, torch.float32: _F32}[y.dtype]
    lsb = _lam_args(lam, B, H, plan.D)
    idx = _device(codes, scales, lam, y)
    _check(_on(idx, library().kvq_decode, plan.handle, _ptr(codes), _ptr(scales), B, H, Tcap, t0, y.shape[2],
               _ptr(lam), lsb, _ptr(y), dt,
               y.stride(0), y.stride(1), y.stride(2), _stream(idx)))


def rotate(plan: Plan, x, lam, w):
    """w [B, H, T, D] fp32 = lambda * (R x) (the encoder's transform alone)."""
    import torch
    _req(x.dtype == torch.float16 and lam.dtype == torch.float32 and w.dtype == torch.float32,
         "x must be fp16, lambda and w fp32")
    _req(lam.is_contiguous(), "lambda must be contiguous")
    B, H, T, sb, sh, st = _x_args(x, plan.D)
    _req(w.is_contiguous() and tuple(w.shape) == (B, H, T, plan.D), f"w must be contiguous {(B, H, T, plan.D)}")
    lsb = _lam_args(lam, B, H, plan.D)
    idx = _device(x, lam, w)
    _check(_on(idx, library().kvq_rotate, plan.handle, _ptr(x), B, H, T, sb, sh, st, _ptr(lam),
               lsb, _ptr(w), _stream(idx)))


def attn_workspace_size(D: int, B: int, Hq: int, seq_len: int) -> int:
    n = _sz()
    _check(library().kvq_attn_workspace_size(D, B, Hq, seq_len, ctypes.byref(n)))
    return n.value


def _attn_checks(plan, q, k_codes, k_scales, lam_k, v_codes, v_scales, lam_v, out):
    """Shapes, dtypes and layouts of a decode-step attention call."""
    import torch
    _req(q.dim() == 3 and q.dtype == torch.float16 and q.shape[2] == plan.D, "q must be fp16 [B, Hq, D]")
    B, Hq, D = q.shape
    _req(k_codes.dim() == 4, "codes must be [B, Hkv, Tcap, D*bits/8]")
    Hkv, Tcap = k_codes.shape[1], k_codes.shape[2]
    cshape, sshape = (B, Hkv, Tcap, plan.code_bytes), (B, Hkv, Tcap, D // plan.G)
    for c, sc in ((k_codes, k_scales), (v_codes, v_scales)):
        _req(c.dtype == torch.uint8 and tuple(c.shape) == cshape, f"codes must be uint8 {cshape}")
        _req(sc.dtype == torch.float16 and tuple(sc.shape) == sshape, f"scales must be fp16 {sshape}")
    for lam in (lam_k, lam_v):
        _req(lam.dtype == torch.float32 and tuple(lam.shape) == (Hkv, D), f"lambda must be fp32 [{Hkv}, {D}]")
    _req(tuple(out.shape) == (B, Hq, D), f"out must be [{B}, {Hq}, {D}]")
    _req(out.dtype in (torch.float16, torch.float32), "out must be fp16 or fp32")
    for t in (q, k_codes, k_scales, lam_k, v_codes, v_scales, lam_v, out):
        _req(t.is_contiguous(), "attention tensors must be contiguous")


def attn_decode(plan: Plan, q, k_codes, k_scales, lam_k, v_codes, v_scales, lam_v, seq_len: int,
                sm_scale: float, out, workspace):
    """Decode-step attention over the int4 cache: out [B, Hq, D]."""
    import torch
    _attn_checks(plan, q, k_codes, k_scales, lam_k, v_codes, v_scales, lam_v, out)
    _req(workspace.is_contiguous(), "workspace must be contiguous")
    B, Hq, D = q.shape
    Hkv, Tcap = k_codes.shape[1], k_codes.shape[2]
    dt = {torch.float16: _F16, torch.float32: _F32}[out.dtype]
    idx = _device(q, k_codes, k_scales, lam_k, v_codes, v_scales, lam_v, out, workspace)
    _check(_on(idx, library().kvq_attn_decode, plan.handle, _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(lam_k),
               _ptr(v_codes), _ptr(v_scales), _ptr(lam_v), B, Hq, Hkv, Tcap, seq_len,
               float(sm_scale), _ptr(out), dt, _ptr(workspace),
               workspace.numel() * workspace.element_size(), _stream(idx)))


def attn_decode_noalloc(plan: Plan, q, k_codes, k_scales, lam_k, v_codes, v_scales, lam_v, seq_len: int,
                        sm_scale: float, out):
    """attn_decode with no workspace: the partials go to the library's
    per-GPU buffer (calls that overlap on one GPU race)."""
    import torch
    _attn_checks(plan, q, k_codes, k_scales, lam_k, v_codes, v_scales, lam_v, out)
    B, Hq, D = q.shape
    Hkv, Tcap = k_codes.shape[1], k_codes.shape[2]
    dt = {torch.float16: _F16, torch.float32: _F32}[out.dtype]
    idx = _device(q, k_codes, k_scales, lam_k, v_codes, v_scales, lam_v, out)
    _check(_on(idx, library().kvq_attn_decode_noalloc, plan.handle, _ptr(q), _ptr(k_codes), _ptr(k_scales),
               _ptr(lam_k), _ptr(v_codes), _ptr(v_scales), _ptr(lam_v), B, Hq, Hkv, Tcap, seq_len,
               float(sm_scale), _ptr(out), dt, _stream(idx)))


def attn_decode_f16(q, k, v, seq_len: int, sm_scale: float, out, workspace):
    """The same attention over an fp16 cache k, v [B, Hkv, Tcap, D]."""
    import torch
    _req(q.dim() == 3 and q.dtype == torch.float16, "q must be fp16 [B, Hq, D]")
    B, Hq, D = q.shape
    _req(k.dim() == 4 and k.dtype == torch.float16 and k.shape[0] == B and k.shape[3] == D,
         "k must be fp16 [B, Hkv, Tcap, D]")
    _req(v.dtype == torch.float16 and v.shape == k.shape, "v must match k")
    Hkv, Tcap = k.shape[1], k.shape[2]
    _req(tuple(out.shape) == (B, Hq, D), f"out must be [{B}, {Hq}, {D}]")
    _req(out.dtype in (torch.float16, torch.float32), "out must be fp16 or fp32")
    for t in (q, k, v, out, workspace):
        _req(t.is_contiguous(), "attention tensors must be contiguous")
    dt = {torch.float16: _F16, torch.float32: _F32}[out.dtype]
    idx = _device(q, k, v, out, workspace)
    _check(_on(idx, library().kvq_attn_decode_f16, D, _ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Tcap, seq_len,
               float(sm_scale), _ptr(out), dt, _ptr(workspace),
               workspace.numel() * workspace.element_size(), _stream(idx)))


def diag_shader_clock(out, iters: int = 200):
    """Measurement aid: enqueue the shader-clock probe on the current stream
    of out's device; out is a device int64 tensor of at least 3 elements and
    receives (shader-clock ticks, wall-clock ticks, scratch); 200 iterations
    take about 4 us at 2.4 GHz (one loop step is about 44 cycles).  The clock in
    GHz is out[0] / out[1] * diag_wall_clock_khz() / 1e6, once the stream
    has reached the probe."""
    import torch
    _req(out.dtype == torch.int64 and out.numel() >= 3 and out.is_contiguous(),
         "out must be a contiguous int64 tensor of at least 3 elements")
    idx = _device(out)
    _check(_on(idx, library().kvq_diag_shader_clock, _ptr(out), int(iters), _stream(idx)))


def diag_wall_clock_khz(device: int | None = None) -> int:
    """Rate of the probe's wall clock on a device (the current one by default)."""
    import torch
    idx = torch.cuda.current_device() if device is None else int(device)
    khz = ctypes.c_int32(0)
    _check(_on(idx, library().kvq_diag_wall_clock_khz, ctypes.byref(khz)))
    return int(khz.value)
