"""Seeded synthetic inputs shaped like the paper's KV-cache workloads.

This module only draws random numbers: it holds none of the quantizer's
arithmetic, and both the GPU path and the CPU oracle are fed from it.  The
paper measures on real models (Qwen2.5-1.5B, Gemma-3 1B, Mistral-7B) and
evaluation text that are not available here; these generators stand in for
them with each model's KV shape and a value law that has the properties the
paper's scaling argument is about (per-channel spread and outlier channels;
explainer, "Methodik" item 3, per-channel plus per-group scaling).

Laws (all values rounded to fp16 round-to-nearest-even):
  * ``gaussian_outliers``: N(0, 1) with ``n_out`` outlier channels per head
    multiplied by ``out_mult`` (the small round-trip case).
  * ``channel_spread``: z * std_j with std_j = exp(N(0, 0.5^2)) per
    (layer, kv, head, channel) and round(0.01 D) (at least 1) outlier
    channels per head multiplied by 30 (the prefix-encode cases).
  * ``student_t3``: Student-t with 3 degrees of freedom,
    z0 / sqrt((z1^2 + z2^2 + z3^2) / 3) (the bulk-encode case).
  * lambda ~ lognormal(0, 0.3) per channel; queries ~ N(0, 1).

Every draw comes from a ``torch.Generator`` on the requested device, seeded
from (seed, layer, kv), so a tensor is reproducible on the device it was made
on; tests hand the oracle the generated values themselves.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch

__all__ = [
    "Config", "CONFIGS", "gen", "gaussian_outliers", "channel_spread",
    "student_t3", "lognormal_lambda", "queries", "prefix_inputs", "decode_inputs",
]


def gen(device, *key: int) -> torch.Generator:
    """A generator on ``device`` seeded from an integer key tuple."""
    s = 0x243F6A8885A308D3
    for k in key:
        s = (s * 1000003 + int(k) + 1) % (1 << 62)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _normal(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _outlier_mask(H, D, n_out, g, device):
    """[H, D] float mask, 1 except ``n_out`` channels per head chosen without
    replacement."""
    m = torch.ones(H, D, device=device)
    for h in range(H):
        idx = torch.randperm(D, generator=g, device=device)[:n_out]
        m[h, idx] = 0.0
    return m


def gaussian_outliers(H, T, D, n_out, out_mult, seed, device="cpu", layer=0, kv=0):
    """x [H, T, D] fp16: N(0,1) with n_out outlier channels per head x out_mult."""
    g = gen(device, seed, layer, kv)
    z = _normal((H, T, D), g, device)
    keep = _outlier_mask(H, D, n_out, g, device)
    mult = keep + (1.0 - keep) * out_mult
    return (z * mult[:, None, :]).to(torch.float16)


def n_outliers(D: int) -> int:
    """1% of the channels, at least one."""
    return max(1, int(round(0.01 * D)))


def channel_spread(H, T, D, seed, device="cpu", layer=0, kv=0, out_mult=30.0):
    """x [H, T, D] fp16 with per-channel std exp(N(0, 0.5^2)) and 1% outlier
    channels x out_mult (per head)."""
    g = gen(device, seed, layer, kv)
    std = torch.exp(0.5 * _normal((H, D), g, device))
    keep = _outlier_mask(H, D, n_outliers(D), g, device)
    std = std * (keep + (1.0 - keep) * out_mult)
    z = _normal((H, T, D), g, device)
    return (z * std[:, None, :]).to(torch.float16)


def student_t3(H, T, D, seed, device="cpu", layer=0, kv=0):
    """x [H, T, D] fp16, i.i.d. Student-t(3) = z0 / sqrt((z1^2+z2^2+z3^2)/3)."""
    g = gen(device, seed, layer, kv)
    out = torch.empty((H, T, D), device=device, dtype=torch.float16)
    # draw per head to bound the float32 temporaries
    for h in range(H):
        z = _normal((4, T, D), g, device)
        chi = (z[1] * z[1] + z[2] * z[2] + z[3] * z[3]) / 3.0
        out[h] = (z[0] / torch.sqrt(chi)).to(torch.float16)
    return out


def lognormal_lambda(shape, seed, device="cpu", sigma=0.3, *key):
    """Per-channel lambda ~ lognormal(0, sigma), float32."""
    g = gen(device, seed, *key)
    return torch.exp(sigma * _normal(shape, g, device))


def queries(B, Hq, D, seed, device="cpu"):
    """Decode-step queries q [B, Hq, D] ~ N(0, 1), fp16."""
    g = gen(device, seed, 7)
    return _normal((B, Hq, D), g, device).to(torch.float16)


@dataclass(frozen=True)
class Config:
    """One workload: the call shape and the value law."""
    name: str
    D: int
    B: int          # calls are batched over B (layers x {K, V} for prefixes)
    H: int
    T: int
    law: str
    index: int      # seeds: data = index, lambda = 100 + index, signs = 1000 + index
    Hq: int = 0     # decode steps: query heads (H is then the KV head count)

    @property
    def vectors(self) -> int:
        return self.B * self.H * self.T

    @property
    def data_seed(self) -> int:
        return self.index

    @property
    def lambda_seed(self) -> int:
        return 100 + self.index

    @property
    def sign_seed(self) -> int:
        return 1000 + self.index


CONFIGS = {
    # single K tensor, 2 KV heads x 256 tokens, D=128: round trip
    "small": Config("small-roundtrip-H2-T256-D128", 128, 1, 2, 256, "gaussian20", 1),
    # Qwen2.5-1.5B prefix: 28 layers x {K,V} x 2 KV heads x 4096 tokens, D=128
    "qwen": Config("qwen2.5-1.5b-prefix-28Lx2x2Hx4096-D128", 128, 56, 2, 4096, "spread", 2),
    # Gemma-3-1B prefix: 26 layers x {K,V} x 1 KV head x 4096 tokens, D=256
    "gemma": Config("gemma-3-1b-prefix-26Lx2x1Hx4096-D256", 256, 52, 1, 4096, "spread", 3),
    # decode step: batch 64, Hq 8 / Hkv 2, 32768 cached tokens, D=128
    "decode": Config("gqa-decode-B64-Hq8-Hkv2-L32769-D128", 128, 64, 2, 32768, "spread", 4, 8),
    # the same decode step at Gemma-3 1B's head shape: batch 64, Hq 4 / Hkv 1,
    # 32768 cached tokens, D=256 (the same cache bytes per step as "decode")
    "decode256": Config("gqa-decode-B64-Hq4-Hkv1-L32769-D256", 256, 64, 1, 32768, "spread", 8, 4),
    # Mistral-7B bulk: 32 layers x {K,V}, batch 16 x 8 heads x 8192 tokens, D=128
    "mistral": Config("mistral-7b-bulk-32Lx2-B16-H8-T8192-D128", 128, 16, 8, 8192, "t3", 5),
    # head sizes that are not powers of two (mixed-radix SRFT): the prefix
    # shape of "qwen" (28 layers x {K,V} x 2 KV heads x 4096 tokens) at D=96
    # and D=80
    "d96": Config("prefix-28Lx2x2Hx4096-D96", 96, 56, 2, 4096, "spread", 6),
    "d80": Config("prefix-28Lx2x2Hx4096-D80", 80, 56, 2, 4096, "spread", 7),
}


def prefix_inputs(cfg: Config, device="cpu", T: int | None = None):
    """(x [B, H, T, D] fp16, lambda [B, H, D] fp32) for the prefix configs,
    batch index b = 2 * layer + kv.  ``T`` may shrink the token count (the
    law per (layer, kv, head, channel) is unchanged, only fewer tokens are
    drawn)."""
    T = cfg.T if T is None else T
    xs, lams = [], []
    for b in range(cfg.B):
        layer, kv = divmod(b, 2)
        if cfg.law == "gaussian20":
            x = gaussian_outliers(cfg.H, T, cfg.D, 4, 20.0, cfg.data_seed, device, layer, kv)
        elif cfg.law == "spread":
            x = channel_spread(cfg.H, T, cfg.D, cfg.data_seed, device, layer, kv)
        else:
            x = student_t3(cfg.H, T, cfg.D, cfg.data_seed, device, layer, kv)
        xs.append(x)
        lams.append(lognormal_lambda((cfg.H, cfg.D), cfg.lambda_seed, device, 0.3, layer, kv))
    return torch.stack(xs), torch.stack(lams)


def decode_inputs(B: int, Hkv: int, Hq: int, Tcap: int, D: int, seed: int, device="cpu"):
    """Inputs of a decode step: fp16 K and V [B, Hkv, Tcap, D] with the
    channel-spread law of one layer (per-head channel statistics and outlier
    channels shared across the batch, independent values per sequence),
    lambda_K and lambda_V [Hkv, D], and queries q [B, Hq, D]."""
    out = []
    for kv in (0, 1):
        g = gen(device, seed, 0, kv)
        std = torch.exp(0.5 * _normal((Hkv, D), g, device))
        keep = _outlier_mask(Hkv, D, n_outliers(D), g, device)
        std = std * (keep + (1.0 - keep) * 30.0)
        x = torch.empty((B, Hkv, Tcap, D), device=device, dtype=torch.float16)
        for b in range(B):          # per sequence, to bound the fp32 temporaries
            x[b] = (_normal((Hkv, Tcap, D), g, device) * std[:, None, :]).to(torch.float16)
        out.append(x)
    lam_k = lognormal_lambda((Hkv, D), seed + 100, device, 0.3, 0, 0)
    lam_v = lognormal_lambda((Hkv, D), seed + 100, device, 0.3, 0, 1)
    q = queries(B, Hq, D, seed, device)
    return out[0], out[1], lam_k, lam_v, q
