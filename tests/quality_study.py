"""Synthetic quality study: reconstruction error of the quantized cache for
the rotations and scaling schemes the pages compare.

The abstract reports no measurable difference in KV quality between the
SRFT and the SRHT; the pages also report that per-token 4-bit scaling fails
on models with outlier coordinates while per-channel plus per-group scaling
recovers (explainer, "Methodik" 3), and describe the real-input DFT with its
Hermitian half spectrum unpacked to reals (explainer, "Methodik" 2).  Without
models or evaluation text, this study measures what those choices do to the
relative reconstruction error

    rel_mse = sum ||x - decode(encode(x))||^2 / sum ||x||^2

on seeded synthetic data with the configs' value laws: the channel-spread
law (per-channel std exp(N(0, 0.5^2)), 1% outlier channels x30) at D=128 and
D=256, and i.i.d. Student-t(3) at D=128.  lambda = 1 throughout (the pages'
lambda is learned or calibrated for model quality, which needs data this
study does not have).

Test infrastructure: everything here runs on the CPU oracle.  Run as
``python -m tests.quality_study`` to print the table.
"""

from __future__ import annotations

import numpy as np

import oracle as O
from kv_cache_int4_amd import workloads as W

LAWS = (("spread", 128), ("spread", 256), ("t3", 128))

# (name, rotation, group size (0 = one scale per vector), code bits)
VARIANTS = (
    ("per-token int4 (no rotation)", O.IDENTITY, 0, 4),
    ("per-group G32 int4 (no rotation)", O.IDENTITY, 32, 4),
    ("SRFT G32 int4", O.SRFT, 32, 4),
    ("SRHT G32 int4", O.SRHT, 32, 4),
    ("real-DFT (Hermitian unpack) G32 int4", O.HERMITIAN, 32, 4),
    ("SRFT G16 int4", O.SRFT, 16, 4),
    ("SRHT G16 int4", O.SRHT, 16, 4),
    ("SRFT G32 int8", O.SRFT, 32, 8),
    ("SRHT G32 int8", O.SRHT, 32, 8),
)

SIGN_SEED = 7


def inputs(law: str, D: int, n: int, seed: int = 3) -> np.ndarray:
    """n fp16 vectors of the law (one head, one layer), as numpy [n, D]."""
    if law == "spread":
        x = W.channel_spread(1, n, D, seed)
    elif law == "t3":
        x = W.student_t3(1, n, D, seed)
    else:
        raise ValueError(law)
    return x.reshape(-1, D).numpy()


def rel_mse(x16: np.ndarray, xh: np.ndarray) -> float:
    x = np.asarray(x16, dtype=np.float64)
    return float(((x - np.asarray(xh, dtype=np.float64)) ** 2).sum() / (x ** 2).sum())


def oracle_rel_mse(x16: np.ndarray, rotation: int, G: int, bits: int) -> float:
    D = x16.shape[-1]
    G = G or D
    s = O.plan_signs(D, rotation, SIGN_SEED)
    lam = np.ones(D, dtype=np.float32)
    codes, scales, _ = O.encode(x16, lam, rotation, s, G, bits)
    return rel_mse(x16, O.decode(codes, scales, lam, rotation, s, G, bits))


def table(n: int = 8192):
    """{(law, D): {variant name: rel_mse}}"""
    out = {}
    for law, D in LAWS:
        x = inputs(law, D, n)
        out[(law, D)] = {name: oracle_rel_mse(x, rot, G, bits) for name, rot, G, bits in VARIANTS}
    return out


def markdown(res) -> str:
    cols = [f"{law} D={D}" for law, D in res]
    lines = ["| variant | " + " | ".join(cols) + " |", "|---|" + "---|" * len(cols)]
    for name, *_ in VARIANTS:
        lines.append(f"| {name} | " + " | ".join(f"{res[k][name]:.3e}" for k in res) + " |")
    return "\n".join(lines)


if __name__ == "__main__":
    import sys
    n = int(sys.argv[1]) if len(sys.argv) > 1 else 32768
    print(markdown(table(n)))
