"""The quality study's numbers through the HIP path: relative reconstruction
error of encode + decode (fp32 output) on the GPU, for every variant the
kernels build, against the oracle's on the same inputs."""

import numpy as np
import pytest
import torch

import oracle as O
import kv_cache_int4_amd as K
from tests import quality_study as Q
from tests.test_gpu_parity import say

pytestmark = pytest.mark.gpu

ROT_NAMES = {O.SRFT: "srft", O.SRHT: "srht", O.IDENTITY: "identity"}


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K.library()


def gpu_rel_mse(x16: np.ndarray, rotation: int, G: int, bits: int) -> float:
    N, D = x16.shape
    plan = K.Plan(D, G, ROT_NAMES[rotation], Q.SIGN_SEED, bits=bits)
    x = torch.from_numpy(x16).reshape(1, 1, N, D).cuda()
    lam = torch.ones((1, D), dtype=torch.float32, device="cuda")
    codes = torch.empty((1, 1, N, plan.code_bytes), dtype=torch.uint8, device="cuda")
    scales = torch.empty((1, 1, N, D // G), dtype=torch.float16, device="cuda")
    K.encode(plan, x, lam, codes, scales)
    y = torch.empty((1, 1, N, D), dtype=torch.float32, device="cuda")
    K.decode(plan, codes, scales, lam, y)
    torch.cuda.synchronize()
    return Q.rel_mse(x16, y.cpu().numpy().reshape(N, D))


@pytest.mark.parametrize("law,D", list(Q.LAWS))
def test_gpu_study_matches_oracle(law, D):
    x = Q.inputs(law, D, 65536)
    rows = []
    for name, rot, G, bits in Q.VARIANTS:
        if rot not in ROT_NAMES or G == 0:
            continue
        g = gpu_rel_mse(x, rot, G, bits)
        o = Q.oracle_rel_mse(x, rot, G, bits)
        rows.append((name, g, o))
        assert abs(g / o - 1) < 1e-3, (name, g, o)
    for name, g, o in rows:
        say(f"   {law} D={D} {name}: gpu {g:.4e} oracle {o:.4e}")
