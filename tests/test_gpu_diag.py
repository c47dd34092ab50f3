"""The shader-clock probe the benchmark reads between its phases."""
import pytest
import torch

import kv_cache_int4_amd as K


@pytest.mark.gpu
def test_shader_clock_probe_reads_a_plausible_clock():
    out = torch.zeros(3, dtype=torch.int64, device="cuda:0")
    khz = K.diag_wall_clock_khz()
    assert khz > 0
    for iters in (2000, 20000):
        K.diag_shader_clock(out, iters)
        torch.cuda.synchronize()
        ticks, wall, _ = out.cpu().tolist()
        assert ticks > 0 and wall > 0
        ghz = ticks / wall * khz / 1e6
        print(f"iters {iters}: {ticks} shader ticks over {wall} wall ticks at {khz} kHz = {ghz:.3f} GHz")
        # MI355X: 2.4 GHz peak; the power manager may lower it under load
        assert 0.2 < ghz < 3.5
        # the chain of iters dependent FMAs takes at least iters cycles
        assert ticks >= iters
