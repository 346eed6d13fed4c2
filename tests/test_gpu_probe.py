"""The unit probes of ssm_probe.h on the GPU, at small iteration counts: every
wavefront's clock readings advance, the effective clock is plausible, and the
chains' outputs have the values their recurrences converge to."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,per_cu", [(0, 8), (1, 8), (2, 8), (3, 2)])
def test_probe_runs_and_reads_clocks(kind, per_cu):
    import torch

    import adjoint_gradients_amd as agm

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = cus * per_cu
    waves = wgs * agm.SSM_PROBE_WAVES_PER_WG
    iters = 4000
    print(f"case probe kind={kind} wgs={wgs} iters={iters}", flush=True)
    sink = torch.empty(wgs * 256, device="cuda:0", dtype=torch.float32)
    clk = torch.zeros(waves * 4, device="cuda:0", dtype=torch.int64)
    agm.ssm_probe_units(kind, wgs, iters, sink, clk)
    torch.cuda.synchronize()
    c = clk.view(waves, 4).cpu().numpy()
    assert (c[:, 1] > c[:, 0]).all() and (c[:, 3] > c[:, 2]).all()
    khz = agm.ssm_probe_wall_clock_khz()
    assert khz > 0
    ghz = np.median((c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / (khz * 1e3))) / 1e9
    assert 0.3 < ghz < 3.5, ghz
    s = sink.cpu().numpy()
    assert np.isfinite(s).all()
    if kind == 0:
        # x <- x a + b converges to b / (1 - a) = 1 (within 4000 steps of a = 1 - 2^-10: 2% left)
        assert np.allclose(s, 8.0, rtol=0.1)
    elif kind == 1:
        # x <- 2^-x converges to the fixed point of x = 2^-x
        xs = 0.641185744504986
        assert np.allclose(s, 8 * xs, rtol=1e-3)
    elif kind == 3:
        # each accumulator element gains 16 * 2^-6 * 2^-5 = 2^-7 a step: 64 elements of iters * 2^-7
        assert np.allclose(s, 64 * iters * 2.0 ** -7, rtol=1e-5)
    assert not math.isnan(float(s.sum()))
