"""The benchmark's floor probes (libmxfp4_probes.so) run and give sane
figures: an empty launch costs something, streaming a buffer is not faster
than HBM's peak allows, the matrix-instruction probe does not exceed the FP4
peak and reports a shader clock in the plausible range."""
import pytest

import bench
from tests.gpu_util import torch_cuda

pytestmark = pytest.mark.gpu


def test_floor_probes_run_and_are_plausible():
    torch = torch_cuda()
    out = bench.floors(torch, steps=4, samples=3, names=["c2"])
    assert 0.5 < out["empty_kernel_us"]["median"] < 50
    s = out["stream_b_us"]["M32_N4096_K512"]
    assert s["bytes"] == 4096 * 512 // 2 + 4096 * 16  # codes + scales (4096 rows x 16 groups, no padding needed)
    assert s["gbs"] < bench.HBM_PEAK_GBS * 1.05
    for m in out["mfma"]:
        assert 0 < m["tflops"] <= bench.FP4_PEAK_TFLOPS * 1.05
        assert 1000 < m["shader_mhz"] < 3000
        assert m["cycles_per_instruction_per_wave"] >= 15.5
