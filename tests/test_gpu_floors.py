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


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_phase_probe_matches_library_and_stamps_are_ordered(name):
    """The stamped copy of the fused kernel writes the library's C bit for
    bit, and every wave's stamps come in phase order."""
    torch = torch_cuda()
    import block_scaled_mxfp4_bf16_amd as mx
    out = bench.phases(torch, mx, steps=2, names=[name])[name]
    assert "skipped" not in out, out
    assert out["c_matches_library"]
    for ph in bench.PHASE_NAMES:
        assert out["wave_phase_us"][ph]["min"] >= 0.0
    assert 0.0 < out["first_entry_to_last_completion_us"]["median"] < 1000.0
    assert out["entry_spread_us"]["median"] <= out["first_entry_to_last_completion_us"]["median"]


def test_wide_phase_probe_matches_library_and_stamps_are_ordered():
    """The stamped copy of the large-M K loop writes the library's C bit for
    bit (at 256 x 7168 x 7168, after the same A quantization), and the
    phases it reports are non-negative."""
    torch = torch_cuda()
    import block_scaled_mxfp4_bf16_amd as mx
    out = bench.wide_phases(torch, mx, steps=2)
    assert "skipped" not in out, out
    assert out["c_matches_library"]
    for ph in bench.WIDE_PHASE_NAMES:
        assert out["workgroup_phase_us"][ph]["median"] >= 0.0
    assert 0.0 < out["first_entry_to_last_completion_us"]["median"] < 1000.0
    assert len(out["median_completion_by_xcd_us"]) >= 1


@pytest.mark.parametrize("shuffled", [False, True])
def test_quantize_timing_runs_and_is_plausible(shuffled):
    """The bench's timing of the standalone quantization of A: a positive
    time, and no faster than HBM's peak allows for the bytes it moves."""
    torch = torch_cuda()
    import block_scaled_mxfp4_bf16_amd as mx
    r = bench.time_quantize(torch, mx, bench.workload("c2"), shuffled, steps=8, samples=2, min_bytes=1 << 22)
    assert r["us_per_call"] > 0
    assert r["gbs"] < bench.HBM_PEAK_GBS * 1.05
    assert r["scales"] == ("shuffled" if shuffled else "raw")
