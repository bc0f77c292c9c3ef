"""Host-side logic of bench.py: the algorithmic byte and FLOP counts, the
matrix-instruction count of a product, the two rocprofv3 counter summaries
(on small synthetic counter files), and the one-GPU guard.  No GPU needed."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import synthetic as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size", "Kernel_Id",
          "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
          "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_counters(d, rows):
    """rows: (dispatch, grid, kernel, counter, value, start_ns, end_ns)"""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for disp, grid, kern, ctr, val, t0, t1 in rows:
            w.writerow({"Correlation_Id": disp, "Dispatch_Id": disp, "Agent_Id": "Agent 1", "Queue_Id": 1,
                        "Process_Id": 1, "Thread_Id": 1, "Grid_Size": grid, "Kernel_Id": 1, "Kernel_Name": kern,
                        "Workgroup_Size": 256, "LDS_Block_Size": 0, "Scratch_Size": 0, "VGPR_Count": 0,
                        "Accum_VGPR_Count": 0, "SGPR_Count": 0, "Counter_Name": ctr, "Counter_Value": val,
                        "Start_Timestamp": t0, "End_Timestamp": t1})


def test_algorithmic_bytes_and_flops():
    # M=32 N=4096 K=512: A bf16 + B e2m1 + B e8m0 + C bf16, each once
    assert bench.alg_bytes(32, 4096, 512) == 2 * 32 * 512 + 4096 * 512 // 2 + 4096 * 512 // 32 + 2 * 32 * 4096
    assert bench.alg_bytes(32, 4096, 512) == 1409024
    assert bench.alg_flops(256, 7168, 7168) == 26306674688


def test_expected_matrix_instructions():
    # 16 x 16 x 128 instructions: row tiles padded to 16, half steps counted whole
    assert bench.expected_mfma(256, 7168, 7168) == 16 * 448 * 56
    assert bench.expected_mfma(8, 2112, 7168) == 1 * 132 * 56
    assert bench.expected_mfma(17, 32, 192) == 2 * 2 * 2
    for c in ("c1", "c2", "c3", "c4", "c5"):
        w = syn.CONFIGS[c]
        # every instruction does 2 * 16 * 16 * 128 FLOPs, padding included
        assert bench.expected_mfma(w.M, w.N, w.K) * 65536 >= bench.alg_flops(w.M, w.N, w.K)


def test_summarize_mfma_on_synthetic_counters(tmp_path, capsys):
    wide = "void mxfp4::gemm_wide_kernel<4, 7, 4, 2, false, false>(unsigned char const*)"
    fused = "void mxfp4::gemm_kernel<1, 2, 1, 4, 1, false, 16, 0, false>(unsigned short const*)"  # c2's schedule
    quant = "mxfp4::quant_quad_kernel(unsigned short const*)"
    rows = []
    for i, ns in enumerate([16000, 16400, 17000]):  # median duration 16400
        d = 10 + i
        rows += [(d, 65536, wide, "SQ_INSTS_MFMA", 401408, 1000, 1000 + ns),
                 (d, 65536, wide, "SQ_VALU_MFMA_BUSY_CYCLES", 401408 * 16, 1000, 1000 + ns)]
    fused_q = "void mxfp4::gemm_kernel<1, 2, 1, 4, 1, true, 16, 0, false>(unsigned short const*)"  # c2, gemm_q
    rows += [(20, 32768, fused, "SQ_INSTS_MFMA", 2048, 0, 4000),
             (20, 32768, fused, "SQ_VALU_MFMA_BUSY_CYCLES", 2048 * 16, 0, 4000),
             (22, 32768, fused_q, "SQ_INSTS_MFMA", 2048, 0, 3000),
             (22, 32768, fused_q, "SQ_VALU_MFMA_BUSY_CYCLES", 2048 * 16, 0, 3000),
             (21, 57344, quant, "SQ_INSTS_MFMA", 0, 0, 3000)]  # not a GEMM: ignored
    write_counters(str(tmp_path / "pmc"), rows)
    bench.summarize_mfma(str(tmp_path / "pmc"), ["c2", "c5"], "cmd")
    out = json.loads(capsys.readouterr().out)
    assert out["command"] == "cmd"
    ks = {k["kernel"]: k for k in out["kernels"]}
    assert set(ks) == {wide.split("(")[0], fused.split("(")[0], fused_q.split("(")[0]}
    w = ks[wide.split("(")[0]]
    assert w["dispatches"] == 3 and w["mfma_instructions"] == 401408
    assert w["workload"] == syn.CONFIGS["c5"].name
    assert w["busy_cycles_per_instruction"] == 16.0 and w["duration_ns"] == 16400
    assert w["matrix_busy_frac_at_2400MHz"] == pytest.approx(401408 * 16 / (1024 * 2.4 * 16400), abs=1e-4)
    assert ks[fused.split("(")[0]]["workload"] == syn.CONFIGS["c2"].name
    assert ks[fused_q.split("(")[0]]["workload"] == syn.CONFIGS["c2"].name + " (A pre-quantized)"


def test_summarize_pmc_scales_by_the_copy_calibration(tmp_path, monkeypatch, capsys):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    gemm = "void mxfp4::gemm_wide_kernel<4, 7, 4, 2, false, false>(unsigned char const*)"
    quant = "mxfp4::quant_quad_kernel(unsigned short const*)"
    copy = "__amd_rocclr_copyBuffer"
    cal = bench.CALIBRATION_BYTES
    # FETCH_SIZE reads half of a cold copy's bytes, WRITE_SIZE all of them (KiB per dispatch)
    fetch = [(1, 1 << 20, copy, "FETCH_SIZE", 64, 0, 1), (2, 1 << 26, copy, "FETCH_SIZE", cal / 2 / 1024, 0, 1)]
    write = [(1, 1 << 20, copy, "WRITE_SIZE", 64, 0, 1), (2, 1 << 26, copy, "WRITE_SIZE", cal / 1024, 0, 1)]
    prep = "mxfp4::quantize_raw_kernel<false>(unsigned short const*)"  # once per run: not part of a call
    fetch.append((3, 1 << 20, prep, "FETCH_SIZE", 99999, 0, 1))
    write.append((3, 1 << 20, prep, "WRITE_SIZE", 99999, 0, 1))
    fetch.append((4, 1 << 30, copy, "FETCH_SIZE", 100, 0, 1))  # a larger grid, fewer bytes than the calibration
    write.append((4, 1 << 30, copy, "WRITE_SIZE", 100, 0, 1))
    for i, (f, w) in enumerate([(700, 256), (720, 256), (760, 256)]):
        fetch.append((10 + 2 * i, 65536, gemm, "FETCH_SIZE", f, 0, 1))
        write.append((10 + 2 * i, 65536, gemm, "WRITE_SIZE", w, 0, 1))
        fetch.append((11 + 2 * i, 4096, quant, "FETCH_SIZE", 100, 0, 1))
        write.append((11 + 2 * i, 4096, quant, "WRITE_SIZE", 30, 0, 1))
    write_counters(str(tmp_path / "f"), fetch)
    write_counters(str(tmp_path / "w"), write)
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "cmd")
    out = json.loads(capsys.readouterr().out)
    assert out["copy_calibration"] == {"fetch": 0.5, "write": 1.0}
    k = out["kernels"]["void mxfp4::gemm_wide_kernel<4, 7, 4, 2, false, false>"]
    assert k["fetch_bytes"] == 720 * 1024 * 2  # median, divided by the fetch scale
    assert k["write_bytes"] == 256 * 1024 and k["dispatches"] == [3, 3]
    assert set(out["kernels"]) == {"void mxfp4::gemm_wide_kernel<4, 7, 4, 2, false, false>", "mxfp4::quant_quad_kernel"}
    assert out["fetch_bytes_per_call"] == 720 * 2048 + 100 * 2048
    assert out["write_bytes_per_call"] == 256 * 1024 + 30 * 1024
    assert out["hbm_bytes_per_call"] == out["fetch_bytes_per_call"] + out["write_bytes_per_call"]
    with open(tmp_path / "traffic.json") as f:
        assert json.load(f)["kernel_source_hash"] == bench.kernel_source_hash()
    # the bench reports traffic only while the hash matches the sources
    assert bench.measured_traffic() == out["hbm_bytes_per_call"]
    with open(tmp_path / "traffic.json", "w") as f:
        json.dump(dict(out, kernel_source_hash="0" * 16), f)
    assert bench.measured_traffic() is None


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "p_4x2880x512", "p_256x3072x1536"])
@pytest.mark.parametrize("steps", [1, 5, 20, 100, 2000])
def test_rotation_is_cold_at_any_step_count(name, steps):
    """A multiple of `steps` sets, at least 1 GiB of them, covered by whole
    graphs: every call's set was last touched >= 1 GiB of other sets ago."""
    w = bench.workload(name)
    per = bench.set_bytes(w.M, w.N, w.K)
    sets, graphs = bench.rotation(per, steps)
    assert sets % steps == 0 and graphs * steps == sets
    assert sets * per >= bench.COLD_BYTES
    assert (sets - steps) * per < bench.COLD_BYTES or sets == steps  # no more than needed
    assert (sets - 1) * per >= bench.COLD_BYTES - per


def test_set_bytes_counts_the_padded_scales():
    # N = 2112 pads to 2304 scale rows; K/32 = 224 is already a multiple of 8
    assert bench.set_bytes(8, 2112, 7168) == 2 * 8 * 7168 + 2112 * 3584 + 2304 * 224 + 2 * 8 * 2112


def test_percentile_and_roofline_blocks():
    assert bench.percentile([3.0], 10) == 3.0
    assert bench.percentile([1.0, 2.0, 3.0, 4.0, 5.0], 50) == 3.0
    assert bench.percentile([1.0, 2.0, 3.0, 4.0, 5.0], 10) == pytest.approx(1.4)
    r = bench.roofline(256, 7168, 7168, 10.0, "mfma")
    assert r["unit"] == "TFLOP/s" and r["peak"] == 10100.0
    assert r["achieved"] == pytest.approx(2 * 256 * 7168 * 7168 / 1e-5 / 1e12, abs=0.1)
    assert r["frac"] == pytest.approx(r["achieved"] / 10100.0, abs=1e-4)
    h = bench.roofline(32, 4096, 512, 2.0, "hbm")
    assert h["unit"] == "GB/s" and h["achieved"] == pytest.approx(1409024 / 2e-6 / 1e9, abs=0.1)
    assert bench.bound_of(256) == "mfma" and bench.bound_of(64) == "hbm"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 1
    assert "one GPU" in r.stderr and r.stdout == ""


def test_load_sclk_mean_over_xcds():
    assert bench.load_sclk_mhz(None) is None
    assert bench.load_sclk_mhz({"mem_0": 2000}) is None
    c = {"gfx_0": 2400, "gfx_1": 2300, "mem_0": 2000, "socclk_0": 74, "replays": 580}
    assert bench.load_sclk_mhz(c) == 2350.0
