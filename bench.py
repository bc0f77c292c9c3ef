#!/usr/bin/env python3
"""Benchmark of the fused MXFP4 GEMM (A bf16 quantized on the fly) on one MI355X.

A step is one call of the whole per-call path -- quantize A in registers,
multiply by the preshuffled MXFP4 B, reduce, store bf16 C -- over one batch of
synthetic input.  B is prepared once, outside the timed region, by the
library's own quantize and preshuffle kernels.

Timing: K steps are captured into one HIP graph and replayed; the timed
region is that replay, bracketed by device synchronizations, with HIP events
recorded on the replay stream.  In the default "cold" mode consecutive steps
cycle through enough copies of (A, B, scales, C) -- at least 1 GiB -- that
each step's inputs come from HBM rather than L2 or the 256 MB MALL.

Each configuration is then timed a second time on a single buffer set
("warm_us_per_call": inputs stay in L2 and the MALL), for context; the
reported value is always the cold one.

Prints one JSON line.  The headline workload is M=32, N=4096, K=512; the
line also carries every measured configuration under "per_config".
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 matrix peak, TFLOP/s
HEADLINE = "c2"
# What decides the headline GEMM's code: its kernel sources, plus the
# schedule the library picks for the headline shape (hashed with them).
KERNEL_SOURCES = ["block_scaled_mxfp4_bf16_amd/csrc/gemm_kernels.hip", "block_scaled_mxfp4_bf16_amd/csrc/mxfp4_device.hpp",
                  "block_scaled_mxfp4_bf16_amd/csrc/mxfp4_internal.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_M32_N4096_K512.json")
CALIBRATION_BYTES = 256 << 20


def calibration_copy(torch):
    """A plain device copy of known size whose source is cold: 256 MiB
    written, then 1 GiB written to push it out of L2 and the MALL, then
    copied.  Counter runs scale HBM counters by what they read for it."""
    src = torch.empty(CALIBRATION_BYTES, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    evict = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    evict.fill_(2)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, evict, dst
    torch.cuda.empty_cache()


def kernel_source_hash():
    import hashlib
    import block_scaled_mxfp4_bf16_amd as mx
    import synthetic as syn
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    w = syn.CONFIGS[HEADLINE]
    h.update(str(mx.mxfp4_gemm_schedule_name(w.M, w.N, w.K)).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the kernel as it is now; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def alg_bytes(M, N, K):
    """A bf16 + B e2m1 + B e8m0 + C bf16, each counted once."""
    return 2 * M * K + N * K // 2 + N * K // 32 + 2 * M * N


def alg_flops(M, N, K):
    return 2 * M * N * K


def prepare(torch, mx, w, sets):
    import numpy as np
    dev = torch.device("cuda", 0)
    a = torch.from_numpy(w.a_bits().view(np.int16)).view(torch.bfloat16).to(dev)
    b = torch.from_numpy(w.b_bits().view(np.int16)).view(torch.bfloat16).to(dev)
    qb, sb = mx.quantize(b)
    bw, bs = mx.preshuffle_b(qb, sb)
    del b, qb, sb
    out = []
    for i in range(sets):
        if i == 0:
            out.append((a, bw, bs, torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)))
        else:
            out.append((a.clone(), bw.clone(), bs.clone(), torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()
    return out


def time_config(torch, mx, w, steps, warmup, cold):
    M, N, K = w.M, w.N, w.K
    per_set = alg_bytes(M, N, K) + N * K // 32
    sets = min(512, max(2, math.ceil((1 << 30) / per_set))) if cold else 1
    bufs = prepare(torch, mx, w, sets)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        mx.mxfp4_reserve(M, N, K, stream=stream)
        for i in range(warmup):
            A, Bw, Bs, C = bufs[i % sets]
            mx.mxfp4_gemm(A, Bw, Bs, C, M, N, K, stream=stream)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            A, Bw, Bs, C = bufs[i % sets]
            mx.mxfp4_gemm(A, Bw, Bs, C, M, N, K, stream=stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()  # first replay uploads the graph
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = ev0.elapsed_time(ev1) / steps
    del g, bufs
    torch.cuda.empty_cache()
    us = kern_ms * 1e3
    return {
        "M": M, "N": N, "K": K,
        "schedule": mx.mxfp4_gemm_schedule_name(M, N, K),
        "buffer_sets": sets,
        "us_per_call": round(us, 4),
        "wall_ms_per_step": wall * 1e3 / steps,
        "tflops": alg_flops(M, N, K) / (us * 1e-6) / 1e12,
        "alg_gbs": alg_bytes(M, N, K) / (us * 1e-6) / 1e9,
        "hbm_frac": alg_bytes(M, N, K) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "mfma_frac": alg_flops(M, N, K) / (us * 1e-6) / 1e12 / FP4_PEAK_TFLOPS,
    }


def time_prepare_b(torch, mx, w, steps=50):
    """One-launch B preparation (quantize + both shuffles) of a workload's B,
    cold: consecutive calls cycle through >= 1 GiB of bf16 B copies."""
    import numpy as np
    N, K = w.N, w.K
    b = torch.from_numpy(w.b_bits().view(np.int16)).view(torch.bfloat16).to("cuda")
    sets = max(2, math.ceil((1 << 30) / (2 * N * K)))
    bs_in = [b] + [b.clone() for _ in range(sets - 1)]
    bw = torch.empty((N // 16, (K // 2) * 16), dtype=torch.uint8, device="cuda")
    bs = torch.empty(mx.mxfp4_shuffled_scale_bytes(N, K), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(3):
            mx.mxfp4_prepare_b(bs_in[i % sets], N, K, bw, bs, stream=stream)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            mx.mxfp4_prepare_b(bs_in[i % sets], N, K, bw, bs, stream=stream)
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    nbytes = 2 * N * K + N * K // 2 + mx.mxfp4_shuffled_scale_bytes(N, K)
    del g, bs_in, b
    torch.cuda.empty_cache()
    return {"N": N, "K": K, "us_per_call": round(us, 3), "bytes": nbytes, "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "buffer_sets": sets}


def cpu_baseline(w, budget_s=12.0):
    """The oracle as it stands, single-threaded, on whole calls of the
    headline workload (quantize A, exact GEMM, round) until the budget is
    spent."""
    import oracle
    qb, sb = oracle.quantize(w.b_bits())
    a = w.a_bits()
    oracle.mxfp4_gemm_bf16(a, qb, sb)  # load + page in
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.mxfp4_gemm_bf16(a, qb, sb)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": alg_flops(w.M, w.N, w.K) * n / el / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": "%d whole calls of %s (quantize A + fp64 GEMM + bf16 rounding), %.1f s" % (n, w.name, el)}


def _pmc_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize_pmc(fetch_dir, write_dir, command):
    """Turn two rocprofv3 --pmc runs of the headline bench (FETCH_SIZE, then
    WRITE_SIZE; KiB per dispatch) into HBM bytes per GEMM launch.  The scale
    of each counter is calibrated on the plain copy kernels of the same runs
    (the clones of B, of known size, made while preparing the buffer sets)."""
    import synthetic as syn
    w = syn.CONFIGS[HEADLINE]
    bw_bytes = w.N * w.K // 2

    def per_kernel(rows, counter):
        gemm, copy = [], []
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            name = r["Kernel_Name"]
            if "gemm_kernel" in name:
                gemm.append(v)
            elif "copyBuffer" in name:
                copy.append((int(r["Grid_Size"]), v))
        # the calibration copy is the largest copy of the run
        big = max(g for g, _ in copy)
        return gemm, [v for g, v in copy if g == big]

    fg, fc = per_kernel(_pmc_rows(fetch_dir), "FETCH_SIZE")
    wg, wc = per_kernel(_pmc_rows(write_dir), "WRITE_SIZE")
    med = lambda v: sorted(v)[len(v) // 2]
    f_scale = med(fc) / CALIBRATION_BYTES  # counter bytes per byte copied
    w_scale = med(wc) / CALIBRATION_BYTES
    fetch = med(fg) / f_scale
    write = med(wg) / w_scale
    out = {"workload": w.name, "kernel_source_hash": kernel_source_hash(), "command": command,
           "gemm_dispatches": [len(fg), len(wg)], "fetch_bytes_per_launch": round(fetch),
           "write_bytes_per_launch": round(write), "hbm_bytes_per_launch": round(fetch + write),
           "algorithmic_bytes": alg_bytes(w.M, w.N, w.K), "copy_calibration": {"fetch": f_scale, "write": w_scale}}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def expected_mfma(M, N, K):
    """Matrix instructions the product needs at 16 x 16 x 128 per
    instruction: 16-row tiles (rows past M padded), 16-column subtiles,
    128-wide K steps (a final 64-wide half step counted whole)."""
    return ((M + 15) // 16) * (N // 16) * ((K + 127) // 128)


def summarize_mfma(pmc_dir, configs, command):
    """Turn a rocprofv3 --pmc run (SQ_INSTS_MFMA, SQ_VALU_MFMA_BUSY_CYCLES)
    of the bench into matrix-unit use per GEMM kernel: instructions and busy
    SIMD cycles per dispatch (medians), the dispatch's own duration from the
    same run, and busy cycles over what 1024 SIMDs offer in that time at the
    nominal 2.4 GHz.  At full FP4 rate one 16x16x128 instruction keeps its
    SIMD's matrix unit busy 16 cycles."""
    import synthetic as syn
    groups = {}
    for r in _pmc_rows(pmc_dir):
        if "gemm" not in r["Kernel_Name"]:
            continue
        key = (r["Kernel_Name"].split("(")[0], int(r["Grid_Size"]))
        d = groups.setdefault(key, {})
        disp = d.setdefault(r["Dispatch_Id"], {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        disp[r["Counter_Name"]] = float(r["Counter_Value"])
    med = lambda v: sorted(v)[len(v) // 2]
    want = {expected_mfma(w.M, w.N, w.K): w.name for w in (syn.CONFIGS[c] for c in configs)}
    out = {"command": command, "kernels": []}
    for (name, grid), d in sorted(groups.items()):
        ds = list(d.values())
        inst = med([x.get("SQ_INSTS_MFMA", 0.0) for x in ds])
        busy = med([x.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for x in ds])
        ns = med([x["ns"] for x in ds])
        out["kernels"].append({
            "kernel": name, "grid": grid, "dispatches": len(ds), "workload": want.get(int(inst)),
            "mfma_instructions": int(inst), "busy_simd_cycles": int(busy),
            "busy_cycles_per_instruction": round(busy / inst, 2) if inst else None,
            "duration_ns": ns, "matrix_busy_frac_at_2400MHz": round(busy / (1024 * 2.4 * ns), 4) if ns else None})
    print(json.dumps(out, indent=1))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc":
        summarize_pmc(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-mfma":
        summarize_mfma(sys.argv[2], sys.argv[3].split(","), " ".join(sys.argv[4:]))
        return
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--configs", default="c1,c2,c3,c4,c5", help="configurations measured under per_config")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-b-prep", action="store_true", help="skip timing the one-launch B preparation")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the second, warm timing (one buffer set, so inputs stay in L2 and MALL)")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="first run a cold 256 MiB device copy (for scaling HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this operation is built and timed on a single MI355X "
              "(N-sharding of B across GPUs needs no collective and is not implemented); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(1)

    import torch
    import block_scaled_mxfp4_bf16_amd as mx
    import synthetic as syn

    torch.cuda.set_device(0)
    if args.pmc_calibration:
        calibration_copy(torch)
    names = [c for c in args.configs.split(",") if c]
    if HEADLINE not in names:
        names.insert(0, HEADLINE)
    per = {}
    for name in names:
        w = syn.CONFIGS[name]
        r = time_config(torch, mx, w, args.steps, args.warmup, cold=True)
        if not args.no_warm:
            # context only: the same calls on one buffer set, inputs warm in L2 and MALL
            r["warm_us_per_call"] = time_config(torch, mx, w, args.steps, args.warmup, cold=False)["us_per_call"]
        per[w.name] = r
        print("[bench] %s: %.3f us/call cold%s, %.1f TFLOP/s, %.0f GB/s (%.1f%% of HBM), schedule %s"
              % (w.name, r["us_per_call"], "" if args.no_warm else " (%.3f warm)" % r["warm_us_per_call"],
                 r["tflops"], r["alg_gbs"], 100 * r["hbm_frac"], r["schedule"]),
              file=sys.stderr, flush=True)

    hw = syn.CONFIGS[HEADLINE]
    h = per[hw.name]
    print("[bench] kernel source hash %s" % kernel_source_hash(), file=sys.stderr, flush=True)
    line = {
        "metric": "us/call and TFLOPS per (M,N,K); % of HBM or MXFP4-MFMA roofline",
        "value": h["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["wall_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 (e2m1 x e2m1 scaled MFMA, f32 accumulate, bf16 out)",
        "data": "synthetic (Philox-4x32-10 + Box-Muller N(0,1) bf16, seeded)",
        "config": {"workload": hw.name, "M": hw.M, "N": hw.N, "K": hw.K,
                   "cache": "cold: %d rotating buffer sets" % h["buffer_sets"], "schedule": h["schedule"]},
        "us_per_call": h["us_per_call"],
        "roofline": {
            "bound": "hbm",
            "achieved": round(h["alg_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(h["hbm_frac"], 4),
            "traffic": measured_traffic(),
        },
        "per_config": per,
    }
    if not args.no_b_prep:
        # offline weight preparation (not part of a call): its own throughput
        line["b_prep"] = {}
        for name in ("c2", "c5"):
            w = syn.CONFIGS[name]
            r = time_prepare_b(torch, mx, w)
            line["b_prep"][w.name] = r
            print("[bench] B prep %dx%d: %.2f us, %.0f GB/s (%.1f%% of HBM)" % (w.N, w.K, r["us_per_call"], r["gbs"],
                                                                           100 * r["hbm_frac"]),
                  file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(hw)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
