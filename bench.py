#!/usr/bin/env python3
"""Benchmark of the MXFP4 GEMM (A bf16 quantized on the fly) on one MI355X.

A step is one call of the whole per-call path -- quantize A, multiply by the
preshuffled MXFP4 B with scaled FP4 matrix instructions, reduce, store bf16 C
-- over one batch of synthetic input.  B is prepared once, outside the timed
region, by the library's own quantize and preshuffle kernels.

Cold by construction, at any step count: every configuration gets S copies
("sets") of (A, B, scales, C), S a multiple of --steps with S * set bytes >=
1 GiB (4x the 256 MB MALL).  The calls cycle through the sets in order, so a
set is touched again only after every other set has been: each call's inputs
were last read >= 1 GiB of other traffic ago and come from HBM.  The calls
are captured as S / steps HIP graphs of --steps calls each, replayed in turn
so the rotation continues from one replay to the next.

Timed region: one replay of the first graph (exactly --steps calls, each on
its own set), bracketed by device synchronizations, with HIP events recorded
on the replay stream; ms_per_step is that replay's event time / steps.
Statistics: one more graph holds whole rotations (every set in order, at
least 200 calls), so that the cost of launching a graph is spread as it is
over a long run of calls; --samples replays of it, each timed by events,
give the median, p10 and p90 of the time per call (us_per_call, value).

The headline is the largest configuration, M=256 N=7168 K=7168, reported as
TFLOP/s against the dense MXFP4 matrix peak.  Every configuration (the five
of the method's workloads and the other leaderboard shapes on the pages) is
reported under per_config with its own roofline block; for context each is
also timed warm (one set, inputs resident in L2 and the MALL), and the five
method workloads from an A quantized beforehand (mxfp4_gemm_q, cold, under
per_config.<workload>.prequantized_a).

Prints one JSON line.
"""
import argparse
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 matrix peak, TFLOP/s
HEADLINE = "c5"
COLD_BYTES = 1 << 30           # footprint of one rotation: 4x the 256 MB MALL
# What decides the kernels' code: the library sources, plus the schedule the
# library picks for the headline shape (hashed with them).
KERNEL_SOURCE_DIR = "block_scaled_mxfp4_bf16_amd/csrc"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_M256_N7168_K7168.json")
CALIBRATION_BYTES = 256 << 20


def alg_bytes(M, N, K):
    """A bf16 + B e2m1 + B e8m0 + C bf16, each counted once."""
    return 2 * M * K + N * K // 2 + N * K // 32 + 2 * M * N


NOMINAL_SCLK_MHZ = 2400.0       # the clock the published matrix peak assumes


def load_sclk_mhz(clocks):
    """Mean shader clock over the XCDs (amd-smi's gfx_<i> domains) from a
    reading taken under load, or None."""
    if not clocks:
        return None
    v = [x for k, x in clocks.items() if k.startswith("gfx_") and isinstance(x, (int, float)) and x > 0]
    return sum(v) / len(v) if v else None


def alg_flops(M, N, K):
    return 2 * M * N * K


def expected_mfma(M, N, K):
    """Matrix instructions the product needs at 16 x 16 x 128 per
    instruction: 16-row tiles (rows past M padded), 16-column subtiles,
    128-wide K steps (a final 64-wide half step counted whole)."""
    return ((M + 15) // 16) * (N // 16) * ((K + 127) // 128)


def set_bytes(M, N, K):
    """Device bytes of one buffer set: A, B codes, padded B scales, C."""
    scales = ((N + 255) // 256 * 256) * ((K // 32 + 7) // 8 * 8)
    return 2 * M * K + N * K // 2 + scales + 2 * M * N


def rotation(per_set, steps, min_bytes=COLD_BYTES):
    """(sets, graphs): the least multiple of `steps` sets whose footprint is
    at least min_bytes, and the number of `steps`-call graphs that cover them."""
    need = max(1, math.ceil(min_bytes / per_set))
    sets = steps * math.ceil(need / steps)
    return sets, sets // steps


def percentile(v, q):
    """Linear-interpolated percentile of a list (q in [0, 100])."""
    s = sorted(v)
    if len(s) == 1:
        return s[0]
    x = (len(s) - 1) * q / 100.0
    i = int(math.floor(x))
    j = min(i + 1, len(s) - 1)
    return s[i] + (s[j] - s[i]) * (x - i)


def roofline(M, N, K, us, bound):
    """Roofline block for one configuration at `us` microseconds per call:
    algorithmic bytes against HBM, or algorithmic FLOPs against the MXFP4
    matrix peak."""
    if bound == "mfma":
        achieved = alg_flops(M, N, K) / (us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP4_PEAK_TFLOPS, 4)}
    achieved = alg_bytes(M, N, K) / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4)}


def bound_of(M):
    """The method's targets: HBM roofline at small M, matrix peak from 256 rows."""
    return "mfma" if M >= 256 else "hbm"


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
    d = os.path.join(ROOT, KERNEL_SOURCE_DIR)
    for rel in sorted(os.listdir(d)):
        if rel.startswith("probe"):
            continue  # the measurement probes are not part of the library
        with open(os.path.join(d, rel), "rb") as f:
            h.update(rel.encode())
            h.update(f.read())
    w = syn.CONFIGS[HEADLINE]
    h.update(str(mx.mxfp4_gemm_schedule_name(w.M, w.N, w.K)).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per call of the headline workload from the committed counter
    summary, if it was taken on the kernels as they are now; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_call")


def gpu_clocks():
    """Current GPU clocks as amd-smi reports them: MHz per clock domain
    (gfx_0..7 are the eight XCDs' shader clocks), or the error."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True, text=True,
                           timeout=30)
        if r.returncode != 0:
            return {"error": (r.stderr or r.stdout).strip()[-300:]}
        return compact_clocks(json.loads(r.stdout))
    except Exception as e:  # the clocks are context; the measurement does not depend on them
        return {"error": repr(e)[-300:]}


def compact_clocks(d):
    """{domain: MHz} from amd-smi's JSON (a list of GPUs, or one GPU)."""
    g = d["gpu_data"][0] if isinstance(d, dict) and "gpu_data" in d else (d[0] if isinstance(d, list) else d)
    out = {}
    for name, v in g.get("clock", {}).items():
        if isinstance(v, dict) and isinstance(v.get("clk"), dict):
            out[name] = v["clk"].get("value")
    return out


def cpu_model():
    try:
        for line in subprocess.run(["lscpu"], capture_output=True, text=True, timeout=30).stdout.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return None


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


def time_config(torch, mx, w, steps, warmup, samples, cold=True, clocks_under_load=False):
    """Time `steps`-call graph replays of the workload (see the module
    docstring).  Returns the per-call figures of the first timed replay (the
    contract's timed region) and the statistics over `samples` replays.
    With clocks_under_load, the replays then go on (untimed) while amd-smi
    reads the clocks from another thread, so the reading is taken under this
    workload's load rather than at idle."""
    M, N, K = w.M, w.N, w.K
    per_set = set_bytes(M, N, K)
    sets, graphs = rotation(per_set, steps) if cold else (1, 1)
    bufs = prepare(torch, mx, w, sets)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        mx.mxfp4_reserve(M, N, K, stream=stream)
        for i in range(warmup):
            A, Bw, Bs, C = bufs[i % sets]
            mx.mxfp4_gemm(A, Bw, Bs, C, M, N, K, stream=stream)
    stream.synchronize()
    gs = []
    for j in range(graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                A, Bw, Bs, C = bufs[(j * steps + i) % sets]
                mx.mxfp4_gemm(A, Bw, Bs, C, M, N, K, stream=stream)
        gs.append(g)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for g in gs:
            g.replay()  # the first replay of a graph uploads it
    torch.cuda.synchronize()

    # the timed region: one replay, exactly `steps` calls
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        gs[0].replay()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timed_us = e0.elapsed_time(e1) * 1e3 / steps
    # statistics: a graph of whole rotations, continuing after graph 0
    rounds = max(1, math.ceil(200 / sets))
    long_calls = rounds * sets
    lg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(lg, stream=stream):
        for i in range(long_calls):
            A, Bw, Bs, C = bufs[(steps + i) % sets]
            mx.mxfp4_gemm(A, Bw, Bs, C, M, N, K, stream=stream)
    with torch.cuda.stream(stream):
        lg.replay()  # upload
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    with torch.cuda.stream(stream):
        for s in range(samples):
            ev[s][0].record(stream)
            lg.replay()
            ev[s][1].record(stream)
    torch.cuda.synchronize()
    us = [a.elapsed_time(b) * 1e3 / long_calls for a, b in ev]
    del lg
    load_clocks = None
    if clocks_under_load:
        import threading
        box = {}
        t = threading.Thread(target=lambda: box.setdefault("c", gpu_clocks()))
        t0 = time.perf_counter()
        k = 0
        with torch.cuda.stream(stream):
            # a second of continuous load first (the clock readings are
            # averaged over a window), then more while amd-smi runs (bounded)
            while time.perf_counter() - t0 < 1.0:
                for _ in range(20):
                    gs[k % graphs].replay()
                    k += 1
                stream.synchronize()
            t.start()
            while t.is_alive() and time.perf_counter() - t0 < 30:
                for _ in range(20):
                    gs[k % graphs].replay()
                    k += 1
                stream.synchronize()
        t.join()
        load_clocks = dict(box.get("c") or {}, replays=k, seconds=round(time.perf_counter() - t0, 2))
    del gs, bufs
    torch.cuda.empty_cache()
    med = percentile(us, 50)
    r = {
        "M": M, "N": N, "K": K,
        "schedule": mx.mxfp4_gemm_schedule_name(M, N, K),
        "cache": ("cold: %d buffer sets of %d bytes (%.2f GiB) cycled in order; each call's set last touched %d "
                  "calls earlier" % (sets, per_set, sets * per_set / 2 ** 30, sets)) if cold else
                 "warm: one buffer set (inputs resident in L2 and MALL)",
        "buffer_sets": sets, "set_bytes": per_set, "footprint_bytes": sets * per_set,
        "timed_us_per_call": round(timed_us, 4),
        "timed_wall_ms": round(wall * 1e3, 4),
        "samples": samples, "calls_per_sample": long_calls,
        "us_per_call": round(med, 4),
        "us_p10": round(percentile(us, 10), 4), "us_p90": round(percentile(us, 90), 4),
        "us_min": round(min(us), 4), "us_max": round(max(us), 4),
        "tflops": alg_flops(M, N, K) / (med * 1e-6) / 1e12,
        "alg_gbs": alg_bytes(M, N, K) / (med * 1e-6) / 1e9,
        "hbm_frac": alg_bytes(M, N, K) / (med * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "mfma_frac": alg_flops(M, N, K) / (med * 1e-6) / 1e12 / FP4_PEAK_TFLOPS,
    }
    r["roofline"] = roofline(M, N, K, med, bound_of(M))
    if load_clocks is not None:
        r["clocks_under_load"] = load_clocks
    return r


def time_config_q(torch, mx, w, steps, samples):
    """The pre-quantized-A entry point (mxfp4_gemm_q) on the workload: A is
    quantized once, outside the timed region, to codes and shuffled scales
    (the form a caller that reuses one A quantization across GEMMs holds),
    and the calls cycle cold through buffer sets as in time_config.  Median,
    p10 and p90 over `samples` replays of a graph of whole rotations."""
    import numpy as np
    M, N, K = w.M, w.N, w.K
    dev = torch.device("cuda", 0)
    a = torch.from_numpy(w.a_bits().view(np.int16)).view(torch.bfloat16).to(dev)
    b = torch.from_numpy(w.b_bits().view(np.int16)).view(torch.bfloat16).to(dev)
    qb, sb = mx.quantize(b)
    bw, bs = mx.preshuffle_b(qb, sb)
    aq, as_ = mx.quantize(a, shuffled_scales=True)
    del a, b, qb, sb
    per_set = aq.numel() + as_.numel() + bw.numel() + bs.numel() + 2 * M * N
    sets, _ = rotation(per_set, steps)
    bufs = [(aq, as_, bw, bs)] + [(aq.clone(), as_.clone(), bw.clone(), bs.clone()) for _ in range(sets - 1)]
    bufs = [t + (torch.empty((M, N), dtype=torch.bfloat16, device=dev),) for t in bufs]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        mx.mxfp4_reserve(M, N, K, stream=stream)
        for i in range(3):
            mx.mxfp4_gemm_q(*bufs[i % sets], M, N, K, stream=stream)
    stream.synchronize()
    rounds = max(1, math.ceil(200 / sets))
    calls = rounds * sets
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(calls):
            mx.mxfp4_gemm_q(*bufs[i % sets], M, N, K, stream=stream)
    with torch.cuda.stream(stream):
        g.replay()  # upload
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    with torch.cuda.stream(stream):
        for k in range(samples):
            ev[k][0].record(stream)
            g.replay()
            ev[k][1].record(stream)
    torch.cuda.synchronize()
    us = [x.elapsed_time(y) * 1e3 / calls for x, y in ev]
    del g, bufs
    torch.cuda.empty_cache()
    med = percentile(us, 50)
    return {"schedule": mx.mxfp4_gemm_q_schedule_name(M, N, K), "us_per_call": round(med, 4),
            "us_p10": round(percentile(us, 10), 4), "us_p90": round(percentile(us, 90), 4),
            "tflops": alg_flops(M, N, K) / (med * 1e-6) / 1e12, "buffer_sets": sets, "set_bytes": per_set}


def time_prepare_b(torch, mx, w, steps=50):
    """One-launch B preparation (quantize + both shuffles) of a workload's B,
    cold: consecutive calls cycle through >= 1 GiB of bf16 B copies."""
    import numpy as np
    N, K = w.N, w.K
    b = torch.from_numpy(w.b_bits().view(np.int16)).view(torch.bfloat16).to("cuda")
    sets = max(2, math.ceil(COLD_BYTES / (2 * N * K)))
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


def time_quantize(torch, mx, w, shuffled, steps=50, samples=5, min_bytes=COLD_BYTES):
    """The standalone quantization (mxfp4_quantize) of a workload's A, raw or
    with shuffled scales, cold: the calls cycle in order through copies of A
    in one buffer of >= 1 GiB (several graphs of `steps` calls cover them
    all), median over `samples` replays of the whole rotation.  Bytes: bf16 A
    read, codes and scales written."""
    import numpy as np
    M, K = w.M, w.K
    a = torch.from_numpy(w.a_bits().view(np.int16)).view(torch.bfloat16).to("cuda")
    sets, graphs = rotation(2 * M * K, steps, min_bytes)
    big = torch.empty((sets, M, K), dtype=torch.bfloat16, device="cuda")
    big.copy_(a.unsqueeze(0).expand(sets, M, K))
    q = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    s_bytes = mx.mxfp4_shuffled_scale_bytes(M, K) if shuffled else M * (K // 32)
    sc = torch.empty(s_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(3):
            mx.mxfp4_quantize(big[i], M, K, q, sc, shuffled, stream=stream)
    stream.synchronize()
    gs = []
    for j in range(graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                mx.mxfp4_quantize(big[j * steps + i], M, K, q, sc, shuffled, stream=stream)
        gs.append(g)
    with torch.cuda.stream(stream):
        for g in gs:
            g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(samples):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            ev0.record(stream)
            for g in gs:
                g.replay()
            ev1.record(stream)
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) * 1e3 / sets)
    us = percentile(times, 50)
    nbytes = 2 * M * K + M * K // 2 + s_bytes
    del gs, big
    torch.cuda.empty_cache()
    return {"M": M, "K": K, "scales": "shuffled" if shuffled else "raw", "us_per_call": round(us, 3), "bytes": nbytes,
            "gbs": round(nbytes / (us * 1e-6) / 1e9, 1), "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "buffer_sets": sets}


CPU_SAMPLE_ROWS = 8  # rows of the headline workload's A in the oracle's sample


def _cpu_leg(rows, budget_s):
    """Whole calls of the oracle (quantize A, fp32 group-accumulated GEMM,
    bf16 rounding) on the first `rows` rows of the headline workload, until
    the budget is spent: (TFLOP/s, calls, seconds, threads)."""
    import oracle
    import synthetic as syn
    w = syn.CONFIGS[HEADLINE]
    qb, sb = oracle.quantize(w.b_bits())
    a = w.a_bits()[:rows].copy()
    oracle.mxfp4_gemm_bf16(a, qb, sb, f32acc=True)  # load + page in
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.mxfp4_gemm_bf16(a, qb, sb, f32acc=True)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return alg_flops(rows, w.N, w.K) * n / el / 1e12, n, el, oracle.num_threads()


def cpu_baseline(threads, budget_s=10.0):
    """The oracle as it stands, on the host's cores: all `threads` threads,
    then one thread (each leg in a child process, so its OpenMP thread count
    is fixed at start; neither touches the GPU)."""
    import synthetic as syn
    w = syn.CONFIGS[HEADLINE]
    legs = {}
    for nt in (threads, 1):
        code = ("import json, sys; sys.path.insert(0, %r); import bench; "
                "print(json.dumps(bench._cpu_leg(%d, %r)))" % (ROOT, CPU_SAMPLE_ROWS, budget_s))
        env = dict(os.environ, OMP_NUM_THREADS=str(nt), HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
        out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600,
                             check=True).stdout
        legs[nt] = json.loads(out.strip().splitlines()[-1])
    v, n, el, used = legs[threads]
    v1, n1, el1, _ = legs[1]
    sample = ("%d whole calls (quantize A + fp32 group-accumulated GEMM + bf16 rounding) on rows 0-%d of %s "
              "(%d x %d x %d), %.1f s" % (n, CPU_SAMPLE_ROWS - 1, w.name, CPU_SAMPLE_ROWS, w.N, w.K, el))
    return {"value": v, "unit": "TFLOP/s", "cores": used, "kind": "oracle", "sample": sample,
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_thread": {"value": v1, "unit": "TFLOP/s", "cores": 1,
                              "sample": "%d whole calls, %.1f s" % (n1, el1)}}


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
    WRITE_SIZE; KiB per dispatch) into HBM bytes per call: per kernel of the
    call (the library's kernels), the median over its dispatches, summed.
    Each counter is scaled by what it reads for a plain copy of known size
    (the largest copy of the run: the 256 MiB calibration copy)."""
    import synthetic as syn
    w = syn.CONFIGS[HEADLINE]
    med = lambda v: sorted(v)[len(v) // 2]

    def per_kernel(rows, counter):
        kern, copy = {}, []
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            name = r["Kernel_Name"]
            if "mxfp4::" in name:
                kern.setdefault(name.split("(")[0], []).append(v)
            elif "copyBuffer" in name:
                copy.append(v)
        # the calibration copy moves more bytes than any other copy of the run
        return kern, max(copy)

    fk, fc = per_kernel(_pmc_rows(fetch_dir), "FETCH_SIZE")
    wk, wc = per_kernel(_pmc_rows(write_dir), "WRITE_SIZE")
    f_scale = fc / CALIBRATION_BYTES  # counter bytes per byte copied
    w_scale = wc / CALIBRATION_BYTES
    # a call's kernels run once per call; the B preparation runs once per run
    most = max(len(v) for v in fk.values())
    kernels = {}
    for name in sorted(set(fk) | set(wk)):
        if len(fk.get(name, [])) < most / 2:
            continue
        kernels[name] = {"dispatches": [len(fk.get(name, [])), len(wk.get(name, []))],
                         "fetch_bytes": round(med(fk[name]) / f_scale) if name in fk else 0,
                         "write_bytes": round(med(wk[name]) / w_scale) if name in wk else 0}
    fetch = sum(k["fetch_bytes"] for k in kernels.values())
    write = sum(k["write_bytes"] for k in kernels.values())
    out = {"workload": w.name, "kernel_source_hash": kernel_source_hash(), "command": command, "kernels": kernels,
           "fetch_bytes_per_call": fetch, "write_bytes_per_call": write, "hbm_bytes_per_call": fetch + write,
           "algorithmic_bytes": alg_bytes(w.M, w.N, w.K), "copy_calibration": {"fetch": f_scale, "write": w_scale}}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def kernel_signature(w, quantized_a=False):
    """The GEMM kernel instantiation the library runs for a workload (with
    quantized_a: the call of mxfp4_gemm_q), as the profiler names it
    (without namespace): gemm_kernel<MT, NT, WN, WK, KPW, pre-quantized,
    staged rows, epilogue, phase stamps (always off)> or
    gemm_wide_kernel<MW, NW, W, D, LDS-staged B, phase stamps (always off)>,
    read off the schedule name."""
    import re
    import block_scaled_mxfp4_bf16_amd as mx
    name = (mx.mxfp4_gemm_q_schedule_name if quantized_a else mx.mxfp4_gemm_schedule_name)(w.M, w.N, w.K)
    m = re.match(r"(wide|widel)_mt(\d+)_nt(\d+)_w(\d+)_d(\d+)_split\d+$", name)
    if m:
        return "gemm_wide_kernel<%s, %s, %s, %s, %s, false>" % (m.group(2), m.group(3), m.group(4), m.group(5),
                                                               "true" if m.group(1) == "widel" else "false")
    m = re.match(r"mt(\d+)_nt(\d+)_wn(\d+)_wk(\d+)_kpw(\d+)_(split|streamk)\d+(.*)$", name)
    rest = m.group(7)
    epi = 2 if m.group(6) == "streamk" else (1 if rest.endswith("_at") else 0)
    return "gemm_kernel<%s, %s, %s, %s, %s, %s, %d, %d, false>" % (m.group(1), m.group(2), m.group(3), m.group(4), m.group(5),
                                                           "true" if "_pq" in rest else "false",
                                                           8 if "_r8" in rest else 16, epi)


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
    by_sig = {}
    for c in configs:
        w = syn.CONFIGS.get(c) or syn.EXTRA_SHAPES[c]
        by_sig.setdefault(kernel_signature(w), []).append((expected_mfma(w.M, w.N, w.K), w.name))
        # the bench times mxfp4_gemm_q on the five configurations only
        if c in syn.CONFIGS and kernel_signature(w, True) != kernel_signature(w):
            by_sig.setdefault(kernel_signature(w, True), []).append(
                (expected_mfma(w.M, w.N, w.K), w.name + " (A pre-quantized)"))

    def workload_of(kernel, inst):
        # the instantiation, then the instruction count where workloads share
        # one (a schedule whose waves x steps overrun K issues more)
        c = by_sig.get(kernel.replace("void ", "").split("mxfp4::")[-1], [])
        exact = [n for i, n in c if i == inst]
        return exact[0] if exact else (c[0][1] if len(c) == 1 else None)
    out = {"command": command, "kernels": []}
    for (name, grid), d in sorted(groups.items()):
        ds = list(d.values())
        inst = med([x.get("SQ_INSTS_MFMA", 0.0) for x in ds])
        busy = med([x.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for x in ds])
        ns = med([x["ns"] for x in ds])
        out["kernels"].append({
            "kernel": name, "grid": grid, "dispatches": len(ds),
            "workload": workload_of(name, int(inst)),
            "mfma_instructions": int(inst), "busy_simd_cycles": int(busy),
            "busy_cycles_per_instruction": round(busy / inst, 2) if inst else None,
            "duration_ns": ns, "matrix_busy_frac_at_2400MHz": round(busy / (1024 * 2.4 * ns), 4) if ns else None})
    print(json.dumps(out, indent=1))


PROBES_LIB = os.path.join(ROOT, "block_scaled_mxfp4_bf16_amd", "libmxfp4_probes.so")


def floors(torch, steps, samples, names):
    """Floors of this machine, measured with the probe library: one launch of
    an empty kernel; the least time to stream each workload's B (codes and
    padded scales) from memory in one launch of plain coalesced loads (cold
    rotation as for the GEMM, the best of several grid sizes); and the
    scaled FP4 matrix instructions' issue rate with the shader clock
    (s_memtime against the 100 MHz s_memrealtime) measured alongside.
    All timed as graph replays of `steps` launches, median over `samples`."""
    import ctypes
    L = ctypes.CDLL(PROBES_LIB)
    P, I = ctypes.c_void_p, ctypes.c_int
    L.mxfp4_probe_empty.argtypes = [P]
    L.mxfp4_probe_stream.argtypes = [P, ctypes.c_size_t, P, I, P]
    L.mxfp4_probe_mfma.argtypes = [P, P, I, I, P]
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream

    def graph_time(call, count):
        gs = []
        for j in range(count):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(steps):
                    call(j * steps + i)
            gs.append(g)
        with torch.cuda.stream(stream):
            for g in gs:
                g.replay()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
        with torch.cuda.stream(stream):
            for k in range(samples):
                ev[k][0].record(stream)
                gs[k % count].replay()
                ev[k][1].record(stream)
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 / steps for a, b in ev]
        return percentile(us, 50), percentile(us, 10), percentile(us, 90)

    out = {}
    med, p10, p90 = graph_time(lambda i: L.mxfp4_probe_empty(sh), 1)
    out["empty_kernel_us"] = {"median": round(med, 3), "p10": round(p10, 3), "p90": round(p90, 3)}
    print("[floors] empty kernel: %.3f us per launch" % med, file=sys.stderr, flush=True)
    sink = torch.empty(8192 * 256, dtype=torch.int32, device="cuda")
    out["stream_b_us"] = {}
    for name in names:
        w = workload(name)
        nbytes = w.N * w.K // 2 + ((w.N + 255) // 256 * 256) * ((w.K // 32 + 7) // 8 * 8)
        nbytes = (nbytes + 15) // 16 * 16
        sets, graphs = rotation(nbytes, steps)
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(sets)]
        best = None
        for wgs in (256, 512, 1024, 2048):
            if wgs * 256 * 16 > nbytes * 4:
                continue
            med, p10, p90 = graph_time(
                lambda i, wgs=wgs: L.mxfp4_probe_stream(bufs[i % sets].data_ptr(), nbytes, sink.data_ptr(), wgs, sh),
                graphs)
            if best is None or med < best[0]:
                best = (med, wgs)
        del bufs
        torch.cuda.empty_cache()
        out["stream_b_us"][w.name] = {"bytes": nbytes, "us": round(best[0], 3), "workgroups": best[1],
                                      "gbs": round(nbytes / (best[0] * 1e-6) / 1e9, 1)}
        print("[floors] stream %s B (%d bytes): %.3f us (%d workgroups)" % (w.name, nbytes, best[0], best[1]),
              file=sys.stderr, flush=True)
    out["mfma"] = []
    for wgs, iters in ((256, 4096), (1024, 1024)):
        o = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
        st = torch.zeros(wgs * 4, dtype=torch.int64, device="cuda")
        med, p10, p90 = graph_time(lambda i: L.mxfp4_probe_mfma(o.data_ptr(), st.data_ptr(), wgs, iters, sh), 1)
        t = st.view(wgs, 4).cpu().tolist()
        ticks = sorted(r[1] - r[0] for r in t)[wgs // 2]
        real = sorted(r[3] - r[2] for r in t)[wgs // 2]
        inst = wgs * 4 * iters * 8
        flops = inst * 65536
        out["mfma"].append({
            "workgroups": wgs, "waves_per_simd": wgs // 256, "instructions": inst, "us": round(med, 3),
            "tflops": round(flops / (med * 1e-6) / 1e12, 1),
            "shader_mhz": round(ticks / real * 100.0, 1) if real else None,
            "cycles_per_instruction_per_wave": round(ticks / (iters * 8), 2)})
        print("[floors] MFMA %d workgroups: %.3f us, %.0f TFLOP/s, shader clock %s MHz, %.2f cycles per "
              "instruction per wave" % (wgs, med, flops / (med * 1e-6) / 1e12, out["mfma"][-1]["shader_mhz"],
                                        out["mfma"][-1]["cycles_per_instruction_per_wave"]),
              file=sys.stderr, flush=True)
    return out


# The split-1 schedules the phase probe instantiates with stamps, by probe
# index: (workload, schedule name the library must pick for it).
# workload: (probe entry `which`, schedule, m tiles, subtiles, column waves per workgroup)
PHASE_PROBES = {"c1": (2, "mt1_nt2_wn1_wk4_kpw3_split1", 1, 2, 1), "c2": (0, "mt1_nt2_wn1_wk4_kpw1_split1", 1, 2, 1),
                "c3": (1, "mt1_nt1_wn1_wk14_kpw4_split1_r8", 1, 1, 1),
                "c4": (3, "mt1_nt2_wn4_wk4_kpw4_split1", 1, 2, 4)}
PHASE_NAMES = ["loads_issued", "a_staged", "products_done", "c_stores_issued", "c_stores_complete"]


def phases(torch, mx, steps, names=("c2", "c3")):
    """Where the time of one small-M call goes: the probe library's copy of
    the fused kernel (the library's code, built with its flags, plus six
    100 MHz real-time stamps per wave) runs the workload under the cold
    rotation of the GEMM timing, in graphs of `steps` calls.  Per wave the
    phases are entry -> loads issued -> A staged (A has arrived, been
    quantized and written to LDS) -> products done (B has arrived and the
    matrix instructions issued; with several K waves, the partial sums are in
    LDS) -> C stores issued -> C stores complete.  Reported: the medians and
    90th percentiles of each phase over all waves of the last graph's calls;
    the spread of wave entry times within a call (how long the launch takes
    to start every workgroup); the span from the first entry to the last
    completion; and the stamped calls' time per call from the graph replay,
    beside the library's own.  The stamped C is checked bit for bit against
    the library's."""
    import ctypes
    L = ctypes.CDLL(PROBES_LIB)
    P, I = ctypes.c_void_p, ctypes.c_int
    L.mxfp4_probe_phases.argtypes = [I, P, P, P, P, P, ctypes.c_size_t, I, I, I, I, P]
    L.mxfp4_probe_phases_waves.argtypes = [I]
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream
    out = {}
    for name in names:
        which, sched, mt, nt, wn = PHASE_PROBES[name]
        w = workload(name)
        M, N, K = w.M, w.N, w.K
        if mx.mxfp4_gemm_schedule_name(M, N, K) != sched:
            out[name] = {"skipped": "the library picks %s" % mx.mxfp4_gemm_schedule_name(M, N, K)}
            continue
        waves = L.mxfp4_probe_phases_waves(which)
        grid = (N // (16 * nt * wn)) * ((M + 16 * mt - 1) // (16 * mt))
        words = grid * waves * 8
        sets, graphs = rotation(set_bytes(M, N, K), steps)
        bufs = prepare(torch, mx, w, sets)
        stamps = [torch.zeros(words, dtype=torch.int64, device="cuda") for _ in range(steps)]
        ref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def call(i):
            A, Bw, Bs, C = bufs[i % sets]
            rc = L.mxfp4_probe_phases(which, A.data_ptr(), Bw.data_ptr(), Bs.data_ptr(), C.data_ptr(),
                                      stamps[i % steps].data_ptr(), words, M, N, K, 0, sh)
            if rc != 0:
                raise RuntimeError("phase probe %s: error %d" % (name, rc))

        with torch.cuda.stream(stream):
            mx.mxfp4_reserve(M, N, K, stream=stream)
            mx.mxfp4_gemm(bufs[0][0], bufs[0][1], bufs[0][2], ref, M, N, K, stream=stream)
            call(0)
        stream.synchronize()
        same = bool(torch.equal(ref.view(torch.int16), bufs[0][3].view(torch.int16)))

        def graph_us(fn):
            gs = []
            for j in range(graphs):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for i in range(steps):
                        fn(j * steps + i)
                gs.append(g)
            with torch.cuda.stream(stream):
                for g in gs:
                    g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                for g in gs:
                    g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / (graphs * steps)

        lib_us = graph_us(lambda i: mx.mxfp4_gemm(bufs[i % sets][0], bufs[i % sets][1], bufs[i % sets][2],
                                                  bufs[i % sets][3], M, N, K, stream=stream))
        stamped_us = graph_us(call)
        per_phase = [[] for _ in PHASE_NAMES]
        spread, span = [], []
        for st in stamps:
            t = st.view(grid * waves, 8)[:, :6].cpu().tolist()
            for r in t:
                for k in range(5):
                    per_phase[k].append((r[k + 1] - r[k]) * 0.01)
            spread.append((max(r[0] for r in t) - min(r[0] for r in t)) * 0.01)
            span.append((max(r[5] for r in t) - min(r[0] for r in t)) * 0.01)
        out[name] = {
            "schedule": sched, "workgroups": grid, "waves_per_workgroup": waves,
            "library_us_per_call": round(lib_us, 3), "stamped_us_per_call": round(stamped_us, 3),
            "c_matches_library": same,
            "wave_phase_us": {n: {"median": round(percentile(v, 50), 3), "p90": round(percentile(v, 90), 3),
                                  "min": round(min(v), 3), "max": round(max(v), 3)}
                              for n, v in zip(PHASE_NAMES, per_phase)},
            "entry_spread_us": {"median": round(percentile(spread, 50), 3), "p90": round(percentile(spread, 90), 3)},
            "first_entry_to_last_completion_us": {"median": round(percentile(span, 50), 3),
                                                  "p90": round(percentile(span, 90), 3)},
        }
        print("[phases] %s: %s" % (name, json.dumps(out[name])), file=sys.stderr, flush=True)
        del bufs, stamps
        torch.cuda.empty_cache()
    return out


WIDE_PHASE_SCHEDULE = "wide_mt4_nt7_w4_d2_split1"
WIDE_PHASE_NAMES = ["k_loop", "partials_in_lds", "sums_and_c_stores_issued", "c_stores_complete"]


def wide_phases(torch, mx, steps, name="c5"):
    """Where the time of a large-M call goes: the probe library runs the
    library's A quantization and its 64 x 112-tile K loop with five 100 MHz
    real-time stamps per wave (entry, K loop done, partial tiles in LDS, C
    stores issued, complete), two launches per call as the library does,
    under the cold rotation of the GEMM timing.  Reported per workgroup
    (medians and 90th percentiles over the last graph's calls): the K loop
    from the first wave's entry to the last wave's last product, the
    partial tiles' trip into LDS, the summing and C stores, and their
    completion; per call: the spread of workgroup entries and of K-loop
    ends, and the span from the first entry to the last completion; per
    XCD: the median completion time.  The stamped C is checked bit for bit
    against the library's."""
    import ctypes
    L = ctypes.CDLL(PROBES_LIB)
    P, I = ctypes.c_void_p, ctypes.c_int
    L.mxfp4_probe_wide_operand_bytes.argtypes = [I, I]
    L.mxfp4_probe_wide_operand_bytes.restype = ctypes.c_size_t
    L.mxfp4_probe_wide_quant.argtypes = [P, P, I, I, P]
    L.mxfp4_probe_wide_phases.argtypes = [P, P, P, P, P, ctypes.c_size_t, I, I, I, P]
    w = workload(name)
    M, N, K = w.M, w.N, w.K
    if mx.mxfp4_gemm_schedule_name(M, N, K) != WIDE_PHASE_SCHEDULE:
        return {"skipped": "the library picks %s" % mx.mxfp4_gemm_schedule_name(M, N, K)}
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream
    G = (N // 112) * ((M + 63) // 64)
    words = G * 4 * 8
    sets, graphs = rotation(set_bytes(M, N, K), steps)
    bufs = prepare(torch, mx, w, sets)
    aop = torch.zeros(L.mxfp4_probe_wide_operand_bytes(M, K), dtype=torch.uint8, device="cuda")
    stamps = [torch.zeros(words, dtype=torch.int64, device="cuda") for _ in range(steps)]
    ref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def call(i):
        A, Bw, Bs, C = bufs[i % sets]
        rc = L.mxfp4_probe_wide_quant(A.data_ptr(), aop.data_ptr(), M, K, sh)
        rc = rc or L.mxfp4_probe_wide_phases(aop.data_ptr(), Bw.data_ptr(), Bs.data_ptr(), C.data_ptr(),
                                             stamps[i % steps].data_ptr(), words, M, N, K, sh)
        if rc != 0:
            raise RuntimeError("wide phase probe: error %d" % rc)

    with torch.cuda.stream(stream):
        mx.mxfp4_reserve(M, N, K, stream=stream)
        mx.mxfp4_gemm(bufs[0][0], bufs[0][1], bufs[0][2], ref, M, N, K, stream=stream)
        call(0)
    stream.synchronize()
    same = bool(torch.equal(ref.view(torch.int16), bufs[0][3].view(torch.int16)))

    def graph_us(fn):
        gs = []
        for j in range(graphs):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(steps):
                    fn(j * steps + i)
            gs.append(g)
        with torch.cuda.stream(stream):
            for g in gs:
                g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for g in gs:
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (graphs * steps)

    lib_us = graph_us(lambda i: mx.mxfp4_gemm(bufs[i % sets][0], bufs[i % sets][1], bufs[i % sets][2],
                                              bufs[i % sets][3], M, N, K, stream=stream))
    stamped_us = graph_us(call)
    per_wg = {n: [] for n in WIDE_PHASE_NAMES}
    entry_spread, loop_end_spread, span = [], [], []
    xcd_end = {}
    for st in stamps:
        t = st.view(G, 4, 8)[:, :, :6].cpu().tolist()
        T0 = min(min(wv[0] for wv in wg) for wg in t)
        ends = []
        for wg in t:
            ent = min(wv[0] for wv in wg)
            le = max(wv[1] for wv in wg)
            per_wg["k_loop"].append((le - ent) * 0.01)
            per_wg["partials_in_lds"].append((max(wv[2] for wv in wg) - le) * 0.01)
            per_wg["sums_and_c_stores_issued"].append(percentile([wv[3] - wv[2] for wv in wg], 50) * 0.01)
            per_wg["c_stores_complete"].append(percentile([wv[4] - wv[3] for wv in wg], 50) * 0.01)
            ends.append(le)
            xcd_end.setdefault(int(wg[0][5]), []).append((max(wv[4] for wv in wg) - T0) * 0.01)
        entry_spread.append((max(min(wv[0] for wv in wg) for wg in t) - T0) * 0.01)
        loop_end_spread.append((max(ends) - min(ends)) * 0.01)
        span.append((max(max(wv[4] for wv in wg) for wg in t) - T0) * 0.01)
    q = lambda v: {"median": round(percentile(v, 50), 3), "p90": round(percentile(v, 90), 3)}
    out = {"workload": w.name, "schedule": WIDE_PHASE_SCHEDULE, "workgroups": G, "waves_per_workgroup": 4,
           "library_us_per_call": round(lib_us, 3), "stamped_us_per_call": round(stamped_us, 3),
           "c_matches_library": same,
           "workgroup_phase_us": {n: q(v) for n, v in per_wg.items()},
           "entry_spread_us": q(entry_spread), "k_loop_end_spread_us": q(loop_end_spread),
           "first_entry_to_last_completion_us": q(span),
           "median_completion_by_xcd_us": {str(x): round(percentile(v, 50), 3) for x, v in sorted(xcd_end.items())}}
    print("[phases] %s: %s" % (name, json.dumps(out)), file=sys.stderr, flush=True)
    del bufs, stamps
    torch.cuda.empty_cache()
    return out


def workload(name):
    import synthetic as syn
    return syn.CONFIGS.get(name) or syn.EXTRA_SHAPES[name]


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc":
        summarize_pmc(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-mfma":
        summarize_mfma(sys.argv[2], sys.argv[3].split(","), " ".join(sys.argv[4:]))
        return
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--samples", type=int, default=30, help="timed replays per configuration for the statistics")
    ap.add_argument("--configs", default="c1,c2,c3,c4,c5,p_4x2880x512,p_16x2112x7168,p_32x2880x512,p_256x3072x1536",
                    help="configurations measured under per_config (the headline is always measured)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-b-prep", action="store_true",
                    help="skip timing the one-launch B preparation and the standalone quantization of A")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the second, warm timing (one buffer set, so inputs stay in L2 and MALL)")
    ap.add_argument("--no-clocks", action="store_true", help="skip reading the GPU clocks with amd-smi")
    ap.add_argument("--no-gemm-q", action="store_true",
                    help="skip timing mxfp4_gemm_q (A quantized beforehand) on the five method workloads")
    ap.add_argument("--floors", action="store_true",
                    help="measure the machine's floors with the probe library instead (launch, B streaming, "
                         "matrix-instruction rate and clock, and the per-phase timing of the small-M kernel for "
                         "c2 and c3 and of the large-M kernel for c5 when listed) and print them as one JSON line")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="first run a cold 256 MiB device copy (for scaling HBM counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this operation is built and timed on a single MI355X "
              "(N-sharding of B across GPUs needs no collective and is not implemented); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(1)
    if args.steps < 1 or args.samples < 1:
        print("--steps and --samples must be at least 1", file=sys.stderr)
        sys.exit(1)

    clocks_before = None if args.no_clocks else gpu_clocks()
    import torch
    import block_scaled_mxfp4_bf16_amd as mx

    torch.cuda.set_device(0)
    if args.floors:
        names = [c for c in args.configs.split(",") if c]
        fl = floors(torch, args.steps, args.samples, names)
        fl["phases"] = phases(torch, mx, args.steps, [n for n in names if n in PHASE_PROBES])
        if "c5" in names:
            fl["phases"]["c5"] = wide_phases(torch, mx, args.steps)
        print(json.dumps({"floors": fl, "steps": args.steps, "samples": args.samples, "clocks": clocks_before}),
              flush=True)
        return
    if args.pmc_calibration:
        calibration_copy(torch)
    names = [c for c in args.configs.split(",") if c]
    if HEADLINE not in names:
        names.insert(0, HEADLINE)
    per = {}
    for name in names:
        w = workload(name)
        r = time_config(torch, mx, w, args.steps, args.warmup, args.samples, cold=True,
                        clocks_under_load=(name == HEADLINE and not args.no_clocks))
        if not args.no_warm:
            # context only: the same calls on one buffer set, inputs warm in L2 and MALL
            r["warm_us_per_call"] = time_config(torch, mx, w, args.steps, args.warmup, args.samples,
                                                cold=False)["us_per_call"]
        if not args.no_gemm_q and name in ("c1", "c2", "c3", "c4", "c5"):
            # context: the same product from an A quantized beforehand
            r["prequantized_a"] = time_config_q(torch, mx, w, args.steps, args.samples)
            print("[bench] %s from pre-quantized A (mxfp4_gemm_q): %.3f us/call cold, schedule %s"
                  % (w.name, r["prequantized_a"]["us_per_call"], r["prequantized_a"]["schedule"]),
                  file=sys.stderr, flush=True)
        per[w.name] = r
        print("[bench] %s: %.3f us/call cold (p10 %.3f, p90 %.3f%s), %.1f TFLOP/s, %.0f GB/s, %.1f%% of %s "
              "roofline, schedule %s"
              % (w.name, r["us_per_call"], r["us_p10"], r["us_p90"],
                 "" if args.no_warm else "; %.3f warm" % r["warm_us_per_call"], r["tflops"], r["alg_gbs"],
                 100 * r["roofline"]["frac"], r["roofline"]["bound"], r["schedule"]),
              file=sys.stderr, flush=True)

    hw = workload(HEADLINE)
    h = per[hw.name]
    print("[bench] kernel source hash %s" % kernel_source_hash(), file=sys.stderr, flush=True)
    rl = dict(h["roofline"])
    rl["traffic"] = measured_traffic()
    rl["timed"] = "whole call (every launch of one mxfp4_gemm), HIP events on the replay stream"
    line = {
        "metric": "us/call and TFLOPS per (M,N,K); % of HBM or MXFP4-MFMA roofline",
        "value": h["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["timed_us_per_call"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 (e2m1 x e2m1 scaled MFMA, f32 accumulate, bf16 out)",
        "data": "synthetic (Philox-4x32-10 + Box-Muller N(0,1) bf16, seeded)",
        "config": {"workload": hw.name, "M": hw.M, "N": hw.N, "K": hw.K, "cache": h["cache"],
                   "schedule": h["schedule"]},
        "us_per_call": h["us_per_call"],
        "us_p10": h["us_p10"],
        "us_p90": h["us_p90"],
        "roofline": rl,
        "per_config": per,
    }
    if not args.no_b_prep:
        # offline weight preparation (not part of a call): its own throughput
        line["b_prep"] = {}
        for name in ("c2", "c5"):
            w = workload(name)
            r = time_prepare_b(torch, mx, w)
            line["b_prep"][w.name] = r
            print("[bench] B prep %dx%d: %.2f us, %.0f GB/s (%.1f%% of HBM)" % (w.N, w.K, r["us_per_call"], r["gbs"],
                                                                           100 * r["hbm_frac"]),
                  file=sys.stderr, flush=True)
        # the standalone quantization of A (mxfp4_quantize), raw and with shuffled scales
        line["quantize_a"] = {}
        for name in ("c2", "c5"):
            w = workload(name)
            line["quantize_a"][w.name] = {}
            for shuffled in (False, True):
                r = time_quantize(torch, mx, w, shuffled)
                line["quantize_a"][w.name][r["scales"]] = r
                print("[bench] quantize A %dx%d (%s scales): %.2f us, %.0f GB/s (%.1f%% of HBM)"
                      % (w.M, w.K, r["scales"], r["us_per_call"], r["gbs"], 100 * r["hbm_frac"]), file=sys.stderr,
                      flush=True)
    if not args.no_clocks:
        line["clocks"] = {"before": clocks_before, "under_headline_load": h.get("clocks_under_load"),
                          "after": gpu_clocks()}
        mhz = load_sclk_mhz(h.get("clocks_under_load"))
        if mhz:
            # the matrix peak scales with the shader clock: the same fractions
            # against the peak at the clock measured under load
            line["clocks"]["sclk_under_load_mhz"] = round(mhz, 1)
            for r in per.values():
                r["mfma_frac_at_load_sclk"] = r["mfma_frac"] * NOMINAL_SCLK_MHZ / mhz
    if not args.no_cpu_baseline:
        threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
        line["cpu_baseline"] = cpu_baseline(threads)
        print("[bench] oracle on the host: %.4g TFLOP/s on %d threads, %.4g on one"
              % (line["cpu_baseline"]["value"], line["cpu_baseline"]["cores"],
                 line["cpu_baseline"]["single_thread"]["value"]), file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
