"""Time every compiled schedule that can serve a GEMM shape, on the GPU.

    python -m block_scaled_mxfp4_bf16_amd.tune 32x4096x512 [MxNxK ...] [--steps 50] [--top 10]
                                             [--confirm 3] [--json out.json] [--quantized-a]

For each shape: random bf16 A and B (B prepared with mxfp4_prepare_b), then
for each name from mxfp4_list_schedules, the calls are captured in HIP graphs
of `steps` calls and a full pass over them is replayed between events.  The
calls cycle, in order, through a multiple of `steps` copies of (A, B, scales,
C) totalling at least 1 GiB (4x the MALL), so every call reads its inputs
from HBM, as a call in a real workload would.  The best `top` are then re-timed
`confirm` times in alternation, with the built-in choice among them, so that
drift over the run cannot decide the ranking.  Pin the winner with
mxfp4_set_schedule_override(name).
"""
import argparse
import json
import math
import sys

import torch

import block_scaled_mxfp4_bf16_amd as mx


def prepare(M, N, K, quantized_a, steps, min_bytes=1 << 30, seed=0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    a = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn((N, K), generator=g, device="cuda").to(torch.bfloat16)
    bw, bs = mx.prepare_b(b)
    del b
    if quantized_a:
        aq, as_ = mx.quantize(a, shuffled_scales=True)
        a_in = (aq, as_)
        a_bytes = aq.numel() + as_.numel()
    else:
        a_in = (a,)
        a_bytes = 2 * M * K
    per_set = a_bytes + bw.numel() + bs.numel() + 2 * M * N
    need = math.ceil(min_bytes / per_set)
    sets = steps * math.ceil(need / steps)
    bufs = []
    for i in range(sets):
        clone = (lambda t: t) if i == 0 else (lambda t: t.clone())
        bufs.append(tuple(clone(t) for t in a_in) + (clone(bw), clone(bs),
                    torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
    torch.cuda.synchronize()
    return bufs


def call(M, N, K, quantized_a, buf, stream):
    if quantized_a:
        aq, as_, bw, bs, c = buf
        mx.mxfp4_gemm_q(aq, as_, bw, bs, c, M, N, K, stream=stream)
    else:
        a, bw, bs, c = buf
        mx.mxfp4_gemm(a, bw, bs, c, M, N, K, stream=stream)


def time_schedule(M, N, K, quantized_a, bufs, stream, name, steps):
    """Microseconds per call under schedule `name` (None: the built-in choice)."""
    mx.mxfp4_set_schedule_override(name)
    try:
        with torch.cuda.stream(stream):
            mx.mxfp4_reserve(M, N, K, stream=stream)
            for i in range(3):
                call(M, N, K, quantized_a, bufs[i % len(bufs)], stream)
        stream.synchronize()
        gs = []
        for j in range(len(bufs) // steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(steps):
                    call(M, N, K, quantized_a, bufs[j * steps + i], stream)
            gs.append(g)
        with torch.cuda.stream(stream):
            for g in gs:
                g.replay()  # the first replay uploads the graph
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for g in gs:
                g.replay()  # every set once, in order
            e1.record(stream)
        torch.cuda.synchronize()
        del gs
        return e0.elapsed_time(e1) * 1e3 / len(bufs)
    finally:
        mx.mxfp4_set_schedule_override(None)


def tune(M, N, K, quantized_a=False, steps=50, top=10, confirm=3, log=print, min_bytes=1 << 30):
    """Time every schedule for (M, N, K); see the module docstring.  The
    buffer sets total at least `min_bytes` (the default keeps every call's
    inputs out of the caches; smaller is for quick checks only)."""
    names = mx.mxfp4_list_schedules(M, N, K, quantized_a)
    if not names:
        raise ValueError("no schedule serves %dx%dx%d" % (M, N, K))
    builtin = (mx.mxfp4_gemm_q_schedule_name if quantized_a else mx.mxfp4_gemm_schedule_name)(M, N, K)
    bufs = prepare(M, N, K, quantized_a, steps, min_bytes)
    stream = torch.cuda.Stream()
    times = {}
    for i, n in enumerate(names):
        times[n] = time_schedule(M, N, K, quantized_a, bufs, stream, n, steps)
        if (i + 1) % 100 == 0:
            log("  %dx%dx%d: %d of %d schedules timed" % (M, N, K, i + 1, len(names)))
    ranked = sorted(times, key=times.get)
    finalists = ranked[:top] + ([builtin] if builtin not in ranked[:top] else [])
    again = {n: [] for n in finalists}
    for _ in range(confirm):
        for n in finalists:
            again[n].append(time_schedule(M, N, K, quantized_a, bufs, stream, n, steps))
    final = sorted(finalists, key=lambda n: sum(again[n]) / len(again[n]))
    res = {"shape": [M, N, K], "quantized_a": bool(quantized_a), "builtin": builtin, "times_us": times,
           "confirmed_us": {n: sum(v) / len(v) for n, v in again.items()}, "best": final[0]}
    b = res["confirmed_us"][builtin]
    log("%dx%dx%d%s: %d schedules; built-in %s %.3f us; best %s %.3f us (%.1f%% faster)"
        % (M, N, K, " (quantized A)" if quantized_a else "", len(names), builtin, b, final[0],
           res["confirmed_us"][final[0]], 100 * (1 - res["confirmed_us"][final[0]] / b)))
    for n in final:
        log("  %-40s %.3f%s" % (n, res["confirmed_us"][n], "  (built-in)" if n == builtin else ""))
    del bufs
    torch.cuda.empty_cache()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("shapes", nargs="+", help="MxNxK")
    ap.add_argument("--steps", type=int, default=50, help="calls per graph (the sets are a multiple of this)")
    ap.add_argument("--top", type=int, default=10)
    ap.add_argument("--confirm", type=int, default=3)
    ap.add_argument("--quantized-a", action="store_true", help="time mxfp4_gemm_q (A given as codes and scales)")
    ap.add_argument("--json", help="write every timing here")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        sys.exit("tune needs a GPU")
    out = []
    for shape in args.shapes:
        M, N, K = map(int, shape.lower().split("x"))
        out.append(tune(M, N, K, args.quantized_a, args.steps, args.top, args.confirm,
                        log=lambda s: print(s, flush=True)))
    if args.json:
        with open(args.json, "w") as f:
            json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
