"""GPU parity of the fused GEMM against the oracle, element by element:
|C - C_ref| <= 1e-2 * |C_ref| + 1e-2 with C_ref the oracle's fp64 result on
the same seeded inputs; B is given to the GPU as the oracle prepared it."""
import numpy as np
import pytest

import block_scaled_mxfp4_bf16_amd as mx
import oracle
import synthetic as syn
from tests.gpu_util import (assert_close, bf16_dev_to_bits, bits_to_f64, prepare_b, to_dev_u16_as_bf16,
                            to_dev_u8, torch_cuda)

pytestmark = pytest.mark.gpu


class Case:
    def __init__(self, torch, a_bits, b_bits):
        self.torch = torch
        self.M, self.K = a_bits.shape
        self.N = b_bits.shape[0]
        self.a_bits = a_bits
        self.qb, self.sb, bw, bs = prepare_b(b_bits)
        self.A = to_dev_u16_as_bf16(torch, a_bits)
        self.Bw = to_dev_u8(torch, bw)
        self.Bs = to_dev_u8(torch, bs)

    def run(self):
        C = mx.gemm(self.A, self.Bw, self.Bs, self.N)
        self.torch.cuda.synchronize()
        return bf16_dev_to_bits(C)

    def ref(self):
        qa, sa = oracle.quantize(self.a_bits)
        return oracle.gemm_f64(qa, sa, self.qb, self.sb)

    def ref_sampled(self, ms, ns):
        qa, sa = oracle.quantize(self.a_bits)
        return oracle.gemm_f64_sampled(qa, sa, self.qb, self.sb, ms, ns)


def make(torch, M, N, K, seed):
    return Case(torch, syn.normal_bf16(seed, syn.STREAM_A, (M, K)), syn.normal_bf16(seed, syn.STREAM_B, (N, K)))


SMALL = [(1, 32, 64), (5, 64, 192), (16, 96, 256), (17, 160, 320), (33, 64, 512), (64, 128, 1024),
         (100, 96, 384), (8, 2112, 448), (3, 32, 1088), (48, 64, 128), (130, 224, 2112)]


@pytest.mark.parametrize("M,N,K", SMALL)
def test_small_shapes_match_oracle(M, N, K):
    torch = torch_cuda()
    c = make(torch, M, N, K, seed=M * 7 + N + K)
    assert_close(c.run(), c.ref(), "gemm %dx%dx%d" % (M, N, K))


def test_one_hot_b_reproduces_fused_quantization_exactly():
    """With B[n][k] = 1 at k = n, C[:, n] is the dequantized A column n: the
    fused in-register quantization must equal the oracle's bit for bit
    (the values are e2m1 times powers of two, exact in bf16)."""
    torch = torch_cuda()
    M, N, K = 24, 256, 256
    a = syn.normal_bf16(17, syn.STREAM_A, (M, K))
    a[3, 32:64] = 0  # a zero group
    a[5, 0:32] = 0x8000
    b = np.zeros((N, K), dtype=np.uint16)
    b[np.arange(N), np.arange(N)] = 0x3F80
    for mode in (0, 1):
        mx.mxfp4_set_quant_mode(mode)
        try:
            got = Case(torch, a, b).run()
        finally:
            mx.mxfp4_set_quant_mode(0)
        qa, sa = oracle.quantize(a)
        want = oracle.bf16_from_f64(oracle.dequantize(qa, sa)[:, :N])
        # -0.0 and +0.0 products sum to +0.0 in the matrix unit; compare values
        assert np.array_equal(bits_to_f64(got), bits_to_f64(want)), "mode %d" % mode


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_config_full_match(name):
    torch = torch_cuda()
    w = syn.CONFIGS[name]
    c = Case(torch, w.a_bits(), w.b_bits())
    assert_close(c.run(), c.ref(), name)


def test_config_c5_full_match():
    """M=256, N=7168, K=7168: all 1,835,008 outputs against the oracle's fp64
    product (the oracle runs its outputs in parallel; a few seconds)."""
    torch = torch_cuda()
    w = syn.CONFIGS["c5"]
    c = Case(torch, w.a_bits(), w.b_bits())
    assert_close(c.run(), c.ref(), "c5")


@pytest.mark.parametrize("name", list(syn.EXTRA_SHAPES))
def test_leaderboard_shapes(name):
    """The other leaderboard shapes on the pages, every output compared."""
    torch = torch_cuda()
    w = syn.EXTRA_SHAPES[name]
    c = Case(torch, w.a_bits(), w.b_bits())
    assert_close(c.run(), c.ref(), name)


# A spread over the compiled kernels: one and many waves along N and K,
# one and several steps per wave, single- and multi-workgroup K splits.
SCHEDULES = ["mt1_nt1_wn1_wk1_kpw1_split17", "mt1_nt1_wn1_wk4_kpw1_split5", "mt1_nt2_wn2_wk2_kpw2_split5",
             "mt1_nt1_wn4_wk4_kpw2_split3", "mt1_nt1_wn1_wk16_kpw2_split1", "mt2_nt1_wn4_wk2_kpw2_split5",
             "mt2_nt2_wn2_wk4_kpw1_split5", "mt4_nt1_wn8_wk1_kpw2_split9", "mt4_nt2_wn4_wk1_kpw2_split9",
             "mt4_nt1_wn2_wk4_kpw2_split3", "mt4_nt2_wn1_wk2_kpw2_split5",
             # pre-quantized mode: here bf16 A is quantized into the workspace by a launch of its
             # own, in the caller's layout, which the GEMM then reads
             "mt4_nt2_wn2_wk2_kpw4_split3_pq", "mt1_nt1_wn2_wk8_kpw1_split3_pq", "mt8_nt1_wn2_wk2_kpw4_split3_pq",
             "mt2_nt2_wn1_wk1_kpw4_split5_pq", "mt4_nt4_wn1_wk2_kpw4_split3_pq",
             # large-M kernel: waves split K, A quantized once
             "wide_mt4_nt2_w8_d2_split1", "wide_mt4_nt4_w8_d3_split3", "wide_mt8_nt2_w8_d2_split2"]


@pytest.mark.parametrize("sched", SCHEDULES)
def test_every_schedule_matches_oracle_and_is_deterministic(sched):
    torch = torch_cuda()
    c = make(torch, 40, 256, 2048 + 64, seed=3)
    mx.mxfp4_set_schedule_override(sched)
    try:
        if mx.mxfp4_gemm_schedule_name(c.M, c.N, c.K) is None:
            pytest.skip("schedule cannot cover this K")
        first = c.run()
        second = c.run()
    finally:
        mx.mxfp4_set_schedule_override(None)
    assert np.array_equal(first, second)
    assert_close(first, c.ref(), sched)


def test_hw_and_sw_encoders_give_identical_c():
    torch = torch_cuda()
    w = syn.CONFIGS["c4"]
    c = Case(torch, w.a_bits(), w.b_bits())
    hw = c.run()
    mx.mxfp4_set_quant_mode(1)
    try:
        sw = c.run()
    finally:
        mx.mxfp4_set_quant_mode(0)
    assert np.array_equal(hw, sw)


def test_gemm_ex_with_caller_workspace():
    """M=8 N=2112 K=7168 with K split over two workgroups (named: the
    built-in choice for this shape needs no workspace)."""
    torch = torch_cuda()
    w = syn.CONFIGS["c3"]
    c = Case(torch, w.a_bits(), w.b_bits())
    mx.mxfp4_set_schedule_override("mt1_nt2_wn1_wk8_kpw4_split2_r8")
    try:
        need = mx.mxfp4_gemm_workspace_bytes(c.M, c.N, c.K)
        assert need > 0
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        outs = []
        for _ in range(3):
            C = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
            mx.mxfp4_gemm_ex(c.A, c.Bw, c.Bs, C, c.M, c.N, c.K, ws, need)
            torch.cuda.synchronize()
            outs.append(bf16_dev_to_bits(C))
        assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
        assert np.array_equal(outs[0], c.run())
        # the tickets are left at zero for the next call
        assert int(ws[:65536].count_nonzero()) == 0
    finally:
        mx.mxfp4_set_schedule_override(None)
    assert_close(outs[0], c.ref(), "c3 through a caller workspace")


def test_single_split_default_needs_no_workspace():
    """The built-in choice at M=8 N=2112 K=7168 covers K in one workgroup
    per column tile: no workspace, and mxfp4_gemm_ex accepts none."""
    torch = torch_cuda()
    w = syn.CONFIGS["c3"]
    assert mx.mxfp4_gemm_workspace_bytes(w.M, w.N, w.K) == 0
    c = Case(torch, w.a_bits(), w.b_bits())
    C = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
    mx.mxfp4_gemm_ex(c.A, c.Bw, c.Bs, C, c.M, c.N, c.K, None, 0)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_dev_to_bits(C), c.run())


def test_reserve_then_repeated_calls_are_identical():
    torch = torch_cuda()
    c = make(torch, 16, 3072, 1536, seed=1)
    mx.mxfp4_reserve(c.M, c.N, c.K)
    runs = [c.run() for _ in range(5)]
    for r in runs[1:]:
        assert np.array_equal(r, runs[0])


def test_workspace_reused_across_shapes_with_more_tiles():
    """A split-K shape with few tiles and a large partial region, then one
    with more tiles on the same stream: the second one's tickets must not
    land on the first one's partial sums."""
    torch = torch_cuda()
    first = make(torch, 130, 224, 2112, seed=21)   # 21 tiles, 5 splits of 16x64-row tiles
    second = make(torch, 16, 3072, 1536, seed=22)  # 96 tiles, 3 splits
    assert_close(first.run(), first.ref(), "first shape")
    assert_close(second.run(), second.ref(), "second shape")
    assert_close(first.run(), first.ref(), "first shape again")


# The split-K epilogues the built-in choice never picks.  Stream-K: G
# workgroups, each an equal run of the tiles x K steps iterations; at
# 40x256x2112 with 32-column tiles there are 24 tiles x 17 steps = 408
# iterations, so G = 13 gives runs of 31-32 steps (whole tiles stored
# directly plus partial ones), 24 one whole tile each, 50 runs of 8-9 steps
# that cross tile boundaries; with 64-column tiles (12 tiles, 204
# iterations) G = 204 gives every tile 17 one-step contributors.
STREAMK_CASES = [("mt1_nt2_wn1_wk8_kpw4_streamk13", 40, 256, 2112), ("mt1_nt2_wn1_wk8_kpw4_streamk24", 40, 256, 2112),
                 ("mt1_nt2_wn1_wk8_kpw4_streamk50", 40, 256, 2112), ("mt1_nt1_wn4_wk4_kpw4_streamk204", 40, 256, 2112),
                 ("mt1_nt1_wn4_wk4_kpw4_streamk7_r8", 5, 256, 2112), ("mt1_nt2_wn1_wk8_kpw4_streamk256_r8", 8, 2112, 7168),
                 ("mt1_nt2_wn1_wk8_kpw2_streamk300", 16, 3072, 1536), ("mt1_nt2_wn4_wk4_kpw4_streamk256", 64, 7168, 2048),
                 ("mt1_nt1_wn2_wk4_kpw4_streamk97", 17, 128, 4160)]
# Float-atomic split-K: uneven splits, a half step at the end of K, rows past M.
ATOMIC_CASES = [("mt1_nt2_wn1_wk8_kpw4_split3_at", 40, 256, 2112), ("mt1_nt1_wn4_wk4_kpw4_split5_at", 33, 128, 4160),
                ("mt1_nt2_wn1_wk8_kpw4_split2_r8_at", 8, 2112, 7168), ("mt1_nt1_wn4_wk4_kpw4_split4_r8_at", 3, 128, 2112),
                ("mt1_nt2_wn1_wk4_kpw4_split4_at", 16, 2112, 7168)]


def run_forced(c, sched, times):
    mx.mxfp4_set_schedule_override(sched)
    try:
        assert mx.mxfp4_gemm_schedule_name(c.M, c.N, c.K) == sched
        return [c.run() for _ in range(times)]
    finally:
        mx.mxfp4_set_schedule_override(None)


@pytest.mark.parametrize("sched,M,N,K", STREAMK_CASES)
def test_streamk_matches_oracle_and_is_deterministic(sched, M, N, K):
    torch = torch_cuda()
    c = make(torch, M, N, K, seed=M + N + K + 5)
    runs = run_forced(c, sched, 3)
    assert np.array_equal(runs[0], runs[1]) and np.array_equal(runs[0], runs[2])
    assert_close(runs[0], c.ref(), "%s %dx%dx%d" % (sched, M, N, K))


@pytest.mark.parametrize("sched,M,N,K", ATOMIC_CASES)
def test_atomic_split_matches_oracle(sched, M, N, K):
    """Every run within tolerance of the oracle; runs may differ in the
    last bits, since the atomics add in arrival order.  In between, a
    ticketed split-K call on another shape leaves its partial sums in the
    same workspace: the zero-fill launch must clear them."""
    torch = torch_cuda()
    c = make(torch, M, N, K, seed=M + N + K + 6)
    ref = c.ref()
    for r in run_forced(c, sched, 2):
        assert_close(r, ref, sched)
    other = make(torch, 40, 256, 2112, seed=8)
    for r in run_forced(other, "mt1_nt1_wn1_wk4_kpw1_split17", 1):
        assert_close(r, other.ref(), "ticketed split between atomic runs")
    for r in run_forced(c, sched, 1):
        assert_close(r, ref, sched + " after another shape")


@pytest.mark.parametrize("sched,M,N,K", [STREAMK_CASES[2], STREAMK_CASES[5], ATOMIC_CASES[0], ATOMIC_CASES[2]])
def test_split_epilogues_in_an_exact_caller_workspace(sched, M, N, K):
    """mxfp4_gemm_ex with a workspace of exactly the size the library asks
    for, its partial-sum region filled with non-zero bytes."""
    torch = torch_cuda()
    c = make(torch, M, N, K, seed=M + N + K + 7)
    mx.mxfp4_set_schedule_override(sched)
    try:
        need = mx.mxfp4_gemm_workspace_bytes(M, N, K)
        ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
        ws[:65536] = 0
        C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        mx.mxfp4_gemm_ex(c.A, c.Bw, c.Bs, C, M, N, K, ws, need)
        torch.cuda.synchronize()
    finally:
        mx.mxfp4_set_schedule_override(None)
    assert_close(bf16_dev_to_bits(C), c.ref(), sched)
    assert int(ws[:65536].count_nonzero()) == 0  # tickets left at zero


RAGGED_SCHEDULES = ["wide_mt4_nt7_w4_d2_split1", "wide_mt8_nt2_w8_d2_split2", "widel_mt4_nt7_w4_d3_split1"]


@pytest.mark.parametrize("sched", RAGGED_SCHEDULES)
def test_k_loop_kernels_ragged(sched):
    """K loop with a step count that is not a multiple of the prefetch depth
    or of the waves, a half step (K % 128 == 64), and rows past the last
    full row tile."""
    torch = torch_cuda()
    c = make(torch, 70, 224, 1088, seed=9)
    mx.mxfp4_set_schedule_override(sched)
    try:
        assert mx.mxfp4_gemm_schedule_name(c.M, c.N, c.K) == sched
        got = c.run()
        again = c.run()
    finally:
        mx.mxfp4_set_schedule_override(None)
    assert np.array_equal(got, again)
    assert_close(got, c.ref(), sched)


R8_SCHEDULES = ["mt1_nt1_wn1_wk16_kpw4_split1_r8", "mt1_nt1_wn2_wk8_kpw2_split2_r8", "mt1_nt2_wn1_wk8_kpw4_split1_r8",
                "mt1_nt1_wn1_wk4_kpw1_split5_r8", "mt1_nt1_wn4_wk4_kpw4_split2_r8", "mt1_nt1_wn1_wk1_kpw4_split5_r8"]


@pytest.mark.parametrize("sched", R8_SCHEDULES)
@pytest.mark.parametrize("M", [1, 5, 8])
def test_eight_row_staging_matches_oracle(sched, M):
    """A staged in 8-row blocks (rows 8..15 of the matrix operand fed as
    zeros), with a half step at the end of K and a split that is uneven."""
    torch = torch_cuda()
    c = make(torch, M, 256, 2048 + 64, seed=40 + M)
    mx.mxfp4_set_schedule_override(sched)
    try:
        assert mx.mxfp4_gemm_schedule_name(c.M, c.N, c.K) == sched
        first = c.run()
        second = c.run()
    finally:
        mx.mxfp4_set_schedule_override(None)
    assert np.array_equal(first, second)
    assert_close(first, c.ref(), "%s M=%d" % (sched, M))


# Large-M kernel: (schedule, M, N, K) with partial row tiles, row tiles past
# the quantized quads, half steps at the end of K, and uneven K splits.
WIDE_CASES = [("wide_mt4_nt7_w8_d2_split1", 130, 224, 1088), ("wide_mt4_nt7_w4_d2_split3", 70, 448, 2112),
              ("wide_mt8_nt2_w8_d2_split2", 200, 128, 1600), ("wide_mt8_nt2_w8_d2_split1", 129, 96, 640),
              ("wide_mt4_nt3_w8_d3_split1", 256, 192, 512), ("wide_mt4_nt6_w8_d2_split4", 96, 192, 4096),
              ("wide_mt4_nt2_w8_d4_split1", 17, 64, 256), ("wide_mt4_nt4_w8_d3_split1", 256, 512, 1024),
              ("wide_mt4_nt8_w8_d2_split5", 80, 256, 2112), ("wide_mt4_nt1_w8_d4_split3", 64, 96, 448),
              ("wide_mt8_nt3_w8_d2_split1", 140, 96, 8192), ("wide_mt4_nt4_w8_d2_split2", 66, 64, 64),
              # B staged through a per-wave LDS ring: a partial first round, several
              # full rounds, uneven splits
              ("widel_mt4_nt7_w4_d4_split1", 130, 224, 1088), ("widel_mt4_nt7_w4_d3_split3", 70, 448, 2112),
              ("widel_mt4_nt4_w8_d2_split1", 256, 512, 1024), ("widel_mt4_nt2_w8_d4_split2", 96, 192, 4096),
              ("widel_mt4_nt8_w4_d3_split1", 80, 256, 8192), ("widel_mt4_nt7_w4_d4_split1", 200, 448, 7168)]


@pytest.mark.parametrize("sched,M,N,K", WIDE_CASES)
def test_wide_kernel_matches_oracle(sched, M, N, K):
    torch = torch_cuda()
    c = make(torch, M, N, K, seed=M + N + K)
    mx.mxfp4_set_schedule_override(sched)
    try:
        assert mx.mxfp4_gemm_schedule_name(c.M, c.N, c.K) == sched
        first = c.run()
        second = c.run()
    finally:
        mx.mxfp4_set_schedule_override(None)
    assert np.array_equal(first, second)
    assert_close(first, c.ref(), "%s %dx%dx%d" % (sched, M, N, K))


# Calls captured into a HIP graph: the default small-M path, ticketed split K
# (tickets must be back at zero after every replay), the float-atomic
# epilogue (its zero fill is a kernel node), and the two-launch large-M path.
GRAPH_CASES = [(None, 32, 4096, 512), ("mt1_nt2_wn1_wk8_kpw4_split2_r8", 8, 2112, 7168),
               ("mt1_nt1_wn4_wk4_kpw4_split4", 16, 512, 4096), ("mt1_nt2_wn1_wk8_kpw4_split2_at", 16, 256, 7168),
               ("wide_mt4_nt7_w4_d2_split3", 130, 448, 2112)]


@pytest.mark.parametrize("sched,M,N,K", GRAPH_CASES)
def test_graph_replays_match_eager(sched, M, N, K):
    """Several calls captured in one graph, replayed four times with the
    program's own eager work and synchronizations in between; every replay's
    C equals the eager call's bit for bit (the atomic epilogue: within the
    tolerance, its addition order varies) and the oracle's within tolerance."""
    torch = torch_cuda()
    c = make(torch, M, N, K, seed=M + K)
    mx.mxfp4_set_schedule_override(sched)
    try:
        if sched is not None:
            assert mx.mxfp4_gemm_schedule_name(M, N, K) == sched
        stream = torch.cuda.Stream()
        outs = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
        with torch.cuda.stream(stream):
            mx.mxfp4_reserve(M, N, K, stream=stream)
            mx.mxfp4_gemm(c.A, c.Bw, c.Bs, outs[0], M, N, K, stream=stream)
        stream.synchronize()
        eager = bf16_dev_to_bits(outs[0])
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for C in outs:
                mx.mxfp4_gemm(c.A, c.Bw, c.Bs, C, M, N, K, stream=stream)
        exact = sched is None or not sched.endswith("_at")
        for rep in range(4):
            for C in outs:
                C.fill_(float("nan"))  # eager work between replays; a replay must overwrite all of C
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                g.replay()
            stream.synchronize()
            other = c.run()  # an eager call on the default stream between replays
            for i, C in enumerate(outs):
                got = bf16_dev_to_bits(C)
                if exact:
                    assert np.array_equal(got, eager), (sched, rep, i)
                else:
                    assert_close(got, bits_to_f64(eager), "%s replay %d call %d" % (sched, rep, i))
            if exact:
                assert np.array_equal(other, eager)
        del g
    finally:
        mx.mxfp4_set_schedule_override(None)
    assert_close(eager, c.ref(), "graph case %s %dx%dx%d" % (sched, M, N, K))


# A quantized once, handed to the GEMM: (schedule or None for the default, M, N, K)
GEMM_Q_CASES = [("mt4_nt1_wn2_wk4_kpw4_split1_pq", 64, 7168, 2048), ("mt1_nt1_wn1_wk8_kpw4_split2_pq", 8, 2112, 7168),
                ("mt2_nt1_wn1_wk1_kpw4_split1_pq", 32, 4096, 512), ("mt4_nt2_wn2_wk2_kpw4_split3_pq", 40, 256, 2112),
                ("wide_mt4_nt7_w4_d2_split1", 130, 224, 1088), ("wide_mt8_nt2_w8_d2_split2", 200, 128, 1600),
                ("wide_mt4_nt1_w8_d4_split3", 65, 96, 448), ("widel_mt4_nt7_w4_d4_split1", 130, 224, 1088),
                # eight waves of eight steps: ragged rows and a half step at the end of K,
                # and a K split whose second part starts on an odd step
                ("mt1_nt1_wn1_wk8_kpw8_split1_pq", 5, 640, 1088), ("mt1_nt1_wn1_wk8_kpw8_split2_pq", 13, 224, 7488)]


@pytest.mark.parametrize("sched,M,N,K", GEMM_Q_CASES)
def test_gemm_q_equals_gemm_under_the_same_schedule(sched, M, N, K):
    """Quantizing A with mxfp4_quantize and calling mxfp4_gemm_q gives the
    same bits as mxfp4_gemm on the bf16 A under the same schedule: the
    operand bytes are identical and so is the arithmetic."""
    torch = torch_cuda()
    c = make(torch, M, N, K, seed=3 * M + N + K)
    aq, as_ = mx.quantize(c.A, shuffled_scales=True)
    mx.mxfp4_set_schedule_override(sched)
    try:
        assert mx.mxfp4_gemm_q_schedule_name(M, N, K) == sched
        cq = bf16_dev_to_bits(mx.gemm_q(aq, as_, c.Bw, c.Bs, N))
        cf = c.run()
    finally:
        mx.mxfp4_set_schedule_override(None)
    assert np.array_equal(cq, cf)
    assert_close(cq, c.ref(), sched)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"] + list(syn.EXTRA_SHAPES))
def test_gemm_q_default_schedule_on_oracle_quantized_a(name):
    """mxfp4_gemm_q fed the oracle's own quantized A (codes and shuffled
    scales) under its default schedule matches the oracle's product, every
    output compared."""
    torch = torch_cuda()
    w = syn.CONFIGS.get(name) or syn.EXTRA_SHAPES[name]
    c = Case(torch, w.a_bits(), w.b_bits())
    qa, sa = oracle.quantize(c.a_bits)
    aq = to_dev_u8(torch, qa)
    as_ = to_dev_u8(torch, oracle.shuffle_scales(sa, c.M, c.K))
    assert mx.mxfp4_gemm_q_schedule_name(c.M, c.N, c.K).endswith("_pq")
    got = bf16_dev_to_bits(mx.gemm_q(aq, as_, c.Bw, c.Bs, c.N))
    torch.cuda.synchronize()
    assert_close(got, c.ref(), name)


# Shapes outside the tuned table: the default schedule choice for small,
# ragged and large M, long and half-step K, narrow and odd-tile N.
DEFAULT_SHAPES = [(1, 32, 64), (3, 96, 4160), (17, 288, 448), (48, 1024, 1024), (65, 96, 192), (100, 224, 2112),
                  (300, 64, 1088), (513, 288, 640), (64, 32, 8192),
                  # above 64 rows the estimated-time choice between the kernel families: the
                  # large-M kernel, a fused one (ragged M), 256-column fused tiles
                  (192, 2048, 4096), (129, 3584, 2048), (160, 4096, 2048)]


def _random_shapes(n, seed=2026, max_mnk=1.5e9):
    """Seeded shapes for the built-in choice off the tuned table: M 1-300, N a
    multiple of 32 up to 4096, K a multiple of 64 up to 8192, small enough
    for the oracle to finish in a fraction of a second each."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.integers(1, 301))
        N = 32 * int(rng.integers(1, 129))
        K = 64 * int(rng.integers(1, 129))
        if M * N * K <= max_mnk:
            out.append((M, N, K))
    return out


RANDOM_SHAPES = _random_shapes(24)


@pytest.mark.parametrize("M,N,K", RANDOM_SHAPES)
def test_builtin_choice_on_random_shapes_matches_oracle(M, N, K):
    """Whatever schedule the built-in choice picks (table, cost model, large-M
    kernel), mxfp4_gemm and mxfp4_gemm_q match the oracle on every output."""
    torch = torch_cuda()
    c = make(torch, M, N, K, seed=M + 7 * N + 13 * K)
    ref = c.ref()
    assert_close(c.run(), ref, "gemm %dx%dx%d (%s)" % (M, N, K, mx.mxfp4_gemm_schedule_name(M, N, K)))
    aq, as_ = mx.quantize(c.A, shuffled_scales=True)
    got_q = bf16_dev_to_bits(mx.gemm_q(aq, as_, c.Bw, c.Bs, N))
    assert_close(got_q, ref, "gemm_q %dx%dx%d (%s)" % (M, N, K, mx.mxfp4_gemm_q_schedule_name(M, N, K)))


@pytest.mark.parametrize("M,N,K", DEFAULT_SHAPES)
def test_default_schedules_match_oracle(M, N, K):
    torch = torch_cuda()
    c = make(torch, M, N, K, seed=5 * M + 3 * N + K)
    ref = c.ref()
    assert_close(c.run(), ref, "gemm %dx%dx%d (%s)" % (M, N, K, mx.mxfp4_gemm_schedule_name(M, N, K)))
    aq, as_ = mx.quantize(c.A, shuffled_scales=True)
    got_q = bf16_dev_to_bits(mx.gemm_q(aq, as_, c.Bw, c.Bs, N))
    assert_close(got_q, ref, "gemm_q %dx%dx%d (%s)" % (M, N, K, mx.mxfp4_gemm_q_schedule_name(M, N, K)))
    need = mx.mxfp4_gemm_workspace_bytes(M, N, K)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mx.mxfp4_gemm_ex(c.A, c.Bw, c.Bs, C, M, N, K, ws if need else None, need)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_dev_to_bits(C), c.run())


def test_tuner_times_every_listed_schedule():
    """The tuning module on a small shape: every listed schedule is timed,
    the finalists include the built-in choice, and the best one is listed."""
    torch_cuda()
    from block_scaled_mxfp4_bf16_amd import tune
    res = tune.tune(16, 256, 512, steps=10, top=2, confirm=1, log=lambda s: None, min_bytes=4 << 20)
    names = mx.mxfp4_list_schedules(16, 256, 512)
    assert set(res["times_us"]) == set(names)
    assert all(t > 0 for t in res["times_us"].values())
    assert res["builtin"] in res["confirmed_us"] and res["best"] in names
    assert mx.mxfp4_gemm_schedule_name(16, 256, 512) == res["builtin"]  # the override is cleared afterwards


def test_long_k_at_few_rows_uses_the_large_m_kernel_sampled():
    """M=40 N=3584 K=14336: the estimated-time choice takes the large-M
    kernel below 64 rows when K is long and N wide; sampled outputs against
    the oracle one by one, every row tile and a spread of columns."""
    torch = torch_cuda()
    M, N, K = 40, 3584, 14336
    assert mx.mxfp4_gemm_schedule_name(M, N, K).startswith("wide_")
    c = make(torch, M, N, K, seed=77)
    got = c.run()
    rng = np.random.default_rng(7)
    ms = np.concatenate([np.arange(M), rng.integers(0, M, 1200)])
    ns = np.concatenate([rng.integers(0, N, M), rng.integers(0, N, 1200)])
    assert_close(got[ms, ns], c.ref_sampled(ms, ns), "40x3584x14336 sampled")


def test_tuner_with_quantized_a():
    """The tuning module in its pre-quantized-A mode (mxfp4_gemm_q): every
    listed pre-quantized schedule is timed and the built-in one is among the
    finalists."""
    torch_cuda()
    from block_scaled_mxfp4_bf16_amd import tune
    res = tune.tune(32, 256, 1024, quantized_a=True, steps=10, top=1, confirm=1, log=lambda s: None,
                    min_bytes=4 << 20)
    assert set(res["times_us"]) == set(mx.mxfp4_list_schedules(32, 256, 1024, True))
    assert res["builtin"] == mx.mxfp4_gemm_q_schedule_name(32, 256, 1024)
    assert res["builtin"] in res["confirmed_us"]


# Tiles with an odd number of 16-column subtiles per wave (every other tile
# starts on an odd column group, whose B scales sit in the upper half of a
# scale dword) and 32 x 96 tiles; split K, rows past M and a final half step.
ODD_TILE_CASES = [("mt1_nt7_wn1_wk4_kpw4_split1", 64, 7168, 2048), ("mt1_nt7_wn1_wk8_kpw2_split2", 20, 448, 2112),
                  ("mt1_nt7_wn1_wk16_kpw1_split1", 5, 224, 1024), ("mt1_nt7_wn1_wk2_kpw8_split3", 17, 448, 4160),
                  ("mt2_nt6_wn1_wk4_kpw3_split1", 256, 3072, 1536), ("mt2_nt3_wn2_wk4_kpw3_split2", 40, 288, 1600),
                  ("mt2_nt6_wn1_wk6_kpw2_split1", 33, 192, 1536), ("mt2_nt3_wn2_wk2_kpw6_split1", 70, 96, 1536),
                  ("mt2_nt2_wn3_wk4_kpw3_split1", 256, 3072, 1536), ("mt2_nt1_wn6_wk2_kpw6_split1", 40, 192, 1536),
                  ("mt1_nt1_wn7_wk2_kpw8_split2", 9, 224, 4096), ("mt2_nt2_wn3_wk3_kpw4_split2", 31, 96, 2112)]


@pytest.mark.parametrize("sched,M,N,K", ODD_TILE_CASES)
def test_odd_and_wide_tiles_match_oracle(sched, M, N, K):
    torch = torch_cuda()
    c = make(torch, M, N, K, seed=M + N + K + 9)
    mx.mxfp4_set_schedule_override(sched)
    try:
        assert mx.mxfp4_gemm_schedule_name(M, N, K) == sched
        first = c.run()
        second = c.run()
    finally:
        mx.mxfp4_set_schedule_override(None)
    assert np.array_equal(first, second)
    assert_close(first, c.ref(), "%s %dx%dx%d" % (sched, M, N, K))


def test_concurrent_streams_keep_separate_workspaces():
    """Two streams run a split-K shape (16 x 2112 x 7168 splits K four ways,
    so every call uses its stream's tickets and partial tiles) interleaved,
    with no synchronization between the streams; every result equals the
    one computed alone, bit for bit, and that one is within the tolerance of
    the oracle."""
    torch = torch_cuda()
    M, N, K = 16, 2112, 7168
    assert "split4" in mx.mxfp4_gemm_schedule_name(M, N, K)
    cases = [make(torch, M, N, K, seed=31), make(torch, M, N, K, seed=32)]
    cases[1].Bw, cases[1].Bs, cases[1].qb, cases[1].sb = cases[0].Bw, cases[0].Bs, cases[0].qb, cases[0].sb
    alone = [c.run() for c in cases]
    mm, nn = (g.ravel() for g in np.meshgrid(np.arange(0, M, 3), np.arange(0, N, 97), indexing="ij"))
    for j, (c, a) in enumerate(zip(cases, alone)):
        assert_close(a[mm, nn], c.ref_sampled(mm, nn), "stream case %d sampled" % j)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for c, s in zip(cases, streams):
        mx.mxfp4_reserve(M, N, K, stream=s)
    torch.cuda.synchronize()
    outs = [[torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(20)] for _ in cases]
    for i in range(20):
        for j, (c, s) in enumerate(zip(cases, streams)):
            mx.mxfp4_gemm(c.A, c.Bw, c.Bs, outs[j][i], M, N, K, stream=s)
    torch.cuda.synchronize()
    for j in range(2):
        for i in range(20):
            assert np.array_equal(bf16_dev_to_bits(outs[j][i]), alone[j]), (j, i)
