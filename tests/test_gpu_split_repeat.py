"""The split-K epilogues under repetition.  Each case runs the GEMM 500
times in a row on the same inputs into the same output and compares every
result with the first, byte for byte, stopping at the first difference.
The ticketed and stream-K epilogues add their partial sums in a fixed
order, so any lost, stale or doubly counted partial, or a ticket not back
at zero, changes the bytes.  The first result is also checked against the
oracle.  Cases: the M=8 N=2112 K=7168 workload split over two workgroups,
the leaderboard's 16 x 2112 x 7168 at its built-in split of four, a large-M
split, and stream-K grids whose runs cross tile boundaries."""
import numpy as np
import pytest

import block_scaled_mxfp4_bf16_amd as mx
import oracle
import synthetic as syn
from tests.gpu_util import assert_close, bf16_dev_to_bits, prepare_b, to_dev_u16_as_bf16, to_dev_u8, torch_cuda

pytestmark = pytest.mark.gpu

REPEATS = 500
CASES = [("mt1_nt2_wn1_wk8_kpw4_split2_r8", 8, 2112, 7168),
         (None, 16, 2112, 7168),  # the built-in choice: split 4
         ("wide_mt4_nt4_w8_d3_split3", 100, 512, 4096),
         ("mt1_nt2_wn1_wk8_kpw4_streamk256_r8", 8, 2112, 7168),
         ("mt1_nt2_wn1_wk8_kpw2_streamk300", 16, 3072, 1536),
         ("mt1_nt1_wn2_wk4_kpw4_streamk97", 17, 128, 4160)]


@pytest.mark.parametrize("sched,M,N,K", CASES)
def test_split_epilogue_is_bit_stable_over_repeats(sched, M, N, K):
    torch = torch_cuda()
    a = syn.normal_bf16(M + K, syn.STREAM_A, (M, K))
    b = syn.normal_bf16(M + K, syn.STREAM_B, (N, K))
    qb, sb, bw, bs = prepare_b(b)
    A, Bw, Bs = to_dev_u16_as_bf16(torch, a), to_dev_u8(torch, bw), to_dev_u8(torch, bs)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mx.mxfp4_set_schedule_override(sched)
    try:
        name = mx.mxfp4_gemm_schedule_name(M, N, K)
        assert name is not None and ("split1" not in name), name
        mx.gemm(A, Bw, Bs, N, out=C)
        first = C.clone()
        torch.cuda.synchronize()
        for i in range(REPEATS - 1):
            mx.gemm(A, Bw, Bs, N, out=C)
            assert bool(torch.equal(C, first)), "%s %dx%dx%d: run %d differs from the first" % (name, M, N, K, i + 2)
    finally:
        mx.mxfp4_set_schedule_override(None)
    qa, sa = oracle.quantize(a)
    assert_close(bf16_dev_to_bits(first), oracle.gemm_f64(qa, sa, qb, sb), "%s %dx%dx%d" % (name, M, N, K))
