"""mxfp4_gemm_noalloc, the entry point that allocates nothing, against
mxfp4_gemm, both called through the C ABI.  Calls in a row on one GPU share
the library's scratch array: a large-M shape (its quantized A operand lives
in the scratch), then a smaller split-K shape (tickets and partial sums in
the scratch) twice, so the second of those also checks that the first left
its tickets at zero.  Each result must equal mxfp4_gemm's bit for bit (same
schedule, fixed summation order) and match the oracle within the method's
tolerance."""
import numpy as np
import pytest

import block_scaled_mxfp4_bf16_amd as mx
import oracle
import synthetic as syn
from tests.gpu_util import assert_close, bf16_dev_to_bits, prepare_b, to_dev_u16_as_bf16, to_dev_u8, torch_cuda

pytestmark = pytest.mark.gpu


def call_both(torch, M, N, K, seed):
    assert mx.mxfp4_gemm_workspace_bytes(M, N, K) > 0  # the schedule uses scratch
    a = syn.normal_bf16(seed, syn.STREAM_A, (M, K))
    b = syn.normal_bf16(seed, syn.STREAM_B, (N, K))
    qb, sb, bw, bs = prepare_b(b)
    A = to_dev_u16_as_bf16(torch, a)
    Bw = to_dev_u8(torch, bw)
    Bs = to_dev_u8(torch, bs)
    ref_c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    got_c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    L = mx.lib()
    stream = torch.cuda.current_stream().cuda_stream
    assert L.mxfp4_gemm(A.data_ptr(), Bw.data_ptr(), Bs.data_ptr(), ref_c.data_ptr(), M, N, K, stream) == 0
    assert L.mxfp4_gemm_noalloc(A.data_ptr(), Bw.data_ptr(), Bs.data_ptr(), got_c.data_ptr(), M, N, K, stream) == 0
    torch.cuda.synchronize()
    got = bf16_dev_to_bits(got_c)
    assert np.array_equal(got, bf16_dev_to_bits(ref_c)), "%dx%dx%d differs from mxfp4_gemm" % (M, N, K)
    qa, sa = oracle.quantize(a)
    assert_close(got, oracle.gemm_f64(qa, sa, qb, sb), "noalloc %dx%dx%d" % (M, N, K))
    return got


def test_noalloc_equals_gemm_on_consecutive_calls_second_smaller():
    torch = torch_cuda()
    assert mx.mxfp4_gemm_schedule_name(256, 4096, 7168).startswith("wide_")
    call_both(torch, 256, 4096, 7168, seed=31)
    assert "split4" in mx.mxfp4_gemm_schedule_name(16, 2112, 7168)
    first = call_both(torch, 16, 2112, 7168, seed=32)
    again = call_both(torch, 16, 2112, 7168, seed=32)
    assert np.array_equal(first, again)


def test_noalloc_refuses_what_does_not_fit():
    torch = torch_cuda()
    x = torch.zeros(16, dtype=torch.uint8, device="cuda")
    p = x.data_ptr()
    rc = mx.lib().mxfp4_gemm_noalloc(p, p, p, p, 4096, 4096, 8192, torch.cuda.current_stream().cuda_stream)
    assert rc == 3  # MXFP4_ERR_WORKSPACE, before anything is enqueued
