"""GPU parity at the edges of the size range the C ABI accepts.  Every
operand stays below 2^31 bytes (the kernels address memory with 32-bit
offsets): here the largest A and the largest C, through the quantizer, the
GEMM and the pre-quantized GEMM, and a K too long for the fused small-M
kernels (the large-M kernel, which loops over K, serves it).  Expected
values come from the oracle on the same host bytes, on sampled rows or
outputs where the whole product is too big to compute on the CPU."""
import numpy as np
import pytest

import block_scaled_mxfp4_bf16_amd as mx
import oracle
import synthetic as syn
from tests.gpu_util import assert_close, bf16_dev_to_bits, prepare_b, to_dev_u16_as_bf16, to_dev_u8, torch_cuda

pytestmark = pytest.mark.gpu


def large_a(M, K, seed):
    """[M, K] bf16 bits: a seeded N(0,1) block of 1024 rows, repeated; in
    copy c (rows 1024c ...) the 32-element groups that a hash of (c, row,
    group) selects change sign, so rows 1024 apart differ in about half of
    their groups and a row read from the wrong place shows."""
    block = syn.normal_bf16(seed, syn.STREAM_A, (1024, K))
    G = K // 32
    r = np.arange(1024, dtype=np.uint64)[:, None] + np.uint64(1)
    g = np.arange(G, dtype=np.uint64)[None, :] + np.uint64(1)
    out = np.empty((M, K), dtype=np.uint16)
    for c in range((M + 1023) // 1024):
        h = (r * np.uint64(0x9E3779B1) + g * np.uint64(0x85EBCA77) + np.uint64(c + 1) * np.uint64(0xC2B2AE3D))
        flip = (((h & np.uint64(0xFFFFFFFF)) >> np.uint64(16)) & np.uint64(1)).astype(np.uint16) * np.uint16(0x8000)
        n = min(1024, M - 1024 * c)
        out[1024 * c:1024 * c + n] = block[:n] ^ np.repeat(flip[:n], 32, axis=1)
    return out


def test_largest_a():
    """M x K x 2 = 2^31 - 65536 bytes of A (the largest multiple-of-64 K for
    M = 32767 below 2^31 bytes): quantize, the default GEMM and the
    pre-quantized GEMM, checked on sampled rows, including the last."""
    torch = torch_cuda()
    M, N, K = 32767, 32, 32768
    assert M * K * 2 < 2 ** 31
    a = large_a(M, K, seed=31)
    b = syn.normal_bf16(32, syn.STREAM_B, (N, K))
    qb, sb, bw, bs = prepare_b(b)
    rows = np.array([0, 1, 15, 16, 1023, 1024, 8191, 16383, 16384, 24575, 32704, 32765, 32766]
                    + list(np.random.default_rng(3).integers(0, M, 19)), dtype=np.int64)
    qa, sa = oracle.quantize(a[rows])
    ref = oracle.gemm_f64(qa, sa, qb, sb)
    A = to_dev_u16_as_bf16(torch, a)
    del a
    Bw, Bs = to_dev_u8(torch, bw), to_dev_u8(torch, bs)
    idx = torch.from_numpy(rows).cuda()
    print("largest A: %s" % mx.mxfp4_gemm_schedule_name(M, N, K), flush=True)
    C = mx.gemm(A, Bw, Bs, N)
    torch.cuda.synchronize()
    assert_close(bf16_dev_to_bits(C[idx]), ref, "gemm, largest A")
    del C
    q, s = mx.quantize(A)
    torch.cuda.synchronize()
    assert np.array_equal(q[idx].cpu().numpy(), qa) and np.array_equal(s[idx].cpu().numpy(), sa)
    del q, s
    aq, as_ = mx.quantize(A, shuffled_scales=True)
    del A
    Cq = mx.gemm_q(aq, as_, Bw, Bs, N)
    torch.cuda.synchronize()
    assert_close(bf16_dev_to_bits(Cq[idx]), ref, "gemm_q, largest A")


def test_largest_c():
    """M x N x 2 = 2,145,320,... bytes of C, the largest 32-column multiple
    below 2^31 bytes for M = 32767; sampled outputs, including the last row
    and column."""
    torch = torch_cuda()
    M, N, K = 32767, 32736, 64
    assert M * N * 2 < 2 ** 31
    a = syn.normal_bf16(33, syn.STREAM_A, (M, K))
    b = syn.normal_bf16(33, syn.STREAM_B, (N, K))
    qb, sb, bw, bs = prepare_b(b)
    qa, sa = oracle.quantize(a)
    rng = np.random.default_rng(4)
    ms = np.concatenate([[0, M - 1, M - 1, 0, 16384], rng.integers(0, M, 3000)]).astype(np.int64)
    ns = np.concatenate([[0, N - 1, 0, N - 1, 16383], rng.integers(0, N, 3000)]).astype(np.int64)
    ref = oracle.gemm_f64_sampled(qa, sa, qb, sb, ms, ns)
    A = to_dev_u16_as_bf16(torch, a)
    Bw, Bs = to_dev_u8(torch, bw), to_dev_u8(torch, bs)
    print("largest C: %s" % mx.mxfp4_gemm_schedule_name(M, N, K), flush=True)
    C = mx.gemm(A, Bw, Bs, N)
    torch.cuda.synchronize()
    got = bf16_dev_to_bits(C[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()])
    assert_close(got, ref, "largest C")


def test_k_beyond_the_fused_kernels():
    """M = 16 with K = 262144 (2048 steps): more than 16 splits of any fused
    kernel cover, so the large-M kernel serves it, for gemm and gemm_q."""
    torch = torch_cuda()
    M, N, K = 16, 64, 262144
    a = syn.normal_bf16(34, syn.STREAM_A, (M, K))
    b = syn.normal_bf16(34, syn.STREAM_B, (N, K))
    qb, sb, bw, bs = prepare_b(b)
    qa, sa = oracle.quantize(a)
    ref = oracle.gemm_f64(qa, sa, qb, sb)
    assert mx.mxfp4_gemm_schedule_name(M, N, K).startswith("wide_")
    A = to_dev_u16_as_bf16(torch, a)
    Bw, Bs = to_dev_u8(torch, bw), to_dev_u8(torch, bs)
    C = mx.gemm(A, Bw, Bs, N)
    aq, as_ = mx.quantize(A, shuffled_scales=True)
    Cq = mx.gemm_q(aq, as_, Bw, Bs, N)
    torch.cuda.synchronize()
    assert_close(bf16_dev_to_bits(C), ref, "gemm, K = 262144")
    assert_close(bf16_dev_to_bits(Cq), ref, "gemm_q, K = 262144")
