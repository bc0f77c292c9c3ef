"""Pins for the oracle's GEMM and output rounding (CPU only).

- exact rational brute force on tiny shapes, reading codes through the e2m1
  table fixture and scales as exact powers of two;
- inputs that quantize losslessly, where the GEMM must equal numpy's fp64
  matmul of the original values exactly;
- a one-hot B, which returns the dequantized A columns;
- the bf16 output rounding against exact rational rounding and hand cases.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synthetic import bf16_bits_to_f32, f32_to_bf16_bits, normal_bf16
from tests.conftest import read_golden

TABLE = {int(c): Fraction(v) if v != "-0.0" else Fraction(0) for c, v in read_golden("e2m1_table.txt")}
MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def exact_gemm(qa, sa, qb, sb):
    M, KB = qa.shape
    N = qb.shape[0]
    K = 2 * KB
    C = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                ca = (int(qa[m, k // 2]) >> (4 * (k % 2))) & 0xF
                cb = (int(qb[n, k // 2]) >> (4 * (k % 2))) & 0xF
                acc += (TABLE[ca] * Fraction(2) ** (int(sa[m, k // 32]) - 127)
                        * TABLE[cb] * Fraction(2) ** (int(sb[n, k // 32]) - 127))
            C[m][n] = acc
    return C


def exact_bf16_bits(q: Fraction) -> int:
    """Round an exact rational to bf16 (nearest, ties to even), normal range."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * 128  # [128, 256)
    r = int(scaled)
    rem = scaled - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    if r == 256:
        r = 128
        e += 1
    return sign | ((e + 127) << 7) | (r - 128)


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 64, 1), (2, 3, 64, 2), (3, 2, 128, 3), (4, 4, 96, 4)])
def test_gemm_matches_exact_rational_brute_force(M, N, K, seed):
    a = normal_bf16(seed, 0, (M, K))
    b = normal_bf16(seed, 1, (N, K))
    qa, sa = oracle.quantize(a)
    qb, sb = oracle.quantize(b)
    C = oracle.gemm_f64(qa, sa, qb, sb)
    ex = exact_gemm(qa, sa, qb, sb)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(C[m, n]) - ex[m][n]) <= abs(ex[m][n]) * Fraction(1, 2 ** 50)
            assert oracle.bf16_from_f64(np.array([C[m, n]]))[0] == exact_bf16_bits(ex[m][n])


def lossless(rng, rows, K, tmin=-3, tmax=3):
    """Rows whose 32-groups are e2m1 magnitudes times 2^t with the group max
    from the representable set, so quantization is the identity."""
    G = K // 32
    x = np.empty((rows, K), dtype=np.float32)
    for r in range(rows):
        for g in range(G):
            top = rng.choice(MAGS[1:])
            vals = rng.choice(MAGS[MAGS <= top], size=32) * rng.choice([-1.0, 1.0], size=32)
            vals[rng.integers(32)] = top
            x[r, 32 * g: 32 * g + 32] = vals * 2.0 ** rng.integers(tmin, tmax + 1)
    xb = f32_to_bf16_bits(x)
    assert np.array_equal(bf16_bits_to_f32(xb), x)
    return xb, x.astype(np.float64)


@pytest.mark.parametrize("M,N,K", [(16, 32, 256), (5, 48, 320), (33, 64, 128)])
def test_gemm_equals_numpy_matmul_on_lossless_inputs(M, N, K):
    rng = np.random.default_rng(M * 1000 + N)
    ab, av = lossless(rng, M, K)
    bb, bv = lossless(rng, N, K)
    qa, sa = oracle.quantize(ab)
    qb, sb = oracle.quantize(bb)
    C = oracle.gemm_f64(qa, sa, qb, sb)
    assert np.array_equal(C, av @ bv.T)


def test_gemm_one_hot_b_returns_dequantized_a():
    M, N, K = 7, 64, 128
    a = normal_bf16(99, 0, (M, K))
    b = np.zeros((N, K), dtype=np.uint16)
    b[np.arange(N), np.arange(N)] = 0x3F80  # 1.0
    qa, sa = oracle.quantize(a)
    qb, sb = oracle.quantize(b)
    C = oracle.gemm_f64(qa, sa, qb, sb)
    deq = oracle.dequantize(qa, sa)
    assert np.array_equal(C, deq[:, :N])
    # and dequant(A) is close to A (|err| <= half a step of the group grid)
    av = bf16_bits_to_f32(a).astype(np.float64)
    step = np.ldexp(1.0, sa.astype(np.int64) - 127).repeat(32, axis=1)
    assert np.all(np.abs(deq - av) <= step + 1e-300)


def test_sampled_equals_full():
    a = normal_bf16(5, 0, (24, 256))
    b = normal_bf16(5, 1, (48, 256))
    qa, sa = oracle.quantize(a)
    qb, sb = oracle.quantize(b)
    C = oracle.gemm_f64(qa, sa, qb, sb)
    rng = np.random.default_rng(0)
    ms = rng.integers(0, 24, 50)
    ns = rng.integers(0, 48, 50)
    got = oracle.gemm_f64_sampled(qa, sa, qb, sb, ms, ns)
    assert np.allclose(got, C[ms, ns], rtol=1e-14, atol=0)


def test_whole_path_is_quantize_then_gemm_then_round():
    a = normal_bf16(6, 0, (9, 192))
    b = normal_bf16(6, 1, (32, 192))
    qa, sa = oracle.quantize(a)
    qb, sb = oracle.quantize(b)
    want = oracle.bf16_from_f64(oracle.gemm_f64(qa, sa, qb, sb))
    assert np.array_equal(oracle.mxfp4_gemm_bf16(a, qb, sb), want)


def test_bf16_rounding_hand_cases():
    cases = [
        (1.0 + 2.0 ** -8, 0x3F80),            # tie -> even (1.0)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie -> even (1 + 2^-6)
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),
        (-2.5, 0xC020),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (2.0 ** 130, 0x7F80),                 # overflow -> inf
        (2.0 ** -133, 0x0001),                # smallest bf16 subnormal
        (2.0 ** -134, 0x0000),                # tie with 0 -> even (0)
        (3 * 2.0 ** -134, 0x0002),            # tie 1|2 subnormal ulps -> even (2)
    ]
    got = oracle.bf16_from_f64(np.array([c[0] for c in cases]))
    assert [int(g) for g in got] == [c[1] for c in cases]


def test_bf16_rounding_matches_integer_rne_on_f32_values():
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * np.float32(1e3)
    want = f32_to_bf16_bits(x)
    got = oracle.bf16_from_f64(x.astype(np.float64))
    assert np.array_equal(got, want)
