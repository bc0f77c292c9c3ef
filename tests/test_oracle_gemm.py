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


# ---------------------------------------------------------------- fp32 accumulation

def group_terms(qa, sa, qb, sb):
    """Exact per-group terms t[m, n, g] = sum over the group of deq(A) deq(B)
    (numpy fp64 on dequantized values: every product and every 32-term sum
    of e2m1 x e2m1 x powers of two within one group is exact)."""
    M, N, K = qa.shape[0], qb.shape[0], qa.shape[1] * 2
    da = oracle.dequantize(qa, sa).reshape(M, K // 32, 32)
    db = oracle.dequantize(qb, sb).reshape(N, K // 32, 32)
    return np.einsum("mgj,ngj->mng", da, db)


def f32_ascending(terms):
    """Reference fp32 accumulation, one element at a time: round each group
    term to fp32 and add in ascending group order with numpy float32 adds."""
    acc = np.float32(0.0)
    for t in terms:
        acc = np.float32(acc + np.float32(t))
    return acc


@pytest.mark.parametrize("M,N,K,seed", [(2, 3, 256, 1), (3, 5, 512, 2), (1, 4, 1024, 3)])
def test_gemm_f32_matches_elementwise_fp32_emulation(M, N, K, seed):
    a = normal_bf16(seed, 0, (M, K))
    b = normal_bf16(seed, 1, (N, K))
    a[0, :32] = f32_to_bf16_bits(np.float32(1e4) * bf16_bits_to_f32(a[0, :32]))  # one large group
    qa, sa = oracle.quantize(a)
    qb, sb = oracle.quantize(b)
    C = oracle.gemm_f32(qa, sa, qb, sb)
    t = group_terms(qa, sa, qb, sb)
    for m in range(M):
        for n in range(N):
            assert C[m, n] == f32_ascending(t[m, n]), (m, n)


def test_gemm_f32_equals_f64_where_the_sums_are_exact():
    """All scale bytes 127 and K = 512: every partial sum is a multiple of
    1/4 below 2^12, exact in fp32, so the two accumulations agree exactly."""
    rng = np.random.default_rng(11)
    M, N, K = 9, 40, 512
    qa = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    qb = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = np.full((M, K // 32), 127, dtype=np.uint8)
    sb = np.full((N, K // 32), 127, dtype=np.uint8)
    c32 = oracle.gemm_f32(qa, sa, qb, sb)
    c64 = oracle.gemm_f64(qa, sa, qb, sb)
    assert np.array_equal(c32.astype(np.float64), c64)


def test_gemm_f32_adds_groups_in_ascending_order():
    """Three groups, each with a single nonzero product, so the group terms
    are exactly +-2^25 and 1.  Row 0 has terms (2^25, 1, -2^25): in fp32 and
    ascending order (2^25 + 1) rounds to 2^25 (the fp32 spacing there is 4),
    and the sum is 0.  Row 1 has (2^25, -2^25, 1) and sums to 1.  fp64 gives
    1 for both, and adding row 0's groups in any order that pairs 2^25 with
    -2^25 first gives 1: only ascending fp32 accumulation gives (0, 1)."""
    K = 96
    qa = np.zeros((2, K // 2), dtype=np.uint8)
    qb = np.zeros((1, K // 2), dtype=np.uint8)
    sa = np.full((2, 3), 127, dtype=np.uint8)
    sb = np.full((1, 3), 127, dtype=np.uint8)
    # codes: 2 = 1.0, 0xA = -1.0; element 0 of each group
    qb[0, 0] = qb[0, 16] = qb[0, 32] = 0x02
    # row 0: +2^25, +1, -2^25 ; row 1: +2^25, -2^25, +1
    qa[0, 0], qa[0, 16], qa[0, 32] = 0x02, 0x02, 0x0A
    qa[1, 0], qa[1, 16], qa[1, 32] = 0x02, 0x0A, 0x02
    sa[0] = [127 + 25, 127, 127 + 25]
    sa[1] = [127 + 25, 127 + 25, 127]
    C = oracle.gemm_f32(qa, sa, qb, sb)
    assert C[0, 0] == 0.0   # 2^25 + 1 rounds to 2^25, then cancels
    assert C[1, 0] == 1.0   # 2^25 - 2^25 = 0, then + 1
    assert list(oracle.gemm_f64(qa, sa, qb, sb)[:, 0]) == [1.0, 1.0]


@pytest.mark.parametrize("M,N,K,seed", [(16, 96, 1536, 1), (8, 64, 7168, 3), (32, 64, 2048, 4)])
def test_gemm_f32_gap_to_f64_within_summation_bound(M, N, K, seed):
    """|C32 - C64| <= gamma_G * sum_g |t_g| with gamma_G = G u / (1 - G u),
    u = 2^-24: the error bound of recursive summation of G terms, each
    term itself rounded once to fp32 (Higham, Accuracy and Stability of
    Numerical Algorithms, 2nd ed., section 4.2).  Far below the method's
    tolerance of 1e-2 |C| + 1e-2."""
    a = normal_bf16(seed, 0, (M, K))
    b = normal_bf16(seed, 1, (N, K))
    qa, sa = oracle.quantize(a)
    qb, sb = oracle.quantize(b)
    c32 = oracle.gemm_f32(qa, sa, qb, sb).astype(np.float64)
    c64 = oracle.gemm_f64(qa, sa, qb, sb)
    t = group_terms(qa, sa, qb, sb)
    G = K // 32
    u = 2.0 ** -24
    gamma = (G + 1) * u / (1 - (G + 1) * u)
    bound = gamma * np.abs(t).sum(axis=2)
    assert np.all(np.abs(c32 - c64) <= bound)
    assert np.all(np.abs(c32 - c64) <= 1e-3 * (1e-2 * np.abs(c64) + 1e-2))


def test_whole_path_with_f32_accumulation():
    a = normal_bf16(8, 0, (5, 256))
    b = normal_bf16(8, 1, (32, 256))
    qa, sa = oracle.quantize(a)
    qb, sb = oracle.quantize(b)
    want = oracle.bf16_from_f64(oracle.gemm_f32(qa, sa, qb, sb).astype(np.float64))
    assert np.array_equal(oracle.mxfp4_gemm_bf16(a, qb, sb, f32acc=True), want)


def test_results_do_not_depend_on_thread_count(tmp_path):
    """The parallel loops split independent outputs only: one thread and
    many give the same bytes (run in a child process with OMP_NUM_THREADS=1)."""
    import os
    import subprocess
    import sys
    out = str(tmp_path / "one.npy")
    code = ("import sys, numpy as np, oracle, synthetic as s\n"
            "a = s.normal_bf16(21, 0, (12, 1024)); b = s.normal_bf16(21, 1, (80, 1024))\n"
            "qa, sa = oracle.quantize(a); qb, sb = oracle.quantize(b)\n"
            "assert oracle.num_threads() == 1\n"
            "np.save(sys.argv[1], np.concatenate([oracle.gemm_f64(qa, sa, qb, sb).ravel(), "
            "oracle.gemm_f32(qa, sa, qb, sb).astype(np.float64).ravel()]))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, OMP_NUM_THREADS="1", PYTHONPATH=root)
    subprocess.run([sys.executable, "-c", code, out], env=env, check=True, cwd=root)
    one = np.load(out)
    a = normal_bf16(21, 0, (12, 1024))
    b = normal_bf16(21, 1, (80, 1024))
    qa, sa = oracle.quantize(a)
    qb, sb = oracle.quantize(b)
    many = np.concatenate([oracle.gemm_f64(qa, sa, qb, sb).ravel(),
                           oracle.gemm_f32(qa, sa, qb, sb).astype(np.float64).ravel()])
    assert oracle.num_threads() > 1 or os.cpu_count() == 1
    assert np.array_equal(one, many)
