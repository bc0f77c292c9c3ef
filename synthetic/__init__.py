"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no part of the method's arithmetic (no quantization, no
layout shuffles, no GEMM); it only draws bf16 bit patterns.  Both the HIP path
and the CPU oracle receive the same bytes from it.

Generator: Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC 2011), a counter-based generator, turned into
N(0,1) draws by the Box-Muller transform, rounded to f32 and then to bf16 with
round-to-nearest-even.  The leaderboard harness on the pages draws A then B
from N(0,1) in bf16 with one seeded generator and asserts K % 64 == 0
(submission 608632, the patched input generator); the draw order here follows
that, the bit stream does not (the pages' CUDA generator is not reproducible
off-GPU and need not be: both sides get the same bytes).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)
_KEY_TAG = 0x6D786634  # second key word, fixed

STREAM_A = 0
STREAM_B = 1
STREAM_PICK = 2


def philox4x32_10(ctr: np.ndarray, key0: int, key1: int) -> np.ndarray:
    """Philox-4x32 with 10 rounds.  ctr: uint32 [n, 4] -> uint32 [n, 4]."""
    c = [ctr[:, i].astype(np.uint64) for i in range(4)]
    k0, k1 = key0 & 0xFFFFFFFF, key1 & 0xFFFFFFFF
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & 0xFFFFFFFF
            k1 = (k1 + _W1) & 0xFFFFFFFF
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
    return np.stack([x.astype(np.uint32) for x in c], axis=1)


def uniform_u32(seed: int, stream: int, n: int) -> np.ndarray:
    """n uint32 words from counters (i, stream, 0, 0), i = 0.. ."""
    blocks = (n + 3) // 4
    ctr = np.zeros((blocks, 4), dtype=np.uint32)
    ctr[:, 0] = np.arange(blocks, dtype=np.uint64).astype(np.uint32)
    ctr[:, 1] = stream
    return philox4x32_10(ctr, seed, _KEY_TAG).reshape(-1)[:n]


def normal_f32(seed: int, stream: int, n: int, chunk: int = 1 << 22) -> np.ndarray:
    """n N(0,1) draws as float32 (Box-Muller on pairs of Philox words)."""
    out = np.empty(n, dtype=np.float32)
    npairs = (n + 1) // 2
    done = 0
    while done < npairs:
        cnt = min(chunk, npairs - done)
        # pair p uses words 2p, 2p+1 of the stream; counters are generated per chunk
        first_block = (2 * done) // 4
        last_block = (2 * (done + cnt) + 3) // 4
        ctr = np.zeros((last_block - first_block, 4), dtype=np.uint32)
        ctr[:, 0] = np.arange(first_block, last_block, dtype=np.uint64).astype(np.uint32)
        ctr[:, 1] = stream
        words = philox4x32_10(ctr, seed, _KEY_TAG).reshape(-1)
        off = 2 * done - 4 * first_block
        w = words[off: off + 2 * cnt].astype(np.float64)
        u1 = (w[0::2] + 1.0) / 4294967296.0  # (0, 1]
        u2 = w[1::2] / 4294967296.0          # [0, 1)
        r = np.sqrt(-2.0 * np.log(u1))
        z = np.empty(2 * cnt, dtype=np.float64)
        z[0::2] = r * np.cos(2.0 * np.pi * u2)
        z[1::2] = r * np.sin(2.0 * np.pi * u2)
        lo = 2 * done
        hi = min(n, lo + 2 * cnt)
        out[lo:hi] = z[: hi - lo].astype(np.float32)
        done += cnt
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, stream: int, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return f32_to_bf16_bits(normal_f32(seed, stream, n)).reshape(shape)


def pick_groups(seed: int, total: int, count: int) -> np.ndarray:
    """count distinct indices of [0, total), partial Fisher-Yates on Philox words."""
    w = uniform_u32(seed, STREAM_PICK, count).astype(np.float64) / 4294967296.0
    perm = np.arange(total, dtype=np.int64)
    for i in range(count):
        j = i + int(w[i] * (total - i))
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[:count])


def scale_groups_by(a_bits: np.ndarray, groups: np.ndarray, factor: float) -> np.ndarray:
    """Multiply the listed 32-element groups (row-major group index) by a power of two."""
    rows, K = a_bits.shape
    g = a_bits.reshape(rows * (K // 32), 32).copy()
    f = bf16_bits_to_f32(g[groups]) * np.float32(factor)
    g[groups] = f32_to_bf16_bits(f)
    return g.reshape(rows, K)


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    seed: int
    scaled_group_frac: float = 0.0  # fraction of A's 32-groups multiplied by 8

    def a_bits(self) -> np.ndarray:
        a = normal_bf16(self.seed, STREAM_A, (self.M, self.K))
        if self.scaled_group_frac > 0:
            total = self.M * self.K // 32
            count = int(round(self.scaled_group_frac * total))
            a = scale_groups_by(a, pick_groups(self.seed, total, count), 8.0)
        return a

    def b_bits(self) -> np.ndarray:
        return normal_bf16(self.seed, STREAM_B, (self.N, self.K))


# The five measured configurations (M x N x K), with their seeds.
CONFIGS = {
    "c1": Workload("M16_N3072_K1536", 16, 3072, 1536, seed=1),
    "c2": Workload("M32_N4096_K512", 32, 4096, 512, seed=2),
    "c3": Workload("M8_N2112_K7168", 8, 2112, 7168, seed=3),
    "c4": Workload("M64_N7168_K2048_wide_scales", 64, 7168, 2048, seed=4, scaled_group_frac=0.01),
    "c5": Workload("M256_N7168_K7168", 256, 7168, 7168, seed=5),
}

# Further leaderboard shapes listed on the pages (parity cases only).
EXTRA_SHAPES = {
    "p_4x2880x512": Workload("M4_N2880_K512", 4, 2880, 512, seed=11),
    "p_16x2112x7168": Workload("M16_N2112_K7168", 16, 2112, 7168, seed=12),
    "p_32x2880x512": Workload("M32_N2880_K512", 32, 2880, 512, seed=13),
    "p_256x3072x1536": Workload("M256_N3072_K1536", 256, 3072, 1536, seed=14),
}
