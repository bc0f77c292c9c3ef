"""Pins for the oracle's layout transforms (CPU only).

The oracle writes both shuffles in address form.  The pages print other forms
of the same layouts: the scale shuffle as a view/permute (submission 608632,
_shuffle_scales) and its in-kernel inverse (submission 608632, kernel v7, the
b_scales reshape/permute), and two inverses of the B preshuffle (submission
608632, kernel v7, the b reshape/permute; submission 711914,
_unshuffle_b_preshuffle).  Those forms are restated below with numpy and the
oracle must agree with each.
"""
import numpy as np
import pytest

import oracle


def page_view_permute_shuffle(raw, rows, G):
    """Scale shuffle as a view/permute: (rows/32, 2, 16, G/8, 2, 4) ->
    order (0, 3, 5, 2, 4, 1), flattened per 32-row block."""
    s = raw.reshape(rows // 32, 2, 16, G // 8, 2, 4).transpose(0, 3, 5, 2, 4, 1)
    return np.ascontiguousarray(s).reshape(rows // 32, G * 32)


def page_kernel_unshuffle_scales(sh_block, BN, BK):
    """In-kernel scale unshuffle of a [BN/32, BK/32*32] byte block to
    [BN, BK/32]: reshape (BN/32, BK/256, 4, 16, 2, 2, 1), permute
    (0, 5, 3, 1, 4, 2, 6)."""
    s = sh_block.reshape(BN // 32, BK // 256, 4, 16, 2, 2, 1).transpose(0, 5, 3, 1, 4, 2, 6)
    return np.ascontiguousarray(s).reshape(BN, BK // 32)


def page_kernel_unshuffle_b_v7(b, BN, BK):
    """[BN/16, (BK/2)*16] -> [BN, BK/2]: reshape (1, BN/16, BK/64, 2, 16, 16),
    permute (0, 1, 4, 2, 3, 5)."""
    x = b.reshape(1, BN // 16, BK // 64, 2, 16, 16).transpose(0, 1, 4, 2, 3, 5)
    return np.ascontiguousarray(x).reshape(BN, BK // 2)


def page_unshuffle_b_711914(b_wide, BN, BK):
    """(BN/16, WIDE_K) -> (BK/2, BN): reshape (BN/16, BK/64, 2, 16, 16),
    permute (1, 2, 4, 0, 3)."""
    x = b_wide.reshape(BN // 16, BK // 64, 2, 16, 16).transpose(1, 2, 4, 0, 3)
    return np.ascontiguousarray(x).reshape(BK // 2, BN)


def rand_bytes(seed, shape):
    return np.random.default_rng(seed).integers(0, 256, size=shape, dtype=np.uint8)


@pytest.mark.parametrize("rows,K", [(32, 256), (256, 512), (64, 2048), (2112, 7168), (96, 1536), (4096, 512)])
def test_scale_shuffle_matches_view_permute_form(rows, K):
    G = K // 32
    raw = rand_bytes(rows * 7 + K, (rows, G))
    sh = oracle.shuffle_scales(raw, rows, K)
    Gp = (G + 7) // 8 * 8
    rp = (rows + 255) // 256 * 256
    assert sh.shape == (rp // 32, Gp * 32)
    # the printed form needs G % 8 == 0 and rows % 32 == 0: pad like the buffer does
    padded = np.full((rp, Gp), 127, dtype=np.uint8)
    padded[:rows, :G] = raw
    assert np.array_equal(sh, page_view_permute_shuffle(padded, rp, Gp))


@pytest.mark.parametrize("rows,K", [(32, 64), (48, 96), (16, 1536), (8, 7168), (300, 160)])
def test_scale_shuffle_padding_and_round_trip(rows, K):
    G = K // 32
    raw = rand_bytes(rows + K, (rows, G))
    sh = oracle.shuffle_scales(raw, rows, K)
    assert sh.size == oracle.shuffled_scale_bytes(rows, K)
    assert np.array_equal(oracle.unshuffle_scales(sh, rows, K), raw)
    # every byte not addressed by a real (row, group) is the fill value 127
    mask = np.ones(sh.size, dtype=bool)
    idx = np.arange(rows * G, dtype=np.int64)
    r, g = idx // G, idx % G
    Gp = (G + 7) // 8 * 8
    addr = (r % 32) // 16 + 2 * ((g % 8) // 4) + 4 * (r % 16) + 64 * (g % 4) + 256 * (g // 8) + (r // 32) * 32 * Gp
    mask[addr] = False
    assert np.all(sh.reshape(-1)[mask] == 127)
    assert len(np.unique(addr)) == rows * G


@pytest.mark.parametrize("N,K,BN,BK", [(64, 512, 64, 256), (256, 1024, 128, 512), (2112, 7168, 64, 256)])
def test_kernel_scale_unshuffle_inverts_oracle(N, K, BN, BK):
    G = K // 32
    raw = rand_bytes(N + 3 * K, (N, G))
    sh = oracle.shuffle_scales(raw, N, K)
    for n0 in range(0, N - BN + 1, BN):
        for k0 in range(0, K - BK + 1, BK):
            block = sh[n0 // 32: (n0 + BN) // 32, (k0 // 32) * 32: (k0 // 32) * 32 + (BK // 32) * 32]
            nat = page_kernel_unshuffle_scales(block, BN, BK)
            assert np.array_equal(nat, raw[n0:n0 + BN, k0 // 32:(k0 + BK) // 32])


@pytest.mark.parametrize("N,K", [(16, 64), (32, 256), (128, 512), (2112, 7168), (3072, 1536)])
def test_b_preshuffle_matches_both_printed_inverses(N, K):
    bq = rand_bytes(N * 5 + K, (N, K // 2))
    sh = oracle.preshuffle_b(bq)
    assert sh.shape == (N // 16, (K // 2) * 16)
    assert np.array_equal(page_kernel_unshuffle_b_v7(sh, N, K), bq)
    assert np.array_equal(page_unshuffle_b_711914(sh, N, K), bq.T)
    assert np.array_equal(oracle.unpreshuffle_b(sh, N, K), bq)


def test_b_preshuffle_tile_is_one_operand_block():
    """Tile (g, t) holds rows 16g..16g+15, bytes 16t..16t+15 of each row,
    row-major, 256 bytes contiguous."""
    N, K = 32, 128
    bq = np.arange(N * K // 2, dtype=np.int64).reshape(N, K // 2).astype(np.uint8)
    sh = oracle.preshuffle_b(bq).reshape(-1)
    g, t = 1, 2
    tile = sh[g * (K // 2) * 16 + t * 256: g * (K // 2) * 16 + (t + 1) * 256].reshape(16, 16)
    assert np.array_equal(tile, bq[16 * g: 16 * g + 16, 16 * t: 16 * t + 16])
