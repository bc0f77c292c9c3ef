"""Shared helpers for the GPU parity tests: seeded inputs, oracle-prepared B,
and the tolerance of the method (|C - C_ref| <= 1e-2 * |C_ref| + 1e-2)."""
import numpy as np
import pytest

import oracle

RTOL = 1e-2
ATOL = 1e-2


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


def to_dev_u16_as_bf16(torch, bits: np.ndarray):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def to_dev_u8(torch, a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev_to_bits(t) -> np.ndarray:
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def prepare_b(b_bits: np.ndarray):
    """Oracle-quantized B in natural layout plus the oracle's shuffled layouts."""
    N, K = b_bits.shape
    qb, sb = oracle.quantize(b_bits)
    return qb, sb, oracle.preshuffle_b(qb), oracle.shuffle_scales(sb, N, K)


def assert_close(got_bits: np.ndarray, ref: np.ndarray, what: str):
    got = bits_to_f64(got_bits)
    err = np.abs(got - ref)
    lim = RTOL * np.abs(ref) + ATOL
    bad = err > lim
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join("%s: got %r ref %r" % (tuple(i), got[tuple(i)], ref[tuple(i)]) for i in idx)
        raise AssertionError("%s: %d of %d outside |d| <= 1e-2|ref| + 1e-2; first: %s"
                             % (what, int(bad.sum()), bad.size, detail))
