"""The seeded input generator: Philox-4x32-10 known-answer vectors (from the
Random123 distribution that accompanies Salmon et al., SC 2011), draw
statistics and the wide-scale group pick of the M=64 workload."""
import numpy as np

import oracle
import synthetic as syn


def test_philox_known_answers():
    kat = [
        ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
        ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
        ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
         (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
    ]
    for ctr, key, want in kat:
        got = syn.philox4x32_10(np.array([ctr], dtype=np.uint32), *key)[0]
        assert tuple(int(x) for x in got) == want


def test_normal_draws_look_normal():
    z = syn.normal_f32(1, 0, 1 << 18).astype(np.float64)
    assert abs(z.mean()) < 0.01
    assert abs(z.std() - 1.0) < 0.01
    assert abs(np.mean(np.abs(z) < 1.0) - 0.6827) < 0.005


def test_chunking_does_not_change_the_stream():
    a = syn.normal_f32(3, 1, 10001, chunk=1 << 22)
    b = syn.normal_f32(3, 1, 10001, chunk=777)
    assert np.array_equal(a, b)


def test_streams_and_seeds_differ():
    a = syn.normal_bf16(1, syn.STREAM_A, (4, 64))
    b = syn.normal_bf16(1, syn.STREAM_B, (4, 64))
    c = syn.normal_bf16(2, syn.STREAM_A, (4, 64))
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_wide_scale_workload_shifts_exactly_41_groups_by_three():
    w = syn.CONFIGS["c4"]
    base = syn.normal_bf16(w.seed, syn.STREAM_A, (w.M, w.K))
    a = w.a_bits()
    _, s0 = oracle.quantize(base)
    q1, s1 = oracle.quantize(a)
    q0, _ = oracle.quantize(base)
    diff = (s1.astype(int) - s0.astype(int)).reshape(-1)
    assert np.count_nonzero(diff) == 41 == round(0.01 * w.M * w.K / 32)
    assert set(diff[diff != 0].tolist()) == {3}
    assert np.array_equal(q0, q1)  # codes unchanged under a power-of-two shift


def test_inputs_are_finite_bf16():
    for w in list(syn.CONFIGS.values())[:3]:
        a = w.a_bits()
        assert a.dtype == np.uint16 and a.shape == (w.M, w.K)
        assert np.all(((a >> 7) & 0xFF) != 0xFF)
        assert w.K % 64 == 0
