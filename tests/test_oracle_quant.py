"""Pins for the oracle's quantizer (CPU only).

Each test checks the oracle against something other than itself: the e2m1
format's closed form, the constants printed on the pages, hand-derived cases,
an exhaustive nearest-value search written with numpy, and exact power-of-two
identities that follow from the definition.
"""
import numpy as np
import pytest

import oracle
from synthetic import bf16_bits_to_f32, f32_to_bf16_bits, normal_bf16
from tests.conftest import read_golden

MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def bf16(v):
    """Exact float -> bf16 bits (asserts exact representability)."""
    b = f32_to_bf16_bits(np.asarray(v, dtype=np.float32))
    assert np.all(bf16_bits_to_f32(b) == np.asarray(v, dtype=np.float32)), v
    return int(b.reshape(-1)[0]) if np.ndim(v) == 0 else b


def finite_bf16_all():
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return x[((x >> 7) & 0xFF) != 0xFF]


# ---------------------------------------------------------------- e2m1 table

def test_e2m1_table_matches_format_definition():
    rows = read_golden("e2m1_table.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = oracle.e2m1_value(int(code))
        want = float(val)
        assert got == want and np.signbit(got) == np.signbit(want), (code, got, want)


def test_page_constants_are_consistent():
    c = {r[0]: r[1] for r in read_golden("page_constants.txt")}
    magic = np.float32(float(c["denorm_magic_f32"]))
    assert magic == np.float32(2.0 ** 22)
    assert int(np.array(magic).view(np.uint32)) == int(c["denorm_magic_bits"]) == 149 << 23
    assert int(c["normal_bias_add"], 16) == (((1 - 127) << 23) + (1 << 21) - 1) & 0xFFFFFFFF
    # The amax rounding constants add 1/4 ulp of the 2-bit leading mantissa
    # and clear the mantissa: rounds up iff mantissa >= 0.75.
    assert int(c["amax_round_add"], 16) == 1 << 21
    assert int(c["amax_round_mask"], 16) == 0xFF800000
    assert oracle.e2m1_value(int(c["saturate_code"])) == 6.0


# ---------------------------------------------------------------- encoder

def nearest_even_search(x_bits, s):
    """Nearest e2m1 magnitude by explicit distance search (numpy, fp64),
    ties to the even code, sign kept.  Independent of the oracle's C code."""
    xv = bf16_bits_to_f32(x_bits).astype(np.float64)
    v = np.abs(xv) * np.ldexp(1.0, 127 - s)
    v = np.minimum(v, 16.0)  # above 7 the nearest is 6 either way; keeps |v - m| exact
    d = np.abs(v[:, None] - MAGS[None, :])
    best = d.min(axis=1)
    cand = d == best[:, None]
    first = np.argmax(cand, axis=1)
    two = cand.sum(axis=1) == 2
    # a tie is always between consecutive codes c, c+1: take the even one
    code = np.where(two & (first % 2 == 1), first + 1, first)
    sign = (x_bits >> 15).astype(np.int64)
    return (code | (sign << 3)).astype(np.uint8)


def test_encoder_exhaustive_three_formulations():
    """All finite bf16 x all scale bytes 0..254: the integer midpoint
    encoder == the oracle's fp64 distance search == this file's numpy
    nearest-even search."""
    x = finite_bf16_all()
    for s in range(255):
        a = oracle.encode_many(x, s)
        b = oracle.encode_nearest_many(x, s)
        c = nearest_even_search(x, s)
        assert np.array_equal(a, b), s
        assert np.array_equal(a, c), (s, np.nonzero(a != c)[0][:5])


def test_encoder_hand_cases():
    for v, code in read_golden("encode_cases.txt"):
        v = float(v)
        for s in (127, 100, 140):
            xb = bf16(np.float32(v) * np.float32(2.0 ** (s - 127)))
            assert oracle.encode(int(xb), s) == int(code), (v, s)


# ---------------------------------------------------------------- scale byte

@pytest.mark.parametrize("amax,expect", [
    (1.0, 125), (1.5, 125), (1.7421875, 125),   # below 1.75: exponent kept
    (1.75, 126), (1.9921875, 126),             # 1.75 and above: rounds up
    (2.0, 126), (6.0, 127), (7.0, 128 - 0),    # 6 = 1.5*2^2 -> E=129; 7 = 1.75*2^2 -> E=130
])
def test_scale_byte_spot_values(amax, expect):
    g = np.zeros(32, dtype=np.uint16)
    g[5] = bf16(amax)
    g[9] = bf16(-amax / 4)
    assert oracle.scale_byte(g) == expect
    g[5] = bf16(-amax)  # sign does not matter
    assert oracle.scale_byte(g) == expect


def test_scale_byte_extremes():
    z = np.zeros(32, dtype=np.uint16)
    assert oracle.scale_byte(z) == 0
    assert oracle.scale_byte(np.full(32, 0x8000, dtype=np.uint16)) == 0  # all -0.0
    big = z.copy()
    big[0] = 0x7F7F  # largest finite bf16: rounds up to the inf pattern, E = 255
    assert oracle.scale_byte(big) == 253
    tiny = z.copy()
    tiny[3] = 0x0001  # smallest subnormal
    assert oracle.scale_byte(tiny) == 0


def test_scale_byte_puts_group_max_in_range():
    """Away from the clamps the chosen scale maps amax into [3.5, 7):
    amax/2^(s-127) is in [4, 7) when amax is not rounded up and in [3.5, 4)
    when it is (mantissa >= 0.75)."""
    a = normal_bf16(123, 0, (512, 256))
    q, s = oracle.quantize(a)
    g = bf16_bits_to_f32(a).astype(np.float64).reshape(512, 8, 32)
    amax = np.abs(g).max(axis=2)
    v = amax * np.ldexp(1.0, 127 - s.astype(np.int64))
    assert np.all(v >= 3.5) and np.all(v < 7.0)
    frac = amax / np.ldexp(1.0, np.floor(np.log2(amax)).astype(np.int64))
    assert np.all((v < 4.0) == (frac >= 1.75))


# ---------------------------------------------------------------- groups

def test_zero_and_negative_zero_groups():
    x = np.zeros((2, 64), dtype=np.uint16)
    x[1, :] = 0x8000
    q, s = oracle.quantize(x)
    assert np.all(s == 0)
    assert np.all(q[0] == 0x00) and np.all(q[1] == 0x88)


def test_saturating_group():
    """amax = 1.703125 * 2^e is not rounded up, so the scale is 2^(e-2) and
    the max element maps to 6.8125 -> saturates to 6 (code 7)."""
    e = 3
    g = np.zeros(32, dtype=np.float32)
    g[0] = 1.703125 * 2.0 ** e
    g[1] = 5.0 * 2.0 ** (e - 2)   # tie 4|6 -> 4 (code 6)
    g[2] = 5.5 * 2.0 ** (e - 2)   # -> 6 (code 7)
    g[3] = -0.125 * 2.0 ** (e - 2)  # -> -0 (code 8)
    q, s = oracle.quantize(bf16(g).reshape(1, 32))
    assert s[0, 0] == 127 + e - 2
    codes = np.stack([q[0] & 0xF, q[0] >> 4], axis=1).reshape(-1)
    assert list(codes[:4]) == [7, 6, 7, 8]


def test_nibble_order_even_low():
    g = np.zeros(32, dtype=np.float32)
    g[0], g[1] = 6.0, 0.5  # scale 2^0 (amax 6 -> E = 129 -> s = 127)
    q, s = oracle.quantize(bf16(g).reshape(1, 32))
    assert s[0, 0] == 127
    assert q[0, 0] == (7 | (1 << 4))


# ---------------------------------------------------------------- power of two

def test_power_of_two_shift_equivariance():
    """quant(2^j x) = (codes(x), s(x) + j) while no clamp binds: bf16 * 2^j is
    exact and the whole computation only sees exponents shift."""
    a = normal_bf16(7, 0, (64, 256))
    q0, s0 = oracle.quantize(a)
    for j in (-20, -3, 1, 3, 40):
        aj = f32_to_bf16_bits(bf16_bits_to_f32(a) * np.float32(2.0 ** j))
        qj, sj = oracle.quantize(aj)
        assert np.array_equal(qj, q0)
        assert np.array_equal(sj.astype(int), s0.astype(int) + j)


@pytest.mark.parametrize("top", [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
def test_exactly_representable_groups_round_trip(top):
    """A group of e2m1 values times 2^t whose largest magnitude is top * 2^t
    dequantizes back to itself exactly."""
    rng = np.random.default_rng(int(top * 10))
    allowed = MAGS[MAGS <= top]
    for t in (-30, -2, 0, 5, 60):
        vals = rng.choice(allowed, size=(8, 32)) * rng.choice([-1.0, 1.0], size=(8, 32))
        vals[:, 0] = top * rng.choice([-1.0, 1.0], size=8)
        x = (vals * 2.0 ** t).astype(np.float32)
        xb = bf16(x)
        q, s = oracle.quantize(xb)
        back = oracle.dequantize(q, s).reshape(8, 32)
        assert np.array_equal(back, x.astype(np.float64)), (top, t)


def test_non_finite_input_rejected():
    x = np.zeros((1, 32), dtype=np.uint16)
    x[0, 4] = 0x7F80
    with pytest.raises(ValueError):
        oracle.quantize(x)
