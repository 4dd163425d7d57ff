"""CPU pins for the seeded generator's FP8 E4M3 codec (OCP e4m3fn: sign, 4
exponent bits with bias 7, 3 mantissa bits, subnormals m * 2^-9, NaN at
S.1111.111, no infinities, largest finite 448).  The expected values below
follow from that definition by hand, not from the codec."""
import numpy as np

from workloads import FP8_MAX, f32_to_fp8_bits, fp8_bits_to_f32, round_to_fp8


def test_decode_known_codes():
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
             0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x58: 16.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0,
             0xB8: -1.0, 0xFE: -448.0}
    got = fp8_bits_to_f32(np.array(list(table), np.uint8))
    assert np.array_equal(got, np.array(list(table.values()), np.float32))
    assert np.isnan(fp8_bits_to_f32(np.array([0x7F, 0xFF], np.uint8))).all()
    z = fp8_bits_to_f32(np.array([0x80], np.uint8))[0]
    assert z == 0.0 and np.signbit(z)
    assert FP8_MAX == 448.0


def test_every_finite_code_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8_bits_to_f32(codes)
    fin = ~np.isnan(vals)
    assert fin.sum() == 254
    assert np.array_equal(f32_to_fp8_bits(vals[fin]), codes[fin])


def test_rounding_ties_go_to_even():
    x = np.array([1.0 + 1 / 16, 1.0 + 3 / 16, 17.0, 19.0, 2.0 ** -10, 3 * 2.0 ** -10, -(1.0 + 1 / 16)])
    # 1.0625 sits between 1.0 (m=0) and 1.125 (m=1): even is 1.0;
    # 1.1875 between 1.125 (m=1) and 1.25 (m=2): 1.25; 17 between 16 (m=0) and 18: 16;
    # 19 between 18 (m=1) and 20 (m=2): 20; 2^-10 is half the smallest subnormal: 0;
    # 1.5 subnormal units: 2 units
    assert list(f32_to_fp8_bits(x)) == [0x38, 0x3A, 0x58, 0x5A, 0x00, 0x02, 0xB8]


def test_saturation_and_signed_zero():
    x = np.array([448.0, 463.9, 464.0, 1e6, -1e6, 0.0, -0.0])
    assert list(f32_to_fp8_bits(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80]


def test_rounding_error_bound_and_monotonic():
    rng = np.random.default_rng(0)
    x = np.sort(np.concatenate([rng.standard_normal(20000) * 4, rng.uniform(-0.02, 0.02, 5000)]))
    r = round_to_fp8(x).astype(np.float64)
    assert np.all(np.diff(r) >= 0)
    normal = np.abs(x) >= 2.0 ** -6
    assert np.all(np.abs(r - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal] + 1e-12)
    assert np.all(np.abs(r - x)[~normal] <= 2.0 ** -10 + 1e-12)
