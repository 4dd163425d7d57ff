"""CPU pins for the seeded generator's FP8 codecs: E4M3 (OCP e4m3fn: sign, 4
exponent bits with bias 7, 3 mantissa bits, subnormals m * 2^-9, NaN at
S.1111.111, no infinities, largest finite 448).  The expected values below
follow from that definition by hand, not from the codec."""
import numpy as np

from workloads import (E5M2_MAX, FP8_MAX, e5m2_bits_to_f32, f32_to_e5m2_bits, f32_to_fp8_bits, fp8_bits_to_f32,
                       round_to_e5m2, round_to_fp8)


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


# --- FP8 E5M2 (OCP: sign, 5 exponent bits with bias 15, 2 mantissa bits,
# subnormals m * 2^-16, S.11111.00 infinity, S.11111.xx (xx != 0) NaN, largest
# finite 57344).  Values below follow from that definition by hand.

def test_e5m2_decode_known_codes():
    table = {0x00: 0.0, 0x01: 2.0 ** -16, 0x03: 3 * 2.0 ** -16, 0x04: 2.0 ** -14, 0x38: 0.5, 0x3C: 1.0,
             0x3D: 1.25, 0x3F: 1.75, 0x40: 2.0, 0x4C: 16.0, 0x78: 32768.0, 0x7B: 57344.0, 0xBC: -1.0,
             0xFB: -57344.0}
    got = e5m2_bits_to_f32(np.array(list(table), np.uint8))
    assert np.array_equal(got, np.array(list(table.values()), np.float32))
    inf = e5m2_bits_to_f32(np.array([0x7C, 0xFC], np.uint8))
    assert inf[0] == np.inf and inf[1] == -np.inf
    assert np.isnan(e5m2_bits_to_f32(np.array([0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF], np.uint8))).all()
    z = e5m2_bits_to_f32(np.array([0x80], np.uint8))[0]
    assert z == 0.0 and np.signbit(z)
    assert E5M2_MAX == 57344.0


def test_e5m2_every_finite_code_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    vals = e5m2_bits_to_f32(codes)
    fin = np.isfinite(vals)
    assert fin.sum() == 248
    assert np.array_equal(f32_to_e5m2_bits(vals[fin]), codes[fin])


def test_e5m2_rounding_ties_go_to_even():
    x = np.array([1.125, 1.375, 1.625, 1.875, 2.0 ** -17, 3 * 2.0 ** -17, 5 * 2.0 ** -17, 9.0, -1.125])
    # 1.125 between 1.0 (m=0) and 1.25 (m=1): even is 1.0; 1.375 between 1.25 and
    # 1.5 (m=2): 1.5; 1.625 between 1.5 and 1.75 (m=3): 1.5; 1.875 between 1.75
    # and 2.0 (carry to the next exponent, m=0): 2.0; 2^-17 is half the smallest
    # subnormal: 0; 1.5 units: 2; 2.5 units: 2; 9 between 8 and 10 (m=1): 8
    assert list(f32_to_e5m2_bits(x)) == [0x3C, 0x3E, 0x3E, 0x40, 0x00, 0x02, 0x02, 0x48, 0xBC]


def test_e5m2_saturation_and_signed_zero():
    x = np.array([57344.0, 60000.0, 61440.0, 1e9, -1e9, 0.0, -0.0])
    assert list(f32_to_e5m2_bits(x)) == [0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0x00, 0x80]


def test_e5m2_rounding_error_bound_and_monotonic():
    rng = np.random.default_rng(1)
    x = np.sort(np.concatenate([rng.standard_normal(20000) * 4, rng.uniform(-1e-4, 1e-4, 5000)]))
    r = round_to_e5m2(x).astype(np.float64)
    assert np.all(np.diff(r) >= 0)
    normal = np.abs(x) >= 2.0 ** -14
    assert np.all(np.abs(r - x)[normal] <= 2.0 ** -3 * np.abs(x)[normal] + 1e-12)
    assert np.all(np.abs(r - x)[~normal] <= 2.0 ** -17 + 1e-15)


def test_e5m2_values_are_exact_in_bfloat16():
    """Every finite e5m2 value is representable in bf16 (8 exponent bits, 7
    mantissa bits), which the kernels rely on when they widen rows."""
    from workloads import round_to_bf16
    vals = e5m2_bits_to_f32(np.arange(256, dtype=np.uint8))
    fin = vals[np.isfinite(vals)]
    assert np.array_equal(round_to_bf16(fin), fin)


def test_codecs_agree_with_torch_conversions():
    """torch's own float8 casts (round to nearest even) give the same bits for
    in-range values, subnormals included."""
    torch = __import__("pytest").importorskip("torch")
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(4000) * 50, rng.standard_normal(4000) * 1e-3,
                        rng.standard_normal(2000) * 1e-5]).astype(np.float32)
    t = torch.from_numpy(x)
    e4 = t[torch.from_numpy(np.abs(x) < 440)].to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f32_to_fp8_bits(x[np.abs(x) < 440]), e4)
    e5 = t.to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(f32_to_e5m2_bits(x), e5)
