"""Pins of the number formats: e4m3 from its definition's special values, torch's CPU casts as an
independent library routine, exhaustive round trips and tie cases; bf16 against torch."""
import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, e4m3_decode, e4m3_encode, e4m3_quantise, f32_bits_to_f64


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0**-9), (0x07, 7 * 2.0**-9), (0x08, 2.0**-6), (0x38, 1.0), (0x39, 1.125),
    (0x40, 2.0), (0x7E, 448.0), (0x80, -0.0), (0xB8, -1.0), (0xFE, -448.0), (0x77, 240.0), (0x30, 0.5),
])
def test_e4m3_special_values(code, value):
    got = e4m3_decode(np.array([code], np.uint8))[0]
    assert got == value and np.signbit(got) == np.signbit(value)


def test_e4m3_nan_codes():
    d = e4m3_decode(np.array([0x7F, 0xFF], np.uint8))
    assert np.isnan(d).all()
    assert np.isfinite(e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))).all()


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(mine)
    assert np.array_equal(mine[ok], ref[ok])


def test_e4m3_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), codes)


def test_e4m3_ties_go_to_even_code():
    # midpoint of 1.0 (0x38) and 1.125 (0x39) -> 0x38; of 1.125 and 1.25 (0x3A) -> 0x3A
    assert e4m3_encode(np.float32([1.0625, 1.1875]))[0] == 0x38
    assert e4m3_encode(np.float32([1.0625, 1.1875]))[1] == 0x3A
    # subnormal midpoint: 0.5 * 2^-9 -> 0x00, 1.5 * 2^-9 -> 0x02, 2.5*2^-9 -> 0x02
    got = e4m3_encode(np.float32([0.5 * 2.0**-9, 1.5 * 2.0**-9, 2.5 * 2.0**-9]))
    assert got.tolist() == [0x00, 0x02, 0x02]
    # subnormal/normal boundary: midpoint of 7*2^-9 (0x07) and 2^-6 (0x08) -> 0x08
    assert e4m3_encode(np.float32([7.5 * 2.0**-9]))[0] == 0x08


def test_e4m3_saturates():
    got = e4m3_encode(np.float32([448.0, 460.0, 464.0, 1e9, np.inf, -500.0, -np.inf]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_e4m3_encode_matches_torch_on_in_range_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), ref)


def test_e4m3_quantise_power_of_two_scale_is_exact_shift():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(10000) * 3).astype(np.float32)
    for k in (-3, 0, 2):
        s = 2.0**k
        assert np.array_equal(e4m3_quantise(x, s), e4m3_encode(x * np.float32(2.0**-k)))


def test_e4m3_quantise_largest_value_maps_to_largest_code():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(4096) * 2.7).astype(np.float32)
    amax = float(np.abs(x).max())
    s = float(np.float32(amax / 448.0))
    codes = e4m3_quantise(x, s)
    assert (codes & 0x7F).max() == 0x7E
    err = np.abs(e4m3_decode(codes) * s - x.astype(np.float64))
    # relative half-ulp of e4m3 is 2^-4 of the value, plus the subnormal step near zero
    assert (err <= np.abs(x) * 2.0**-4 + s * 2.0**-10 + 1e-12).all()


def test_bf16_and_f32_bits_match_torch():
    rng = np.random.default_rng(4)
    x = torch.from_numpy(rng.standard_normal(100000).astype(np.float32) * 100)
    xb = x.to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits_to_f64(bits), xb.to(torch.float64).numpy())
    fbits = x.view(torch.int32).numpy().view(np.uint32)
    assert np.array_equal(f32_bits_to_f64(fbits), x.to(torch.float64).numpy())


def test_bf16_fp8_table_equals_elementwise_round_trip():
    """The memoised table of stored fp8 values (one entry per bf16 bit pattern) equals quantise then
    decode evaluated element by element, for every pattern, NaN positions included."""
    from oracle.run import bf16_fp8_table
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16_bits_to_f64(bits).astype(np.float32)
    for s in (0.0103, 1.0, float(np.float32(4.7 / 448.0))):
        want = e4m3_decode(e4m3_quantise(x, s)) * float(np.float32(s))
        got = bf16_fp8_table(s)[bits]
        assert np.array_equal(np.isnan(got), np.isnan(want))
        ok = ~np.isnan(want)
        assert np.array_equal(got[ok], want[ok])
