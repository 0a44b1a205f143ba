"""Pins of the oracle's element encodes (fp8 e4m3fn, bf16) against library routines
and brute force. CPU only."""
import numpy as np
import pytest
import torch

import oracle

ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def torch_fp8(x_f32):
    return torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_bf16(x_f32):
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_e4m3fn_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # closed-form landmarks of the OCP format
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert ours[0x38] == 1.0 and ours[0x80] == 0.0 and np.signbit(ours[0x80])


def test_e4m3fn_encode_every_bf16_value_matches_torch():
    x = bf16_bits_to_f32(ALL_BF16)
    assert np.array_equal(oracle.f32_to_e4m3fn(x), torch_fp8(x))


def test_e4m3fn_encode_random_f32_matches_torch():
    rng = np.random.default_rng(11)
    # random bit patterns concentrated on the fp8 range, plus raw patterns
    mag = np.exp2(rng.uniform(-12, 10, size=60000)).astype(np.float32)
    sgn = np.where(rng.random(60000) < 0.5, -1, 1).astype(np.float32)
    raw = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([mag * sgn, raw])
    assert np.array_equal(oracle.f32_to_e4m3fn(x), torch_fp8(x))


def test_e4m3fn_encode_brute_force_nearest():
    """Independent definition: nearest finite code by exhaustive search, ties to the
    even code, NaN once the nearest point lies past the top (448 + half a step)."""
    vals = oracle.e4m3fn_to_f64(np.arange(128, dtype=np.uint8))  # non-negative codes
    finite = np.flatnonzero(~np.isnan(vals))
    rng = np.random.default_rng(5)
    grid_mid = (vals[finite][1:] + vals[finite][:-1]) / 2  # exact ties
    xs = np.concatenate([
        rng.uniform(0, 470, 3000), np.exp2(rng.uniform(-11, -5, 2000)), grid_mid,
        vals[finite], [463.99, 464.0, 464.01, 500.0]]).astype(np.float32)
    got = oracle.f32_to_e4m3fn(xs)
    for x, g in zip(xs.astype(np.float64), got):
        d = np.abs(vals[finite] - x)
        best = finite[d == d.min()]
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        if x > 464.0:
            want = 0x7F
        assert g == want, (x, g, want)


def test_e4m3fn_encode_specials():
    x = np.array([np.inf, -np.inf, np.nan, -np.nan, 448.0, 464.0, 464.00003, -0.0, 2**-10],
                 dtype=np.float32)
    assert list(oracle.f32_to_e4m3fn(x)) == [0x7F, 0xFF, 0x7F, 0xFF, 0x7E, 0x7E, 0x7F, 0x80, 0x00]


@pytest.mark.parametrize("scale", [0.05, 0.04])
def test_scaled_encode_every_bf16_matches_torch_division_then_cast(scale):
    """Exhaustive: all 65,536 bf16 inputs; torch's fp32 division is IEEE, its cast RNE."""
    ours = oracle.encode_bf16_to_fp8_scaled(ALL_BF16, scale)
    x = torch.from_numpy(bf16_bits_to_f32(ALL_BF16).copy())
    ref = (x / torch.tensor(scale, dtype=torch.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(ours, ref.view(torch.uint8).numpy())


def test_bf16_encode_random_f32_matches_torch():
    rng = np.random.default_rng(7)
    raw = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    x = raw.view(np.float32)
    x = x[~np.isnan(x)]
    ties = ((rng.integers(0, 2**16, 5000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[~np.isnan(ties)]
    x = np.concatenate([x, ties, np.array([3.4028235e38, -3.4028235e38, 1e-45, -0.0],
                                          dtype=np.float32)])
    assert np.array_equal(oracle.f32_to_bf16(x), torch_bf16(x))


def test_bf16_encode_nan_reading():
    """NaN stays NaN with its sign (reading R5); torch maps every NaN to one pattern, so
    only NaN-ness is checked against the mathematics here and the exact bits are pinned
    by the stated rule."""
    u = np.array([0x7F800001, 0xFFC00001, 0x7FFFFFFF, 0x7FC00000], dtype=np.uint32)
    got = oracle.f32_to_bf16(u.view(np.float32))
    assert all(((g >> 7) & 0xFF) == 0xFF and (g & 0x7F) != 0 for g in got)
    assert list(got) == [0x7FC0, 0xFFC0, 0x7FFF, 0x7FC0]


def test_bf16_widen_is_exact_and_round_trips():
    x = bf16_bits_to_f32(ALL_BF16)
    ok = ~np.isnan(x)
    assert np.array_equal(oracle.f32_to_bf16(x[ok]), ALL_BF16[ok])


def test_array_encode_equals_the_scalar_encodes_and_torch():
    """The array entry used by the exhaustive GPU sweep is the scalar encodes
    element by element: 300k fp32 bit patterns drawn over every class (normals,
    subnormals, zeros, infinities, NaNs of every payload), against the scalar
    oracle calls and against torch's casts (NaN-ness only for bf16 NaNs)."""
    rng = np.random.default_rng(32)
    bits = rng.integers(0, 1 << 32, size=300_000, dtype=np.uint64).astype(np.uint32)
    bits[:64] = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x00000001,
                          0x807FFFFF, 0x43E00000, 0x43E80000, 0x43EFFFFF, 0x43F00000] * 5 + [1, 2, 3, 4],
                         dtype=np.uint32)
    x = bits.view(np.float32)
    b16 = oracle.encode_f32_array(x, oracle.BF16)
    f8 = oracle.encode_f32_array(x, oracle.FP8_E4M3FN)
    sample = slice(0, 3000)
    assert np.array_equal(b16[sample], oracle.f32_to_bf16(x[sample]))
    assert np.array_equal(f8[sample], oracle.f32_to_e4m3fn(x[sample]))
    nan = np.isnan(x)
    tb = torch_bf16(x)
    assert np.array_equal(b16[~nan], tb[~nan])
    assert np.all((b16[nan] & 0x7FFF) > 0x7F80)
    assert np.array_equal(f8, torch_fp8(x))
