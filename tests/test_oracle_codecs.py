"""Pins of the oracle's number-format codecs against library dtype tables and
the formats' published value sets (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import codecs


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    assert np.nanmax(got) == 448.0


def _e4m3_grid():
    v = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = np.unique(v[~np.isnan(v)])
    return v


def test_round_e4m3_matches_torch_cast_on_midpoints_and_random():
    grid = _e4m3_grid()
    mids = (grid[:-1] + grid[1:]) / 2  # exact ties, representable in fp32
    rng = np.random.default_rng(0)
    rnd = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1, 30, 300)])
    vals = np.concatenate([grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                           rnd, [460.0, 464.0, 470.0, 1e6, -1e6, 2 ** -10, 2 ** -9 * 1.5]])
    vals32 = vals.astype(np.float32)
    ref = torch.from_numpy(vals32).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.round_e4m3_sat(vals32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e2m1_decode_matches_ocp_value_set():
    # OCP MX E2M1 magnitudes for codes 0..7, negatives for codes 8..15
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    table = table + [-t for t in table]
    got = codecs.e2m1_decode_nibbles(np.arange(16, dtype=np.uint8))
    assert list(got) == table


def test_e2m1_unpack_low_nibble_first():
    got = codecs.e2m1_unpack(np.array([[0x21, 0xF0]], dtype=np.uint8))
    assert got.tolist() == [[1, 2, 0, 15]]


def test_ue8m0_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = codecs.ue8m0_decode(b)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_bf16_decode_and_round_match_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(50000).astype(np.float32) * 10,
                        np.array([1e-40, -3e-39, 3.0e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32)])
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(codecs.bf16_decode(bits), ref)
    assert np.array_equal(codecs.round_bf16(x.astype(np.float64)), ref)


@pytest.mark.parametrize("v,expect", [(1.0625, 1.0), (1.06261, 1.125), (1.1875, 1.25), (-1.3125, -1.25),
                                      (460.0, 448.0), (1000.0, 448.0), (0.0, 0.0)])
def test_round_e4m3_hand_values(v, expect):
    # grid around 1: step 1/8, ties to even mantissa; saturation at 448
    assert codecs.round_e4m3_sat(np.array([v]))[0] == expect
