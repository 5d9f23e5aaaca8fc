"""Pins of the oracle's E4M3 codec against the OCP format definition and torch."""
import numpy as np
import pytest
import torch

from oracle import e4m3_decode_table, e4m3_encode, E4M3_MAX


def test_special_values_from_format_definition():
    t = e4m3_decode_table()
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0      # largest finite
    assert t[0x01] == 2.0 ** -9                          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9                      # largest subnormal
    assert t[0x08] == 2.0 ** -6                          # smallest normal
    assert t[0x38] == 1.0                                # exponent field 7 = bias
    assert t[0x39] == 1.125
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t[[c for c in range(256) if c not in (0x7F, 0xFF)]]).all()
    assert E4M3_MAX == 448.0


def test_table_is_monotone_in_code_for_each_sign():
    t = e4m3_decode_table()
    pos = t[:0x7F]
    assert (np.diff(pos) > 0).all()
    assert np.array_equal(t[0x80:0xFF], -pos)


def test_round_trip_every_finite_code():
    t = e4m3_decode_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(e4m3_encode(t[codes]), codes.astype(np.uint8))


def test_ties_go_to_even_mantissa():
    # between 1.0 (0x38) and 1.125 (0x39): midpoint 1.0625 -> 0x38 (even)
    # between 1.125 (0x39) and 1.25 (0x3A): midpoint 1.1875 -> 0x3A (even)
    got = e4m3_encode(np.array([1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10]))
    # 2^-10 is the midpoint of 0 and 2^-9 -> 0 (even); 3*2^-10 midpoint of
    # 2^-9 (0x01) and 2^-8 (0x02) -> 0x02 (even)
    assert list(got) == [0x38, 0x3A, 0xB8, 0x00, 0x02]


def test_saturation_nan_and_signed_zero():
    got = e4m3_encode(np.array([448.0, 460.0, 464.0, 1e30, np.inf, -np.inf, np.nan, -0.0, 0.0]))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F, 0x80, 0x00]


def test_matches_torch_float8_in_range():
    # Library pin: torch's float8_e4m3fn cast (round-to-nearest-even) on
    # finite values below the overflow threshold.
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * s
                        for s in (1e-3, 0.05, 1.0, 30.0, 200.0)])
    x = x[np.abs(x) < 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), ref)


def test_encode_is_nearest():
    t = e4m3_decode_table()
    fin = t[:0x7F]
    rng = np.random.default_rng(3)
    x = rng.uniform(0, 448, 5000)
    codes = e4m3_encode(x)
    err = np.abs(t[codes] - x)
    best = np.abs(fin[None, :] - x[:, None]).min(axis=1)
    assert np.array_equal(err, best)
