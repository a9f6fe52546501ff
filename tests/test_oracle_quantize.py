"""Pins for the oracle's E4M3 encoder, quantisation and paged cache inserts.

The encoder is checked against the format itself (every finite code
round-trips, midpoints between neighbouring codes go to the even code, values
just off a midpoint go to the nearer one), against torch.float8_e4m3fn's CPU
cast where that cast does not saturate (|x| <= 464; beyond, torch gives NaN
where the stated rule saturates), and against the saturation / NaN rule by
direct values.  The inserts are checked against rows placed by hand.
"""
import math

import numpy as np
import pytest
import torch

import oracle

TABLE = oracle.e4m3_table()
FINITE = np.array([c for c in range(256) if not math.isnan(TABLE[c])], np.uint8)
POS = np.array(sorted((c for c in FINITE if c < 0x80), key=lambda c: TABLE[c]), np.uint8)


def test_every_finite_code_round_trips():
    assert np.array_equal(oracle.encode_e4m3(TABLE[FINITE]), FINITE)


def test_midpoints_go_to_the_even_code():
    lo, hi = POS[:-1], POS[1:]
    mid = (TABLE[lo] + TABLE[hi]) / 2.0
    got = oracle.encode_e4m3(mid)
    want = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(got, want)
    # mirror for negative values: the sign bit is set, the magnitude code the same
    assert np.array_equal(oracle.encode_e4m3(-mid), want | 0x80)


def test_values_just_off_a_midpoint_go_to_the_nearer_code():
    lo, hi = POS[:-1], POS[1:]
    mid = (TABLE[lo] + TABLE[hi]) / 2.0
    below = np.nextafter(mid.astype(np.float32), np.float32(-np.inf)).astype(np.float64)
    above = np.nextafter(mid.astype(np.float32), np.float32(np.inf)).astype(np.float64)
    assert np.array_equal(oracle.encode_e4m3(below), lo)
    assert np.array_equal(oracle.encode_e4m3(above), hi)


def test_matches_torch_cast_where_it_does_not_saturate():
    g = torch.Generator().manual_seed(17)
    x = torch.cat([
        (torch.rand(40000, generator=g, dtype=torch.float64) * 928 - 464).float(),
        (torch.randn(20000, generator=g, dtype=torch.float64) * 0.01).float(),   # subnormal range
        torch.tensor(np.concatenate([(TABLE[POS[:-1]] + TABLE[POS[1:]]) / 2]), dtype=torch.float32),
    ])
    want = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_e4m3(x.numpy().astype(np.float64)), want)


def test_saturation_nan_and_signed_zero():
    big = [448.0, 463.99, 464.0, 465.0, 479.0, 1e30, math.inf]
    assert oracle.encode_e4m3(big).tolist() == [0x7E] * len(big)
    assert oracle.encode_e4m3([-v for v in big]).tolist() == [0xFE] * len(big)
    assert oracle.encode_e4m3([math.nan]).tolist() == [0x7F]
    assert oracle.encode_e4m3([0.0, -0.0, -1e-9, 1e-9]).tolist() == [0x00, 0x80, 0x80, 0x00]
    # 2^-10 is the midpoint between 0 and the smallest subnormal: ties to 0
    assert oracle.encode_e4m3([2.0 ** -10, 2.0 ** -10 * 1.001]).tolist() == [0x00, 0x01]


@pytest.mark.parametrize("scale", [1.0, 0.5, 2.0, 2.0 ** -8, 3.0])
def test_quantize_divides_by_the_scale(scale):
    # exact multiples: dividing a code's value times a power of two by that
    # power is exact, so the code comes back
    if math.log2(scale).is_integer():
        x = (TABLE[FINITE] * scale).astype(np.float32)
        assert np.array_equal(oracle.quantize_e4m3(x, scale), FINITE)
    # the quotient is one float32 division: 3 * 1.25 / 3 is exactly 1.25 in
    # float32, and 1 / 3 lies between the codes for 0.3125 and 0.34375
    x = np.array([3.0 * 1.25, 1.0], np.float32)
    got = oracle.quantize_e4m3(x, 3.0)
    if scale == 3.0:
        assert got.tolist() == [0x3A, 0x2B]   # 1.25 = 1.010b; 1/3 -> 0.34375 = 1.011b * 2^-2


def test_insert_index_k_places_rows_by_slot():
    cache = np.full((3, 128, 128), 0x55, np.uint8)
    codes = np.array([[0x38] * 128, [0x40] * 128, [0x30] * 128, [0xB8] * 128, [0x01] * 128],
                     np.uint8)
    k = TABLE[codes].astype(np.float32) * 2.0          # scale 2: values are 2 * code value
    slots = np.array([130, -1, 0, 383, 5])
    oracle.insert_index_k(cache, k, slots, 2.0)
    want = np.full((3, 128, 128), 0x55, np.uint8)
    want[1, 2] = codes[0]
    want[0, 0] = codes[2]
    want[2, 127] = codes[3]
    want[0, 5] = codes[4]
    assert np.array_equal(cache, want)


def test_insert_kv_splits_k_and_v_per_head():
    cache = np.full((2, 2, 128, 256), 0x55, np.uint8)
    k = np.zeros((2, 2, 128), np.float32)
    v = np.zeros((2, 2, 128), np.float32)
    k[0, 0], k[0, 1], k[1, 0], k[1, 1] = 1.0, 2.0, -1.0, 0.5
    v[0, 0], v[0, 1], v[1, 0], v[1, 1] = 4.0, -4.0, 8.0, 0.25
    oracle.insert_kv(cache, k, v, np.array([129, 7]), 1.0, 4.0)
    want = np.full((2, 2, 128, 256), 0x55, np.uint8)
    want[1, 0, 1, :128], want[1, 1, 1, :128] = 0x38, 0x40     # K of token 0 (scale 1)
    want[1, 0, 1, 128:], want[1, 1, 1, 128:] = 0x38, 0xB8     # V of token 0 / 4
    want[0, 0, 7, :128], want[0, 1, 7, :128] = 0xB8, 0x30
    want[0, 0, 7, 128:], want[0, 1, 7, 128:] = 0x40, 0x18     # 8/4 = 2, 0.25/4 = 2^-4
    assert np.array_equal(cache, want)
