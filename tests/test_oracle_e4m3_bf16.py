"""Pins for the oracle's E4M3 decode and bfloat16 rounding."""
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_table_matches_torch_cast_exhaustively():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = oracle.e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(tab))
    assert nan.sum() == 2
    assert np.array_equal(ref[~nan], tab[~nan])
    # sign bit of zero
    assert math.copysign(1.0, tab[0x80]) == -1.0


def test_e4m3_golden_values():
    tab = oracle.e4m3_table()
    n = 0
    for line in open(os.path.join(GOLDEN, "e4m3_codes.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()[:2]
        code = int(code, 16)
        if val == "nan":
            assert math.isnan(tab[code])
        else:
            assert tab[code] == float(val), hex(code)
            if val.startswith("-"):
                assert math.copysign(1.0, tab[code]) == -1.0
        n += 1
    assert n >= 15


def test_e4m3_values_are_integer_multiples_of_2_pow_minus_9():
    tab = oracle.e4m3_table()
    fin = tab[np.isfinite(tab)]
    scaled = fin * 512.0
    assert np.all(scaled == np.round(scaled))
    assert np.max(np.abs(scaled)) == 448 * 512 < 2 ** 18


def test_round_bf16_matches_torch():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(100000, generator=g, dtype=torch.float64) * 3
    ref = x.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(x.numpy())
    assert np.array_equal(ref, got)


def test_round_bf16_ties_to_even():
    # 1 + 2^-8 is exactly halfway between bf16 1.0 and 1 + 2^-7: ties go to even (1.0)
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties go to 1 + 2^-6
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, float("nan")])
    bits = oracle.round_bf16(vals)
    back = oracle.bf16_bits_to_float(bits)
    assert back[0] == 1.0
    assert back[1] == 1 + 2 ** -6
    assert back[2] == -1.0
    assert back[3] == 0.0
    assert math.isnan(back[4])
