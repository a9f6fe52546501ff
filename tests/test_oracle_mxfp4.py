"""Pins for the oracle's MXFP4 index keys (E2M1 elements, E8M0 block scales).

E2M1 values against a hand-worked table (tests/golden/e2m1_codes.txt), E8M0
against torch's float8_e8m0fnu decode, the encoder by round-trips and ties, the
block quantiser by exact blocks, worked scale choices, clamping and NaN, the
nibble layout by a hand case, and the MXFP4 scoring path against the E4M3 one
on keys that both formats hold exactly.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_codes.txt")


def test_e2m1_table_matches_hand_values():
    want = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        code, value = line.split()[:2]
        want[int(code, 16)] = float(value)
    t = oracle.e2m1_table()
    assert sorted(want) == list(range(16))
    for c, v in want.items():
        assert t[c] == v and math.copysign(1, t[c]) == math.copysign(1, v), (c, t[c], v)


def test_e8m0_matches_torch_decode():
    codes = torch.arange(255, dtype=torch.uint8)
    want = codes.view(torch.float8_e8m0fnu).float().double().numpy()
    assert np.array_equal(oracle.e8m0_value(codes.numpy()), want)
    assert np.isnan(oracle.e8m0_value([0xFF]))[0]


def test_e2m1_round_trip_ties_and_saturation():
    t = oracle.e2m1_table()
    assert oracle.encode_e2m1(t).tolist() == list(range(16))
    # midpoints go to the even code
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    assert oracle.encode_e2m1(mids).tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert oracle.encode_e2m1([-0.75, -5.0]).tolist() == [0xA, 0xE]
    assert oracle.encode_e2m1([0.26, 1.76, 5.01, 7.0, 1e9, -1e9]).tolist() == [1, 4, 7, 7, 7, 0xF]


def test_block_scale_choice_clamp_and_nan():
    def scales(block_values):
        return oracle.quantize_mxfp4(np.asarray(block_values, np.float64).reshape(1, 128))[1][0].tolist()
    z = np.zeros(32)
    # amax 6 -> floor(log2 6) = 2 -> exponent 0; amax 0.5 -> -3; amax 2^-20 -> -22
    assert scales(np.concatenate([z + 6, z + 0.5, z + 2.0 ** -20, z])) == [127, 124, 105, 0]
    # clamped exponents: 2^-140 -> -127 (elements round to 0); 2^140 -> 127 (saturate)
    d, s = oracle.quantize_mxfp4(np.concatenate([z + 2.0 ** -140, z + 2.0 ** 140, z, z]).reshape(1, 128))
    assert s[0].tolist() == [0, 254, 0, 0]
    v = oracle.decode_mxfp4(d, s)[0]
    assert np.all(v[:32] == 0) and np.all(v[32:64] == 6 * 2.0 ** 127)
    nan_block = np.concatenate([z, z, z, z])
    nan_block[40] = np.nan
    d, s = oracle.quantize_mxfp4(nan_block.reshape(1, 128))
    assert s[0].tolist() == [0, 0xFF, 0, 0] and np.all(d[0, 16:32] == 0)
    inf_block = np.concatenate([z + 1, z, z, z])
    inf_block[3] = -np.inf
    assert oracle.quantize_mxfp4(inf_block.reshape(1, 128))[1][0].tolist() == [0xFF, 0, 0, 0]


def test_exact_blocks_reproduce_their_codes():
    rng = np.random.default_rng(2)
    t = oracle.e2m1_table()
    codes = rng.integers(0, 16, (50, 4, 32))
    codes[:, :, 0] = rng.choice([6, 7, 14, 15], (50, 4))      # magnitude 4 or 6: floor(log2 amax) = 2
    exps = rng.integers(-20, 20, (50, 4))
    x = t[codes] * np.ldexp(1.0, exps)[..., None]
    d, s = oracle.quantize_mxfp4(x.reshape(50, 128))
    assert np.array_equal(s, (exps + 127).astype(np.uint8))
    assert np.array_equal(oracle.decode_mxfp4(d, s), x.reshape(50, 128))


def test_nibble_layout_hand_case():
    data = np.zeros((1, 64), np.uint8)
    data[0, 0] = 0x21            # element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    data[0, 63] = 0xF7           # element 126 = 6, element 127 = -6
    scales = np.array([[128, 127, 127, 126]], np.uint8)
    v = oracle.decode_mxfp4(data, scales)[0]
    assert v[0] == 1.0 and v[1] == 2.0 and v[126] == 3.0 and v[127] == -3.0
    assert np.count_nonzero(v) == 4


def test_insert_mxfp4_places_rows():
    cache = oracle.Mxfp4Keys(np.full((2, 128, 64), 0x55, np.uint8), np.full((2, 128, 4), 0x55, np.uint8))
    k = np.zeros((3, 128), np.float32)
    k[0] = 6.0
    k[2, :32] = -0.5
    oracle.insert_index_k_mxfp4(cache, k, np.array([129, -1, 0]))
    assert np.all(cache.data[1, 1] == 0x77) and cache.scales[1, 1].tolist() == [127] * 4
    assert np.all(cache.data[0, 0, :16] == 0xEE) and cache.scales[0, 0].tolist() == [124, 0, 0, 0]
    assert np.all(cache.data[0, 0, 16:] == 0)
    untouched = np.ones((2, 128), bool)
    untouched[1, 1] = untouched[0, 0] = False
    assert np.all(cache.data[untouched] == 0x55)


def test_mxfp4_scores_equal_e4m3_scores_on_shared_values():
    """Keys whose values both formats hold exactly (E2M1 values times 2^e with
    small e are E4M3 values) must score the same through either cache."""
    rng = np.random.default_rng(3)
    pages, hq = 6, 2
    t = oracle.e2m1_table()
    codes = rng.integers(0, 16, (pages, 128, 4, 32))
    exps = rng.integers(-3, 3, (pages, 128, 4))
    vals = (t[codes] * np.ldexp(1.0, exps)[..., None]).reshape(pages, 128, 128)
    d, s = oracle.quantize_mxfp4(vals)
    assert np.array_equal(oracle.decode_mxfp4(d, s), vals)
    e4 = oracle.encode_e4m3(vals)
    assert np.array_equal(oracle.decode_e4m3(e4), vals)
    cu_q, cu_k = np.array([0, 40, 50]), np.array([0, 500, 260])
    bt = np.array([[3, 0, 5, 1], [2, 4, -1, -1]], np.int32)
    q = oracle.encode_e4m3(rng.standard_normal((50, hq, 128)))
    a = oracle.index_scores(cu_q, cu_k, bt, q, e4, 0.5, 2.0)
    b = oracle.index_scores(cu_q, cu_k, bt, q, oracle.Mxfp4Keys(d, s), 0.5, 2.0)
    assert np.array_equal(a, b)
