"""Pins for the oracle's MXFP4 K|V pages as the attention reads them (each
element's code value times its block scale, rounded to E4M3).

The staged codes against hand-worked values (tests/golden/mxfp4_kv_staged.txt),
against torch's float8_e4m3fn cast of every (code, scale) product clamped to
the E4M3 range, exact agreement with decode_mxfp4 wherever the products are
E4M3 values, the element and block placement by hand-placed bytes, and the
attention over the staged cache against dense attention over decode_mxfp4
values.
"""
import os

import numpy as np
import torch

import oracle
from helpers import PAGE, D, varlen, random_codes, scatter_pages

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_kv_staged.txt")


def test_staged_codes_match_hand_values():
    t = oracle.mxfp4_staged_table()
    n = 0
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        code, scale, want = line.split()[:3]
        assert t[int(scale), int(code, 16)] == int(want, 16), line
        n += 1
    assert n >= 15


def test_staged_codes_match_torch_cast():
    """Every (scale, code) below the NaN scale: torch's E4M3 cast (nearest even)
    of the exact product clamped to +-448 (the saturation rule)."""
    t = oracle.mxfp4_staged_table()
    e2m1 = oracle.e2m1_table()
    for sc in range(255):
        v = np.clip(e2m1 * 2.0 ** (sc - 127), -448.0, 448.0)
        want = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(t[sc], want), sc
    assert np.all(t[255] == 0x7F)


def test_staged_values_equal_mxfp4_values_in_exact_range():
    """Scales 2^-5 .. 2^6 keep every product an E4M3 value: reading through E4M3
    changes nothing."""
    rng = np.random.default_rng(1)
    data = rng.integers(0, 256, (3, 2, 5, 128), dtype=np.uint8)
    scales = rng.integers(122, 134, (3, 2, 5, 8), dtype=np.uint8)
    got = oracle.decode_e4m3(oracle.mxfp4_kv_as_e4m3(data, scales))
    want_k = oracle.decode_mxfp4(data[..., :64], scales[..., :4])
    want_v = oracle.decode_mxfp4(data[..., 64:], scales[..., 4:])
    assert np.array_equal(got[..., :128], want_k)
    assert np.array_equal(got[..., 128:], want_v)


def test_element_and_block_placement():
    data = np.zeros((1, 128), np.uint8)
    scales = np.full((1, 8), 127, np.uint8)
    data[0, 5] = 0x71          # K elements 10 (low nibble, 0.5) and 11 (high nibble, 6)
    data[0, 64 + 20] = 0xA2    # V elements 40 (1.0) and 41 (-1.0)
    scales[0, 0] = 128         # K block 0 (elements 0..31) doubled
    scales[0, 5] = 125         # V block 1 (elements 32..63) quartered
    got = oracle.decode_e4m3(oracle.mxfp4_kv_as_e4m3(data, scales))[0]
    want = np.zeros(256)
    want[10], want[11] = 1.0, 12.0
    want[128 + 40], want[128 + 41] = 0.25, -0.25
    assert np.array_equal(got, want)


def test_attention_over_staged_cache_is_dense_attention():
    """Every visible page selected, scales in the exact range: the oracle's
    attention over the staged cache equals torch SDPA in float64 over the
    MXFP4 values (K and V global scales applied as for the E4M3 cache)."""
    rng = np.random.default_rng(7)
    Hq, Hkv = 4, 2
    cu_q, cu_k, bt, num_pages = varlen([40, 17], [700, 200], spare=1, seed=3)
    total_q, total_k = int(cu_q[-1]), int(cu_k[-1])
    q = random_codes(rng, (total_q, Hq, D), 0x48)
    rows_d = rng.integers(0, 256, (total_k, Hkv, 128), dtype=np.uint8)
    rows_s = rng.integers(124, 128, (total_k, Hkv, 8), dtype=np.uint8)
    data = scatter_pages(rows_d, cu_k, bt, num_pages, (Hkv, 128)).transpose(0, 2, 1, 3).copy()
    scales = scatter_pages(rows_s, cu_k, bt, num_pages, (Hkv, 8)).transpose(0, 2, 1, 3).copy()
    _, pos = oracle.query_positions(cu_q, cu_k)
    sel = np.full((total_q, 1, 16), -1, np.int32)
    for i, p in enumerate(pos):
        v = int(p // PAGE + 1)
        sel[i, 0, :v] = np.arange(v)
    sm, qs, ks, vs = 0.0883883, 0.5, 1.5, 0.75
    got = oracle.sparse_attention(cu_q, cu_k, bt, q, oracle.mxfp4_kv_as_e4m3(data, scales), sel,
                                  sm, qs, ks, vs)
    dec = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).double()
    for b in range(2):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1]); k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        sq, sk = q1 - q0, k1 - k0
        Q = dec(q[q0:q1]).transpose(0, 1) * qs
        K = torch.from_numpy(oracle.decode_mxfp4(rows_d[k0:k1, :, :64], rows_s[k0:k1, :, :4]))
        V = torch.from_numpy(oracle.decode_mxfp4(rows_d[k0:k1, :, 64:], rows_s[k0:k1, :, 4:]))
        K = K.transpose(0, 1).repeat_interleave(Hq // Hkv, 0) * ks
        V = V.transpose(0, 1).repeat_interleave(Hq // Hkv, 0) * vs
        mask = torch.arange(sk)[None, :] <= torch.arange(sk - sq, sk)[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None], K[None].contiguous(), V[None].contiguous(), attn_mask=mask, scale=sm)[0]
        np.testing.assert_allclose(got[q0:q1], ref.transpose(0, 1).numpy(), rtol=1e-10, atol=1e-12)
