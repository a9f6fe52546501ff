"""GPU parity for the E4M3 quantisation and the paged cache inserts: the HIP
kernels through the C ABI against the oracle, bit for bit."""
import math

import numpy as np
import pytest
import torch

import oracle
from fp8_top_page_amd import msa_insert_index_k, msa_insert_kv, msa_quantize_e4m3

pytestmark = pytest.mark.gpu

TABLE = oracle.e4m3_table()
POS = np.array(sorted((c for c in range(128) if not math.isnan(TABLE[c])), key=lambda c: TABLE[c]))


def _scale(s):
    return torch.tensor([s], dtype=torch.float32, device="cuda")


def _rows(x, width=128):
    """Pad a flat float32 array to whole rows of `width`."""
    n = -(-len(x) // width) * width
    out = np.zeros(n, np.float32)
    out[:len(x)] = x
    return out.reshape(-1, width)


def _special_values():
    mids = (TABLE[POS[:-1]] + TABLE[POS[1:]]) / 2.0
    m32 = mids.astype(np.float32)
    vals = [TABLE[POS], mids, np.nextafter(m32, np.float32(-np.inf)), np.nextafter(m32, np.float32(np.inf)),
            [448.0, 463.99, 464.0, 465.0, 479.0, 480.0, 1e30, np.inf, np.nan, 0.0, -0.0, 1e-30, 2.0 ** -10,
             2.0 ** -10 * 1.001, 2.0 ** -130]]
    v = np.concatenate([np.asarray(a, np.float64) for a in vals]).astype(np.float32)
    rng = np.random.default_rng(3)
    rand = np.concatenate([rng.standard_normal(20000) * 100, rng.standard_normal(20000) * 0.01,
                           rng.uniform(-1000, 1000, 5000)]).astype(np.float32)
    return np.concatenate([v, -v, rand])


@pytest.mark.parametrize("scale", [1.0, 0.5, 3.0, 2.0 ** -8, 0.7371])
def test_quantize_f32_special_values(scale):
    x = _rows(_special_values(), 256)                       # heads = 2
    src = torch.from_numpy(x).cuda()
    dst = torch.full(x.shape, 0x55, dtype=torch.uint8, device="cuda")
    msa_quantize_e4m3(src, _scale(scale), dst)
    torch.cuda.synchronize()
    want = oracle.quantize_e4m3(x, scale)
    got = dst.cpu().numpy()
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, (f"{bad[0].size} codes differ, first at {x[bad][:4]}: "
                              f"got {got[bad][:4]}, want {want[bad][:4]}")


@pytest.mark.parametrize("scale", [1.0, 3.0])
def test_quantize_every_bf16_value(scale):
    bits = np.arange(65536, dtype=np.uint32)
    x = (bits << 16).view(np.float32).reshape(-1, 128)       # every bfloat16, widened exactly
    src = torch.from_numpy((bits.astype(np.uint16)).view(np.int16).reshape(-1, 128)).cuda().view(torch.bfloat16)
    dst = torch.empty(src.shape, dtype=torch.uint8, device="cuda")
    msa_quantize_e4m3(src, _scale(scale), dst)
    torch.cuda.synchronize()
    want = oracle.quantize_e4m3(x, scale)
    got = dst.cpu().numpy()
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} codes differ (bf16 inputs {x[bad][:4]})"


def _slots(n_tokens, num_pages, seed, holes=0.1, out_of_range=0.02):
    rng = np.random.default_rng(seed)
    slots = rng.permutation(num_pages * 128)[:n_tokens].astype(np.int64)
    r = rng.random(n_tokens)
    slots[r < holes] = -1
    slots[(r >= holes) & (r < holes + out_of_range)] = num_pages * 128 + 5   # skipped
    return slots


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_insert_index_k(dtype):
    n, pages = 1500, 20
    g = torch.Generator().manual_seed(4)
    k = (torch.randn(n, 128, generator=g) * 3).to(dtype)
    slots = _slots(n, pages, 5)
    cache = torch.full((pages, 128, 128), 0x55, dtype=torch.uint8, device="cuda")
    msa_insert_index_k(k.cuda(), torch.from_numpy(slots).cuda(), _scale(0.0625), cache, pages)
    torch.cuda.synchronize()
    want = np.full((pages, 128, 128), 0x55, np.uint8)
    oracle.insert_index_k(want, k.float().numpy(), np.where(slots < pages * 128, slots, -1), 0.0625)
    assert np.array_equal(cache.cpu().numpy(), want)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_insert_kv(dtype):
    n, pages, hkv = 900, 12, 2
    g = torch.Generator().manual_seed(6)
    k = (torch.randn(n, hkv, 128, generator=g) * 2).to(dtype)
    vbig = (torch.randn(n, hkv + 1, 128, generator=g) * 600).to(dtype)   # V strided, saturates
    v = vbig[:, :hkv]
    slots = _slots(n, pages, 7)
    cache = torch.full((pages, hkv, 128, 256), 0x55, dtype=torch.uint8, device="cuda")
    kd, vd = k.cuda(), vbig.cuda()[:, :hkv]
    msa_insert_kv(kd, vd, torch.from_numpy(slots).cuda(), _scale(1.0), _scale(0.5), cache, pages, hkv)
    torch.cuda.synchronize()
    want = np.full((pages, hkv, 128, 256), 0x55, np.uint8)
    oracle.insert_kv(want, k.float().numpy(), v.float().numpy(),
                     np.where(slots < pages * 128, slots, -1), 1.0, 0.5)
    assert np.array_equal(cache.cpu().numpy(), want)


def test_insert_large_batch_sampled():
    """A whole 32K-token prefill chunk into a 4-head cache: sampled tokens checked."""
    n, pages, hkv = 32768, 300, 4
    g = torch.Generator(device="cuda").manual_seed(8)
    k = torch.randn(n, hkv, 128, generator=g, device="cuda", dtype=torch.bfloat16)
    v = torch.randn(n, hkv, 128, generator=g, device="cuda", dtype=torch.bfloat16)
    slots = torch.from_numpy(_slots(n, pages, 9, holes=0.0, out_of_range=0.0)).cuda()
    cache = torch.zeros((pages, hkv, 128, 256), dtype=torch.uint8, device="cuda")
    msa_insert_kv(k, v, slots, _scale(1.0), _scale(1.0), cache, pages, hkv)
    torch.cuda.synchronize()
    idx = np.random.default_rng(10).choice(n, 64, replace=False)
    s = slots.cpu().numpy()[idx]
    got = cache.cpu().numpy()[s // 128, :, s % 128]
    kk, vv = k.float().cpu().numpy()[idx], v.float().cpu().numpy()[idx]
    want = np.concatenate([oracle.quantize_e4m3(kk, 1.0), oracle.quantize_e4m3(vv, 1.0)], axis=-1)
    assert np.array_equal(got, want)
