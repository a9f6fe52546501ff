"""GPU parity for MXFP4 index keys: the insert (bit-exact against the oracle)
and scoring from MXFP4 keys through both scorer kernels (prefill and
page-parallel decode), with selection, CSR and attention on top."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fp8_top_page_amd import msa_insert_index_k_mxfp4
from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath
from parity import (check_attention, check_csr, check_scores, check_selection_invariants,
                    check_topk_exact_on_gpu_scores, sample_queries, to_np)

pytestmark = pytest.mark.gpu

E2M1 = oracle.e2m1_table()


def _special_rows():
    """Rows of 128 whose blocks test the block rule: zeros, NaN, inf, exact E2M1
    blocks, ties after scaling, tiny (subnormal) and huge magnitudes."""
    rng = np.random.default_rng(1)
    z = np.zeros(32, np.float32)
    blocks = [
        z, z + np.float32(-0.0), np.r_[z[:31], np.nan], np.r_[np.inf, z[1:]],
        E2M1[rng.integers(0, 16, 32)] * 8.0, E2M1[rng.integers(0, 16, 32)] * 2.0 ** -30,
        np.r_[6.0, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75, -5.0, 0.25, z[:22]] * 2.0 ** 5,
        rng.standard_normal(32) * 1e-40, rng.standard_normal(32) * 1e37,
        np.r_[4.0, 3.9999, 7.9, z[:29]], rng.standard_normal(32), rng.standard_normal(32) * 300,
    ]
    rows = np.concatenate([np.asarray(b, np.float32) for b in blocks])
    rows = np.concatenate([rows, rng.standard_normal(4 * 32 * 40).astype(np.float32)])
    return rows.reshape(-1, 128)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_insert_mxfp4_matches_oracle(dtype):
    k = torch.from_numpy(_special_rows()).to(dtype)
    n, pages = k.shape[0], 4
    rng = np.random.default_rng(2)
    slots = rng.permutation(pages * 128)[:n].astype(np.int64)
    slots[::7] = -1
    slots[3] = pages * 128 + 9                      # past the cache: skipped
    data = torch.full((pages, 128, 64), 0x55, dtype=torch.uint8, device="cuda")
    scales = torch.full((pages, 128, 4), 0x55, dtype=torch.uint8, device="cuda")
    msa_insert_index_k_mxfp4(k.cuda(), torch.from_numpy(slots).cuda(), data, scales, pages)
    torch.cuda.synchronize()
    want = oracle.Mxfp4Keys(np.full((pages, 128, 64), 0x55, np.uint8), np.full((pages, 128, 4), 0x55, np.uint8))
    oracle.insert_index_k_mxfp4(want, k.float().numpy(), np.where(slots < pages * 128, slots, -1))
    assert np.array_equal(scales.cpu().numpy(), want.scales)
    assert np.array_equal(data.cpu().numpy(), want.data)


def _random_mxfp4(num_pages, seed):
    rng = np.random.default_rng(seed)
    data = rng.integers(0, 256, (num_pages, 128, 64), dtype=np.uint8)
    scales = rng.integers(118, 131, (num_pages, 128, 4)).astype(np.uint8)
    return data, scales


def _run(inp, data, scales):
    db = DeviceBatch.from_inputs(inp)
    db.use_mxfp4_keys(data, scales)
    path = MsaPath(db)
    path.run()
    torch.cuda.synchronize()
    return path


@pytest.mark.parametrize("sq,sk,H,Hq,Hkv", [
    ((256,), (1024,), 1, 8, 1),                       # tiny prefill, every query
    ((128, 300), (4096, 2000), 2, 16, 2),             # short chunks over a prefix, ragged
    ((700,), (9000,), 4, 32, 4),                      # H = 4, causal pages
    ((64, 3, 50, 0), (9000, 200, 64, 500), 1, 8, 1),  # decode-like: page-parallel kernel
    ((32, 7, 1), (5000, 40, 70000), 2, 16, 2),
    ((16, 9), (3000, 777), 4, 8, 4),
    ((8,) * 40, (12800,) * 40, 1, 8, 1),              # 280 items: several per scorer block
])
def test_scores_from_mxfp4_keys(sq, sk, H, Hq, Hkv):
    print(f"\n[parity] mxfp4 keys sq={sq} sk={sk} H={H}", flush=True)
    inp = workloads.make_inputs(workloads.custom("mxfp4", 13, sq, sk, H, Hq, Hkv))
    data, scales = _random_mxfp4(inp.num_pages, 14)
    path = _run(inp, data, scales)
    scores = to_np(path.scores)
    queries = np.arange(inp.total_q) if inp.total_q <= 512 else sample_queries(inp, 48)
    ref = oracle.index_scores(inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table, inp.index_q,
                              oracle.Mxfp4Keys(data, scales), inp.index_q_scale,
                              inp.index_k_scale, queries=queries)
    check_scores(inp, scores, queries, ref=ref)
    sel = to_np(path.topk)[:, 0, :]
    check_selection_invariants(inp, sel)
    check_topk_exact_on_gpu_scores(inp, scores, sel)
    check_csr(inp, sel, to_np(path.row_ptr), to_np(path.q_indices))
    att_q = queries[:64]
    check_attention(inp, sel, to_np(path.out.float()).reshape(inp.total_q, Hq, 128), att_q)


def test_long_context_mxfp4_sampled():
    """2,048 queries at the end of a 262,144-token KV from MXFP4 keys: sampled scores."""
    inp = workloads.make_inputs(workloads.custom("mxfp4_long", 15, (2048,), (262144,), 1, 8, 1),
                                attention=False)
    data, scales = _random_mxfp4(inp.num_pages, 16)
    db = DeviceBatch.from_inputs(inp)
    db.use_mxfp4_keys(data, scales)
    path = MsaPath(db)
    path.score()
    torch.cuda.synchronize()
    queries = sample_queries(inp, 16)
    ref = oracle.index_scores(inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table, inp.index_q,
                              oracle.Mxfp4Keys(data, scales), inp.index_q_scale,
                              inp.index_k_scale, queries=queries)
    check_scores(inp, to_np(path.scores), queries, ref=ref)
