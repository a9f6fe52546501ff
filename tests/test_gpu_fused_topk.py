"""GPU: the fused decode scores + top-16 call (msa_index_score_topk) against the
separate calls (msa_index_score, then msa_topk_select on its scores), which the
workload parity tests check against the oracle: the selections must be equal
bit for bit, including the equal-score rule (lower page first) and the forced
recent pages, on decode batches of 1, 2 and 4 index heads, ragged query counts,
short and very long contexts (many work items per request) and an empty request.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath
from parity import check_selection_invariants, check_topk_exact_on_gpu_scores, to_np

pytestmark = pytest.mark.gpu


def _both(inp, n_local=1, zero_keys=False):
    db = DeviceBatch.from_inputs(inp)
    if zero_keys:                                   # every score 0: ties everywhere
        db.k_cache.zero_()
    sep = MsaPath(db, n_local=n_local)
    sep.score()
    sep.select()
    fused = MsaPath(db, n_local=n_local)
    fused.topk.fill_(-7)
    fused.score_select()
    torch.cuda.synchronize()
    return to_np(sep.scores), to_np(sep.topk)[:, 0, :], to_np(fused.topk)[:, 0, :]


def _compare(inp, n_local=1, zero_keys=False):
    scores, sep, fused = _both(inp, n_local, zero_keys)
    bad = np.nonzero(np.any(sep != fused, axis=1))[0]
    assert len(bad) == 0, (f"{len(bad)} queries differ, e.g. {bad[0]}: separate "
                           f"{sep[bad[0]].tolist()} fused {fused[bad[0]].tolist()}")
    check_selection_invariants(inp, fused, n_local=n_local)
    return scores, fused


@pytest.mark.parametrize("name", ["decode_b16", "decode_b64"])
def test_fused_equals_separate_on_decode_workloads(name):
    print(f"\n[fused-topk] {name}", flush=True)
    inp = workloads.make_inputs(workloads.WORKLOADS[name], attention=False)
    scores, fused = _compare(inp)
    check_topk_exact_on_gpu_scores(inp, scores, fused)


@pytest.mark.parametrize("H,n_local", [(1, 1), (2, 3), (4, 16), (1, 2)])
def test_fused_ragged_decode_shapes(H, n_local):
    """Requests of 1 .. 64/H queries over contexts from one page to 300K tokens
    (about 2350 pages: many items per request), and an empty request."""
    qmax = 64 // H
    sq = [1, qmax, 3, 0, qmax // 2, 7 % qmax + 1, qmax]
    sk = [5, 300, 3000, 900, 300000, 20000, 130000]
    inp = workloads.make_inputs(workloads.custom(f"fused_h{H}", 40 + H, sq, sk, H, 8, 1),
                                attention=False)
    scores, fused = _compare(inp, n_local=n_local)
    check_topk_exact_on_gpu_scores(inp, scores, fused, n_local=n_local)


def test_fused_equal_scores_take_lower_pages():
    inp = workloads.make_inputs(workloads.custom("fused_ties", 45, [8, 8], [70000, 5000], 1, 8, 1),
                                attention=False)
    _, fused = _compare(inp, zero_keys=True)
    _, pos = oracle.query_positions(inp.cu_seqlens_q, inp.cu_seqlens_k)
    v = pos // 128 + 1
    want = np.stack([np.concatenate([[vi - 1], np.arange(15)]) for vi in v])
    assert np.array_equal(fused, want)
