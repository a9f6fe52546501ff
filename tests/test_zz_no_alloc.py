"""msa_index_score_noalloc (work list in the library's built-in buffer) against
msa_index_score (work list in a caller workspace), through the C ABI: calls in
a row on one stream -- a prefill chunk (one request, planned on the host), then
a decode batch of 80 requests and a smaller ragged batch of 70 (more requests
than the scorer's waves plan themselves, so both go through the plan kernel
and the built-in buffer, the second call smaller than the first), then a
3-request batch that the waves plan -- each bit-identical to the workspace
call's scores, entries past the visible pages left unwritten by both."""
import numpy as np
import pytest
import torch

import workloads
from fp8_top_page_amd import (msa_index_score, msa_index_score_noalloc,
                              msa_index_score_workspace_size)
from fp8_top_page_amd.pipeline import DeviceBatch

pytestmark = pytest.mark.gpu

CASES = [
    ("prefill chunk", (3000,), (40000,), 4),          # 3000 queries, prefill scorer
    ("decode batch", (8,) * 80, (9000,) * 80, 1),     # 640 queries, page-parallel scorer
    ("ragged batch", (200, 0, 50) + (3,) * 67, (5000, 100, 900) + (700,) * 67, 2),   # 451 queries
    ("small batch", (200, 0, 50), (5000, 100, 900), 2),   # 250 queries
]


def _score(db, noalloc):
    ld = (db.max_pages + 3) // 4 * 4
    out = torch.full((db.total_q, ld), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        msa_index_score_noalloc(db.vl, db.index_q, db.H, db.k_cache, db.num_pages, db.iq_scale,
                                db.ik_scale, out)
    else:
        ws = torch.empty(max(msa_index_score_workspace_size(db.vl, db.H), 256), dtype=torch.uint8,
                         device="cuda")
        msa_index_score(db.vl, db.index_q, db.H, db.k_cache, db.num_pages, db.iq_scale,
                        db.ik_scale, out, ws)
    return out


def test_noalloc_scoring_equals_workspace_scoring():
    dbs = []
    for k, (name, sq, sk, H) in enumerate(CASES):
        inp = workloads.make_inputs(workloads.custom(name, 40 + k, sq, sk, H), attention=False)
        dbs.append((name, DeviceBatch.from_inputs(inp)))
    # the built-in buffer keeps the previous call's work list: each smaller call
    # must still produce exactly the workspace call's scores
    for name, db in dbs:
        print(f"\n[no-alloc] {name}: {db.total_q} queries", flush=True)
        got = _score(db, True)
        ref = _score(db, False)
        torch.cuda.synchronize()
        assert torch.equal(torch.isnan(got), torch.isnan(ref)), name
        assert torch.equal(got.nan_to_num(0.0), ref.nan_to_num(0.0)), name
