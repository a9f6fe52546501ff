"""The four calls captured in HIP graphs (torch.cuda.CUDAGraph over the caller's
stream) and replayed: every replay must reproduce the eager results bit for bit.

The calls promise not to allocate, synchronise or read device memory from the
host, so they can be captured; the library clears its own scratch with kernels
(no memset nodes).  Outputs are overwritten with sentinels by eager work between
replays, with synchronisations, so a replay that skips a step shows.
"""
import numpy as np
import pytest
import torch

import workloads
from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["q128_kv32k", "ragged_b8"])
def test_graph_replays_match_eager(name):
    print(f"\n[graph] workload {name}", flush=True)
    inp = workloads.make_inputs(workloads.WORKLOADS[name])
    db = DeviceBatch.from_inputs(inp)
    path = MsaPath(db)
    calls = [path.score, path.select, path.csr, path.attend]
    path.run()
    torch.cuda.synchronize()
    visible = torch.isfinite(path.scores)
    ref = [path.scores[visible].clone(), path.topk.clone(), path.row_ptr.clone(),
           path.q_indices[:int(path.row_ptr[-1])].clone(), path.out.clone()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the calls on the capture stream
        path.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for c in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            c()
        graphs.append(g)
    torch.cuda.synchronize()

    for rep in range(3):
        path.scores.masked_fill_(visible, -3.0)
        path.topk.fill_(-9)
        path.row_ptr.fill_(-9)
        path.q_indices.fill_(-9)
        path.out.fill_(7.0)
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        got = [path.scores[visible], path.topk, path.row_ptr,
               path.q_indices[:int(path.row_ptr[-1])], path.out]
        for k, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {rep}: output {k} differs from the eager run"
        print(f"[graph] {name}: replay {rep} matches eager", flush=True)


def test_graph_replays_quantize_insert_and_mxfp4_scores():
    """The cache-write calls and scoring from MXFP4 keys captured and replayed."""
    from fp8_top_page_amd import (msa_insert_index_k, msa_insert_index_k_mxfp4, msa_insert_kv,
                                  msa_quantize_e4m3)
    print("\n[graph] quantise, inserts, MXFP4 scores", flush=True)
    inp = workloads.make_inputs(workloads.WORKLOADS["decode_b16"], attention=True)
    db = DeviceBatch.from_inputs(inp)
    n, pages = 300, db.num_pages
    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn(n, 2 * 128, generator=g, device="cuda", dtype=torch.bfloat16)
    kv = torch.randn(n, db.Hkv, 128, generator=g, device="cuda")
    slots = torch.randperm(pages * 128, generator=torch.Generator().manual_seed(4))[:n].cuda()
    one = torch.ones(1, device="cuda")
    q8 = torch.empty(n, 256, dtype=torch.uint8, device="cuda")
    kc = torch.zeros(pages, 128, 128, dtype=torch.uint8, device="cuda")
    kvc = torch.zeros(pages, db.Hkv, 128, 256, dtype=torch.uint8, device="cuda")
    d4 = torch.zeros(pages, 128, 64, dtype=torch.uint8, device="cuda")
    s4 = torch.zeros(pages, 128, 4, dtype=torch.uint8, device="cuda")
    # MXFP4 keys for the scorer, from the workload's E4M3 keys
    kf = db.k_cache.view(torch.float8_e4m3fn).float().reshape(-1, 128)
    kd = torch.empty(pages, 128, 64, dtype=torch.uint8, device="cuda")
    ks = torch.empty(pages, 128, 4, dtype=torch.uint8, device="cuda")
    msa_insert_index_k_mxfp4(kf, torch.arange(kf.shape[0], device="cuda"), kd, ks, pages)
    db.use_mxfp4_keys(kd, ks)
    path = MsaPath(db)
    calls = [lambda: msa_quantize_e4m3(x, one, q8),
             lambda: msa_insert_index_k(x[:, :128], slots, one, kc, pages),
             lambda: msa_insert_kv(kv, kv, slots, one, one, kvc, pages, db.Hkv),
             lambda: msa_insert_index_k_mxfp4(x[:, 128:], slots, d4, s4, pages),
             path.score]
    outs = [q8, kc, kvc, d4, s4]
    page, row = slots // 128, slots % 128

    def written():    # the bytes the calls write: all of q8, the slot rows of the caches
        return [q8.clone(), kc[page, row], kvc[page, :, row], d4[page, row], s4[page, row],
                path.scores[visible]]

    for c in calls:
        c()
    torch.cuda.synchronize()
    visible = torch.isfinite(path.scores)
    ref = [t.clone() for t in written()]
    graphs = []
    for c in calls:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            c()
        graphs.append(gr)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(0x5A)
        path.scores.masked_fill_(visible, -3.0)
        torch.cuda.synchronize()
        for gr in graphs:
            gr.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(written(), ref)):
            assert torch.equal(a, b), f"replay {rep}: output {k} differs from the eager run"
        print(f"[graph] quantise/insert/MXFP4: replay {rep} matches eager", flush=True)
