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
