"""msa_check_varlen on the GPU: consistent metadata reads 0, and each planted
contradiction between the device metadata and the host-side sizes sets its
flag (the contradictions are planted on the host, into copies of the arrays;
the check reads only inside the arrays the host-side sizes describe)."""
import numpy as np
import pytest
import torch

import workloads
import fp8_top_page_amd as msa

pytestmark = pytest.mark.gpu
F = msa.BAD_FLAGS


def _batch():
    wl = workloads.custom("edge", 31, (40, 0, 300), (5000, 700, 2000), 1, 8, 1)
    return workloads.make_inputs(wl)


def _run(inp, cu_q=None, cu_k=None, bt=None, num_pages=None, **host):
    dev = torch.device("cuda", 0)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    sizes = dict(total_q=inp.total_q, max_seqlen_q=int(np.diff(inp.cu_seqlens_q).max()),
                 max_seqlen_k=int(np.diff(inp.cu_seqlens_k).max()), total_rows=inp.total_rows,
                 max_pages=inp.max_pages)
    sizes.update(host)
    vl = msa.Varlen(t(inp.cu_seqlens_q if cu_q is None else cu_q),
                    t(inp.cu_seqlens_k if cu_k is None else cu_k),
                    t(inp.block_table if bt is None else bt), **sizes)
    flags = torch.full((1,), -1, dtype=torch.int32, device=dev)
    msa.msa_check_varlen(vl, inp.num_pages if num_pages is None else num_pages, flags)
    torch.cuda.synchronize()
    return int(flags.item())


def test_consistent_metadata_reads_zero():
    assert _run(_batch()) == 0
    # more used block-table entries than the check's threads: 1,563 pages
    wl = workloads.custom("edge", 32, (64, 5), (200000, 300), 1, 8, 1)
    assert _run(workloads.make_inputs(wl)) == 0


def test_each_contradiction_sets_its_flag():
    inp = _batch()
    cu_q, cu_k, bt = inp.cu_seqlens_q.copy(), inp.cu_seqlens_k.copy(), inp.block_table.copy()

    c = cu_q.copy(); c[1], c[2] = c[2] + 1, c[2]                # a decrease
    assert _run(inp, cu_q=c) & F["cu_q"]
    c = cu_q.copy(); c[0] = 1                                     # does not start at 0
    assert _run(inp, cu_q=c) & F["cu_q"]

    c = cu_k.copy(); c[1] = cu_k[0] + 10                          # 10 tokens for 40 new ones
    got = _run(inp, cu_k=c)
    # request 1 then holds 5,690 tokens: 45 pages (40 at most), the 40 block-
    # table columns read holding padding; the page total stays 62
    assert got == F["cu_k"] | F["max_k"] | F["pages"] | F["block"], got

    assert _run(inp, max_seqlen_q=200) == F["max_q"]              # request 2 has 300 queries
    got = _run(inp, max_seqlen_k=4000)                            # request 0 has 5000 tokens
    assert got & F["max_k"] and not got & F["pages"]
    small = inp.max_pages - 1                                     # request 0 needs all its pages
    got = _run(inp, max_seqlen_k=small * 128, max_pages=small)
    assert got & F["pages"] and got & F["max_k"]
    assert _run(inp, total_rows=inp.total_rows - 1) == F["rows"]

    b = bt.copy(); b[0, 3] = inp.num_pages                        # past the pool
    assert _run(inp, bt=b) == F["block"]
    b = bt.copy(); b[2, 15] = -1                                  # a used page of request 2
    assert _run(inp, bt=b) == F["block"]
    b = bt.copy(); b[1, bt.shape[1] - 1] = -1                     # an unused column: fine
    assert int(np.ceil(700 / 128)) < bt.shape[1]
    assert _run(inp, bt=b) == 0
    used = max(int(bt[b, :int(np.ceil((cu_k[b + 1] - cu_k[b]) / 128))].max()) for b in range(3))
    assert _run(inp, num_pages=used) == F["block"]                # a pool one page too small
