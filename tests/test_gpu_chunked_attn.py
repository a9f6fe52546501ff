"""GPU parity of the chunked persistent attention (one long request: work items
in chunks of 512 queries, split rows in a ring of three chunk slots, combine
tasks in the same kernel) against the oracle on every query: fresh prefills of
one to many chunks (ragged last chunk), a chunk of new tokens after a cached
prefix, 8 and 16 q-heads per KV head, one selection per KV head, and MXFP4
K|V pages; plus the library's own split path on the same batch cut in two
requests (which does not take the chunked kernel) giving the same outputs."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath
from parity import check_attention, check_csr, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.skip(
    reason="the chunked persistent attention is switched off: its first GPU runs "
           "(1536 queries, three chunks) did not finish; cause not yet found")]


def _run(inp, sel=None, n_sel=1, kv_fp4=None):
    db = DeviceBatch.from_inputs(inp)
    if kv_fp4 is not None:
        db.use_mxfp4_kv(*kv_fp4)
    path = MsaPath(db, n_sel=n_sel)
    if sel is None:
        path.score()
        path.select()
    else:
        path.topk.copy_(torch.from_numpy(sel))
    path.csr()
    path.attend()
    torch.cuda.synchronize()
    return path, to_np(path.topk), to_np(path.out.float()).reshape(inp.total_q, db.Hq, 128)


@pytest.mark.parametrize("sq,sk,Hq,Hkv", [
    ((600,), (600,), 8, 1),          # two chunks, the second ragged
    ((1536,), (1536,), 16, 2),       # exactly three chunks (every ring slot once)
    ((4000,), (4000,), 32, 4),       # eight chunks: ring slots reused
    ((2500,), (9000,), 16, 1),       # new tokens after a cached prefix, 16 q-heads per KV head
])
def test_chunked_attention_every_query(sq, sk, Hq, Hkv):
    print(f"\n[chunked] sq {sq} sk {sk} Hq {Hq} Hkv {Hkv}", flush=True)
    inp = workloads.make_inputs(workloads.custom("chunked", 50 + Hq, sq, sk, 1, Hq, Hkv))
    _, sel, out = _run(inp)
    frac, mx = check_attention(inp, sel[:, 0, :], out, np.arange(inp.total_q))
    print(f"[chunked] ok: frac {frac:.2e} max {mx:.4f}", flush=True)


def test_chunked_attention_per_kv_head_selection():
    inp = workloads.make_inputs(workloads.custom("chunked_sel", 61, (3000,), (3000,), 1, 32, 4))
    sel = workloads.random_topk(inp, n_sel=4, seed=6)
    path, got, out = _run(inp, sel=sel, n_sel=4)
    check_csr(inp, sel, to_np(path.row_ptr), to_np(path.q_indices), n_sel=4)
    check_attention(inp, sel, out, np.arange(inp.total_q), n_sel=4)


def test_chunked_attention_mxfp4_kv():
    inp = workloads.make_inputs(workloads.custom("chunked_fp4", 62, (2100,), (2100,), 1, 16, 2))
    data, scales = workloads.kv_mxfp4(inp, seed=25)
    _, sel, out = _run(inp, kv_fp4=(data, scales))
    check_attention(inp, sel[:, 0, :], out, np.arange(inp.total_q),
                    kv_cache=oracle.mxfp4_kv_as_e4m3(data, scales))


def test_chunked_equals_split_path():
    """The same queries as one request (chunked kernel) and as two requests over
    the same K|V rows (split path): identical bf16 outputs."""
    inp = workloads.make_inputs(workloads.custom("chunked_eq", 63, (2000,), (2000,), 1, 8, 1))
    _, sel, out1 = _run(inp)
    # two requests: the first 1000 queries, then the rest with their own prefix
    cu_q = np.array([0, 1000, 2000], np.int32)
    cu_k = np.array([0, 1000, 3000], np.int32)
    bt = inp.block_table
    pages1 = (1000 + 127) // 128
    bt2 = np.full((2, bt.shape[1]), -1, np.int32)
    bt2[0, :pages1] = bt[0, :pages1]
    bt2[1, :bt.shape[1]] = bt[0]
    db = DeviceBatch(cu_q, cu_k, bt2, inp.index_q, inp.index_k_cache, inp.index_q_scale,
                     inp.index_k_scale, inp.attn_q, inp.kv_cache, inp.attn_q_scale, inp.attn_k_scale,
                     inp.attn_v_scale, inp.softmax_scale)
    path = MsaPath(db)
    path.topk.copy_(torch.from_numpy(sel))
    path.csr()
    path.attend()
    torch.cuda.synchronize()
    out2 = to_np(path.out.float()).reshape(inp.total_q, 8, 128)
    assert np.array_equal(out1, out2)
