"""Parity helpers: run the HIP path, compare with the oracle by the stated rules.

Rules (the tolerances come from the method's own statement of accuracy for the
attention, vLLM PR 60684 Validation: all but 1e-4 of the elements within
atol/rtol 0.05, the rest within 0.25):
  scores     |s_gpu - s_ref| <= 1e-3 * max(|s_ref|, rms_i), rms_i = RMS of query
             i's visible reference scores (a page with one visible token can
             score near 0, where a purely relative bound is undefined)
  selection  integer outputs: the oracle's top-k applied to the GPU's own scores
             must equal the GPU selection exactly; against the oracle end to end,
             sets may differ only by swaps of pages whose reference scores are
             within the score tolerance
  CSR        bit-exact against the oracle CSR of the GPU's selection
  attention  oracle attention on the GPU's selection; fraction of elements with
             |o - r| > 0.05 + 0.05 |r| at most 1e-4, and max |o - r| <= 0.25
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath

PAGE = 128
SCORE_RTOL = 1e-3
ATTN_TOL = 0.05
ATTN_FRAC = 1e-4
ATTN_MAX = 0.25


def run_path(inp, n_local=1, device="cuda", per_head=False):
    db = DeviceBatch.from_inputs(inp, device)
    path = MsaPath(db, n_local=n_local, per_head=per_head)
    path.run()
    torch.cuda.synchronize()
    return path


def to_np(t):
    return t.detach().cpu().numpy()


def positions(inp):
    return oracle.query_positions(inp.cu_seqlens_q, inp.cu_seqlens_k)


def sample_queries(inp, n, seed=0):
    """Deterministic sample: ends of every request, page boundaries, random."""
    cu_q = np.asarray(inp.cu_seqlens_q)
    total = int(cu_q[-1])
    _, pos = positions(inp)
    pick = set()
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        if q1 > q0:
            pick.update([q0, q1 - 1, (q0 + q1) // 2])
    boundary = np.nonzero(pos % PAGE == 0)[0]
    rng = np.random.default_rng(seed)
    if len(boundary):
        pick.update(rng.choice(boundary, size=min(4, len(boundary)), replace=False).tolist())
    rest = max(0, n - len(pick))
    if total:
        pick.update(rng.choice(total, size=min(rest, total), replace=False).tolist())
    return np.array(sorted(pick), np.int64)


def spread_queries(inp, n, seed=0):
    """About n queries spread over the whole batch: the deterministic sample of
    sample_queries plus one query drawn at random from each of n equal slices of
    the query index range, so every scorer q-block and every query range of the
    attention's item order holds sampled queries."""
    total = inp.total_q
    pick = set(sample_queries(inp, 0, seed).tolist())
    rng = np.random.default_rng(seed + 1)
    edges = np.linspace(0, total, num=min(n, total) + 1).astype(np.int64)
    for a, b in zip(edges[:-1], edges[1:]):
        if b > a:
            pick.add(int(rng.integers(a, b)))
    return np.array(sorted(pick), np.int64)


def check_scores(inp, gpu_scores, queries, ref=None):
    """R1 on the visible entries of the sampled queries; unwritten entries stay NaN."""
    if ref is None:
        ref = oracle.index_scores(inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table, inp.index_q,
                                  inp.index_k_cache, inp.index_q_scale, inp.index_k_scale,
                                  queries=queries)
    _, pos = positions(inp)
    worst = 0.0
    for r, i in enumerate(queries):
        v = int(pos[i] // PAGE + 1)
        s_ref = ref[r, :v]
        s_gpu = gpu_scores[i, :v].astype(np.float64)
        assert np.all(np.isfinite(s_gpu)), f"query {i}: non-finite visible score"
        rms = float(np.sqrt(np.mean(s_ref ** 2)))
        tol = SCORE_RTOL * np.maximum(np.abs(s_ref), rms)
        err = np.abs(s_gpu - s_ref)
        bad = np.nonzero(err > tol)[0]
        assert len(bad) == 0, (f"query {i}: {len(bad)} scores out of tolerance, e.g. page "
                               f"{bad[0]} gpu {s_gpu[bad[0]]} ref {s_ref[bad[0]]}")
        worst = max(worst, float(np.max(err / np.maximum(tol, 1e-300))) if v else 0.0)
        unwritten = gpu_scores[i, v:]
        assert np.all(np.isnan(unwritten)), f"query {i}: entries past the visible pages were written"
    return ref, worst


def check_selection_invariants(inp, sel, topk=16, n_local=1):
    _, pos = positions(inp)
    v = (pos // PAGE + 1).astype(np.int64)
    k = np.minimum(topk, v)
    slots = np.arange(topk)[None, :]
    filled = slots < k[:, None]
    assert np.all(sel[~filled] == -1), "padding must be -1"
    assert np.all((sel >= 0)[filled]) and np.all((sel < v[:, None])[filled]), "page outside 0..v-1"
    for f in range(n_local):
        has = k > f
        assert np.all(sel[has, f] == v[has] - 1 - f), "forced recent pages missing"
    srt = np.sort(np.where(filled, sel, -1 - slots), axis=1)
    assert np.all(np.diff(srt, axis=1) != 0), "duplicate page in a selection"


def check_topk_exact_on_gpu_scores(inp, gpu_scores, gpu_sel, n_local=1, queries=None):
    """The oracle's top-k run on the GPU's own scores must match bit for bit."""
    if queries is None:
        queries = np.arange(inp.total_q)
    ref = oracle.topk_select(inp.cu_seqlens_q, inp.cu_seqlens_k,
                             gpu_scores[queries].astype(np.float64), 16, n_local, queries=queries)
    mism = np.nonzero(np.any(ref != gpu_sel[queries], axis=1))[0]
    assert len(mism) == 0, (f"{len(mism)} selections differ, e.g. query {queries[mism[0]]}: "
                            f"gpu {gpu_sel[queries[mism[0]]].tolist()} oracle {ref[mism[0]].tolist()}")


def check_topk_vs_reference(inp, gpu_sel, ref_scores, queries, n_local=1):
    """Sets equal, except swaps of pages whose reference scores are within tolerance."""
    ref_sel = oracle.topk_select(inp.cu_seqlens_q, inp.cu_seqlens_k, ref_scores, 16, n_local,
                                 queries=queries)
    _, pos = positions(inp)
    swaps = 0
    for r, i in enumerate(queries):
        G = set(int(x) for x in gpu_sel[i] if x >= 0)
        R = set(int(x) for x in ref_sel[r] if x >= 0)
        if G == R:
            continue
        v = int(pos[i] // PAGE + 1)
        s = ref_scores[r, :v]
        rms = float(np.sqrt(np.mean(s ** 2)))
        for p in G - R:
            for pp in R - G:
                assert abs(s[p] - s[pp]) <= SCORE_RTOL * max(abs(s[pp]), rms), (
                    f"query {i}: gpu picked page {p} ({s[p]}) over {pp} ({s[pp]})")
        swaps += len(G - R)
    return swaps


def check_csr(inp, gpu_sel, row_ptr, q_indices, n_sel=1):
    sel = gpu_sel.reshape(gpu_sel.shape[0], n_sel, -1)
    ref_ptr, ref_idx = oracle.k2q_csr(inp.cu_seqlens_q, inp.cu_seqlens_k, sel, inp.total_rows)
    assert np.array_equal(row_ptr, ref_ptr), "row_ptr differs"
    nnz = int(ref_ptr[-1])
    assert np.array_equal(q_indices[:nnz], ref_idx), "q_indices differ"


def check_attention(inp, gpu_sel, gpu_out, queries, n_sel=1, kv_cache=None):
    """kv_cache: the E4M3 K|V cache the reference reads (default inp.kv_cache)."""
    sel = gpu_sel.reshape(gpu_sel.shape[0], n_sel, -1)
    kv = inp.kv_cache if kv_cache is None else kv_cache
    ref = oracle.sparse_attention(inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table, inp.attn_q,
                                  kv, sel, inp.softmax_scale, inp.attn_q_scale,
                                  inp.attn_k_scale, inp.attn_v_scale, queries=queries)
    got = gpu_out[queries].reshape(ref.shape).astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), "non-finite attention output"
    frac = float(np.mean(err > ATTN_TOL + ATTN_TOL * np.abs(ref)))
    mx = float(err.max()) if err.size else 0.0
    assert frac <= ATTN_FRAC, f"{frac:.2e} of elements outside atol/rtol 0.05 (max err {mx:.3f})"
    assert mx <= ATTN_MAX, f"max abs error {mx:.3f} > 0.25"
    return frac, mx
