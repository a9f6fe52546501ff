"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Workloads are the five seeded synthetic batches (tiny 1K prefill, 128 queries
over a 32K prefix, fresh 32K prefill, 2048 queries over a 1M-token KV, ragged
batch of 8) and a decode batch.  Scores, the selection (exact on the GPU's own
scores, and against the oracle end to end up to near-tie swaps) and the CSR
are compared on every query of every workload.  Attention is compared on every
query of the small batches and on at least 2048 queries of the large ones,
spread so that every scorer q-block and every query range of the attention's
item order is sampled.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import (check_attention, check_csr, check_scores, check_selection_invariants,
                    check_topk_exact_on_gpu_scores, check_topk_vs_reference, run_path,
                    spread_queries, to_np)

pytestmark = pytest.mark.gpu

# attention queries per workload (None: every query)
ATTN_SAMPLE = {"tiny_1k": None, "q128_kv32k": None, "fresh_32k": 2048, "q2048_kv1m": None,
               "ragged_b8": 2048, "decode_b16": None}


@functools.lru_cache(maxsize=1)
def _inputs(name):
    return workloads.make_inputs(workloads.WORKLOADS[name])


@pytest.mark.parametrize("name", workloads.ORDER)
def test_workload_parity(name):
    print(f"\n[parity] workload {name}", flush=True)
    inp = _inputs(name)
    path = run_path(inp)
    scores = to_np(path.scores)
    sel = to_np(path.topk)[:, 0, :]
    row_ptr, q_idx = to_np(path.row_ptr), to_np(path.q_indices)
    out = to_np(path.out.float()).reshape(inp.total_q, -1, 128)
    queries = np.arange(inp.total_q)

    ref_scores, worst = check_scores(inp, scores, queries)
    print(f"[parity] {name}: scores ok on all {len(queries)} queries (worst err/tol {worst:.3f})",
          flush=True)
    check_selection_invariants(inp, sel)
    check_topk_exact_on_gpu_scores(inp, scores, sel)
    swaps = check_topk_vs_reference(inp, sel, ref_scores, queries)
    del ref_scores
    print(f"[parity] {name}: selection exact on GPU scores; {swaps} near-tie swaps vs oracle", flush=True)
    check_csr(inp, sel, row_ptr, q_idx)
    print(f"[parity] {name}: CSR bit-exact ({int(row_ptr[-1])} entries)", flush=True)
    n = ATTN_SAMPLE[name]
    att_q = queries if n is None else spread_queries(inp, n)
    frac, mx = check_attention(inp, sel, out, att_q)
    print(f"[parity] {name}: attention ok on {len(att_q)} queries (frac {frac:.2e}, max {mx:.4f})",
          flush=True)


def test_all_pages_selected_equals_dense_attention():
    """Tiny prefill: 8 pages, so the top-16 covers every visible page and the
    block-sparse output must equal dense causal attention (torch, float64, CPU)."""
    inp = _inputs("tiny_1k")
    path = run_path(inp)
    out = to_np(path.out.float()).reshape(inp.total_q, 8, 128)
    dec = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).double()
    sk = 1024
    bt = inp.block_table[0]
    kv = np.concatenate([inp.kv_cache[bt[j], 0] for j in range(8)])        # [1024, 256]
    K = dec(kv[:, :128]) * inp.attn_k_scale
    V = dec(kv[:, 128:]) * inp.attn_v_scale
    Q = dec(inp.attn_q).transpose(0, 1) * inp.attn_q_scale                 # [8, 256, 128]
    pos = torch.arange(sk - 256, sk)
    mask = torch.arange(sk)[None, :] <= pos[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q[None], K[None, None].expand(1, 8, -1, -1), V[None, None].expand(1, 8, -1, -1),
        attn_mask=mask, scale=inp.softmax_scale)[0].transpose(0, 1).numpy()
    err = np.abs(out - ref)
    assert np.mean(err > 0.05 + 0.05 * np.abs(ref)) <= 1e-4 and err.max() <= 0.25


def _small_inputs(seqlen_q, seqlen_k, H=1, Hq=8, Hkv=1, seed=11):
    wl = workloads.custom("edge", seed, seqlen_q, seqlen_k, H, Hq, Hkv)
    return workloads.make_inputs(wl)


@pytest.mark.parametrize("sq,sk,H,Hq,Hkv", [
    ((0, 300, 0, 17), (500, 300, 129, 4000), 2, 16, 2),    # empty requests, ragged tails
    ((1,), (1,), 1, 8, 1),                                   # one token
    ((129,), (257,), 4, 4, 4),                               # one q-head per KV head
    ((600, 70), (20000, 3000), 1, 32, 2),                    # 16 q-heads per KV head
    # decode-like batches (at most 64 / H queries per request: page-parallel scoring)
    ((64, 3, 50, 0), (9000, 200, 64, 500), 1, 8, 1),
    ((32, 7, 1), (5000, 40, 70000), 2, 16, 2),
    ((16, 9), (3000, 777), 4, 8, 4),
    # 40 decode requests of 100 pages plan 280 items of 16 pages: more items
    # than scorer blocks, so blocks score several items in turn
    ((8,) * 40, (12800,) * 40, 1, 8, 1),
    ((4,) * 40, (12800,) * 40, 2, 16, 2),
])
def test_edge_shapes(sq, sk, H, Hq, Hkv):
    print(f"\n[parity] edge shape sq={sq} sk={sk} H={H} Hq={Hq} Hkv={Hkv}", flush=True)
    inp = _small_inputs(sq, sk, H, Hq, Hkv)
    path = run_path(inp)
    scores = to_np(path.scores)
    sel = to_np(path.topk)[:, 0, :]
    queries = np.arange(inp.total_q)
    ref, _ = check_scores(inp, scores, queries)
    check_selection_invariants(inp, sel)
    check_topk_exact_on_gpu_scores(inp, scores, sel)
    check_topk_vs_reference(inp, sel, ref, queries)
    check_csr(inp, sel, to_np(path.row_ptr), to_np(path.q_indices))
    check_attention(inp, sel, to_np(path.out.float()).reshape(inp.total_q, Hq, 128), queries)


@pytest.mark.parametrize("sq,sk,H,Hq,Hkv", [
    ((1500, 700), (40000, 9000), 2, 32, 2),     # 16 q-heads per KV head
    ((1200, 0, 300), (30000, 500, 300), 4, 16, 4),   # 4 per KV head, an empty request
    ((1030,), (70000,), 1, 4, 4),               # one q-head per KV head
])
def test_head_groupings_large_batches(sq, sk, H, Hq, Hkv):
    """Batches of more than 1000 queries with other q-head groupings than the
    workloads' (16, 4 and 1 q-heads per KV head) and an empty request: the
    whole path against the oracle on every query."""
    print(f"\n[parity] head grouping sq={sq} sk={sk} H={H} Hq={Hq} Hkv={Hkv}", flush=True)
    inp = _small_inputs(sq, sk, H, Hq, Hkv, seed=31)
    path = run_path(inp)
    sel = to_np(path.topk)[:, 0, :]
    check_selection_invariants(inp, sel)
    check_csr(inp, sel, to_np(path.row_ptr), to_np(path.q_indices))
    check_attention(inp, sel, to_np(path.out.float()).reshape(inp.total_q, Hq, 128),
                    np.arange(inp.total_q))


def test_per_kv_head_selection_with_repeats_large():
    """One selection per KV head over 1300 queries, some slots repeating a
    page: each (query, KV head) attends to its own distinct pages once."""
    from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath
    inp = _small_inputs((900, 400), (12000, 5000), 1, 16, 2, seed=19)
    sel = workloads.random_topk(inp, n_sel=2, seed=4)
    sel[:, 1, 15] = sel[:, 1, 2]
    sel[:, 0, 13] = np.where(sel[:, 0, 13] >= 0, sel[:, 0, 0], -1)
    db = DeviceBatch.from_inputs(inp)
    path = MsaPath(db, n_sel=2)
    path.topk.copy_(torch.from_numpy(sel))
    path.csr()
    path.attend()
    torch.cuda.synchronize()
    check_csr(inp, sel, to_np(path.row_ptr), to_np(path.q_indices), n_sel=2)
    out = to_np(path.out.float()).reshape(inp.total_q, 16, 128)
    check_attention(inp, sel, out, np.arange(inp.total_q), n_sel=2)


@pytest.mark.parametrize("sq,sk,H", [
    ((300, 40), (9000, 700), 2),
    ((1200,), (30000,), 4),
    ((8,) * 20, (12800,) * 20, 2),              # decode-like: page-parallel scorer
])
def test_per_index_head_selection(sq, sk, H):
    """Index head h scores alone (no head sum) and selects the pages of KV head
    h: per-head scores, per-head top-k, one CSR per KV head and attention
    against the oracle's per-head reading on every query."""
    print(f"\n[parity] per-head selection sq={sq} sk={sk} H=Hkv={H}", flush=True)
    inp = _small_inputs(sq, sk, H, 8 * H, H, seed=23)
    path = run_path(inp, per_head=True)
    scores = to_np(path.scores)                          # [total_q, H, ld]
    sel = to_np(path.topk)                               # [total_q, H, 16]
    queries = np.arange(inp.total_q)
    ref = oracle.index_scores(inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table, inp.index_q,
                              inp.index_k_cache, inp.index_q_scale, inp.index_k_scale,
                              per_head=True)
    for h in range(H):
        check_scores(inp, scores[:, h, :], queries, ref=ref[:, h, :])
        check_selection_invariants(inp, sel[:, h, :])
        check_topk_exact_on_gpu_scores(inp, scores[:, h, :], sel[:, h, :])
        check_topk_vs_reference(inp, sel[:, h, :], ref[:, h, :], queries)
    assert any(not np.array_equal(sel[:, 0], sel[:, h]) for h in range(1, H)), "heads selected alike"
    check_csr(inp, sel, to_np(path.row_ptr), to_np(path.q_indices), n_sel=H)
    check_attention(inp, sel, to_np(path.out.float()).reshape(inp.total_q, 8 * H, 128), queries,
                    n_sel=H)


@pytest.mark.parametrize("sq,sk,H", [((300,), (1000,), 2), ((8, 8, 5), (3000, 5000, 900), 1)])
def test_nan_codes_give_nan_scores(sq, sk, H):
    """A NaN E4M3 code in a visible index key makes that page's score NaN for
    every query that sees the token, and a NaN in a query's index vector makes
    all of its page scores NaN, as the maximum over the products does in the
    oracle (prefill and page-parallel scorers).  The selection ranks NaN
    scores last, ties by page, as the oracle's top-k does on the same scores."""
    from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath
    inp = _small_inputs(sq, sk, H, 8, 1, seed=31)
    kc = inp.index_k_cache.copy()
    bt = np.asarray(inp.block_table)
    kc[bt[0, 1], 17, 5] = 0x7F                  # token 128 + 17 of request 0
    if len(sq) > 1:
        kc[bt[2, 3], 100, 0] = 0x7F             # token 3 * 128 + 100 of request 2
    q = inp.index_q.copy()
    q[3, 0, 9] = 0x7F                           # every score of query 3 (request 0)
    inp.index_k_cache, inp.index_q = kc, q
    db = DeviceBatch.from_inputs(inp)
    path = MsaPath(db)
    path.score()
    path.select()
    torch.cuda.synchronize()
    scores = to_np(path.scores)
    sel = to_np(path.topk)[:, 0, :]
    ref = oracle.index_scores(inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table, inp.index_q,
                              inp.index_k_cache, inp.index_q_scale, inp.index_k_scale)
    _, pos = oracle.query_positions(inp.cu_seqlens_q, inp.cu_seqlens_k)
    n_nan = 0
    for i in range(inp.total_q):
        v = int(pos[i] // 128 + 1)
        r, g = ref[i, :v], scores[i, :v].astype(np.float64)
        assert np.array_equal(np.isnan(r), np.isnan(g)), f"query {i}: NaN pattern differs"
        n_nan += int(np.isnan(r).sum())
        ok = ~np.isnan(r)
        tol = 1e-3 * np.maximum(np.abs(r[ok]), float(np.sqrt(np.mean(r[ok] ** 2))) if ok.any() else 1.0)
        assert np.all(np.abs(g[ok] - r[ok]) <= tol), f"query {i}: scores out of tolerance"
    assert n_nan > 0
    check_topk_exact_on_gpu_scores(inp, scores, sel)


@pytest.mark.parametrize("sq,sk,H", [
    (3000, 40077, 2),      # a chunk over a context: q-blocks of about equal reach
    (3000, 3000, 4),       # a fresh prefill: uneven q-blocks, the plan weighs its sizes
    (2048, 133000, 1),     # two q-blocks over 1,040 pages
    (5, 70000, 1),         # one decode-like request: the page-parallel scorer
    (33000, 33000, 4),     # 129 q-blocks: too many to plan without a plan kernel
])
def test_plans_agree(sq, sk, H):
    """The scorer's work is planned on the host (one request), by the scorer's
    own waves (2..64 requests, at most 128 q-blocks) or by a plan kernel (more).
    One request scored alone, with one empty request after it, and with 65
    empty requests after it -- and with a max_seqlen_k that only bounds its
    length -- must give the same scores bit for bit, and the oracle's on a
    sample."""
    from fp8_top_page_amd import Varlen, msa_index_score, msa_index_score_workspace_size
    from fp8_top_page_amd.pipeline import DeviceBatch
    print(f"\n[parity] plans sq={sq} sk={sk} H={H}", flush=True)
    inp = _small_inputs((sq,), (sk,), H, 8, 1, seed=23)
    db = DeviceBatch.from_inputs(inp)
    ld = (db.max_pages + 3) // 4 * 4

    def score(vl):
        out = torch.full((db.total_q, ld), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(msa_index_score_workspace_size(vl, H), 256), dtype=torch.uint8,
                         device="cuda")
        msa_index_score(vl, db.index_q, H, db.k_cache, db.num_pages, db.iq_scale, db.ik_scale,
                        out, ws)
        torch.cuda.synchronize()
        return out

    def with_empty(n_empty):
        cu_q = torch.tensor([0] + [sq] * (n_empty + 1), dtype=torch.int32, device="cuda")
        cu_k = torch.tensor([0] + [sk] * (n_empty + 1), dtype=torch.int32, device="cuda")
        bt = torch.zeros((n_empty + 1, db.block_table.shape[1]), dtype=torch.int32, device="cuda")
        bt[0] = db.block_table[0]
        return Varlen(cu_q, cu_k, bt, total_q=db.total_q, max_seqlen_q=db.max_seqlen_q,
                      max_seqlen_k=db.max_seqlen_k, total_rows=db.total_rows,
                      max_pages=db.max_pages)

    alone = score(db.vl)
    loose = score(Varlen(db.cu_q, db.cu_k, db.block_table, total_q=db.total_q,
                         max_seqlen_q=db.max_seqlen_q,
                         max_seqlen_k=min(db.max_pages * 128, sk + 100),
                         total_rows=db.total_rows, max_pages=db.max_pages))
    for name, other in (("loose max_seqlen_k", loose), ("one empty request after", score(with_empty(1))),
                        ("65 empty requests after", score(with_empty(65)))):
        assert torch.equal(torch.isnan(alone), torch.isnan(other)), name
        assert torch.equal(alone.nan_to_num(0.0), other.nan_to_num(0.0)), name
    check_scores(inp, to_np(alone), spread_queries(inp, min(sq, 256), seed=3))


def test_empty_batch_is_a_no_op():
    inp = _small_inputs((0, 0), (300, 128))
    path = run_path(inp)
    assert to_np(path.row_ptr).tolist() == [0] * (inp.total_rows + 1)


@pytest.mark.parametrize("n_local", [2, 5, 16])
def test_forced_recent_pages(n_local):
    inp = _small_inputs((300,), (9000,), 2, 16, 2, seed=21)
    path = run_path(inp, n_local=n_local)
    scores = to_np(path.scores)
    sel = to_np(path.topk)[:, 0, :]
    check_selection_invariants(inp, sel, n_local=n_local)
    check_topk_exact_on_gpu_scores(inp, scores, sel, n_local=n_local)
    check_csr(inp, sel, to_np(path.row_ptr), to_np(path.q_indices))


def test_topk_exact_ties_take_lower_pages():
    """Scores with massive exact ties (all equal; coarse levels; a tied top
    level) fed straight to the selection kernel: the result must equal the
    oracle's (equal scores go to the lower page)."""
    from types import SimpleNamespace
    from fp8_top_page_amd import msa_topk_select
    from fp8_top_page_amd.pipeline import DeviceBatch
    sq, sk = np.array([64, 64]), np.array([8192 * 128, 5000])
    cu_q = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(sk)]).astype(np.int32)
    pages = (sk + 127) // 128
    bt = np.zeros((2, pages.max()), np.int32)               # never read by the selection
    dummy_q = np.zeros((128, 1, 128), np.uint8)
    db = DeviceBatch(cu_q, cu_k, bt, dummy_q, np.zeros((1, 128, 128), np.uint8), 1.0, 1.0)
    meta = SimpleNamespace(cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, total_q=128)
    rng = np.random.default_rng(0)
    ld = (db.max_pages + 3) // 4 * 4
    for kind in ("equal", "levels", "tied_top"):
        print(f"\n[parity] top-k ties: {kind}", flush=True)
        if kind == "equal":
            s = np.full((128, ld), 1.5, np.float32)
        elif kind == "levels":
            s = rng.integers(0, 4, size=(128, ld)).astype(np.float32)
        else:
            s = rng.standard_normal((128, ld)).astype(np.float32)
            s[:, ::7] = 9.0
        st = torch.from_numpy(s).cuda()
        out = torch.full((128, 16), -7, dtype=torch.int32, device="cuda")
        msa_topk_select(db.vl, st, 16, 1, out)
        torch.cuda.synchronize()
        check_topk_exact_on_gpu_scores(meta, s, to_np(out))


@pytest.mark.parametrize("kind", ["random", "levels", "late_top"])
def test_topk_rows_longer_than_one_chunk(kind):
    """Rows of more candidate pages than the block kernel holds in registers at
    once (8192): requests of 11,719 and 20,313 pages, so the selection runs its
    chunked passes (one, two and three re-reads of the row).  Random rows,
    rows of four score levels (many exact ties, more candidates than the LDS
    list holds) and rows whose best pages all lie past the first chunk; the
    result must equal the oracle's selection on the same scores."""
    from types import SimpleNamespace
    from fp8_top_page_amd import msa_topk_select
    from fp8_top_page_amd.pipeline import DeviceBatch
    print(f"\n[parity] top-k over several chunks: {kind}", flush=True)
    sq, sk = np.array([16, 8]), np.array([1_500_000, 2_600_000])
    cu_q = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(sk)]).astype(np.int32)
    pages = (sk + 127) // 128
    bt = np.zeros((2, pages.max()), np.int32)               # never read by the selection
    db = DeviceBatch(cu_q, cu_k, bt, np.zeros((24, 1, 128), np.uint8),
                     np.zeros((1, 128, 128), np.uint8), 1.0, 1.0)
    meta = SimpleNamespace(cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, total_q=24)
    rng = np.random.default_rng(7)
    ld = (db.max_pages + 3) // 4 * 4
    if kind == "random":
        s = rng.standard_normal((24, ld)).astype(np.float32)
    elif kind == "levels":
        s = rng.integers(0, 4, size=(24, ld)).astype(np.float32)
    else:
        s = rng.standard_normal((24, ld)).astype(np.float32)
        s[:, 8192:] += 10.0
        s[:, 8192 + 3000:8192 + 3040] += 20.0               # the winners, two chunks in
    st = torch.from_numpy(s).cuda()
    out = torch.full((24, 16), -7, dtype=torch.int32, device="cuda")
    msa_topk_select(db.vl, st, 16, 1, out)
    torch.cuda.synchronize()
    check_topk_exact_on_gpu_scores(meta, s, to_np(out))


@pytest.mark.parametrize("pages", [300, 1500, 3000, 8000])
@pytest.mark.parametrize("kind", ["near_top", "near_many", "negative"])
def test_topk_keys_equal_in_their_top_bits(pages, kind):
    """Scores that agree in their top 16 bits and differ below them (40 such
    pages at the top; 3,000 of them, more than the candidate list holds;
    all-negative rows with near ties).  Rows of 2,049..8,192 pages (3,000 and
    8,000) bound the selection by those 16 bits alone until the exact rank;
    300 and 1,500 pages take the wave-per-query and block-per-query kernels.
    The result must equal the oracle's selection on the same scores."""
    from types import SimpleNamespace
    from fp8_top_page_amd import msa_topk_select
    from fp8_top_page_amd.pipeline import DeviceBatch
    print(f"\n[parity] top-k near ties: {kind}, {pages} pages", flush=True)
    sq, sk = np.array([16, 8]), np.array([pages * 128, pages * 64 + 77])
    cu_q = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(sk)]).astype(np.int32)
    pg = (sk + 127) // 128
    bt = np.zeros((2, pg.max()), np.int32)                  # never read by the selection
    db = DeviceBatch(cu_q, cu_k, bt, np.zeros((24, 1, 128), np.uint8),
                     np.zeros((1, 128, 128), np.uint8), 1.0, 1.0)
    meta = SimpleNamespace(cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, total_q=24)
    rng = np.random.default_rng(pages + len(kind))
    ld = (db.max_pages + 3) // 4 * 4 + 4
    s = rng.standard_normal((24, ld)).astype(np.float32)
    n_tied = 40 if kind == "near_top" else 3000
    for r in range(24):
        b = 0 if r < 16 else 1
        vis = (int(sk[b]) - int(sq[b]) + (r - int(cu_q[b]))) // 128 + 1
        cols = rng.choice(vis, size=min(n_tied, vis - 1), replace=False)
        # 5.0 plus multiples of 2^-20 of it: equal top 16 bits, distinct low bits
        s[r, cols] = np.float32(5.0) * (1 + rng.integers(0, 60, size=len(cols)) * 2.0 ** -20)
    if kind == "negative":
        s = -np.abs(s) - np.float32(1.0)
        s[:, ::3] = np.float32(-1.25) * (1 + rng.integers(0, 60, size=s[:, ::3].shape) * 2.0 ** -20)
    s = s.astype(np.float32)
    st = torch.from_numpy(s).cuda()
    out = torch.full((24, 16), -7, dtype=torch.int32, device="cuda")
    msa_topk_select(db.vl, st, 16, 1, out)
    torch.cuda.synchronize()
    check_topk_exact_on_gpu_scores(meta, s, to_np(out))


def test_per_kv_head_selection_and_random_topk():
    """One selection per KV head, drawn like the benchmark script's case():
    CSR and attention against the oracle on that selection."""
    from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath
    inp = _small_inputs((700, 300), (5000, 300), 1, 16, 2, seed=8)
    sel = workloads.random_topk(inp, n_sel=2, seed=3)
    db = DeviceBatch.from_inputs(inp)
    path = MsaPath(db, n_sel=2)
    path.topk.copy_(torch.from_numpy(sel))
    path.csr()
    path.attend()
    torch.cuda.synchronize()
    check_csr(inp, sel, to_np(path.row_ptr), to_np(path.q_indices), n_sel=2)
    out = to_np(path.out.float()).reshape(inp.total_q, 16, 128)
    q = np.arange(0, inp.total_q, 7)
    check_attention(inp, sel, out, q, n_sel=2)


def test_page_listed_twice_is_merged_once():
    """The C ABI takes any selection: one that repeats a page in a query's slots
    must give the CSR of its distinct pages (each query once per row) and
    attention over each page's tokens once, as the oracle computes."""
    from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath
    inp = _small_inputs((300, 40), (6000, 900), 1, 8, 1, seed=14)
    sel = workloads.random_topk(inp, n_sel=1, seed=9)
    sel[:, 0, 15] = sel[:, 0, 1]                 # slot 15 repeats slot 1 (or stays -1)
    sel[:, 0, 14] = np.where(sel[:, 0, 14] >= 0, sel[:, 0, 0], -1)   # and the local page
    db = DeviceBatch.from_inputs(inp)
    path = MsaPath(db)
    path.topk.copy_(torch.from_numpy(sel))
    path.csr()
    path.attend()
    torch.cuda.synchronize()
    check_csr(inp, sel[:, 0, :], to_np(path.row_ptr), to_np(path.q_indices))
    out = to_np(path.out.float()).reshape(inp.total_q, 8, 128)
    check_attention(inp, sel[:, 0, :], out, np.arange(inp.total_q))


def test_page_listed_twice_over_many_row_chunks():
    """Repeated pages where one CSR build block cannot hold all of a query's
    rows: 1,563 pages per selection head (rows in two chunks of 1,024), the
    local page (in the second chunk) and an older page each listed twice, plus
    a second request over 700 pages.  CSR bit-exact, attention on every query
    against the oracle."""
    from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath
    inp = _small_inputs((48, 20), (200000, 89600), 1, 16, 2, seed=23)
    sel = workloads.random_topk(inp, n_sel=2, seed=6)
    sel[:, 0, 12] = np.where(sel[:, 0, 12] >= 0, sel[:, 0, 0], -1)   # the local page again
    sel[:, 1, 15] = sel[:, 1, 3]                                      # an older page again
    sel[:, 1, 7] = np.where(sel[:, 1, 7] >= 0, sel[:, 1, 0], -1)
    db = DeviceBatch.from_inputs(inp)
    path = MsaPath(db, n_sel=2)
    path.topk.copy_(torch.from_numpy(sel))
    path.csr()
    path.attend()
    torch.cuda.synchronize()
    assert inp.total_rows > 1024                   # the CSR build's rows come in two chunks
    check_csr(inp, sel, to_np(path.row_ptr), to_np(path.q_indices), n_sel=2)
    out = to_np(path.out.float()).reshape(inp.total_q, 16, 128)
    check_attention(inp, sel, out, np.arange(inp.total_q), n_sel=2)

def test_large_csr_grid_random_topk():
    """A CSR large enough that its per-block totals go through the separate
    prefix-scan launch (16384 queries of one request over 4160 pages, plus a
    short second request): CSR bit-exact, attention on sampled queries."""
    from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath
    inp = _small_inputs((16384, 100), (532480, 5000), 1, 8, 1, seed=12)
    sel = workloads.random_topk(inp, n_sel=1, seed=5)
    db = DeviceBatch.from_inputs(inp)
    path = MsaPath(db)
    path.topk.copy_(torch.from_numpy(sel))
    print("\n[parity] large CSR grid: csr + attention", flush=True)
    path.csr()
    path.attend()
    torch.cuda.synchronize()
    check_csr(inp, sel[:, 0, :], to_np(path.row_ptr), to_np(path.q_indices))
    out = to_np(path.out.float()).reshape(inp.total_q, 8, 128)
    q = np.concatenate([np.arange(0, 16384, 1021), np.arange(16384, inp.total_q, 9)])
    check_attention(inp, sel[:, 0, :], out, q)


def test_block_table_permutation_is_bitwise_invariant():
    """Moving pages physically (another block table) changes no output bit."""
    a = _small_inputs((200, 90), (3000, 700), 2, 16, 2, seed=4)
    b = _small_inputs((200, 90), (3000, 700), 2, 16, 2, seed=4)
    # re-place b's pages with a different permutation of the same pool
    rng = np.random.default_rng(123)
    perm = rng.permutation(a.num_pages).astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm), dtype=np.int32)
    bt = a.block_table.copy()
    valid = bt >= 0
    bt[valid] = perm[bt[valid]]
    b.block_table = bt
    b.index_k_cache = np.ascontiguousarray(a.index_k_cache[inv])
    b.kv_cache = np.ascontiguousarray(a.kv_cache[inv])
    pa, pb = run_path(a), run_path(b)
    assert torch.equal(pa.scores.nan_to_num(-1.0), pb.scores.nan_to_num(-1.0))
    assert torch.equal(pa.topk, pb.topk)
    assert torch.equal(pa.out, pb.out)


def test_repeatable():
    inp = _small_inputs((500,), (40000,), 4, 32, 4, seed=9)
    p1, p2 = run_path(inp), run_path(inp)
    assert torch.equal(p1.scores.nan_to_num(-1.0), p2.scores.nan_to_num(-1.0))
    assert torch.equal(p1.topk, p2.topk)
    assert torch.equal(p1.row_ptr, p2.row_ptr) and torch.equal(p1.q_indices, p2.q_indices)
    assert torch.equal(p1.out, p2.out)
