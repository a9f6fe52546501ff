"""Pins for oracle.topk_select and oracle.k2q_csr."""
import json
import os

import numpy as np
import pytest

import oracle
from helpers import CODE, PAGE, D, varlen, scatter_pages

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def check_selection_invariants(cu_q, cu_k, sel, topk=16, n_local=1):
    """Invariants of the case() construction: local page forced, no future page,
    k = min(topk, visible), no duplicates, -1 only in the tail."""
    _, pos = oracle.query_positions(cu_q, cu_k)
    for i in range(sel.shape[0]):
        v = int(pos[i] // PAGE + 1)
        k = min(topk, v)
        row = sel[i]
        assert np.all(row[k:] == -1)
        got = row[:k]
        assert np.all(got >= 0) and np.all(got < v)
        assert len(set(got.tolist())) == k
        assert got[0] == v - 1
        for f in range(min(n_local, k)):
            assert got[f] == v - 1 - f


def test_hand_ranking_cases():
    spec = json.load(open(os.path.join(GOLDEN, "topk_hand_case.json")))
    cu_q, cu_k, bt, num_pages = varlen([1], [2560], seed=5)
    q = np.zeros((1, 1, D), np.uint8)
    q[0, 0, 0] = CODE[1.0]
    for case in spec["cases"]:
        rows = np.zeros((2560, D), np.uint8)
        for j in range(20):
            code = eval(case["code_of_page"], {"j": j})
            rows[PAGE * j:PAGE * (j + 1), 0] = code
        kc = scatter_pages(rows, cu_k, bt, num_pages, (D,))
        sc = oracle.index_scores(cu_q, cu_k, bt, q, kc, 1.0, 1.0)
        if "scores" in case:
            assert sc[0].tolist() == case["scores"]
        sel = oracle.topk_select(cu_q, cu_k, sc, 16, case["n_local"])
        assert sel[0].tolist() == case["expected"], case["name"]


def test_all_visible_when_at_most_16_pages():
    rng = np.random.default_rng(0)
    cu_q, cu_k = np.array([0, 300, 310], np.int32), np.array([0, 1024, 3000], np.int32)
    _, pos = oracle.query_positions(cu_q, cu_k)
    sc = rng.standard_normal((310, 30))
    sel = oracle.topk_select(cu_q, cu_k, sc)
    check_selection_invariants(cu_q, cu_k, sel)
    for i in range(300):                     # first request has 8 pages: all selected
        v = int(pos[i] // PAGE + 1)
        assert sorted(sel[i, :v].tolist()) == list(range(v))


@pytest.mark.parametrize("n_local", [1, 2, 3])
def test_brute_force_sort(n_local):
    rng = np.random.default_rng(n_local)
    cu_q = np.array([0, 40, 45], np.int32)
    cu_k = np.array([0, 3000, 3000 + 5000], np.int32)
    _, pos = oracle.query_positions(cu_q, cu_k)
    # coarse values force many exact ties
    sc = rng.integers(-3, 4, size=(45, 40)).astype(np.float64)
    sel = oracle.topk_select(cu_q, cu_k, sc, 16, n_local)
    check_selection_invariants(cu_q, cu_k, sel, 16, n_local)
    for i in range(45):
        v = int(pos[i] // PAGE + 1)
        nf = min(n_local, v)
        rest = sorted(range(v - nf), key=lambda p: (-sc[i, p], p))
        expect = [v - 1 - f for f in range(nf)] + rest[:min(16, v) - nf]
        assert sel[i, :len(expect)].tolist() == expect


def test_csr_is_transpose_of_selection():
    rng = np.random.default_rng(7)
    cu_q = np.array([0, 50, 53, 90], np.int32)
    cu_k = np.array([0, 2000, 2000 + 700, 2700 + 5000], np.int32)
    req, pos = oracle.query_positions(cu_q, cu_k)
    pages = (np.diff(cu_k) + PAGE - 1) // PAGE
    total_rows = int(pages.sum())
    base = np.concatenate([[0], np.cumsum(pages)])
    for n_sel in (1, 2):
        sel = np.stack([oracle.topk_select(cu_q, cu_k, rng.standard_normal((90, 60)))
                        for _ in range(n_sel)], axis=1)
        row_ptr, qidx = oracle.k2q_csr(cu_q, cu_k, sel, total_rows)
        nnz = int((sel >= 0).sum())
        assert row_ptr[0] == 0 and row_ptr[-1] == nnz == len(qidx)
        assert np.all(np.diff(row_ptr) >= 0)
        # brute force, row by row: scan every query's selection
        for g in range(n_sel):
            for b in range(3):
                for j in range(pages[b]):
                    r = g * total_rows + base[b] + j
                    want = [i for i in range(90) if req[i] == b and j in sel[i, g].tolist()]
                    assert qidx[row_ptr[r]:row_ptr[r + 1]].tolist() == want
        # every query is in its own local row
        for i in range(90):
            r = base[req[i]] + pos[i] // PAGE
            assert i in qidx[row_ptr[r]:row_ptr[r + 1]].tolist()


def test_csr_lists_a_query_once_per_row():
    """A page listed twice in one selection is one CSR entry: the rows of a
    selection with repeats equal the brute-force rows of the distinct pages."""
    cu_q = np.array([0, 4], np.int32)
    cu_k = np.array([0, 1000], np.int32)
    sel = np.full((4, 1, 16), -1, np.int32)
    sel[0, 0, :5] = [5, 1, 1, 5, 3]
    sel[1, 0, :3] = [5, 5, 5]
    sel[2, 0, :4] = [7, 0, 7, 0]
    sel[3, 0, :2] = [7, 2]
    row_ptr, qidx = oracle.k2q_csr(cu_q, cu_k, sel, 8)
    rows = [qidx[row_ptr[r]:row_ptr[r + 1]].tolist() for r in range(8)]
    assert rows == [[2], [0], [3], [0], [], [0, 1], [], [2, 3]]
