"""Pins for oracle.index_scores (page score = scaled max over visible tokens of sum_h q_h . k)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from helpers import CODE, PAGE, D, varlen, random_codes, scatter_pages

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand_case():
    spec = json.load(open(os.path.join(GOLDEN, "score_hand_case.json")))
    s = spec["setup"]
    cu_q, cu_k, bt, num_pages = varlen([s["seqlen_q"]], [s["seqlen_k"]], block_tables=[s["block_table"]])
    n = s["seqlen_q"]
    q = np.zeros((n, s["index_heads"], D), np.uint8)
    q[:, 0, 0] = CODE[1.0]
    q[:, 1, 1] = CODE[2.0]
    rows = np.zeros((s["seqlen_k"], D), np.uint8)
    cyc = s["k_dim0_cycle"]
    for t in range(s["seqlen_k"]):
        rows[t, 0] = CODE[cyc[t % len(cyc)]]
    for t in s["k_dim1_ones_at"]:
        rows[t, 1] = CODE[1.0]
    kc = scatter_pages(rows, cu_k, bt, num_pages, (D,))
    return spec, (cu_q, cu_k, bt, q, kc, s["q_scale"], s["k_scale"])


def test_hand_case_golden():
    spec, args = _hand_case()
    sc = oracle.index_scores(*args)
    for pos, page, val in spec["expected"]:
        exp = -np.inf if val == "-inf" else float(val)
        assert sc[pos, page] == exp, (pos, page, sc[pos, page], exp)


def test_hand_case_per_head_golden():
    """The per-head reading (each index head scored alone) on the same hand case."""
    spec, args = _hand_case()
    sc = oracle.index_scores(*args, per_head=True)
    assert sc.shape[1] == 2
    for pos, page, head, val in spec["per_head_expected"]:
        exp = -np.inf if val == "-inf" else float(val)
        assert sc[pos, head, page] == exp, (pos, page, head, sc[pos, head, page], exp)


def _brute_scores(cu_q, cu_k, bt, q, kc, qs, ks, per_head=False):
    """Per-token Python loops; decode through torch's float8 cast (not the oracle table).
    per_head: one score per (query, index head, page), no sum over heads."""
    dec = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).double().tolist()
    out = {}
    for b in range(len(cu_q) - 1):
        sq = int(cu_q[b + 1] - cu_q[b]); sk = int(cu_k[b + 1] - cu_k[b])
        for qi in range(sq):
            i = int(cu_q[b]) + qi
            pos = sk - sq + qi
            qv = [dec(q[i, h]) for h in range(q.shape[1])]
            for j in range(pos // PAGE + 1):
                for hs in ([[h] for h in range(len(qv))] if per_head else [range(len(qv))]):
                    best = None
                    for t in range(PAGE * j, min(PAGE * j + PAGE, pos + 1)):
                        kv = dec(kc[bt[b, j], t - PAGE * j])
                        acc = 0.0
                        for h in hs:
                            for d in range(D):
                                acc += qv[h][d] * kv[d]
                        best = acc if best is None else max(best, acc)
                    out[(i, hs[0], j) if per_head else (i, j)] = best * qs * ks
    return out


@pytest.mark.parametrize("H", [1, 2, 4])
def test_brute_force_tiny(H):
    rng = np.random.default_rng(10 + H)
    cu_q, cu_k, bt, num_pages = varlen([5, 3], [200, 131], spare=2, seed=H)
    total_q, total_k = int(cu_q[-1]), int(cu_k[-1])
    q = random_codes(rng, (total_q, H, D))
    rows = random_codes(rng, (total_k, D))
    kc = scatter_pages(rows, cu_k, bt, num_pages, (D,))
    sc = oracle.index_scores(cu_q, cu_k, bt, q, kc, 0.75, 1.5)
    ref = _brute_scores(cu_q, cu_k, bt, q, kc, 0.75, 1.5)
    seen = set()
    for (i, j), v in ref.items():
        assert sc[i, j] == pytest.approx(v, rel=1e-12, abs=1e-12), (i, j)
        seen.add((i, j))
    # every other entry is not visible
    for i in range(total_q):
        for j in range(sc.shape[1]):
            if (i, j) not in seen:
                assert sc[i, j] == -np.inf


def test_scale_and_block_table_invariance():
    rng = np.random.default_rng(3)
    cu_q, cu_k, bt, num_pages = varlen([40, 7], [300, 520], spare=3, seed=1)
    q = random_codes(rng, (int(cu_q[-1]), 2, D))
    rows = random_codes(rng, (int(cu_k[-1]), D))
    kc = scatter_pages(rows, cu_k, bt, num_pages, (D,))
    base = oracle.index_scores(cu_q, cu_k, bt, q, kc, 0.5, 0.25)
    # doubling q_scale doubles every visible score exactly
    dbl = oracle.index_scores(cu_q, cu_k, bt, q, kc, 1.0, 0.25)
    fin = np.isfinite(base)
    assert np.array_equal(dbl[fin], 2 * base[fin])
    # moving pages physically (new permutation) changes nothing
    _, _, bt2, _ = varlen([40, 7], [300, 520], spare=3, seed=99)
    kc2 = scatter_pages(rows, cu_k, bt2, num_pages, (D,))
    assert np.array_equal(oracle.index_scores(cu_q, cu_k, bt2, q, kc2, 0.5, 0.25), base)
    # an extra all-zero index head changes nothing
    q3 = np.concatenate([q, np.zeros_like(q[:, :1])], axis=1)
    assert np.array_equal(oracle.index_scores(cu_q, cu_k, bt, q3, kc, 0.5, 0.25), base)
    # scores are exact: integer multiples of 2^-18 times the scale product
    units = base[fin] / (0.5 * 0.25) * 2.0 ** 18
    assert np.all(units == np.round(units))


def test_query_subset_matches_full():
    rng = np.random.default_rng(4)
    cu_q, cu_k, bt, num_pages = varlen([30, 10], [700, 260], seed=2)
    q = random_codes(rng, (int(cu_q[-1]), 1, D))
    rows = random_codes(rng, (int(cu_k[-1]), D))
    kc = scatter_pages(rows, cu_k, bt, num_pages, (D,))
    full = oracle.index_scores(cu_q, cu_k, bt, q, kc, 1.0, 1.0)
    sub = [0, 5, 29, 30, 39]
    part = oracle.index_scores(cu_q, cu_k, bt, q, kc, 1.0, 1.0, queries=sub)
    assert np.array_equal(part, full[sub])


def test_planted_mistakes_are_caught(monkeypatch):
    """A wrong causal bound or a dropped index head in the oracle fails the hand case."""
    spec, args = _hand_case()
    real_positions = oracle.msa.query_positions

    def shifted(cu_q, cu_k):
        req, pos = real_positions(cu_q, cu_k)
        return req, pos + 1                     # off-by-one position
    monkeypatch.setattr(oracle.msa, "query_positions", shifted)
    with pytest.raises(AssertionError):
        test_hand_case_golden()
    monkeypatch.setattr(oracle.msa, "query_positions", real_positions)

    cu_q, cu_k, bt, q, kc, qs, ks = args
    q_one_head = q[:, :1].copy()                # drop head 1
    sc = oracle.index_scores(cu_q, cu_k, bt, q_one_head, kc, qs, ks)
    assert sc[255, 1] != 0.5 and sc[100, 0] != 0.375


@pytest.mark.parametrize("H", [2, 4])
def test_per_head_brute_force_tiny(H):
    rng = np.random.default_rng(20 + H)
    cu_q, cu_k, bt, num_pages = varlen([4, 3], [190, 140], spare=1, seed=H)
    total_q, total_k = int(cu_q[-1]), int(cu_k[-1])
    q = random_codes(rng, (total_q, H, D))
    rows = random_codes(rng, (total_k, D))
    kc = scatter_pages(rows, cu_k, bt, num_pages, (D,))
    sc = oracle.index_scores(cu_q, cu_k, bt, q, kc, 0.75, 1.5, per_head=True)
    ref = _brute_scores(cu_q, cu_k, bt, q, kc, 0.75, 1.5, per_head=True)
    assert sc.shape[:2] == (total_q, H)
    for (i, h, j), v in ref.items():
        assert sc[i, h, j] == pytest.approx(v, rel=1e-12, abs=1e-12), (i, h, j)
    assert np.isfinite(sc).sum() == len(ref)


def test_per_head_special_cases():
    """One index head: per head equals summed.  A query whose other heads are
    zero: its scores for the non-zero head equal the summed scores, and the zero
    heads score exactly 0 on every visible page."""
    rng = np.random.default_rng(8)
    cu_q, cu_k, bt, num_pages = varlen([20, 9], [600, 300], seed=5)
    rows = random_codes(rng, (int(cu_k[-1]), D))
    kc = scatter_pages(rows, cu_k, bt, num_pages, (D,))
    q1 = random_codes(rng, (int(cu_q[-1]), 1, D))
    assert np.array_equal(oracle.index_scores(cu_q, cu_k, bt, q1, kc, 0.5, 2.0, per_head=True)[:, 0],
                          oracle.index_scores(cu_q, cu_k, bt, q1, kc, 0.5, 2.0))
    q3 = np.zeros((int(cu_q[-1]), 3, D), np.uint8)
    q3[:, 1] = q1[:, 0]
    ph = oracle.index_scores(cu_q, cu_k, bt, q3, kc, 0.5, 2.0, per_head=True)
    summed = oracle.index_scores(cu_q, cu_k, bt, q3, kc, 0.5, 2.0)
    assert np.array_equal(ph[:, 1], summed)
    vis = np.isfinite(summed)
    assert np.all(ph[:, 0][vis] == 0.0) and np.all(ph[:, 2][vis] == 0.0)
