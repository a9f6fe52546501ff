"""Pins for oracle.sparse_attention: dense causal attention and closed forms."""
import numpy as np
import pytest
import torch

import oracle
from helpers import CODE, PAGE, D, varlen, random_codes, scatter_pages


def _setup(seqlen_q, seqlen_k, Hq, Hkv, seed, spare=2):
    rng = np.random.default_rng(seed)
    cu_q, cu_k, bt, num_pages = varlen(seqlen_q, seqlen_k, spare=spare, seed=seed)
    total_q, total_k = int(cu_q[-1]), int(cu_k[-1])
    q = random_codes(rng, (total_q, Hq, D), 0x48)
    kv_rows = random_codes(rng, (total_k, Hkv, 2 * D), 0x40)
    kv = scatter_pages(kv_rows, cu_k, bt, num_pages, (Hkv, 2 * D)).transpose(0, 2, 1, 3).copy()
    return rng, cu_q, cu_k, bt, q, kv, kv_rows


def _full_selection(cu_q, cu_k, n_sel=1):
    """Every visible page selected (valid when at most 16 pages are visible)."""
    _, pos = oracle.query_positions(cu_q, cu_k)
    sel = np.full((len(pos), n_sel, 16), -1, np.int32)
    for i, p in enumerate(pos):
        v = int(p // PAGE + 1)
        assert v <= 16
        sel[i, :, :v] = np.arange(v)[::-1]
    return sel


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (4, 2)])
def test_dense_causal_equivalence(Hq, Hkv):
    """With every visible page selected, sparse attention is dense causal attention."""
    _, cu_q, cu_k, bt, q, kv, kv_rows = _setup([70, 33], [1000, 300], Hq, Hkv, seed=Hq)
    sel = _full_selection(cu_q, cu_k)
    sm, qs, ks, vs = 0.0883883, 0.5, 1.25, 0.75
    got = oracle.sparse_attention(cu_q, cu_k, bt, q, kv, sel, sm, qs, ks, vs)
    dec = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).double()
    for b in range(2):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1]); k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        sq, sk = q1 - q0, k1 - k0
        Q = dec(q[q0:q1]).transpose(0, 1) * qs                 # [Hq, sq, D]
        KV = dec(kv_rows[k0:k1]).transpose(0, 1)               # [Hkv, sk, 2D]
        K = KV[..., :D].repeat_interleave(Hq // Hkv, 0) * ks
        V = KV[..., D:].repeat_interleave(Hq // Hkv, 0) * vs
        pos = torch.arange(sk - sq, sk)
        mask = torch.arange(sk)[None, :] <= pos[:, None]        # [sq, sk]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None], K[None].contiguous(), V[None].contiguous(), attn_mask=mask, scale=sm)[0]
        np.testing.assert_allclose(got[q0:q1], ref.transpose(0, 1).numpy(), rtol=1e-10, atol=1e-12)


def test_closed_forms():
    _, cu_q, cu_k, bt, q, kv, kv_rows = _setup([300], [300], 8, 1, seed=3)
    sel = _full_selection(cu_q, cu_k)
    # one visible token: output is that token's V (times v_scale)
    out = oracle.sparse_attention(cu_q, cu_k, bt, q, kv, sel, 0.1, 1.0, 1.0, 2.0)
    v0 = oracle.decode_e4m3(kv_rows[0, 0, D:])
    for h in range(8):
        assert np.array_equal(out[0, h], 2.0 * v0)
    # constant V rows: output is that constant
    kv_c = kv.copy()
    kv_c[:, :, :, D:] = CODE[0.5]
    out = oracle.sparse_attention(cu_q, cu_k, bt, q, kv_c, sel, 0.1)
    np.testing.assert_allclose(out, 0.5, rtol=0, atol=1e-14)
    # all-zero K: uniform weights, output is the mean of V over the attended tokens
    kv_z = kv.copy()
    kv_z[:, :, :, :D] = 0
    out = oracle.sparse_attention(cu_q, cu_k, bt, q, kv_z, sel, 0.1, queries=[0, 127, 128, 299])
    V = oracle.decode_e4m3(kv_rows[:, 0, D:])
    for r, i in enumerate([0, 127, 128, 299]):
        np.testing.assert_allclose(out[r, 3], V[:i + 1].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_sparse_subset_and_block_table_invariance():
    rng, cu_q, cu_k, bt, q, kv, kv_rows = _setup([20], [3000], 8, 1, seed=5)
    _, pos = oracle.query_positions(cu_q, cu_k)
    sel = np.full((20, 1, 16), -1, np.int32)
    for i in range(20):
        v = int(pos[i] // PAGE + 1)
        others = rng.permutation(v - 1)[:15]
        sel[i, 0, 0] = v - 1
        sel[i, 0, 1:16] = others
    out = oracle.sparse_attention(cu_q, cu_k, bt, q, kv, sel, 0.09, 0.5)
    # dense attention restricted to the selected tokens (explicit mask)
    dec = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).double()
    Kall = dec(kv_rows[:, 0, :D]); Vall = dec(kv_rows[:, 0, D:])
    for i in (0, 7, 19):
        allowed = torch.zeros(3000, dtype=torch.bool)
        for j in sel[i, 0]:
            allowed[PAGE * j:PAGE * (j + 1)] = True
        allowed[pos[i] + 1:] = False
        Q = dec(q[i]) * 0.5
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None, :, None, :], Kall[None, None].expand(1, 8, -1, -1),
            Vall[None, None].expand(1, 8, -1, -1), attn_mask=allowed[None, None, None], scale=0.09)
        np.testing.assert_allclose(out[i], ref[0, :, 0].numpy(), rtol=1e-10, atol=1e-12)
    # physical page placement does not matter
    _, _, bt2, _ = varlen([20], [3000], spare=2, seed=77)
    kv2 = scatter_pages(kv_rows, cu_k, bt2, kv.shape[0], (1, 2 * D)).transpose(0, 2, 1, 3).copy()
    out2 = oracle.sparse_attention(cu_q, cu_k, bt2, q, kv2, sel, 0.09, 0.5)
    assert np.array_equal(out, out2)


def test_per_kv_head_selection():
    """With one selection per KV head, head g only sees its own pages."""
    rng, cu_q, cu_k, bt, q, kv, kv_rows = _setup([4], [2000], 4, 2, seed=6)
    _, pos = oracle.query_positions(cu_q, cu_k)
    sel = np.full((4, 2, 16), -1, np.int32)
    for i in range(4):
        v = int(pos[i] // PAGE + 1)
        sel[i, 0, :2] = [v - 1, 0]
        sel[i, 1, :2] = [v - 1, 1]
    out = oracle.sparse_attention(cu_q, cu_k, bt, q, kv, sel, 0.1)
    shared0 = oracle.sparse_attention(cu_q, cu_k, bt, q, kv, sel[:, :1], 0.1)
    shared1 = oracle.sparse_attention(cu_q, cu_k, bt, q, kv, sel[:, 1:], 0.1)
    assert np.array_equal(out[:, :2], shared0[:, :2])   # heads 0,1 -> KV head 0 -> selection 0
    assert np.array_equal(out[:, 2:], shared1[:, 2:])   # heads 2,3 -> KV head 1 -> selection 1


def test_page_listed_twice_counts_once():
    """The selection is a set: repeating a page in a query's slots attends to its
    tokens once, so the output equals that of the selection without the repeat."""
    rng, cu_q, cu_k, bt, q, kv, kv_rows = _setup([6], [1500], 8, 1, seed=9)
    _, pos = oracle.query_positions(cu_q, cu_k)
    sel = np.full((6, 1, 16), -1, np.int32)
    dup = sel.copy()
    for i in range(6):
        v = int(pos[i] // PAGE + 1)
        sel[i, 0, :3] = [v - 1, 0, 2]
        dup[i, 0, :6] = [v - 1, 0, 2, 0, v - 1, 2]
    a = oracle.sparse_attention(cu_q, cu_k, bt, q, kv, sel, 0.1, 0.5)
    b = oracle.sparse_attention(cu_q, cu_k, bt, q, kv, dup, 0.1, 0.5)
    assert np.array_equal(a, b)
