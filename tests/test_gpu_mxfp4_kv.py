"""GPU parity of the attention over MXFP4 K|V pages (msa_sparse_attn_prefill_mxfp4)
against the oracle's attention over the same pages read as E4M3
(oracle.mxfp4_kv_as_e4m3), at the attention tolerance (all but 1e-4 of the
elements within atol/rtol 0.05, the rest within 0.25).  The selection and CSR
come from the E4M3 path (scores of the index cache), or from the random
per-KV-head rule; the MXFP4 pages are seeded random codes and scales.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import workloads
from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath
from parity import check_attention, spread_queries, to_np

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def _inputs(name):
    return workloads.make_inputs(workloads.WORKLOADS[name])


def _run(inp, data, scales, n_sel=1, sel=None, k_scale=None, v_scale=None):
    """Score, select and build the CSR from the E4M3 inputs (or take sel), then
    attend over the MXFP4 pages.  Returns (selection, output [q, Hq, 128])."""
    db = DeviceBatch.from_inputs(inp)
    if k_scale is not None:
        db.ak_scale.fill_(k_scale)
        db.av_scale.fill_(v_scale)
    db.use_mxfp4_kv(data, scales)
    path = MsaPath(db, n_sel=n_sel)
    if sel is None:
        path.score()
        path.select()
    else:
        path.topk.copy_(torch.from_numpy(sel))
    path.csr()
    path.attend()
    torch.cuda.synchronize()
    got_sel = to_np(path.topk)
    return got_sel, to_np(path.out.float()).reshape(inp.total_q, db.Hq, 128)


def _check(inp, data, scales, sel, out, queries, n_sel=1, k_scale=None, v_scale=None):
    if k_scale is not None:
        inp = _with_scales(inp, k_scale, v_scale)
    staged = oracle.mxfp4_kv_as_e4m3(data, scales)
    s = sel if n_sel > 1 else sel[:, 0, :]
    return check_attention(inp, s, out, queries, n_sel=n_sel, kv_cache=staged)


def _with_scales(inp, k_scale, v_scale):
    import copy
    c = copy.copy(inp)
    c.attn_k_scale, c.attn_v_scale = k_scale, v_scale
    return c


@pytest.mark.parametrize("name", ["tiny_1k", "q128_kv32k", "decode_b16"])
def test_mxfp4_kv_workloads_every_query(name):
    print(f"\n[mxfp4-kv] {name}", flush=True)
    inp = _inputs(name)
    data, scales = workloads.kv_mxfp4(inp, seed=21)
    sel, out = _run(inp, data, scales)
    frac, mx = _check(inp, data, scales, sel, out, np.arange(inp.total_q))
    print(f"[mxfp4-kv] {name}: {inp.total_q} queries, frac {frac:.2e}, max {mx:.4f}", flush=True)


def test_mxfp4_kv_fresh_32k_spread():
    """The wide attention kernel (items of up to 64 queries, ordered by query
    range): 2048+ queries spread over the batch."""
    print("\n[mxfp4-kv] fresh_32k", flush=True)
    inp = _inputs("fresh_32k")
    data, scales = workloads.kv_mxfp4(inp, seed=22)
    sel, out = _run(inp, data, scales)
    q = spread_queries(inp, 2048)
    frac, mx = _check(inp, data, scales, sel, out, q)
    print(f"[mxfp4-kv] fresh_32k: {len(q)} queries, frac {frac:.2e}, max {mx:.4f}", flush=True)


@pytest.mark.parametrize("sq,sk,Hq,Hkv", [((700, 300), (5000, 300), 16, 2),
                                          ((1500,), (1500,), 64, 4)])
def test_mxfp4_kv_per_kv_head_selection(sq, sk, Hq, Hkv):
    """One random selection per KV head (the benchmark script's rule), 8 and
    16 q-heads per KV head, non-unit K and V global scales."""
    inp = workloads.make_inputs(workloads.custom("mx_kv", 31, sq, sk, 1, Hq, Hkv))
    data, scales = workloads.kv_mxfp4(inp, seed=23)
    sel = workloads.random_topk(inp, n_sel=Hkv, seed=4)
    got, out = _run(inp, data, scales, n_sel=Hkv, sel=sel, k_scale=1.5, v_scale=0.75)
    assert np.array_equal(got, sel)
    _check(inp, data, scales, sel, out, np.arange(inp.total_q), n_sel=Hkv, k_scale=1.5,
           v_scale=0.75)


def test_mxfp4_kv_wide_scale_range():
    """K block scales from 2^-27 to 2^13: products below E4M3's subnormal step,
    subnormal and saturated (K values up to 448 make the softmax nearly one-hot).
    V block scales 2^-9 .. 2^-5 (subnormal products, and outputs small enough for
    the absolute 0.25 bound)."""
    inp = workloads.make_inputs(workloads.custom("mx_kv_wide", 32, (300, 57), (2000, 57), 1, 8, 1))
    data, scales = workloads.kv_mxfp4(inp, seed=24, scale_lo=100, scale_hi=140)
    v = scales[..., 4:]
    live = v != 0xFF
    v[live] = 118 + v[live] % 5
    sel, out = _run(inp, data, scales)
    _check(inp, data, scales, sel, out, np.arange(inp.total_q))
