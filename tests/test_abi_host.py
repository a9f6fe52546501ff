"""C-ABI library: loads, exports every declared symbol, validates on the host.

These tests make no compute call on a GPU: every call here either fails host
validation (before any HIP call) or, where validation passes, runs only in a
container without a GPU (where it must report MSA_ERR_NO_DEVICE).
"""
import ctypes
import os
import re

import pytest
import torch

import fp8_top_page_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

OK, INVALID, UNSUPPORTED, WS_SMALL, HIP, NO_DEV = 0, 1, 2, 3, 4, 5
FAKE = 0x10000           # aligned, never dereferenced on the host
NO_GPU = not torch.cuda.is_available()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(msa_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    L = msa.lib()
    names = declared_functions()
    assert names == sorted([
        "msa_index_score_workspace_size", "msa_index_score", "msa_topk_select",
        "msa_k2q_schedule_size", "msa_build_k2q_csr", "msa_sparse_attn_workspace_size",
        "msa_sparse_attn_prefill", "msa_status_string", "msa_last_error", "msa_abi_version",
        "msa_quantize_e4m3", "msa_insert_index_k", "msa_insert_kv", "msa_index_score_mxfp4",
        "msa_insert_index_k_mxfp4", "msa_index_score_noalloc", "msa_index_score_per_head",
        "msa_sparse_attn_prefill_mxfp4", "msa_index_score_topk",
        "msa_index_score_topk_workspace_size", "msa_check_varlen"]), names
    for n in names:
        assert hasattr(L, n), n
    assert msa.msa_abi_version() == 3


def test_status_strings():
    for st, name in [(OK, "MSA_OK"), (INVALID, "MSA_ERR_INVALID_ARGUMENT"),
                     (UNSUPPORTED, "MSA_ERR_UNSUPPORTED"), (WS_SMALL, "MSA_ERR_WORKSPACE_TOO_SMALL"),
                     (HIP, "MSA_ERR_HIP"), (NO_DEV, "MSA_ERR_NO_DEVICE")]:
        assert msa.msa_status_string(st) == name


def vl(batch=1, total_q=256, max_q=256, max_k=1024, rows=8, max_pages=8, stride=8):
    c = msa._VarlenC(batch=batch, total_q=total_q, max_seqlen_q=max_q, max_seqlen_k=max_k,
                     total_rows=rows, max_pages=max_pages, cu_seqlens_q=FAKE, cu_seqlens_k=FAKE,
                     block_table=FAKE, block_table_stride=stride)
    return c


def score(v, H=1, q_stride=128, ws=None, ld=8, q=FAKE, num_pages=8):
    L = msa.lib()
    if ws is None:
        ws = L.msa_index_score_workspace_size(ctypes.byref(v), H) or 1 << 20
    return L.msa_index_score(ctypes.byref(v), q, q_stride, H, FAKE, num_pages, FAKE, FAKE, FAKE, ld,
                             0x100000, ws, None)


def test_index_score_validation():
    L = msa.lib()
    assert L.msa_index_score(None, FAKE, 128, 1, FAKE, 8, FAKE, FAKE, FAKE, 8, FAKE, 1 << 20, None) == INVALID
    assert score(vl(), H=3) == UNSUPPORTED
    assert score(vl(), H=8) == UNSUPPORTED
    assert score(vl(), q_stride=64) == INVALID          # < H*128
    assert score(vl(), H=2, q_stride=128) == INVALID
    assert score(vl(), q_stride=136) == INVALID         # not a multiple of 16
    assert score(vl(), q=FAKE + 8) == INVALID           # misaligned
    assert score(vl(), ld=7) == INVALID                 # ld < max_pages
    assert score(vl(), ld=10) == INVALID                # ld not a multiple of 4
    assert score(vl(), num_pages=0) == INVALID
    assert score(vl(), ws=16) == WS_SMALL
    assert score(vl(batch=0)) == INVALID
    assert score(vl(max_pages=4, stride=4)) == INVALID  # 4 pages cannot hold 1024 tokens
    assert score(vl(stride=4)) == INVALID               # block table stride < max_pages
    assert score(vl(max_q=2048)) == INVALID             # max_seqlen_q > max_seqlen_k
    assert "ld_scores" in msa.msa_last_error() or msa.msa_last_error()
    # empty batch: valid, nothing to do
    assert score(vl(total_q=0)) == OK


@pytest.mark.skipif(not NO_GPU, reason="checks the no-device path")
def test_valid_calls_report_no_device_without_gpu():
    assert score(vl()) == NO_DEV
    L = msa.lib()
    v = vl()
    assert L.msa_topk_select(ctypes.byref(v), FAKE, 8, 16, 1, FAKE, 16, None) == NO_DEV
    sz = L.msa_k2q_schedule_size(ctypes.byref(v), 1, 16)
    assert L.msa_build_k2q_csr(ctypes.byref(v), FAKE, 16, 0, 1, 16, FAKE, FAKE, 0x100000, sz, None) == NO_DEV


def test_topk_validation():
    L = msa.lib()
    v = vl()
    assert L.msa_topk_select(ctypes.byref(v), FAKE, 8, 8, 1, FAKE, 16, None) == UNSUPPORTED
    assert L.msa_topk_select(ctypes.byref(v), FAKE, 8, 16, 0, FAKE, 16, None) == UNSUPPORTED
    assert L.msa_topk_select(ctypes.byref(v), FAKE, 8, 16, 17, FAKE, 16, None) == UNSUPPORTED
    assert L.msa_topk_select(ctypes.byref(v), FAKE, 8, 16, 1, FAKE, 15, None) == INVALID
    assert L.msa_topk_select(ctypes.byref(v), None, 8, 16, 1, FAKE, 16, None) == INVALID
    assert L.msa_topk_select(ctypes.byref(v), FAKE, 4, 16, 1, FAKE, 16, None) == INVALID


def test_csr_validation():
    L = msa.lib()
    v = vl()
    sz = L.msa_k2q_schedule_size(ctypes.byref(v), 1, 16)
    assert sz > 0
    assert L.msa_k2q_schedule_size(ctypes.byref(v), 2, 16) > sz
    assert L.msa_k2q_schedule_size(ctypes.byref(v), 1, 8) == 0
    assert L.msa_build_k2q_csr(ctypes.byref(v), FAKE, 16, 0, 1, 8, FAKE, FAKE, 0x100000, sz, None) == UNSUPPORTED
    assert L.msa_build_k2q_csr(ctypes.byref(v), FAKE, 16, 0, 0, 16, FAKE, FAKE, 0x100000, sz, None) == INVALID
    assert L.msa_build_k2q_csr(ctypes.byref(v), FAKE, 16, 0, 1, 16, FAKE, FAKE, 0x100000, sz - 1, None) == WS_SMALL
    assert L.msa_build_k2q_csr(ctypes.byref(v), FAKE, 16, 0, 1, 16, FAKE, FAKE, 0x100008, sz, None) == INVALID
    assert L.msa_build_k2q_csr(ctypes.byref(v), FAKE, 32, 8, 2, 16, FAKE, FAKE, 0x100000, 1 << 30, None) == INVALID
    assert L.msa_build_k2q_csr(ctypes.byref(v), None, 16, 0, 1, 16, FAKE, FAKE, 0x100000, sz, None) == INVALID


def attn(v, Hq=8, Hkv=1, n_sel=1, topk=16, q_stride=1024, out_stride=1024, ws=None, sched=None,
         sm=0.088):
    L = msa.lib()
    if sched is None:
        sched = L.msa_k2q_schedule_size(ctypes.byref(v), n_sel, 16) or 1 << 20
    if ws is None:
        ws = L.msa_sparse_attn_workspace_size(ctypes.byref(v), Hq, Hkv, n_sel, 16) or 1 << 20
    return L.msa_sparse_attn_prefill(ctypes.byref(v), FAKE, q_stride, Hq, FAKE, 8, Hkv, FAKE, FAKE,
                                     n_sel, 0x100000, sched, topk, sm, None, None, None, FAKE,
                                     out_stride, 0x200000, ws, None)


def test_attention_validation():
    v = vl()
    assert attn(v, Hq=8, Hkv=3) == UNSUPPORTED
    assert attn(v, topk=8) == UNSUPPORTED
    assert attn(v, n_sel=2) == UNSUPPORTED
    assert attn(v, q_stride=512) == INVALID
    assert attn(v, out_stride=1023) == INVALID
    assert attn(v, out_stride=1028) == INVALID
    assert attn(v, Hq=128, Hkv=1, q_stride=16384, out_stride=16384) == UNSUPPORTED
    assert attn(v, sm=0.0) == INVALID
    assert attn(v, ws=100) == WS_SMALL
    assert attn(v, sched=100) == WS_SMALL
    assert attn(vl(total_q=0)) == OK


def attn_mx(v, scales=FAKE, Hq=8, Hkv=1, topk=16, sm=0.088):
    L = msa.lib()
    sched = L.msa_k2q_schedule_size(ctypes.byref(v), 1, 16) or 1 << 20
    ws = L.msa_sparse_attn_workspace_size(ctypes.byref(v), Hq, Hkv, 1, 16) or 1 << 20
    return L.msa_sparse_attn_prefill_mxfp4(ctypes.byref(v), FAKE, 1024, Hq, FAKE, scales, 8, Hkv,
                                           FAKE, FAKE, 1, 0x100000, sched, topk, sm, None, None,
                                           None, FAKE, 1024, 0x200000, ws, None)


def test_mxfp4_attention_validation():
    """The MXFP4 K|V entry takes the same checks plus its scales pointer."""
    v = vl()
    assert attn_mx(v, scales=None) == INVALID
    assert attn_mx(v, scales=FAKE + 4) == INVALID          # not 8-byte aligned
    assert attn_mx(v, Hq=8, Hkv=3) == UNSUPPORTED
    assert attn_mx(v, topk=8) == UNSUPPORTED
    assert attn_mx(v, sm=0.0) == INVALID
    assert attn_mx(vl(total_q=0), scales=None) == OK


def test_fused_score_topk_validation():
    """The fused decode scores + top-k call: decode-like batches only."""
    L = msa.lib()

    def fz(v, H=1, topk=16, n_local=1, ws=None, stride=16):
        if ws is None:
            ws = L.msa_index_score_topk_workspace_size(ctypes.byref(v), H) or 1 << 20
        return L.msa_index_score_topk(ctypes.byref(v), FAKE, 128 * H, H, FAKE, 8, FAKE, FAKE, topk,
                                      n_local, FAKE, stride, 0x200000, ws, None)
    dec = vl(batch=2, total_q=16, max_q=8)
    assert fz(vl(total_q=100, max_q=100)) == UNSUPPORTED          # 100 > 64 queries
    assert fz(vl(total_q=40, max_q=40), H=2) == UNSUPPORTED       # 40 > 64 / 2
    assert fz(dec, H=3) == UNSUPPORTED
    assert fz(dec, topk=8) == UNSUPPORTED
    assert fz(dec, n_local=0) == UNSUPPORTED
    assert fz(dec, stride=8) == INVALID
    assert fz(dec, ws=64) == WS_SMALL
    a = L.msa_index_score_topk_workspace_size(ctypes.byref(dec), 1)
    assert a > L.msa_index_score_workspace_size(ctypes.byref(dec), 1)
    assert L.msa_index_score_topk_workspace_size(ctypes.byref(dec), 3) == 0


def test_workspace_sizes_grow_with_the_batch():
    L = msa.lib()
    small, big = vl(), vl(total_q=2048, max_q=2048, max_k=1 << 20, rows=8192, max_pages=8192,
                          stride=8192)
    for H in (1, 2, 4):
        a = L.msa_index_score_workspace_size(ctypes.byref(small), H)
        b = L.msa_index_score_workspace_size(ctypes.byref(big), H)
        assert 0 < a <= b
    assert L.msa_index_score_workspace_size(ctypes.byref(small), 3) == 0
    a = L.msa_sparse_attn_workspace_size(ctypes.byref(small), 8, 1, 1, 16)
    b = L.msa_sparse_attn_workspace_size(ctypes.byref(big), 8, 1, 1, 16)
    assert 0 < a < b
    # partial rows: 16 slots x 8 heads x 144 bytes (128 int8 codes, max and sum,
    # 8 block exponents) per query
    assert b >= 2048 * 16 * 8 * 144


@pytest.mark.skipif(not NO_GPU, reason="host-pointer marshalling check, CPU container only")
def test_pipeline_marshalling_on_host_buffers():
    """The binding's argument marshalling (empty and non-empty batches) up to the
    library's device check; nothing is launched without a GPU."""
    import workloads
    from fp8_top_page_amd.pipeline import DeviceBatch, MsaPath
    for sq, sk in [((0, 0), (300, 128)), ((5, 3), (300, 3))]:
        inp = workloads.make_inputs(workloads.custom("m", 1, sq, sk, 2, 16, 2))
        path = MsaPath(DeviceBatch.from_inputs(inp, device="cpu"))
        for step in (path.score, path.select, path.csr, path.attend):
            try:
                step()
            except msa.MsaError as e:
                assert e.status == NO_DEV, e


def test_quantize_and_insert_validation():
    L = msa.lib()
    BF16, F32 = 0, 1
    q = lambda src=FAKE, dt=BF16, n=4, heads=2, ss=256, sc=FAKE, dst=FAKE, ds=256: \
        L.msa_quantize_e4m3(src, dt, n, heads, ss, sc, dst, ds, None)
    assert q(n=0) == OK                       # nothing to do
    assert q(dt=2) == UNSUPPORTED             # not bf16 / f32
    assert q(n=-1) == INVALID
    assert q(heads=0) == INVALID
    assert q(src=None) == INVALID
    assert q(src=FAKE + 8) == INVALID         # source not 16-byte aligned
    assert q(ss=128) == INVALID               # < heads * 128
    assert q(ss=260) == INVALID               # not a multiple of 8
    assert q(sc=None) == INVALID
    assert q(dst=FAKE + 4) == INVALID         # dst not 8-byte aligned
    assert q(ds=200) == INVALID
    if NO_GPU:                                # validation passes: only reachable without a GPU
        assert q() == NO_DEV
    ik = lambda k=FAKE, dt=F32, n=3, ks=128, slots=FAKE, sc=FAKE, cache=FAKE, pages=2: \
        L.msa_insert_index_k(k, dt, n, ks, slots, sc, cache, pages, None)
    assert ik(n=0) == OK
    assert ik(ks=64) == INVALID
    assert ik(slots=None) == INVALID
    assert ik(pages=0) == INVALID
    assert ik(dt=7) == UNSUPPORTED
    if NO_GPU:
        assert ik() == NO_DEV
    kv = lambda k=FAKE, v=FAKE, dt=BF16, n=3, hkv=2, ks=256, vs=256, slots=FAKE, cache=FAKE, pages=2: \
        L.msa_insert_kv(k, v, dt, n, hkv, ks, vs, slots, FAKE, FAKE, cache, pages, None)
    assert kv(n=0) == OK
    assert kv(hkv=0) == INVALID
    assert kv(v=None) == INVALID
    assert kv(vs=128) == INVALID              # < Hkv * 128
    assert kv(cache=FAKE + 2) == INVALID
    if NO_GPU:
        assert kv() == NO_DEV


def test_mxfp4_validation():
    L = msa.lib()
    v = vl()
    ws = L.msa_index_score_workspace_size(ctypes.byref(v), 1)
    sc = lambda kd=FAKE, ks=FAKE, H=1: L.msa_index_score_mxfp4(
        ctypes.byref(v), FAKE, 128 * H, H, kd, ks, 8, FAKE, FAKE, FAKE, 8, 0x100000, ws, None)
    assert sc(ks=None) == INVALID
    assert sc(ks=FAKE + 4) == INVALID         # scales not 16-byte aligned
    assert sc(H=3) == UNSUPPORTED
    if NO_GPU:
        assert sc() == NO_DEV
    ins = lambda k=FAKE, dt=0, n=5, ks=128, slots=FAKE, kd=FAKE, kscale=FAKE, pages=2: \
        L.msa_insert_index_k_mxfp4(k, dt, n, ks, slots, kd, kscale, pages, None)
    assert ins(n=0) == OK
    assert ins(dt=3) == UNSUPPORTED
    assert ins(ks=120) == INVALID
    assert ins(kscale=None) == INVALID
    assert ins(kd=FAKE + 2) == INVALID
    assert ins(pages=0) == INVALID
    if NO_GPU:
        assert ins() == NO_DEV



def test_noalloc_scoring_validation():
    """The no-allocation scorer: the same argument checks as msa_index_score,
    and batches whose work list exceeds its 1 MiB built-in buffer are rejected
    on the host, before any device call."""
    L = msa.lib()

    def na(v, H=1):
        return L.msa_index_score_noalloc(ctypes.byref(v), FAKE, 128 * H, H, FAKE, 8, FAKE, FAKE,
                                         FAKE, 8, None)
    assert L.msa_index_score_noalloc(None, FAKE, 128, 1, FAKE, 8, FAKE, FAKE, FAKE, 8, None) == INVALID
    assert na(vl(), H=3) == UNSUPPORTED
    assert na(vl(total_q=0)) == OK
    big = vl(batch=4096, total_q=1 << 22, max_q=1024, max_k=1 << 20, rows=4096 * 8192,
             max_pages=8192, stride=8192)
    assert L.msa_index_score_workspace_size(ctypes.byref(big), 1) > 1 << 20
    assert na(big) == UNSUPPORTED
    assert "built-in scratch" in msa.msa_last_error()
    if NO_GPU:
        assert na(vl()) == NO_DEV


def test_per_head_scoring_validation():
    L = msa.lib()

    def ph(v, H=2, ld=16, hs=8, ws=1 << 20):
        return L.msa_index_score_per_head(ctypes.byref(v), FAKE, 128 * H, H, FAKE, 8, FAKE, FAKE,
                                          FAKE, ld, hs, 0x100000, ws, None)
    assert ph(vl(), H=3) == UNSUPPORTED
    assert ph(vl(), hs=6) == INVALID              # head stride not a multiple of 4
    assert ph(vl(), hs=4) == INVALID              # head stride < max_pages
    assert ph(vl(), ld=12) == INVALID             # ld cannot hold 2 heads of stride 8
    assert ph(vl(), ws=16) == WS_SMALL
    assert ph(vl(total_q=0)) == OK
    if NO_GPU:
        assert ph(vl()) == NO_DEV


def test_metadata_check_validation():
    """msa_check_varlen rejects bad host arguments before launching anything;
    a valid call without a GPU reports the missing device."""
    L = msa.lib()
    v = vl()
    assert L.msa_check_varlen(None, 8, FAKE, None) == INVALID
    assert L.msa_check_varlen(ctypes.byref(v), 0, FAKE, None) == INVALID
    assert L.msa_check_varlen(ctypes.byref(v), 8, None, None) == INVALID
    assert L.msa_check_varlen(ctypes.byref(vl(stride=4)), 8, FAKE, None) == INVALID
    if NO_GPU:
        assert L.msa_check_varlen(ctypes.byref(v), 8, FAKE, None) == NO_DEV
