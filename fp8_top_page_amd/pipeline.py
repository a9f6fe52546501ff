"""Device buffers and the four-call sequence of the MSA prefill path.

Plumbing only: torch allocates device memory; every step runs in libmsa.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (PAGE, TOPK, Varlen, msa_build_k2q_csr, msa_index_score, msa_index_score_mxfp4,
               msa_index_score_topk, msa_index_score_topk_workspace_size,
               msa_index_score_per_head, msa_index_score_workspace_size, msa_k2q_schedule_size,
               msa_sparse_attn_prefill, msa_sparse_attn_prefill_mxfp4,
               msa_sparse_attn_workspace_size, msa_topk_select)


def _dev(x, device, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


class DeviceBatch:
    """Host arrays of one prefill batch copied to the device, with the host-side sizes."""

    def __init__(self, cu_seqlens_q, cu_seqlens_k, block_table, index_q, index_k_cache,
                 index_q_scale, index_k_scale, attn_q=None, kv_cache=None, attn_q_scale=1.0,
                 attn_k_scale=1.0, attn_v_scale=1.0, softmax_scale=None, device="cuda"):
        cu_q = np.asarray(cu_seqlens_q, np.int64)
        cu_k = np.asarray(cu_seqlens_k, np.int64)
        sq, sk = np.diff(cu_q), np.diff(cu_k)
        pages = (sk + PAGE - 1) // PAGE
        self.total_q = int(cu_q[-1])
        self.max_seqlen_q = int(sq.max()) if len(sq) else 0
        self.max_seqlen_k = int(sk.max()) if len(sk) else 0
        self.total_rows = int(pages.sum())
        self.max_pages = max(int(pages.max()) if len(pages) else 0, 1)
        self.device = device
        self.cu_q = _dev(cu_q.astype(np.int32), device)
        self.cu_k = _dev(cu_k.astype(np.int32), device)
        self.block_table = _dev(np.asarray(block_table, np.int32), device)
        self.vl = Varlen(self.cu_q, self.cu_k, self.block_table, total_q=self.total_q,
                         max_seqlen_q=self.max_seqlen_q, max_seqlen_k=self.max_seqlen_k,
                         total_rows=self.total_rows, max_pages=self.max_pages)
        self.k_fp4 = None            # (data, scales) of MXFP4 index keys, if scored from those
        self.kv_fp4 = None           # (data, scales) of an MXFP4 K|V cache, if attended over that
        self.H = int(index_q.shape[1])
        self.index_q = _dev(np.asarray(index_q).reshape(index_q.shape[0], self.H * 128), device)
        self.k_cache = _dev(index_k_cache, device)
        self.num_pages = int(index_k_cache.shape[0])
        self.iq_scale = torch.tensor([index_q_scale], dtype=torch.float32, device=device)
        self.ik_scale = torch.tensor([index_k_scale], dtype=torch.float32, device=device)
        self.attn_q = None
        if attn_q is not None:
            self.Hq = int(attn_q.shape[1])
            self.Hkv = int(kv_cache.shape[1])
            self.attn_q = _dev(np.asarray(attn_q).reshape(attn_q.shape[0], self.Hq * 128), device)
            self.kv = _dev(kv_cache, device)
            self.aq_scale = torch.tensor([attn_q_scale], dtype=torch.float32, device=device)
            self.ak_scale = torch.tensor([attn_k_scale], dtype=torch.float32, device=device)
            self.av_scale = torch.tensor([attn_v_scale], dtype=torch.float32, device=device)
            self.softmax_scale = float(softmax_scale if softmax_scale is not None else 128 ** -0.5)

    @classmethod
    def from_inputs(cls, inp, device="cuda"):
        return cls(inp.cu_seqlens_q, inp.cu_seqlens_k, inp.block_table, inp.index_q,
                   inp.index_k_cache, inp.index_q_scale, inp.index_k_scale, inp.attn_q,
                   inp.kv_cache, inp.attn_q_scale, inp.attn_k_scale, inp.attn_v_scale,
                   inp.softmax_scale, device)

    def use_mxfp4_keys(self, data, scales):
        """Score from MXFP4 index keys (uint8 [pages, 128, 64] and [pages, 128, 4]),
        host arrays or device tensors."""
        def on_dev(x):
            if isinstance(x, torch.Tensor):
                return x.to(self.device).contiguous()
            return _dev(x, self.device)
        self.k_fp4 = (on_dev(data), on_dev(scales))

    def use_mxfp4_kv(self, data, scales):
        """Attend over an MXFP4 K|V cache (uint8 [pages, Hkv, 128, 128] codes and
        [pages, Hkv, 128, 8] scales), host arrays or device tensors."""
        def on_dev(x):
            if isinstance(x, torch.Tensor):
                return x.to(self.device).contiguous()
            return _dev(x, self.device)
        self.kv_fp4 = (on_dev(data), on_dev(scales))


class MsaPath:
    """Outputs and workspaces for one batch; run the four calls in order.

    per_head=True: each index head h scores alone and selects the pages of KV
    head h (scores [total_q, H, ld], top-k [total_q, H, 16], one CSR per KV
    head); it needs H == num_kv_heads."""

    def __init__(self, db: DeviceBatch, n_local: int = 1, n_sel: int = 1, score_fill=float("nan"),
                 per_head: bool = False):
        self.db = db
        self.n_local = n_local
        self.per_head = per_head
        if per_head:
            n_sel = db.H
            if db.attn_q is not None and db.Hkv != db.H:
                raise ValueError("per-head selection needs as many index heads as KV heads")
        self.n_sel = n_sel
        dev = db.device
        vl = db.vl
        self.ld = (db.max_pages + 3) // 4 * 4
        shape = (db.total_q, db.H, self.ld) if per_head else (db.total_q, self.ld)
        self.scores = torch.full(shape, score_fill, dtype=torch.float32, device=dev)
        self.ws_score = torch.empty(max(msa_index_score_workspace_size(vl, db.H), 256),
                                    dtype=torch.uint8, device=dev)
        self.topk = torch.full((db.total_q, n_sel, TOPK), -7, dtype=torch.int32, device=dev)
        rows = n_sel * db.total_rows
        self.row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
        self.q_indices = torch.empty(max(n_sel * db.total_q * TOPK, 1), dtype=torch.int32, device=dev)
        self.schedule = torch.empty(msa_k2q_schedule_size(vl, n_sel, TOPK), dtype=torch.uint8,
                                    device=dev)
        if db.attn_q is not None:
            self.out = torch.empty((db.total_q, db.Hq * 128), dtype=torch.bfloat16, device=dev)
            self.ws_attn = torch.empty(max(msa_sparse_attn_workspace_size(vl, db.Hq, db.Hkv, n_sel,
                                                                          TOPK), 256),
                                       dtype=torch.uint8, device=dev)

    def score(self, stream=None):
        db = self.db
        if self.per_head:
            msa_index_score_per_head(db.vl, db.index_q, db.H, db.k_cache, db.num_pages,
                                     db.iq_scale, db.ik_scale, self.scores, self.ws_score, stream)
        elif db.k_fp4 is not None:                # MXFP4 index keys
            msa_index_score_mxfp4(db.vl, db.index_q, db.H, db.k_fp4[0], db.k_fp4[1], db.num_pages,
                                  db.iq_scale, db.ik_scale, self.scores, self.ws_score, stream)
        else:
            msa_index_score(db.vl, db.index_q, db.H, db.k_cache, db.num_pages, db.iq_scale,
                            db.ik_scale, self.scores, self.ws_score, stream)

    def score_select(self, stream=None):
        """Decode-like batches: scores and selection in one fused pass (the scores
        buffer is left untouched)."""
        db = self.db
        if not hasattr(self, "ws_fused"):
            self.ws_fused = torch.empty(max(msa_index_score_topk_workspace_size(db.vl, db.H), 256),
                                        dtype=torch.uint8, device=db.device)
        msa_index_score_topk(db.vl, db.index_q, db.H, db.k_cache, db.num_pages, db.iq_scale,
                             db.ik_scale, TOPK, self.n_local, self.topk[:, 0, :], self.ws_fused,
                             stream)

    def select(self, stream=None):
        if self.per_head:                         # one selection per (query, index head)
            for h in range(self.db.H):
                msa_topk_select(self.db.vl, self.scores[:, h, :], TOPK, self.n_local,
                                self.topk[:, h, :], stream)
        else:
            msa_topk_select(self.db.vl, self.scores, TOPK, self.n_local, self.topk[:, 0, :], stream)

    def csr(self, stream=None, topk=None):
        t = self.topk if topk is None else topk
        if self.n_sel == 1 and t.dim() == 3:
            t = t[:, 0, :]
        msa_build_k2q_csr(self.db.vl, t, self.n_sel, TOPK, self.row_ptr, self.q_indices,
                          self.schedule, stream)

    def attend(self, stream=None):
        db = self.db
        if db.kv_fp4 is not None:
            msa_sparse_attn_prefill_mxfp4(db.vl, db.attn_q, db.Hq, db.kv_fp4[0], db.kv_fp4[1],
                                          db.num_pages, db.Hkv, self.row_ptr, self.q_indices,
                                          self.n_sel, self.schedule, TOPK, db.softmax_scale,
                                          db.aq_scale, db.ak_scale, db.av_scale, self.out,
                                          self.ws_attn, stream)
            return
        msa_sparse_attn_prefill(db.vl, db.attn_q, db.Hq, db.kv, db.num_pages, db.Hkv, self.row_ptr,
                                self.q_indices, self.n_sel, self.schedule, TOPK, db.softmax_scale,
                                db.aq_scale, db.ak_scale, db.av_scale, self.out, self.ws_attn,
                                stream)

    def run(self, stream=None):
        self.score(stream)
        self.select(stream)
        self.csr(stream)
        self.attend(stream)
