"""Seeded synthetic inputs for the MSA sparse-prefill path.

This module only draws random numbers and lays them out in the cache and
metadata formats the path consumes.  It holds none of the path's arithmetic
(no scoring, selection, CSR or attention): both the HIP library and the CPU
oracle read the byte arrays produced here.

Formats (MiniMax-M3 MSA pages):
  * index query   [total_q, H, 128] E4M3 bytes, per-tensor fp32 scale
  * index-K cache [num_pages, 128, 128] E4M3 bytes, one 128-byte row per token
    (indexer-CP page, "FP8 rows (128 B per token)"), addressed through the same
    block table as the K|V cache
  * attention query [total_q, Hq, 128] E4M3 bytes, q_scale 0.5
  * K|V cache [num_pages, Hkv, 128, 256] E4M3 bytes, K = [..., :128],
    V = [..., 128:], unit scales (E4M3-query prefill page, benchmark script)
  * MXFP4 K|V cache (kv_mxfp4): data [num_pages, Hkv, 128, 128] (K codes in
    bytes 0..63, V codes in 64..127, two 4-bit codes per byte) and E8M0 block
    scales [num_pages, Hkv, 128, 8] (K blocks 0..3, V blocks 4..7)
  * cu_seqlens_q / cu_seqlens_k [B+1] int32, block_table [B, max_pages] int32
    padded with -1.  New tokens are the last seqlen_q positions of each request.

Unused token rows of partial pages and the spare pool pages are filled with
0x7F (E4M3 NaN) so that a read outside the visible range shows up as NaN.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

PAGE = 128
HEAD_DIM = 128
TOPK = 16
E4M3_MAX = 448.0
POISON = 0x7F
SPARE_PAGES = 4


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    seqlen_q: tuple
    seqlen_k: tuple
    index_heads: int
    q_heads: int
    kv_heads: int
    shift_fraction: float = 0.0  # fraction of tokens shifted along one direction
    shift_sigmas: float = 3.0
    description: str = ""
    # attention-only stand-in: the selection is drawn at random by the rule of the
    # pages' E4M3-query prefill benchmark (random_topk, one selection per KV head)
    random_selection: bool = False

    @property
    def batch(self) -> int:
        return len(self.seqlen_q)


def _ragged_lengths(seed: int, batch: int = 8):
    """Prefix lengths log-uniform in [512, 150000], chunks uniform in {512, 2048, 8192}."""
    g = torch.Generator().manual_seed(seed)
    u = torch.rand(batch, generator=g, dtype=torch.float64)
    prefix = torch.round(torch.exp(math.log(512.0) + u * (math.log(150000.0) - math.log(512.0))))
    chunk_choice = torch.randint(0, 3, (batch,), generator=g)
    chunks = torch.tensor([512, 2048, 8192])[chunk_choice]
    sq = tuple(int(c) for c in chunks)
    sk = tuple(int(p) + int(c) for p, c in zip(prefix, chunks))
    return sq, sk


def _build_workloads():
    ws = {}
    ws["tiny_1k"] = Workload(
        "tiny_1k", 1, (256,), (1024,), 1, 8, 1,
        description="1 request, 256 new tokens at positions 768..1023 of 1024 (8 pages)")
    ws["q128_kv32k"] = Workload(
        "q128_kv32k", 2, (128,), (32768,), 2, 16, 2,
        description="1 request, 128 new tokens after a 32K-token prefix (256 pages)")
    ws["fresh_32k"] = Workload(
        "fresh_32k", 3, (32768,), (32768,), 4, 32, 4, shift_fraction=0.05,
        description="1 request, fresh causal prefill of 32768 tokens, 5% of tokens shifted 3 sigma")
    ws["q2048_kv1m"] = Workload(
        "q2048_kv1m", 4, (2048,), (1048576,), 1, 8, 1,
        description="1 request, 2048 new tokens at the end of 1,048,576 (8192 pages)")
    sq, sk = _ragged_lengths(5)
    ws["ragged_b8"] = Workload(
        "ragged_b8", 5, sq, sk, 2, 16, 2,
        description="8 requests, log-uniform prefixes in [512,150000], chunks in {512,2048,8192}")
    # decode with speculative verification: eight new tokens per request (one
    # decoded plus seven drafts) over a 128K-token context, the shape of the
    # pages' decode-indexer table (16 and 64 requests, eight queries each)
    ws["decode_b16"] = Workload(
        "decode_b16", 6, (8,) * 16, (131072,) * 16, 1, 8, 1,
        description="16 requests, 8 new tokens each after a 131064-token prefix (1024 pages)")
    ws["decode_b64"] = Workload(
        "decode_b64", 7, (8,) * 64, (131072,) * 64, 1, 8, 1,
        description="64 requests, 8 new tokens each after a 131064-token prefix (1024 pages)")
    # The five attention shapes of the E4M3-query prefill benchmark (vLLM PR
    # 60684, Validation): (q-heads, KV heads, new tokens, cached context), one
    # request, random top-16 per KV head with the local page kept; the timed unit
    # there is the CSR build + attention + combine.  Index inputs are minimal
    # (one head) and unused.
    for k, (hq, hkv, q_len, ctx) in enumerate([(16, 1, 8192, 0), (16, 1, 8192, 32768),
                                               (16, 1, 16384, 114688), (64, 4, 8192, 0),
                                               (64, 4, 8192, 32768)]):
        name = f"p2_h{hq}x{hkv}_q{q_len // 1024}k_c{ctx // 1024}k"
        ws[name] = Workload(
            name, 100 + k, (q_len,), (ctx + q_len,), 1, hq, hkv, random_selection=True,
            description=f"attention stand-in: {hq} q-heads / {hkv} KV heads, {q_len} new tokens "
                        f"after {ctx} cached, random top-16 per KV head")
    return ws


WORKLOADS = _build_workloads()
P2_SHAPES = [n for n in WORKLOADS if n.startswith("p2_")]
ORDER = ["tiny_1k", "q128_kv32k", "fresh_32k", "q2048_kv1m", "ragged_b8", "decode_b16"]


def custom(name, seed, seqlen_q, seqlen_k, index_heads=1, q_heads=8, kv_heads=1,
           shift_fraction=0.0):
    """A small workload of arbitrary shape (tests)."""
    return Workload(name, seed, tuple(int(x) for x in seqlen_q), tuple(int(x) for x in seqlen_k),
                    index_heads, q_heads, kv_heads, shift_fraction)


def to_e4m3_bytes(x: torch.Tensor) -> np.ndarray:
    """Round-to-nearest-even E4M3FN codes (library cast), saturated at +-448."""
    x = torch.clamp(x.float(), -E4M3_MAX, E4M3_MAX)
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@dataclass
class Inputs:
    wl: Workload
    cu_seqlens_q: np.ndarray
    cu_seqlens_k: np.ndarray
    block_table: np.ndarray      # [B, max_pages] int32, -1 padded
    num_pages: int
    total_rows: int
    max_pages: int
    # indexer
    index_q: np.ndarray          # [total_q, H, 128] uint8 (E4M3)
    index_k_cache: np.ndarray    # [num_pages, 128, 128] uint8
    index_q_scale: float
    index_k_scale: float
    # attention (optional)
    attn_q: np.ndarray | None = None        # [total_q, Hq, 128] uint8
    kv_cache: np.ndarray | None = None      # [num_pages, Hkv, 128, 256] uint8
    attn_q_scale: float = 0.5
    attn_k_scale: float = 1.0
    attn_v_scale: float = 1.0
    softmax_scale: float = 1.0 / math.sqrt(HEAD_DIM)
    meta: dict = field(default_factory=dict)

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_seqlen_q(self) -> int:
        return int(np.max(np.diff(self.cu_seqlens_q)))

    @property
    def max_seqlen_k(self) -> int:
        return int(np.max(np.diff(self.cu_seqlens_k)))


def _scatter_tokens(rows: torch.Tensor, cu_k, block_table, pool, fill_shape, dtype_bytes):
    """Place logical token rows [total_k, ...] into physical pages [pool, 128, ...]."""
    cache = np.full((pool, PAGE) + fill_shape, POISON, dtype=np.uint8)
    rows = np.asarray(rows)
    for b in range(len(cu_k) - 1):
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        n = k1 - k0
        full = n // PAGE
        phys = block_table[b, :full]
        if full:
            cache[phys] = rows[k0:k0 + full * PAGE].reshape((full, PAGE) + fill_shape)
        rem = n - full * PAGE
        if rem:
            cache[block_table[b, full], :rem] = rows[k0 + full * PAGE:k1]
    return cache


def make_inputs(wl: Workload, attention: bool = True) -> Inputs:
    g = torch.Generator().manual_seed(wl.seed)
    sq = np.array(wl.seqlen_q, dtype=np.int64)
    sk = np.array(wl.seqlen_k, dtype=np.int64)
    assert np.all(sq <= sk) and np.all(sq >= 0)
    B = len(sq)
    cu_q = np.zeros(B + 1, np.int32)
    cu_k = np.zeros(B + 1, np.int32)
    cu_q[1:] = np.cumsum(sq)
    cu_k[1:] = np.cumsum(sk)
    pages = (sk + PAGE - 1) // PAGE
    total_rows = int(pages.sum())
    max_pages = int(pages.max()) if B else 0
    pool = total_rows + SPARE_PAGES
    perm = torch.randperm(pool, generator=g).numpy().astype(np.int32)
    block_table = np.full((B, max(max_pages, 1)), -1, np.int32)
    off = 0
    for b in range(B):
        block_table[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]

    total_q = int(cu_q[-1])
    total_k = int(cu_k[-1])
    H = wl.index_heads
    iq = torch.randn(total_q, H, HEAD_DIM, generator=g)
    ik = torch.randn(total_k, HEAD_DIM, generator=g)
    meta = {}
    if wl.shift_fraction > 0:
        u = torch.randn(HEAD_DIM, generator=g, dtype=torch.float64)
        u = (u / torch.linalg.norm(u)).float()
        n_shift = int(round(wl.shift_fraction * total_k))
        sel = torch.randperm(total_k, generator=g)[:n_shift]
        shift = wl.shift_sigmas * u
        ik[sel] += shift
        # the same logical tokens, where they are also new (query) tokens
        tok_is_shifted = torch.zeros(total_k, dtype=torch.bool)
        tok_is_shifted[sel] = True
        for b in range(B):
            k0 = int(cu_k[b]); q0 = int(cu_q[b])
            first_new = k0 + int(sk[b] - sq[b])
            mask = tok_is_shifted[first_new:first_new + int(sq[b])]
            idx = torch.nonzero(mask).flatten() + q0
            iq[idx] += shift
        meta["shift_tokens"] = n_shift
        meta["shift_norm"] = float(wl.shift_sigmas)
    q_scale = (float(iq.abs().max()) if iq.numel() else E4M3_MAX) / E4M3_MAX
    k_scale = (float(ik.abs().max()) if ik.numel() else E4M3_MAX) / E4M3_MAX
    q_scale = float(np.float32(q_scale))
    k_scale = float(np.float32(k_scale))
    iq_codes = to_e4m3_bytes(iq / q_scale)
    ik_codes = to_e4m3_bytes(ik / k_scale)
    del iq, ik
    k_cache = _scatter_tokens(ik_codes, cu_k, block_table, pool, (HEAD_DIM,), 1)
    del ik_codes

    inp = Inputs(wl, cu_q, cu_k, block_table, pool, total_rows, max_pages,
                 iq_codes, k_cache, q_scale, k_scale, meta=meta)
    if attention:
        aq = torch.randn(total_q, wl.q_heads, HEAD_DIM, generator=g)
        inp.attn_q = to_e4m3_bytes(aq)
        del aq
        kv_codes = np.empty((total_k, wl.kv_heads, 2 * HEAD_DIM), np.uint8)
        step = 1 << 18
        for t0 in range(0, total_k, step):
            t1 = min(total_k, t0 + step)
            x = torch.randn(t1 - t0, wl.kv_heads, 2 * HEAD_DIM, generator=g) * 0.5
            kv_codes[t0:t1] = to_e4m3_bytes(x)
        # [total_k, Hkv, 256] -> pages [pool, 128, Hkv, 256] -> [pool, Hkv, 128, 256]
        cache = _scatter_tokens(kv_codes, cu_k, block_table, pool, (wl.kv_heads, 2 * HEAD_DIM), 1)
        inp.kv_cache = np.ascontiguousarray(cache.transpose(0, 2, 1, 3))
    return inp


def random_topk(inp: Inputs, n_sel: int, seed: int) -> np.ndarray:
    """A random causal selection obeying the rule of the E4M3-query prefill
    benchmark (vLLM PR 60684, Validation): slot 0 holds the query's own
    (local) page, the next min(16, v) - 1 slots hold distinct older visible
    pages drawn uniformly without replacement, in random order, and the
    remaining slots are -1 (v = visible pages of the query).  One selection
    per selection head.  Returns [total_q, n_sel, 16] int32."""
    rng = np.random.default_rng(seed)
    total_q = inp.total_q
    out = np.full((total_q, n_sel, TOPK), -1, np.int32)
    cu_q = np.asarray(inp.cu_seqlens_q, np.int64)
    cu_k = np.asarray(inp.cu_seqlens_k, np.int64)
    for b in range(len(cu_q) - 1):
        first_new = int(cu_k[b + 1] - cu_k[b]) - int(cu_q[b + 1] - cu_q[b])
        for i in range(int(cu_q[b]), int(cu_q[b + 1])):
            own = (first_new + i - int(cu_q[b])) // PAGE     # the query's page
            n_old = min(TOPK - 1, own)                         # older pages to draw
            for g in range(n_sel):
                out[i, g, 0] = own
                if n_old:
                    out[i, g, 1:1 + n_old] = rng.choice(own, size=n_old, replace=False)
    return out


def kv_mxfp4(inp: Inputs, seed: int, scale_lo: int = 124, scale_hi: int = 126):
    """Random MXFP4 K|V pages for the attention of inp's batch: uniform 4-bit
    codes and E8M0 block scales drawn uniformly from [scale_lo, scale_hi] (so
    elements reach 6 * 2^(scale_hi - 127)).  Token rows outside every request
    (unused rows of partial pages, spare pages) get the NaN scale 0xFF, so that
    a read outside the visible range shows up as NaN.
    Returns (data [num_pages, Hkv, 128, 128], scales [num_pages, Hkv, 128, 8])."""
    rng = np.random.default_rng(seed)
    hkv = inp.wl.kv_heads
    data = rng.integers(0, 256, (inp.num_pages, hkv, PAGE, 128), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, (inp.num_pages, hkv, PAGE, 8), dtype=np.uint8)
    valid = np.zeros((inp.num_pages, PAGE), bool)
    cu_k = np.asarray(inp.cu_seqlens_k, np.int64)
    for b in range(len(cu_k) - 1):
        n = int(cu_k[b + 1] - cu_k[b])
        for j in range((n + PAGE - 1) // PAGE):
            valid[inp.block_table[b, j], :min(PAGE, n - j * PAGE)] = True
    scales.transpose(0, 2, 1, 3)[~valid] = 0xFF      # [pages, 128, Hkv, 8] view
    return data, scales
