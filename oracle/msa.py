"""Oracle: a plain, slow CPU implementation of the MSA sparse-prefill path.

TEST INFRASTRUCTURE ONLY.  Imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the library.  It shares no code, table or
constant generator with the HIP path: both sides only read the same seeded
input bytes.

Sources (MiniMax-M3 MSA pages):
  [P1] vLLM PR 60930, "MiniMax M3 FP8 indexer prefill: persistent CuTe scorer"
       (sections Overview, Details: score-only plan/run_scores API, admission
       E4M3 / D128 / page 128 / H in {1,2,4} / sparse_local_block >= 1).
  [P2] vLLM PR 60684, "MSA prefill reads the E4M3 query natively" (Overview,
       Validation: the benchmark script's case() top-k construction and cache
       layout; Details: scales and E4M3 probability rounding).
  [P3] vLLM PR 64631, "NVFP4 index-cache sharding under indexer CP" (Claims,
       Details: FP8 index rows of 128 B per token, ties).
  [P4] vLLM API docs, vllm.models.minimax_m3.nvidia.sparse_attention_msa,
       MiniMaxM3SparseMSAImpl.forward (build_k2q_csr and sparse_atten_func
       call sites, K|V split of the packed page).

Precision: every sum is taken in float64.  E4M3 values are integers times 2^-9
with magnitude below 2^18, so a dot product of up to 4*128 of them is an
integer times 2^-18 below 2^45 and is exact in float64: the scores do not
depend on summation order.  Attention is computed in float64 and rounded to
bfloat16 once.

Pins (each function is checked by tests against something other than itself):
  e4m3_table / decode_e4m3 -- closed form per OCP E4M3FN, exhaustive against
      torch.float8_e4m3fn's CPU cast, and spec values in tests/golden.
  index_scores  -- hand cases with known maxima (tests/golden), brute-force
      per-token Python loops on tiny inputs, scale and block-table invariances.
  topk_select   -- invariants of the case() construction [P2], closed form when
      every visible page fits in 16, brute-force sort on tiny inputs, a hand
      case with a known ranking (tests/golden).
  k2q_csr       -- brute-force transpose of the selection, nnz and row-sum
      identities, each query present in its own local row.
  sparse_attention -- dense causal attention (torch SDPA in float64 with an
      explicit mask) when the selection covers every visible page, closed forms
      (constant V, one visible token, all-zero K gives the mean of V).
  round_bf16    -- torch's bfloat16 cast on random and tie values.
  e2m1_table / e8m0_value / decode_mxfp4 / encode_e2m1 / quantize_mxfp4 --
      the E2M1 value list by hand (tests/golden), torch's E8M0 decode, every
      code round-trips, ties to even, exact blocks reproduce their codes,
      scale choice and saturation by worked values.
  mxfp4_staged_table / mxfp4_kv_as_e4m3 -- hand-worked (code, scale) codes
      (tests/golden), torch's float8_e4m3fn cast of every clamped product, exact
      agreement with decode_mxfp4 wherever the products are E4M3 values, element
      placement by hand-placed bytes, and attention over it equal to dense
      attention over decode_mxfp4 values.
  encode_e4m3 / quantize_e4m3 / insert_* -- every finite code round-trips,
      midpoints between neighbouring codes go to the even code, values just off
      a midpoint go to the nearer code, torch.float8_e4m3fn's CPU cast inside
      its non-saturating range (|x| <= 464), saturation and NaN by the stated
      rule, power-of-two scales exact; inserts against hand-placed rows.
"""
from __future__ import annotations

import math

import numpy as np

PAGE = 128       # tokens per KV page ([P1] admission: page 128)
HEAD_DIM = 128   # D ([P1] admission: D128)


# ----------------------------------------------------------------------------
# E4M3 (OCP E4M3FN, the torch.float8_e4m3fn format the pages use [P2 script])
# ----------------------------------------------------------------------------
def e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes, from the format's definition.

    sign s = bit 7, exponent e = bits 6..3 (bias 7), mantissa m = bits 2..0.
    e == 0: subnormal (-1)^s * m/8 * 2^-6.  e == 15 and m == 7: NaN (no inf).
    Otherwise (-1)^s * (1 + m/8) * 2^(e-7).
    """
    vals = np.empty(256, np.float64)
    for code in range(256):
        s = (code >> 7) & 1
        e = (code >> 3) & 15
        m = code & 7
        sign = -1.0 if s else 1.0
        if e == 0:
            v = sign * (m / 8.0) * 2.0 ** -6
        elif e == 15 and m == 7:
            v = math.nan
        else:
            v = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals[code] = v
    return vals


_E4M3 = e4m3_table()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3 bytes to float64 (unscaled)."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def encode_e4m3(x) -> np.ndarray:
    """Nearest E4M3FN code of each value, ties to the even code, saturating.

    Finite magnitudes at or above 448 and infinities give +-448 (0x7E / 0xFE),
    NaN gives 0x7F, and the sign of zero is kept.  Otherwise, with a = |x|:
    below the smallest normal 2^-6 the code counts multiples of 2^-9 (a
    subnormal, m = round(a / 2^-9), m = 8 being the smallest normal); else
    a = (1 + f) * 2^e with e = floor(log2 a), and the 3-bit mantissa is
    round(f * 8), a carry to 8 moving to the next binade.  Rounding is half to
    even (np.rint).
    """
    x = np.asarray(x, np.float64)
    out = np.empty(x.shape, np.uint8)
    flat, res = x.reshape(-1), out.reshape(-1)
    for k, v in enumerate(flat):
        if math.isnan(v):
            res[k] = 0x7F
            continue
        sign = 0x80 if math.copysign(1.0, v) < 0 else 0
        a = abs(v)
        if a >= 448.0:
            res[k] = sign | 0x7E
            continue
        if a < 2.0 ** -6:
            m = int(np.rint(a / 2.0 ** -9))          # 0 .. 8; 8 is the smallest normal
            res[k] = sign | m
            continue
        _, e2 = math.frexp(a)                        # a = f * 2^e2, f in [0.5, 1)
        e = e2 - 1                                   # a in [2^e, 2^(e+1))
        m = int(np.rint(a / 2.0 ** (e - 3))) - 8     # mantissa in eighths, 0 .. 8
        if m == 8:
            e, m = e + 1, 0
        if e > 8 or (e == 8 and m == 7):             # past 448: saturate
            res[k] = sign | 0x7E
            continue
        res[k] = sign | ((e + 7) << 3) | m
    return out


# ----------------------------------------------------------------------------
# MXFP4 index keys (OCP Microscaling MXFP4: blocks of 32 E2M1 elements sharing
# one E8M0 power-of-two scale) -- the gfx950 analogue of the pages' 4-bit index
# cache [P3 Details: NVFP4 index cache, FP8 query times FP4 key ("Q8KV4")]
# ----------------------------------------------------------------------------
class Mxfp4Keys:
    """An MXFP4 index-K cache: data [num_pages, 128, 64] (element 2i of a row in
    the low nibble of byte i, 2i + 1 in the high nibble) and scales
    [num_pages, 128, 4] E8M0 (block k covers elements 32k .. 32k + 31)."""

    def __init__(self, data, scales):
        self.data = np.asarray(data, np.uint8)
        self.scales = np.asarray(scales, np.uint8)


def e2m1_table() -> np.ndarray:
    """Value of each of the 16 E2M1 codes: sign = bit 3, exponent = bits 2..1
    (bias 1), mantissa = bit 0; exponent 0 is subnormal m * 0.5, otherwise
    (1 + m/2) * 2^(e-1).  No inf, no NaN; the largest magnitude is 6."""
    vals = np.empty(16, np.float64)
    for code in range(16):
        sign = -1.0 if code & 8 else 1.0
        e, m = (code >> 1) & 3, code & 1
        vals[code] = sign * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return vals


_E2M1 = e2m1_table()


def e8m0_value(codes) -> np.ndarray:
    """E8M0 scale codes: 2^(code - 127); 0xFF is NaN."""
    c = np.asarray(codes, np.int64)
    return np.where(c == 0xFF, np.nan, np.ldexp(1.0, c - 127))


def decode_mxfp4(data, scales) -> np.ndarray:
    """[..., 64] data bytes and [..., 4] scales -> [..., 128] float64 values."""
    data = np.asarray(data, np.uint8)
    codes = np.stack([data & 15, data >> 4], axis=-1).reshape(*data.shape[:-1], 2 * data.shape[-1])
    blocks = _E2M1[codes].reshape(*data.shape[:-1], -1, 32)
    out = blocks * e8m0_value(scales)[..., None]
    return out.reshape(*data.shape[:-1], -1)


def encode_e2m1(v) -> np.ndarray:
    """Nearest E2M1 code of each value, ties to the even code (mantissa bit 0),
    saturating at +-6; the sign of zero is kept."""
    v = np.asarray(v, np.float64)
    mags = _E2M1[:8]                                   # 0, .5, 1, 1.5, 2, 3, 4, 6
    out = np.empty(v.shape, np.uint8)
    flat, res = v.reshape(-1), out.reshape(-1)
    for k, x in enumerate(flat):
        sign = 8 if math.copysign(1.0, x) < 0 else 0
        a = min(abs(x), 6.0)
        d = np.abs(mags - a)
        best = np.nonzero(d == d.min())[0]
        code = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        res[k] = sign | code
    return out


def quantize_mxfp4(x):
    """MXFP4 of rows of 128 values (OCP Microscaling conversion): per block of
    32, the shared exponent is floor(log2(max |v|)) - 2 (2 being the exponent of
    E2M1's largest value, 6 = 1.5 * 2^2), clamped to [-127, 127] (a block of
    zeros takes -127); elements are encode_e2m1(v / 2^exponent), which
    saturates.  A block holding NaN or an infinity gets scale 0xFF (NaN) and
    zero elements.
    Returns (data [..., 64], scales [..., 4])."""
    x = np.asarray(x, np.float64)
    lead = x.shape[:-1]
    blocks = x.reshape(*lead, 4, 32)
    scales = np.empty((*lead, 4), np.uint8)
    codes = np.empty((*lead, 4, 32), np.uint8)
    for idx in np.ndindex(*lead, 4):
        blk = blocks[idx]
        if not np.isfinite(blk).all():
            scales[idx] = 0xFF
            codes[idx] = 0
            continue
        amax = float(np.abs(blk).max())
        e = -127 if amax == 0.0 else min(127, max(-127, math.frexp(amax)[1] - 1 - 2))
        scales[idx] = e + 127
        codes[idx] = encode_e2m1(np.ldexp(blk, -e))
    c = codes.reshape(*lead, 64, 2)
    data = (c[..., 0] | (c[..., 1] << 4)).astype(np.uint8)
    return data, scales


def insert_index_k_mxfp4(cache: Mxfp4Keys, k, slot_mapping):
    """Write index keys of new tokens into an MXFP4 index cache (in place):
    token t with slot s >= 0 goes to row s % 128 of page s // 128."""
    for t, s in enumerate(np.asarray(slot_mapping, np.int64)):
        if s < 0:
            continue
        d, sc = quantize_mxfp4(np.asarray(k[t], np.float32).astype(np.float64)[None])
        cache.data[s // PAGE, s % PAGE] = d[0]
        cache.scales[s // PAGE, s % PAGE] = sc[0]
    return cache


# ----------------------------------------------------------------------------
# MXFP4 K|V pages read through E4M3 [P2 Details: with an E4M3 query the 4-bit
# K|V kernel turns each code times its block scale into E4M3 before the FP8
# products, and applies the K global scale to the scores and the V global scale
# to the output; the reference of its test is the cache as that kernel reads
# it.  Here the 4-bit format is MXFP4, the one gfx950's matrix cores take.]
# ----------------------------------------------------------------------------
class Mxfp4KV:
    """An MXFP4 K|V cache: data [num_pages, Hkv, 128, 128] (bytes 0..63 hold the
    token's 128 K elements, bytes 64..127 its 128 V elements, element 2i in the
    low nibble of byte i as in Mxfp4Keys) and scales [num_pages, Hkv, 128, 8]
    E8M0 (bytes 0..3: the K blocks of 32 elements, 4..7: the V blocks)."""

    def __init__(self, data, scales):
        self.data = np.asarray(data, np.uint8)
        self.scales = np.asarray(scales, np.uint8)


def mxfp4_staged_table() -> np.ndarray:
    """[256, 16] E4M3 code of (E2M1 code value) x 2^(scale - 127) for every
    (scale, code), rounded by encode_e4m3 (nearest, ties to even, saturating at
    448); the NaN scale 0xFF gives NaN codes."""
    t = np.empty((256, 16), np.uint8)
    for sc in range(256):
        t[sc] = encode_e4m3(_E2M1 * e8m0_value(sc))
    return t


_STAGED = mxfp4_staged_table()


def mxfp4_kv_as_e4m3(data, scales) -> np.ndarray:
    """The E4M3 K|V cache [..., 256] (K = [..., :128], V = [..., 128:]) that the
    attention reads from MXFP4 K|V rows: data [..., 128], scales [..., 8]."""
    data = np.asarray(data, np.uint8)
    scales = np.asarray(scales, np.uint8)
    codes = np.stack([data & 15, data >> 4], axis=-1).reshape(*data.shape[:-1], 2 * data.shape[-1])
    block = np.repeat(scales, 32, axis=-1)            # element j belongs to block j // 32
    return _STAGED[block, codes]


# ----------------------------------------------------------------------------
# E4M3 quantisation and the paged cache write [P2 Overview: a fused insert
# kernel writes the query in E4M3 and the new tokens' K|V into the packed cache
# pages; P2 Details: the FP8 cache is written with unit scales; P2 script and
# P4 forward: slot_mapping, one int64 cache slot per token]
# ----------------------------------------------------------------------------
def quantize_e4m3(x, scale) -> np.ndarray:
    """E4M3 codes of x / scale: the quotient taken in float32 (one correctly
    rounded division), then encode_e4m3.  x: float32 values (bf16 inputs are
    widened to float32 exactly first)."""
    with np.errstate(invalid="ignore", over="ignore"):     # inf / NaN inputs are expected
        q = np.asarray(x, np.float32) / np.float32(scale)
    return encode_e4m3(q.astype(np.float64))


def insert_index_k(k_cache, k, slot_mapping, scale):
    """Write the index keys of new tokens into the paged index-K cache.

    k_cache: [num_pages, 128, 128] uint8, updated in place.  k: [n, 128]
    float32.  Token t with slot s = slot_mapping[t] >= 0 goes to row s % 128 of
    page s // 128; tokens with s < 0 are skipped.
    """
    for t, s in enumerate(np.asarray(slot_mapping, np.int64)):
        if s < 0:
            continue
        k_cache[s // PAGE, s % PAGE, :] = quantize_e4m3(k[t], scale)
    return k_cache


def insert_kv(kv_cache, k, v, slot_mapping, k_scale, v_scale):
    """Write K and V of new tokens into the packed K|V cache.

    kv_cache: [num_pages, Hkv, 128, 256] uint8, updated in place; K takes bytes
    [..., :128] of a token's row and V bytes [..., 128:] ([P4] forward: the
    packed page split).  k, v: [n, Hkv, 128] float32.  Token t with slot
    s >= 0 goes to row s % 128 of page s // 128, every KV head; s < 0 skipped.
    """
    for t, s in enumerate(np.asarray(slot_mapping, np.int64)):
        if s < 0:
            continue
        for h in range(k.shape[1]):
            kv_cache[s // PAGE, h, s % PAGE, :HEAD_DIM] = quantize_e4m3(k[t, h], k_scale)
            kv_cache[s // PAGE, h, s % PAGE, HEAD_DIM:] = quantize_e4m3(v[t, h], v_scale)
    return kv_cache


# ----------------------------------------------------------------------------
# Positions [P2 script case(): pos = arange(seq_len - q_len, seq_len),
# visible = pos // 128 + 1, local page = visible - 1]
# ----------------------------------------------------------------------------
def query_positions(cu_q: np.ndarray, cu_k: np.ndarray):
    """Request index and absolute position of every query token.

    New tokens are the last seqlen_q positions of each request's KV:
    pos_i = (seqlen_k_b - seqlen_q_b) + (i - cu_q[b])  (context_lens = seq - q_len).
    """
    cu_q = np.asarray(cu_q, np.int64)
    cu_k = np.asarray(cu_k, np.int64)
    total_q = int(cu_q[-1])
    req = np.empty(total_q, np.int64)
    pos = np.empty(total_q, np.int64)
    for b in range(len(cu_q) - 1):
        q0, q1 = cu_q[b], cu_q[b + 1]
        sq, sk = q1 - q0, cu_k[b + 1] - cu_k[b]
        req[q0:q1] = b
        pos[q0:q1] = (sk - sq) + np.arange(q1 - q0)
    return req, pos


def _request_keys(k_cache, block_table, b, seqlen_k):
    """Logical index-K rows [seqlen_k, 128] of request b, decoded (float64):
    E4M3 bytes [num_pages, 128, 128], or an Mxfp4Keys cache."""
    n_pages = (seqlen_k + PAGE - 1) // PAGE
    phys = np.asarray(block_table[b, :n_pages], np.int64)
    if isinstance(k_cache, Mxfp4Keys):
        rows = decode_mxfp4(k_cache.data[phys], k_cache.scales[phys])
    else:
        rows = decode_e4m3(k_cache[phys])
    return rows.reshape(n_pages * PAGE, HEAD_DIM)[:seqlen_k]


# ----------------------------------------------------------------------------
# Index scores [P1 Overview/Details: the FP8 indexer scores every 128-token KV
# page per query; score-only plan(..., score_out=) / run_scores()]
# ----------------------------------------------------------------------------
def index_scores(cu_q, cu_k, block_table, index_q, k_cache, q_scale, k_scale,
                 queries=None, width=None, per_head=False):
    """Page scores s(i, j), float64, -inf where page j is not visible to query i.

    The pages do not state the reduction over a page's tokens or over index
    heads.  Reading adopted: the score of logical page j for query i is

        q_scale * k_scale * max_{t in page j, t <= pos_i} sum_h sum_d q[i,h,d] * k[t,d]

    with one shared 128-byte index-K row per token ([P3] Details: FP8 rows of
    128 B per token), read through the block table, and only causally visible
    tokens counted.  Pages j >= pos_i // 128 + 1 are not visible.

    index_q: [total_q, H, 128] E4M3 bytes.  k_cache: [num_pages, 128, 128] E4M3
    bytes, or an Mxfp4Keys cache (values = E2M1 element * 2^(scale - 127)).
    queries: optional list of global query indices (default: all).
    Returns [len(queries), width] with width = max pages per request by default.

    per_head=True is the other reading of how selections map to KV heads (the
    top-k buffer is [total_q, H, 16], one selection per KV head, API docs,
    MiniMaxM3SparseMSAImpl.forward): index head h is scored alone,

        s_h(i, j) = q_scale * k_scale * max_{t in page j, t <= pos_i} sum_d q[i,h,d] * k[t,d]

    and the result is [len(queries), H, width].
    """
    cu_q = np.asarray(cu_q, np.int64)
    cu_k = np.asarray(cu_k, np.int64)
    req, pos = query_positions(cu_q, cu_k)
    total_q = int(cu_q[-1])
    if queries is None:
        queries = np.arange(total_q)
    queries = np.asarray(queries, np.int64)
    seqlen_k = np.diff(cu_k)
    if width is None:
        width = int(((seqlen_k + PAGE - 1) // PAGE).max()) if len(seqlen_k) else 0
    H = np.asarray(index_q).shape[1]
    out = np.full((len(queries), H, width) if per_head else (len(queries), width), -np.inf, np.float64)
    scale = float(q_scale) * float(k_scale)
    for b in np.unique(req[queries]) if len(queries) else []:
        sel = np.nonzero(req[queries] == b)[0]
        keys = _request_keys(k_cache, block_table, b, int(seqlen_k[b]))   # [sk, 128]
        chunk = max(1, (1 << 26) // max(1, keys.shape[0]))
        for c0 in range(0, len(sel), chunk):
            rows = sel[c0:c0 + chunk]
            qi = queries[rows]
            last = int(pos[qi].max())
            kk = keys[:last + 1]                                          # [T, 128]
            qq = decode_e4m3(index_q[qi])                                 # [n, H, 128]
            t = np.arange(kk.shape[0])[:, None]
            n_pages = (kk.shape[0] + PAGE - 1) // PAGE
            # summed: one dot product over all index heads; per head: one per head
            groups = [[h] for h in range(qq.shape[1])] if per_head else [range(qq.shape[1])]
            for gi, heads in enumerate(groups):
                dots = np.zeros((kk.shape[0], len(qi)), np.float64)
                for h in heads:
                    dots += kk @ qq[:, h, :].T
                dots[t > pos[qi][None, :]] = -np.inf                      # causal: t <= pos_i
                padded = np.full((n_pages * PAGE, len(qi)), -np.inf)
                padded[:kk.shape[0]] = dots
                page_max = padded.reshape(n_pages, PAGE, len(qi)).max(axis=1)   # [pages, n]
                if per_head:
                    out[rows, gi, :n_pages] = (page_max * scale).T
                else:
                    out[rows, :n_pages] = (page_max * scale).T
    return out


# ----------------------------------------------------------------------------
# Top-k [P2 script case(): the local page (visible - 1) is forced, future pages
# never chosen, k = min(16, visible), -1 padding; P1 "Native Top16"]
# ----------------------------------------------------------------------------
def topk_select(cu_q, cu_k, scores, topk=16, n_local=1, queries=None):
    """Selected logical pages per query, int32 [len(queries), topk].

    Forced pages: the last n_local visible pages, local page first (slot 0),
    then the next older ones.  The remaining min(topk, v) - n_forced slots take
    the highest-scoring older visible pages, ordered by score descending and,
    at equal scores, by lower page index (the pages leave exact-tie order open,
    [P3] Details).  Unused slots are -1.

    scores: [len(queries), >= max visible] (row r belongs to queries[r]).
    """
    req, pos = query_positions(cu_q, cu_k)
    if queries is None:
        queries = np.arange(len(pos))
    queries = np.asarray(queries, np.int64)
    out = np.full((len(queries), topk), -1, np.int32)
    for r, i in enumerate(queries):
        v = int(pos[i] // PAGE + 1)
        k = min(topk, v)
        n_forced = min(n_local, k)
        forced = [v - 1 - f for f in range(n_forced)]
        cand = np.arange(v - n_forced)
        s = np.asarray(scores[r, :v - n_forced], np.float64)
        order = np.lexsort((cand, -s))           # primary: -score, secondary: page
        chosen = forced + [int(c) for c in cand[order[:k - n_forced]]]
        out[r, :k] = chosen
    return out


# ----------------------------------------------------------------------------
# k2q CSR [P4 MiniMaxM3SparseMSAImpl.forward: build_k2q_csr(topk, cu_seqlens_q,
# cu_seqlens_k, 128, ..., total_rows=total_kv_blocks, ...) -> row_ptr, q_indices]
# ----------------------------------------------------------------------------
def k2q_csr(cu_q, cu_k, topk_idx, total_rows=None):
    """Transpose a selection into a KV-page -> query CSR.

    Rows are logical (request, page) pairs, request-major:
    row(b, j) = sum_{b' < b} ceil(seqlen_k_b' / 128) + j, so there are
    total_kv_blocks rows per selection head; selection head g owns rows
    g * total_rows + row.  Each row lists the global indices of the queries
    whose selection contains its page, ascending, each once (a page listed
    twice in one selection is still one entry).

    topk_idx: [total_q, n_sel, K] int (logical pages, -1 = none).
    Returns (row_ptr [n_sel * total_rows + 1] int32, q_indices [nnz] int32).
    """
    cu_q = np.asarray(cu_q, np.int64)
    cu_k = np.asarray(cu_k, np.int64)
    pages = (np.diff(cu_k) + PAGE - 1) // PAGE
    row_base = np.concatenate([[0], np.cumsum(pages)])
    if total_rows is None:
        total_rows = int(row_base[-1])
    req, _ = query_positions(cu_q, cu_k)
    topk_idx = np.asarray(topk_idx)
    n_sel = topk_idx.shape[1]
    rows = [[] for _ in range(n_sel * total_rows)]
    for i in range(topk_idx.shape[0]):           # ascending query order
        b = req[i]
        for g in range(n_sel):
            for j in dict.fromkeys(int(x) for x in topk_idx[i, g] if x >= 0):
                rows[g * total_rows + row_base[b] + j].append(i)
    counts = np.array([len(r) for r in rows], np.int64)
    row_ptr = np.zeros(len(rows) + 1, np.int64)
    row_ptr[1:] = np.cumsum(counts)
    q_indices = np.array([i for r in rows for i in r], np.int64)
    return row_ptr.astype(np.int32), q_indices.astype(np.int32)


# ----------------------------------------------------------------------------
# Sparse attention [P4 forward: sparse_atten_func(q, k, v, row_ptr, q_indices,
# topK=16, blk_kv=128, causal=True, softmax_scale, page_table=block_table);
# P2 Details: q_scale folds into softmax_scale, the K scale applies to the
# scores and the V scale to the output; K|V page split k = [..., :128],
# v = [..., 128:]]
# ----------------------------------------------------------------------------
def sparse_attention(cu_q, cu_k, block_table, q, kv_cache, topk_idx, softmax_scale,
                     q_scale=1.0, k_scale=1.0, v_scale=1.0, queries=None):
    """Exact block-sparse causal attention, float64 [len(queries), Hq, 128].

    For query i, q-head hq and KV head g = hq // (Hq // Hkv), the attended
    tokens are those of the selected pages (selection head g, or the single
    shared selection when topk_idx has one head) at positions <= pos_i.  The
    selection is a set of pages: a page listed twice contributes its tokens
    once.

        z_t = softmax_scale * q_scale * k_scale * sum_d q[i,hq,d] * K[t,g,d]
        out = v_scale * sum_t softmax(z)_t * V[t,g,:]

    A query with no attended token gets 0.
    """
    req, pos = query_positions(cu_q, cu_k)
    if queries is None:
        queries = np.arange(len(pos))
    queries = np.asarray(queries, np.int64)
    topk_idx = np.asarray(topk_idx)
    n_sel = topk_idx.shape[1]
    Hq = q.shape[1]
    Hkv = kv_cache.shape[1]
    group = Hq // Hkv
    seqlen_k = np.diff(np.asarray(cu_k, np.int64))
    logit_scale = float(softmax_scale) * float(q_scale) * float(k_scale)
    out = np.zeros((len(queries), Hq, HEAD_DIM), np.float64)
    for r, i in enumerate(queries):
        b = int(req[i])
        qi = decode_e4m3(q[i])                                  # [Hq, 128]
        for g in range(Hkv):
            sel = topk_idx[i, g if n_sel > 1 else 0]
            tok_k, tok_v = [], []
            for j in dict.fromkeys(int(x) for x in sel if x >= 0):      # distinct pages
                n_vis = min(PAGE, int(pos[i]) - PAGE * j + 1, int(seqlen_k[b]) - PAGE * j)
                if n_vis <= 0:
                    continue
                page = kv_cache[int(block_table[b, j]), g, :n_vis]   # [n, 256]
                tok_k.append(decode_e4m3(page[:, :HEAD_DIM]))
                tok_v.append(decode_e4m3(page[:, HEAD_DIM:]))
            if not tok_k:
                continue
            K = np.concatenate(tok_k)                           # [T, 128]
            V = np.concatenate(tok_v)
            for hq in range(g * group, (g + 1) * group):
                z = logit_scale * (K @ qi[hq])
                w = np.exp(z - z.max())
                out[r, hq] = float(v_scale) * (w @ V) / w.sum()
    return out


# ----------------------------------------------------------------------------
# bfloat16 output [P2 script: out = empty_like(bf16 query)]
# ----------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (nearest, ties to even); returns the uint16 bit patterns.

    float64 is first rounded to float32 (nearest-even), then the low 16 bits of
    the float32 pattern are rounded away: add 0x7FFF plus the lowest kept bit
    and truncate.  NaN stays NaN.
    """
    f = np.asarray(x, np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64."""
    u = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)
