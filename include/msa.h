/*
 * msa.h -- MI355X (gfx950) library for the MiniMax-M3 MSA sparse-prefill path:
 * FP8 (E4M3) page indexer, causal top-16 page selection, KV-page -> query CSR,
 * and block-sparse attention over a paged E4M3 K|V cache.
 *
 * Sources, cited by page and section:
 *   [P1] vLLM PR 60930 (MiniMax M3 FP8 indexer prefill on MSA's persistent
 *        CuTe scorer): Overview, Details (score-only plan/run_scores API, device
 *        planning without host sync, admission: E4M3, D128, page 128,
 *        H in {1,2,4} per rank, sparse_local_block >= 1).
 *   [P2] vLLM PR 60684 (MSA prefill reads the E4M3 query natively): Overview,
 *        Validation (benchmark script: case() top-k construction, packed K|V
 *        pages, q_scale 0.5, unit K/V scales), Details (q_scale folds into the
 *        softmax scale; probabilities rounded to E4M3 per split).
 *   [P3] vLLM PR 64631 (NVFP4 index-cache sharding): Details (FP8 index rows of
 *        128 B per token; exact-tie order is implementation-defined).
 *   [P4] vLLM API docs, vllm.models.minimax_m3.nvidia.sparse_attention_msa:
 *        MiniMaxM3SparseMSAImpl.forward (build_k2q_csr and sparse_atten_func
 *        arguments: cu_seqlens_q/k, block size 128, total_rows =
 *        total_kv_blocks, page_table = block_table, topK = 16, causal).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked [host].  `stream` is a
 *     hipStream_t (NULL = the null stream).
 *   - Every call validates its host-side arguments first and returns an error
 *     before launching anything.  On success the work is queued on `stream`
 *     and the call returns without synchronising.  No call allocates memory,
 *     reads device memory from the host, or synchronises, so the calls can be
 *     recorded in a HIP graph ([P1] Details: the scorer plans on device with no
 *     D2H and run_scores does no allocation or sync).
 *   - The caller owns every buffer.  Inputs are only read.  Outputs are
 *     written as documented; workspace contents are private between calls.
 *   - Device data that contradicts the host-side sizes (e.g. a cu_seqlens
 *     entry larger than total_q, a block_table entry >= num_pages) gives
 *     unspecified results; kernels clamp such indices so they do not fault.
 *   - E4M3 means OCP E4M3FN (torch.float8_e4m3fn): bias 7, max 448, no inf.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_PAGE_SIZE 128   /* tokens per KV page ([P1] admission: page 128) */
#define MSA_HEAD_DIM 128    /* D ([P1] admission: D128) */
#define MSA_TOPK 16         /* selected pages per query ([P2] script: TOPK = 16) */

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative or inconsistent size */
  MSA_ERR_UNSUPPORTED = 2,        /* outside the admitted set ([P1] Details: otherwise FMHA is kept) */
  MSA_ERR_WORKSPACE_TOO_SMALL = 3,
  MSA_ERR_HIP = 4,                /* a HIP launch failed; msa_last_error() has the HIP text */
  MSA_ERR_NO_DEVICE = 5
} msa_status_t;

/* Variable-length prefill batch ([P2] script: cu_seqlens_q/k, block_table,
 * total_kv_blocks; [P4] forward: build_k2q_csr arguments).  The struct itself
 * is a host object; the three arrays are device arrays.
 *   Request b has seqlen_q_b = cu_seqlens_q[b+1]-cu_seqlens_q[b] new tokens,
 *   which are the LAST seqlen_q_b of its seqlen_k_b tokens: query token
 *   i (cu_seqlens_q[b] <= i < cu_seqlens_q[b+1]) sits at position
 *   pos_i = seqlen_k_b - seqlen_q_b + (i - cu_seqlens_q[b]).  Requires
 *   0 <= seqlen_q_b <= seqlen_k_b. */
typedef struct {
  int32_t batch;                 /* [host] B >= 1 */
  int32_t total_q;               /* [host] cu_seqlens_q[B] */
  int32_t max_seqlen_q;          /* [host] >= every seqlen_q_b */
  int32_t max_seqlen_k;          /* [host] >= every seqlen_k_b */
  int32_t total_rows;            /* [host] sum_b ceil(seqlen_k_b / 128) = total_kv_blocks */
  int32_t max_pages;             /* [host] >= every ceil(seqlen_k_b / 128); <= block_table_stride */
  const int32_t* cu_seqlens_q;   /* [B+1] non-decreasing, cu_seqlens_q[0] = 0 */
  const int32_t* cu_seqlens_k;   /* [B+1] non-decreasing, cu_seqlens_k[0] = 0 */
  const int32_t* block_table;    /* [B, block_table_stride] logical page -> physical page */
  int64_t block_table_stride;    /* [host] elements between rows of block_table */
} msa_varlen_t;

/* ---------------------------------------------------------------------------
 * 1. Index scores  ([P1] Overview and Details: the FP8 indexer scores every
 *    128-token KV page for each query; score-only plan(..., score_out=) then
 *    run_scores(), planned on device without host sync.)
 *
 * For query i and every logical page j < v_i = pos_i / 128 + 1 of its request:
 *   scores[i * ld_scores + j] =
 *       q_scale * k_scale * max_{t in page j, t <= pos_i}
 *           sum_{h < H} sum_{d < 128} q[i,h,d] * k[block_table[b,j], t % 128, d]
 * (the pages do not state the reductions; this is the reading the library
 * implements: maximum over the causally visible tokens of the page of the sum
 * over index heads of q_h . k).  Entries j >= v_i are NOT written.
 * Products are exact; sums are accumulated in fp32 by the matrix cores.
 *
 *   q          [total_q, H, 128] E4M3, token stride q_stride bytes (>= H*128, multiple of 16)
 *   H          num_index_heads in {1, 2, 4}          (else MSA_ERR_UNSUPPORTED)
 *   k_cache    [num_pages, 128, 128] E4M3: one 128-byte index-K row per token
 *              ([P3] Details), paged through the same block_table
 *   q_scale, k_scale  device fp32 scalars (per-tensor dequantisation scales)
 *   scores     fp32 [total_q, ld_scores], ld_scores >= max_pages and a multiple of 4,
 *              16-byte aligned
 *   workspace  >= msa_index_score_workspace_size(vl, H) bytes, 16-byte aligned
 * ------------------------------------------------------------------------- */
size_t msa_index_score_workspace_size(const msa_varlen_t* vl, int32_t num_index_heads);
msa_status_t msa_index_score(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                             int32_t num_index_heads, const uint8_t* k_cache,
                             int32_t num_pages, const float* q_scale, const float* k_scale,
                             float* scores, int64_t ld_scores, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * 1b. Per-index-head scores: the reading in which index head h selects the
 *     pages of KV head h ([P4] forward: the top-k buffer is [total_q, H, 16],
 *     viewed per KV head; [P2] script: an independent selection per KV head).
 *     The pages leave open how head h's score is formed; here each index head
 *     is scored alone, with no sum over heads:
 *
 *   scores[i * ld_scores + h * head_stride + j] =
 *       q_scale * k_scale * max_{t in page j, t <= pos_i} sum_{d < 128} q[i,h,d] * k[block_table[b,j], t % 128, d]
 *
 * for h < H and every visible page j < v_i; entries j >= v_i are NOT written.
 * Arguments and errors as msa_index_score, plus
 *   head_stride  floats between the rows of consecutive heads of one query:
 *                >= max_pages and a multiple of 4; ld_scores >= (H-1)*head_stride + max_pages
 *   workspace    >= msa_index_score_workspace_size(vl, 1) bytes (the plan is
 *                that of one index head; the size for H heads is also enough)
 * The index-K cache is read once per index head (H scorer passes over one
 * plan); select per head with msa_topk_select on each head's rows (scores +
 * h*head_stride, row stride ld_scores, output topk_idx + h*16 with
 * topk_stride = H*16), then build the CSR with n_sel_heads = H = num_kv_heads.
 * ------------------------------------------------------------------------- */
msa_status_t msa_index_score_per_head(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                                      int32_t num_index_heads, const uint8_t* k_cache,
                                      int32_t num_pages, const float* q_scale,
                                      const float* k_scale, float* scores, int64_t ld_scores,
                                      int64_t head_stride, void* workspace, size_t workspace_bytes,
                                      void* stream);

/* ---------------------------------------------------------------------------
 * 2. Top-k page selection  ([P1] "Native Top16"; [P2] Validation, benchmark
 *    script case(): local page = visible - 1 always kept, future pages never
 *    chosen, k = min(16, visible), -1 padding.)
 *
 * For query i with v_i visible pages: slots 0..f-1 hold the forced pages
 * v_i-1, v_i-2, ..., v_i-f with f = min(n_local, topk, v_i) (slot 0 is the
 * local page); the next min(topk, v_i) - f slots hold the pages
 * j < v_i - f with the highest scores, in descending score order, equal
 * scores ordered by lower page index; remaining slots are -1.  Only
 * scores[i * ld_scores + j] for j < v_i - f are read.
 *   topk       must be 16; 1 <= n_local <= 16 ([P1]: sparse_local_block >= 1)
 *   topk_idx   int32 [total_q, topk_stride], topk_stride >= 16; slots 0..15 written
 * ------------------------------------------------------------------------- */
msa_status_t msa_topk_select(const msa_varlen_t* vl, const float* scores, int64_t ld_scores,
                             int32_t topk, int32_t n_local, int32_t* topk_idx,
                             int64_t topk_stride, void* stream);

/* ---------------------------------------------------------------------------
 * 2b. Fused index scores and top-16 selection for decode-like batches
 *    ([P1] Claims: the top-16 stays a kernel of its own, "Native Top16";
 *    Findings: on short-Q shapes the persistent scorer loses to its schedule's
 *    tail.  Here the selection runs inside the decode scorer's work items.)
 *
 * topk_idx exactly as msa_index_score followed by msa_topk_select on its
 * scores (same tie rule: equal scores go to the lower page), without writing
 * the scores: each scorer work item keeps its pages' scores in LDS and leaves
 * every query's 16 best candidate pages, which a merge reduces to the top 16.
 *   Only batches whose every request has at most 64 / H queries (the decode
 *   scorer's shapes); others get MSA_ERR_UNSUPPORTED.
 *   Arguments as msa_index_score (E4M3 keys) and msa_topk_select (topk == 16,
 *   n_local in [1, 16], topk_idx [total_q, topk_stride] int32).
 *   workspace  >= msa_index_score_topk_workspace_size(vl, H) bytes, 16-byte aligned
 * ------------------------------------------------------------------------- */
size_t msa_index_score_topk_workspace_size(const msa_varlen_t* vl, int32_t num_index_heads);
msa_status_t msa_index_score_topk(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                                  int32_t num_index_heads, const uint8_t* k_cache,
                                  int32_t num_pages, const float* q_scale, const float* k_scale,
                                  int32_t topk, int32_t n_local, int32_t* topk_idx,
                                  int64_t topk_stride, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* ---------------------------------------------------------------------------
 * 3. KV-page -> query CSR  ([P4] forward: build_k2q_csr(topk, cu_seqlens_q,
 *    cu_seqlens_k, 128, ..., total_rows=total_kv_blocks, qhead_per_kv, ...,
 *    return_schedule=True) -> (row_ptr, q_indices, schedule).)
 *
 * Rows are logical (request, page) pairs: row(b, j) = sum_{b'<b}
 * ceil(seqlen_k_b' / 128) + j.  With n_sel_heads selections per query
 * (1 = one selection shared by every KV head; or one per KV head), selection
 * head g owns rows g * total_rows + row.  Row r lists, in ascending order, the
 * global indices of the queries whose selection contains its page:
 *   row_ptr    int32 [n_sel_heads * total_rows + 1], exclusive prefix sums
 *   q_indices  int32, capacity n_sel_heads * total_q * topk
 *   topk_idx   int32, entry (i, g, s) at topk_idx[i * topk_q_stride + g * topk_h_stride + s]
 *              (logical pages; negative = empty slot; pages >= the request's page
 *              count are ignored)
 *   schedule   >= msa_k2q_schedule_size(vl, n_sel_heads, topk) bytes, 16-byte
 *              aligned: the attention's work list, each CSR entry's split slot
 *              and each (query, selection head)'s set of distinct selected pages,
 *              written here and read by msa_sparse_attn_prefill.  Opaque.  It
 *              records each row's physical page as vl->block_table maps it at the
 *              time of this call.
 * ------------------------------------------------------------------------- */
size_t msa_k2q_schedule_size(const msa_varlen_t* vl, int32_t n_sel_heads, int32_t topk);
msa_status_t msa_build_k2q_csr(const msa_varlen_t* vl, const int32_t* topk_idx,
                               int64_t topk_q_stride, int64_t topk_h_stride,
                               int32_t n_sel_heads, int32_t topk, int32_t* row_ptr,
                               int32_t* q_indices, void* schedule, size_t schedule_bytes,
                               void* stream);

/* ---------------------------------------------------------------------------
 * 4. Block-sparse prefill attention  ([P4] forward: sparse_atten_func(q, k, v,
 *    row_ptr, q_indices, topK=16, blk_kv=128, causal=True, softmax_scale, ...,
 *    page_table=block_table, schedule, out); [P2] Overview and Details: E4M3
 *    query over E4M3 K/V with FP8 QK and PV products, probabilities rounded to
 *    E4M3, q_scale folded into the softmax scale, K scale on the scores, V scale
 *    on the output; packed page split k = [..., :128], v = [..., 128:].)
 *
 * For query i, q-head hq, KV head g = hq / (Hq / Hkv), over the tokens t of the
 * pages listed for i in selection head (n_sel_heads == 1 ? 0 : g) with t <= pos_i:
 *   z_t = softmax_scale * q_scale * k_scale * q[i,hq,:] . K[t,g,:]
 *   out[i,hq,:] = v_scale * sum_t softmax(z)_t V[t,g,:]       (bf16, round to nearest even)
 * Each (query, page) pair is computed as one split (online-softmax partial with
 * E4M3 probabilities); the splits are merged by a log-sum-exp combine.
 * Queries with no attended token get 0.
 *   q          [total_q, Hq, 128] E4M3, token stride q_stride bytes (>= Hq*128, multiple of 16)
 *   kv_cache   [num_pages, Hkv, 128, 256] E4M3 (K|V packed per token)
 *   Hq % Hkv == 0, Hkv >= 1, Hq <= 64; n_sel_heads in {1, Hkv}; topk == 16;
 *              total_q * topk * Hq < 2^31 (else MSA_ERR_UNSUPPORTED)
 *   row_ptr, q_indices, schedule: exactly as written by msa_build_k2q_csr for
 *              the same vl, n_sel_heads and topk
 *   q_scale, k_scale, v_scale  device fp32 scalars, or NULL for 1.0
 *   out        bf16 [total_q, Hq, 128], token stride out_stride elements (>= Hq*128,
 *              multiple of 8), 16-byte aligned
 *   workspace  >= msa_sparse_attn_workspace_size(vl, Hq, Hkv, n_sel_heads, topk) bytes
 * ------------------------------------------------------------------------- */
size_t msa_sparse_attn_workspace_size(const msa_varlen_t* vl, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t n_sel_heads, int32_t topk);
msa_status_t msa_sparse_attn_prefill(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                                     int32_t num_q_heads, const uint8_t* kv_cache,
                                     int32_t num_pages, int32_t num_kv_heads,
                                     const int32_t* row_ptr, const int32_t* q_indices,
                                     int32_t n_sel_heads, const void* schedule,
                                     size_t schedule_bytes, int32_t topk, float softmax_scale,
                                     const float* q_scale, const float* k_scale,
                                     const float* v_scale, uint16_t* out, int64_t out_stride,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * 4b. Block-sparse prefill attention over 4-bit K|V pages  ([P2] Details: with
 *    an E4M3 query the 4-bit K|V kernel turns each code times its block scale
 *    into E4M3 before the FP8 products, with the K global scale on the scores
 *    and the V global scale on the output; Claims: 8-13% faster prefill with a
 *    4-bit K|V cache.  The pages' format is NVFP4; on gfx950 it is OCP MXFP4.)
 *
 * Exactly msa_sparse_attn_prefill, with the K|V cache in MXFP4:
 *   kv_data    [num_pages, Hkv, 128, 128] uint8: per token, bytes 0..63 hold the
 *              128 K elements and bytes 64..127 the 128 V elements as E2M1 codes,
 *              element 2i in the low nibble of byte i; 16-byte aligned
 *   kv_scales  [num_pages, Hkv, 128, 8] E8M0: bytes 0..3 scale K elements
 *              32b .. 32b+31 (b = byte), bytes 4..7 the V blocks; 8-byte aligned
 * Each element is read as E4M3: code value x 2^(scale - 127) rounded to the
 * nearest E4M3 value (ties to even), saturating at 448; the scale 0xFF reads
 * as NaN.  k_scale / v_scale are the per-tensor global scales.  Same workspace
 * (msa_sparse_attn_workspace_size), schedule and errors; NULL kv_scales with
 * total_q > 0 is MSA_ERR_INVALID_ARGUMENT.
 * ------------------------------------------------------------------------- */
msa_status_t msa_sparse_attn_prefill_mxfp4(
    const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride, int32_t num_q_heads,
    const uint8_t* kv_data, const uint8_t* kv_scales, int32_t num_pages, int32_t num_kv_heads,
    const int32_t* row_ptr, const int32_t* q_indices, int32_t n_sel_heads, const void* schedule,
    size_t schedule_bytes, int32_t topk, float softmax_scale, const float* q_scale,
    const float* k_scale, const float* v_scale, uint16_t* out, int64_t out_stride,
    void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * 5. E4M3 quantisation and the paged cache write: the step just before the
 *    path ([P2] Overview: a fused insert kernel writes the query in E4M3 and
 *    the new tokens' K|V into the packed cache pages; [P2] Details: the FP8
 *    cache is written with unit scales; [P2] script and [P4] forward:
 *    slot_mapping, one int64 cache slot per token).
 *
 * Every element becomes the E4M3 code nearest to x / scale, the quotient taken
 * as one correctly rounded fp32 division, ties to the even code, saturating:
 * finite values beyond +-448 and +-inf give +-448, NaN gives 0x7F, the sign of
 * zero is kept.  (The pages state neither rounding nor overflow; this is the
 * reading the library implements.)
 *
 *   src_dtype  MSA_DTYPE_BF16 or MSA_DTYPE_F32; source rows of 128 elements,
 *              strides in elements, multiples of 8, base 16-byte aligned
 *   scale      device fp32 scalar
 *   slot_mapping  [n_tokens] int64: token t goes to row s % 128 of physical page
 *              s / 128 (s = slot_mapping[t]); tokens with s < 0 are skipped, and
 *              so are slots >= num_pages * 128.  Distinct tokens must have
 *              distinct slots (otherwise which token's bytes land is unspecified).
 *
 * msa_quantize_e4m3: src [n_rows, heads, 128] -> dst [n_rows, heads, 128] E4M3,
 *   dst row stride dst_stride bytes (>= heads * 128, multiple of 8, base 8-byte
 *   aligned), heads contiguous.  For the attention and index queries.
 * msa_insert_index_k: k [n_tokens, 128] (token stride k_stride) into
 *   k_cache [num_pages, 128, 128] (the index-K layout of section 1).
 * msa_insert_kv: k, v [n_tokens, Hkv, 128] (token strides k_stride / v_stride,
 *   heads contiguous) into kv_cache [num_pages, Hkv, 128, 256]: K to bytes
 *   [..., 0:128] and V to [..., 128:256] of the token's row (the packed page of
 *   section 4), with k_scale and v_scale.
 * Rows of the caches that no token maps to are left as they are.
 * ------------------------------------------------------------------------- */
typedef enum { MSA_DTYPE_BF16 = 0, MSA_DTYPE_F32 = 1 } msa_dtype_t;

msa_status_t msa_quantize_e4m3(const void* src, int32_t src_dtype, int64_t n_rows,
                               int32_t heads, int64_t src_stride, const float* scale,
                               uint8_t* dst, int64_t dst_stride, void* stream);
msa_status_t msa_insert_index_k(const void* k, int32_t src_dtype, int64_t n_tokens,
                                int64_t k_stride, const int64_t* slot_mapping,
                                const float* scale, uint8_t* k_cache, int32_t num_pages,
                                void* stream);
msa_status_t msa_insert_kv(const void* k, const void* v, int32_t src_dtype, int64_t n_tokens,
                           int32_t num_kv_heads, int64_t k_stride, int64_t v_stride,
                           const int64_t* slot_mapping, const float* k_scale,
                           const float* v_scale, uint8_t* kv_cache, int32_t num_pages,
                           void* stream);

/* ---------------------------------------------------------------------------
 * 6. MXFP4 index keys: the 4-bit analogue of the pages' NVFP4 index cache
 *    ([P3] Details: FP8 query times FP4 key in the decode indexer), in the
 *    format gfx950's matrix cores take natively (OCP Microscaling MXFP4).
 *
 * k_data   [num_pages, 128, 64]: a token's 128 key elements as E2M1 codes,
 *          element 2i in the low nibble of byte i, 2i+1 in the high nibble
 * k_scales [num_pages, 128, 4]: E8M0 scale of each 32-element block
 *          (value 2^(code-127), 0xFF = NaN); key value = E2M1 element * 2^(code-127)
 *
 * msa_index_score_mxfp4: msa_index_score (section 1) over such keys, with the
 *   same arguments, layouts and errors; k_scale stays a per-tensor factor.
 *   k_data and k_scales 16-byte aligned.
 * msa_insert_index_k_mxfp4: quantise rows of 128 elements (src as in section
 *   5) per block of 32: exponent = floor(log2(max |x|)) - 2 clamped to
 *   [-127, 127] (-127 for a block of zeros), elements = nearest E2M1 of
 *   x * 2^-exponent, ties to even, saturating at +-6; a block holding NaN or
 *   an infinity gets scale 0xFF and zero elements.  Token t goes to row s % 128
 *   of page s / 128 of both arrays (s = slot_mapping[t]; s < 0 and
 *   s >= num_pages*128 skipped).  (The Microscaling conversion rule; the pages
 *   describe NVFP4, so this format is the reading the library implements.)
 * ------------------------------------------------------------------------- */
msa_status_t msa_index_score_mxfp4(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                                   int32_t num_index_heads, const uint8_t* k_data,
                                   const uint8_t* k_scales, int32_t num_pages,
                                   const float* q_scale, const float* k_scale, float* scores,
                                   int64_t ld_scores, void* workspace, size_t workspace_bytes,
                                   void* stream);
msa_status_t msa_insert_index_k_mxfp4(const void* k, int32_t src_dtype, int64_t n_tokens,
                                      int64_t k_stride, const int64_t* slot_mapping,
                                      uint8_t* k_data, uint8_t* k_scales, int32_t num_pages,
                                      void* stream);

/* ---------------------------------------------------------------------------
 * 7. Index scoring without allocation.  For callers that cannot allocate or
 *    provide device memory (code under HIP graph capture that must not add
 *    allocations, serving loops and harnesses that forbid allocation): exactly
 *    msa_index_score (section 1), same arguments, layouts, results and errors,
 *    except that the scorer's work list lives in a buffer built into the
 *    library instead of a caller workspace.  (Batches of one request, and of
 *    at most 64 requests and 128 query blocks, need no work list: their
 *    scorer plans its work itself and the buffer is not touched.)
 *
 * The built-in buffer holds 1 MiB per GPU (kept until the process ends); a
 * batch whose work list needs more (msa_index_score_workspace_size(vl, H) >
 * 1048576, i.e. hundreds of thousands of queries) is rejected with
 * MSA_ERR_UNSUPPORTED before anything is launched.  Nothing is allocated:
 * the buffer's device address is looked up on the first call on each device.
 * Every call on one GPU shares that GPU's buffer, so calls that overlap in
 * time on one GPU (other streams, other host threads) race and must be
 * ordered by the caller; consecutive calls on one stream are safe.
 * ------------------------------------------------------------------------- */
msa_status_t msa_index_score_noalloc(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                                     int32_t num_index_heads, const uint8_t* k_cache,
                                     int32_t num_pages, const float* q_scale,
                                     const float* k_scale, float* scores, int64_t ld_scores,
                                     void* stream);

/* ---------------------------------------------------------------------------
 * Diagnostics.
 * ------------------------------------------------------------------------- */
const char* msa_status_string(msa_status_t status);  /* static string */
const char* msa_last_error(void);   /* thread-local detail of this thread's last failed call */
int32_t msa_abi_version(void);      /* MSA_ABI_VERSION */
#define MSA_ABI_VERSION 3

/* ---------------------------------------------------------------------------
 * 8. Metadata check, for callers whose device metadata may be wrong.  The
 *    other calls clamp device indices that contradict the host-side sizes so
 *    that they do not fault, and then give unspecified results; this call
 *    reports such contradictions instead.  (The batch layout it checks is the
 *    one the other calls take: [P2] script and [P4] forward, cu_seqlens_q/k,
 *    block_table, total_kv_blocks.)
 *
 * Queues one small kernel on `stream` that writes flags[0] (device int32,
 * overwritten, not accumulated) with the OR of:
 *   MSA_BAD_CU_Q   cu_seqlens_q[0] != 0, a decrease, an entry > total_q, or
 *                  cu_seqlens_q[batch] != total_q
 *   MSA_BAD_CU_K   cu_seqlens_k[0] != 0, a decrease, or a request with more
 *                  new tokens than tokens (seqlen_q_b > seqlen_k_b)
 *   MSA_BAD_MAX_Q  a request with seqlen_q_b > max_seqlen_q
 *   MSA_BAD_MAX_K  a request with seqlen_k_b > max_seqlen_k
 *   MSA_BAD_PAGES  a request with more than max_pages pages
 *   MSA_BAD_ROWS   sum_b ceil(seqlen_k_b / 128) != total_rows
 *   MSA_BAD_BLOCK  a block_table entry of a used page (j < min(pages_b,
 *                  max_pages)) outside [0, num_pages)
 * 0 means the metadata agrees with the host-side sizes.  Reads only inside the
 * arrays the host-side sizes describe; host-side errors as for the other calls.
 * ------------------------------------------------------------------------- */
#define MSA_BAD_CU_Q 1
#define MSA_BAD_CU_K 2
#define MSA_BAD_MAX_Q 4
#define MSA_BAD_MAX_K 8
#define MSA_BAD_PAGES 16
#define MSA_BAD_ROWS 32
#define MSA_BAD_BLOCK 64
msa_status_t msa_check_varlen(const msa_varlen_t* vl, int32_t num_pages, int32_t* flags,
                              void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H_ */
