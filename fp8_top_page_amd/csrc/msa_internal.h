// Internal declarations shared by the host API and the HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "msa.h"

namespace msa {

constexpr int kPage = MSA_PAGE_SIZE;   // tokens per page
constexpr int kDim = MSA_HEAD_DIM;     // head dimension (bytes per E4M3 row)
constexpr int kTopK = MSA_TOPK;

// ---- index scorer tiling -------------------------------------------------
// A work item is (request, block of score_qblock(H) queries, chunk of pages).
// Every wave keeps the fragments of kScoreQueriesPerWave / H queries (all H
// heads) in registers; kScoreWaves waves share one index-K page in LDS.
#ifndef MSA_SCORE_WAVES
#define MSA_SCORE_WAVES 16
#endif
#ifndef MSA_SCORE_QPW
#define MSA_SCORE_QPW 64
#endif
constexpr int kScoreWaves = MSA_SCORE_WAVES;
constexpr int kScoreQueriesPerWave = MSA_SCORE_QPW;
constexpr int score_qtiles(int H) { return kScoreQueriesPerWave / 16 / H; }
constexpr int score_qblock(int H) { return kScoreWaves * 16 * score_qtiles(H); }

// Compute units of the current device (cached per device).
int device_cu_count();

struct ScorePlan {
  int32_t pages_per_item;   // 0: chosen by the device plan
  int64_t max_items;        // host upper bound (grid size before padding)
  size_t workspace_bytes;
};
ScorePlan score_plan(const msa_varlen_t* vl, int H);

struct ScoreArgs {
  msa_varlen_t vl;
  const uint8_t* q;
  int64_t q_stride;
  int H;
  const uint8_t* k_cache;      // E4M3 rows [num_pages, 128, 128], or MXFP4 data [num_pages, 128, 64]
  int32_t num_pages;
  const float* q_scale;
  const float* k_scale;
  float* scores;
  int64_t ld;
  void* workspace;
  ScorePlan plan;
  const uint8_t* k_scales;     // nullptr: E4M3 keys; else MXFP4 block scales [num_pages, 128, 4]
};
hipError_t launch_index_score(const ScoreArgs& a, hipStream_t stream);
// Per-index-head scores: a.H single-head passes over one single-head plan,
// head h's scores at a.scores + h * head_stride (a.plan must be score_plan(vl, 1)).
hipError_t launch_index_score_heads(const ScoreArgs& a, int64_t head_stride, hipStream_t stream);
// Decode-like batches (every request at most 64 / H queries): scores and the
// top-16 selection in one scorer pass plus a merge, without writing scores.
// The workspace holds the plan (a.plan.workspace_bytes) and then
// index_score_topk_extra_bytes of candidate lists.
hipError_t launch_index_score_topk(const ScoreArgs& a, int n_local, int32_t* out,
                                   int64_t out_stride, hipStream_t stream);
size_t index_score_topk_extra_bytes(const ScorePlan& p, int H, int64_t total_q);

// ---- top-k ---------------------------------------------------------------
struct TopkArgs {
  msa_varlen_t vl;
  const float* scores;
  int64_t ld;
  int n_local;
  int32_t* out;
  int64_t out_stride;
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);

// ---- k2q CSR + attention schedule ----------------------------------------
// Queries (CSR entries) per attention work item, at most.
constexpr int kAttnQCMax = 64;

// Long single-request prefills run the attention as one persistent kernel over
// query chunks of 2^kChunkShift queries (work items never cross a chunk): the
// partials of a chunk live in one slot of a ring of kRingSlots chunks, and the
// chunk's combine tasks run in the same kernel once its items are done.
constexpr int kChunkShift = 9;
constexpr bool kChunkedAttention = false;   // off: see sched_layout

struct SchedLayout {
  // byte offsets inside the schedule buffer
  size_t hdr, row_base, blk_tot, items, okey, perm, kstart, rowsel, wbase, bitmap, qslot, smask,
      nib, total;
  int32_t fused;          // chunked persistent attention (items in query chunks, see above)
  int32_t piece_words;    // bitmap words per item piece (items never cross one)
  int64_t n_rows;         // n_sel * total_rows
  int64_t words_per_row;  // bitmap words per row (one bit per query slot, padded)
  int64_t n_units;        // bitmap units (64 consecutive words of the row-major bitmap)
  int64_t n_blocks;       // count/fill blocks
  int64_t max_items;
  int32_t item_q;         // queries (CSR entries) per attention work item, at most
  int32_t order_shift;    // items taken in order of (first query >> order_shift); 0: list order
  int32_t order_keys;     // distinct keys of that order
  int64_t inv_len;        // total_q * n_sel * topk: entries of the (query, slot) -> row table
  int64_t word_chunks;    // row chunks per (request, bitmap word) in the words pass
  int64_t word_blocks;    // blocks of the words pass
};
SchedLayout sched_layout(const msa_varlen_t* vl, int n_sel, int topk);

struct CsrArgs {
  msa_varlen_t vl;
  const int32_t* topk;
  int64_t tq_stride, th_stride;
  int n_sel;
  int32_t* row_ptr;
  int32_t* q_indices;
  uint8_t* sched;
  SchedLayout L;
};
hipError_t launch_k2q_csr(const CsrArgs& a, hipStream_t stream);

// ---- sparse attention -------------------------------------------------------
struct AttnArgs {
  msa_varlen_t vl;
  const uint8_t* q;
  int64_t q_stride;
  int Hq, Hkv, n_sel;
  const uint8_t* kv;           // E4M3 K|V rows [num_pages, Hkv, 128, 256], or MXFP4 codes
                               // [num_pages, Hkv, 128, 128] when kv_scales is set
  int32_t num_pages;
  const int32_t* row_ptr;
  const int32_t* q_indices;
  const uint8_t* sched;
  SchedLayout L;
  float softmax_scale;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  uint16_t* out;
  int64_t out_stride;
  void* workspace;
  const uint8_t* kv_scales;    // MXFP4 E8M0 block scales [num_pages, Hkv, 128, 8], or nullptr
};
size_t attn_workspace_bytes(const msa_varlen_t* vl, int Hq, int Hkv, int n_sel, int topk);
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream);

// ---- E4M3 quantisation / paged cache write ----------------------------------
struct QuantArgs {
  int n_parts;               // 1, or 2 (K and V of the packed cache)
  const void* src[2];
  const float* scale[2];
  int64_t col_off[2];        // destination byte offset inside a row, per part
  int dtype;
  int64_t n_tokens;
  int heads;
  int64_t src_tok_stride[2], src_head_stride;   // elements
  const int64_t* slots;      // nullptr: linear destination
  int64_t max_slot;
  uint8_t* dst;
  int64_t dst_tok_stride, dst_page_stride, dst_head_stride, dst_row_stride;   // bytes
};
hipError_t launch_quantize(const QuantArgs& q, hipStream_t stream);

struct Mx4Args {             // MXFP4 index-key insert
  const void* src;
  int dtype;
  int64_t n_tokens;
  int64_t src_tok_stride;    // elements
  const int64_t* slots;
  int64_t max_slot;
  uint8_t* data;             // [num_pages, 128, 64]
  uint8_t* scales;           // [num_pages, 128, 4]
};
hipError_t launch_insert_mxfp4(const Mx4Args& q, hipStream_t stream);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
// Queries per attention work item: 64 when the rows average at least that many
// (long prefill chunks: each staged page serves more row tiles and is staged
// half as often), else 32 (rows of a few queries, where a row of the local page
// holds many more than the rest and longer items would finish last).
inline int32_t attn_item_queries(const msa_varlen_t* vl) {
  const int64_t per_row =
      ceil_div((int64_t)vl->total_q * kTopK, vl->total_rows > 0 ? vl->total_rows : 1);
  return per_row >= kAttnQCMax ? kAttnQCMax : 32;
}
// Whether the attention stages each 16-row tile of split rows in LDS and writes
// whole rows (rows averaging at least 16 queries: many tiles per item, so the
// staging overlaps other tiles' work), or stores each lane's codes directly
// (rows of a few queries, where an item is one or two tiles and the staging
// round trip would sit on its critical path).
inline bool attn_stage_rows(const msa_varlen_t* vl) {
  return ceil_div((int64_t)vl->total_q * kTopK, vl->total_rows > 0 ? vl->total_rows : 1) >= 16;
}
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace msa
