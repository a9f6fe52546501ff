// FP8 (E4M3) page indexer for gfx950.
//
// Computes, for every query token and every page it can see, the page score
// q_scale * k_scale * max over the page's visible tokens of sum_h q_h . k
// (vLLM PR 60930, Overview and Details: the FP8 indexer scores every 128-token
// page for each query; the work is planned on the device, with no host sync,
// and the scoring call neither allocates nor synchronises).
//
// Design (MI355X):
//  * Planning: one small kernel turns cu_seqlens_q/k into a list of work items
//    (request, block of queries, chunk of pages), causal-trimmed, in the
//    workspace.  It first sums the visible pages of every query block, then
//    tries six chunk sizes (about 1 to 6 items per compute unit) and keeps the
//    one whose items finish first when dealt out in rounds of one per compute
//    unit (each round as long as a full chunk plus the item's start-up), so a
//    batch of uneven query blocks neither leaves a nearly empty last round nor
//    pays many start-ups.  One persistent scorer block per compute unit strides
//    over the items (the item count is known only on the device).
//  * Scoring: tokens are the MFMA M axis, queries the N axis.  Each of the 16
//    waves keeps the E4M3 fragments of 64/H queries (all H heads) in registers
//    for the whole item; index-K pages (16 KiB) stream into a ring of four LDS
//    slots by direct global -> LDS copies and are read by every wave.  The H
//    head products chain into one accumulator (a contraction of length H*128).
//    On the few pages that cross a query's position, token tiles every query
//    of a tile has passed take the plain max, tiles none of them reaches are
//    skipped, and only the tiles in between are masked.
//  * Decode-like batches (every request at most 64/H queries): one wave's
//    queries are all there is, so the waves split each page instead: wave w
//    scores a 16-token slice of one page for all the queries, and the slices'
//    maxima are reduced through LDS.
//  * Epilogue: each lane holds 4 consecutive tokens of one query per 16-token
//    tile; the max over the page's 8 tiles is taken in registers, one lane
//    exchange folds the 4 lane groups into 2, and the two partial maxima go to
//    an LDS tile (8 pages x 2 per query).  At the end of every group of 8 pages
//    the tile is flushed: a lane maxes the 2 partials of each page of a (query,
//    4-page) half group, scales them and stores them, two lanes covering the
//    32 contiguous bytes of a query's group (whole 32-byte write granules of
//    HBM).
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

// Maximum of two floats as v_maximum_f32 (IEEE 754-2019 maximum, a NaN
// operand gives NaN): fmaxf's NaN-dropping form costs a quieting move per
// operand, and a dot product that is NaN (a NaN code in the keys or queries)
// makes the page score NaN, as a plain maximum over the products does.
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

constexpr int kLdsPage = kPage * kDim;       // 16 KiB: 128 rows of 128 B, 16-byte pieces swizzled
constexpr int kThreads = kScoreWaves * 64;
constexpr int kFlush = 16;                   // pages per score-tile flush (decode kernel)
constexpr int kSRow = kFlush + 1;            // score-tile row stride in floats
constexpr int kSRowG = 20;                   // prefill tile: 8 pages x 2 partials, padded (16-byte rows)
constexpr int kMaxItemPages = 256;           // pages per work item, at most
constexpr int kMinItemPages = 4;             // ... and at least
constexpr int kPlanCUs = 256;                // compute units the item sizing aims to fill
constexpr int kPlanRounds = 6;               // item sizes for about k rounds of kPlanCUs items, k = 1..6,
constexpr int kPlanCands = kPlanRounds + 3;   // and three sizes at and just above one round's
constexpr int kPlanLoopItems = 16;           // items per q-block up to which its thread writes them
constexpr int kDirectMaxQBlocks = 128;       // q-blocks of a batch planned without the plan kernel, at most
constexpr int kWavePlanMaxB = 64;            // requests of a batch planned by the scorer's waves, at most

struct ItemHdr {
  int32_t n_items;
  int32_t pages_per_item;                    // chosen by the plan (a multiple of 4 for the decode kernel)
  int32_t pad[62];
};

struct ScoreK {
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* block_table;
  int64_t bt_stride;
  int32_t batch;
  int32_t num_pages;
  int32_t max_pages;
  const uint8_t* q;
  int64_t q_stride;
  const uint8_t* k_cache;
  const float* q_scale;
  const float* k_scale;
  float* scores;
  int64_t ld;
  const ItemHdr* hdr;
  const int4* items;
  const uint8_t* k_scales;   // MXFP4 keys: [num_pages, 128, 4] E8M0 block scales
  uint64_t* cand;            // fused selection (decode kernel): [items, queries, 16] candidate keys
  int2* first_item;          // fused selection: [total_q] (first work item, position) of each query
  int32_t n_local;           // fused selection: forced recent pages
  // A one-request batch planned on the host: direct_items > 0 items of
  // direct_pc pages, q-block by q-block, decoded from these values instead of
  // read from hdr / items (neither is written then).
  int32_t direct_items;
  int32_t direct_pc;
  int32_t direct_sq;         // the request's queries
  int32_t direct_ctx;        // its context: seqlen_k - seqlen_q
  // A batch of at most kWavePlanMaxB requests and kDirectMaxQBlocks q-blocks:
  // every wave plans it from cu_seqlens (wave_plan != 0), with this alignment
  // of the chunk sizes (plan_align), instead of reading hdr / items.
  int32_t wave_plan;
  int32_t plan_align;
};

// ---------------------------------------------------------------------------
// Plan: one block.  Pass 1 sums v (visible pages) over every q-block and
// chooses the pages per item; pass 2 emits the items request by request, q-block
// by q-block, page chunk by page chunk: item = {b, first global query, query
// count, first page}.  For each batch of up to 256 q-blocks one thread per
// q-block counts its page chunks and a block scan places them; the thread then
// writes its q-block's items if every q-block has few, else all threads share
// the batch's items, each finding its q-block by binary search.
// ---------------------------------------------------------------------------
// The sizing helpers below also run on the host, which plans one-request
// batches itself (plan_one_request).
template <class T>
__host__ __device__ constexpr T plan_min(T a, T b) { return a < b ? a : b; }
template <class T>
__host__ __device__ constexpr T plan_max(T a, T b) { return a < b ? b : a; }

__host__ __device__ __forceinline__ int qblock_visible(int ctx, int qf, int qn) {
  return (ctx + qf + qn - 1) / kPage + 1;
}

// Pages per item for about k rounds of kPlanCUs items: the w visible pages of
// all q-blocks cut into k * kPlanCUs chunks, rounded up to a multiple of round,
// within [kMinItemPages, kMaxItemPages].
__host__ __device__ __forceinline__ int cand_pages(int64_t w, int k, int round) {   // round: a power of two
  const int64_t per = (int64_t)kPlanCUs * k;
  const int64_t pc = ((w + per - 1) / per + round - 1) & ~(int64_t)(round - 1);
  return (int)plan_min<int64_t>(kMaxItemPages, plan_max<int64_t>(kMinItemPages, pc));
}
// The candidates: the k = 1..kPlanRounds sizes as multiples of 4, then three
// sizes at and just above one round's: ceil(w / kPlanCUs) + 0, 1, 2 pages (the
// remainder chunks of uneven q-blocks often push a size just past one round,
// and a slightly larger chunk keeps it in one).  align = 4 (the decode kernel,
// whose score flush is 16-byte aligned relative to an item's first page) keeps
// every size a multiple of 4: the last three become the one-round size + 4, 8,
// 12.  The prefill kernel's flush follows absolute 8-page groups: align = 1.
__host__ __device__ __forceinline__ void plan_candidates(int64_t w, int align, int (&cand)[kPlanCands]) {
#pragma unroll
  for (int k = 0; k < kPlanRounds; ++k) cand[k] = cand_pages(w, k + 1, 4);
  const int one = cand_pages(w, 1, align);
#pragma unroll
  for (int j = 0; j < kPlanCands - kPlanRounds; ++j)
    cand[kPlanRounds + j] = plan_min(kMaxItemPages, one + (align == 1 ? j : 4 * (j + 1)));
}
// Predicted run time of n items of at most pc pages, in fifths of a page: the
// items run in rounds of kPlanCUs (one block per compute unit), each round as
// long as a full item, whose start-up (query fragments, first page copies)
// costs about 1.2 pages.  The plan keeps the candidate with the least.
__host__ __device__ __forceinline__ int64_t cand_cost(int64_t n, int pc) {
  return (n + kPlanCUs - 1) / kPlanCUs * (5 * (int64_t)pc + 6);
}
// Block-wide sums of per-thread values over W waves (result in every thread).
template <int W, int N>
__device__ __forceinline__ void block_sum(int (&x)[N], int (*s_red)[N]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = wave_sum(x[i]);
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < N; ++i) s_red[wave][i] = x[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    x[i] = 0;
    for (int k = 0; k < W; ++k) x[i] += s_red[k][i];
  }
  __syncthreads();
}
// Query blocks that all see about the same number of pages (every decode batch,
// a short chunk over a long context) get about one item per compute unit; only
// uneven batches weigh the candidates.
__host__ __device__ __forceinline__ bool plan_uniform(int vmin, int vmax) { return (vmax - vmin) * 8 <= vmax; }

// The candidate with the least predicted time (the first one on ties).
__host__ __device__ __forceinline__ int best_pages(const int (&cand)[kPlanCands], const int (&n)[kPlanCands]) {
  int best = cand[0];
  int64_t best_cost = cand_cost(n[0], best);
  for (int k = 1; k < kPlanCands; ++k) {
    const int64_t c = cand_cost(n[k], cand[k]);
    if (c < best_cost) { best_cost = c; best = cand[k]; }
  }
  return best;
}

__global__ __launch_bounds__(256) void score_plan_kernel(const int32_t* __restrict__ cu_q,
                                                         const int32_t* __restrict__ cu_k, int B,
                                                         int qblock, int align, int64_t max_items,
                                                         ItemHdr* __restrict__ hdr,
                                                         int4* __restrict__ items) {
  __shared__ int wave_tot[4], wave_mx[4];
  __shared__ int s_off[256], s_qf[256], s_qn[256];
  __shared__ int64_t running;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // pass 1: total and spread of the visible pages over all q-blocks; for
  // uneven q-blocks also the chunk count of every candidate item size
  __shared__ int64_t s_w[4];
  __shared__ int s_vmin[4], s_vmax[4];
  __shared__ int s_red[4][kPlanCands];
  int64_t w = 0;
  int vmin = INT32_MAX, vmax = 0;
  for (int b = 0; b < B; ++b) {
    const int sq = cu_q[b + 1] - cu_q[b];
    const int ctx = (cu_k[b + 1] - cu_k[b]) - sq;
    const int nqb = (sq + qblock - 1) / qblock;
    for (int qb = tid; qb < nqb; qb += 256) {
      const int qf = qb * qblock;
      const int v = qblock_visible(ctx, qf, min(sq - qf, qblock));
      w += v;
      vmin = min(vmin, v);
      vmax = max(vmax, v);
    }
  }
  w = wave_sum64(w);
  vmin = wave_min(vmin);
  vmax = wave_max(vmax);
  if (lane == 0) { s_w[wave] = w; s_vmin[wave] = vmin; s_vmax[wave] = vmax; }
  __syncthreads();
  int64_t tw = 0;
  int lo = INT32_MAX, hi = 0;
  for (int k = 0; k < 4; ++k) { tw += s_w[k]; lo = min(lo, s_vmin[k]); hi = max(hi, s_vmax[k]); }
  int pc_all = cand_pages(tw, 1, 4);
  if (!plan_uniform(lo, hi)) {
    int cand[kPlanCands], n[kPlanCands] = {};
    plan_candidates(tw, align, cand);
    for (int b = 0; b < B; ++b) {
      const int sq = cu_q[b + 1] - cu_q[b];
      const int ctx = (cu_k[b + 1] - cu_k[b]) - sq;
      const int nqb = (sq + qblock - 1) / qblock;
      for (int qb = tid; qb < nqb; qb += 256) {
        const int qf = qb * qblock;
        const int v = qblock_visible(ctx, qf, min(sq - qf, qblock));
#pragma unroll
        for (int k = 0; k < kPlanCands; ++k) n[k] += (v + cand[k] - 1) / cand[k];
      }
    }
    block_sum<4>(n, s_red);
    pc_all = best_pages(cand, n);
  }
  if (tid == 0) running = 0;
  __syncthreads();
  const int pc = pc_all;

  // pass 2: emit
  for (int b = 0; b < B; ++b) {
    const int q0 = cu_q[b], sq = cu_q[b + 1] - q0;
    const int sk = cu_k[b + 1] - cu_k[b];
    const int ctx = sk - sq;
    const int nqb = (sq + qblock - 1) / qblock;
    for (int base = 0; base < nqb; base += 256) {
      const int qb = base + tid;
      int nch = 0, qf = 0, qn = 0;
      if (qb < nqb) {
        qf = qb * qblock;
        qn = min(sq - qf, qblock);
        nch = (qblock_visible(ctx, qf, qn) + pc - 1) / pc;
      }
      const int incl = wave_inclusive_scan(nch);
      const int mx = wave_max(nch);
      if (lane == 63) { wave_tot[wave] = incl; wave_mx[wave] = mx; }
      __syncthreads();
      int wave_off = 0, total = 0, maxc = 0;
      for (int k = 0; k < 4; ++k) {
        if (k < wave) wave_off += wave_tot[k];
        total += wave_tot[k];
        maxc = max(maxc, wave_mx[k]);
      }
      const int64_t run = running;
      if (maxc <= kPlanLoopItems) {
        // few chunks per q-block: each q-block's thread writes its own
        const int64_t first = run + wave_off + incl - nch;
        for (int c = 0; c < nch; ++c)
          if (first + c < max_items) items[first + c] = make_int4(b, q0 + qf, qn, c * pc);
      } else {
        // many: every thread takes items, each finding its q-block by search
        s_off[tid] = wave_off + incl - nch;
        s_qf[tid] = qf;
        s_qn[tid] = qn;
        __syncthreads();
        for (int k = tid; k < total; k += 256) {
          int lo = 0, hi = 255;             // last q-block of the batch with s_off <= k
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= k) lo = mid; else hi = mid - 1;
          }
          const int64_t dst = run + k;
          if (dst < max_items) items[dst] = make_int4(b, q0 + s_qf[lo], s_qn[lo], (k - s_off[lo]) * pc);
        }
      }
      __syncthreads();
      if (tid == 0) running = run + total;
      __syncthreads();
    }
  }
  if (tid == 0) {
    hdr->n_items = (int32_t)min<int64_t>(running, max_items);
    hdr->pages_per_item = pc;
  }
}

// Same plan for batches of at most kPlanMaxB requests and kPlanMaxG q-blocks,
// with the request table and the q-block offsets in LDS: every pass is spread
// over all q-blocks (or all items) instead of walking the requests in turn.
constexpr int kPlanThreads = 256;
constexpr int kPlanMaxB = 1024;
constexpr int kPlanMaxG = 4096;

__global__ __launch_bounds__(kPlanThreads) void score_plan_table_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int B, int qblock,
    int align, int64_t max_items, ItemHdr* __restrict__ hdr, int4* __restrict__ items) {
  constexpr int kW = kPlanThreads / 64;
  __shared__ int s_q0[kPlanMaxB], s_sq[kPlanMaxB], s_ctx[kPlanMaxB], s_qbase[kPlanMaxB + 1];
  __shared__ int s_first[kPlanMaxG + 1];
  __shared__ int s_cnt[kW], s_mx[kW];
  __shared__ int64_t s_w[kW];
  __shared__ int s_lo[kW], s_hi[kW];
  __shared__ int s_red[kW][kPlanCands];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  auto block_scan = [&](int x, int* total) {   // exclusive; adds the block total to *total
    const int incl = wave_inclusive_scan(x);
    if (lane == 63) s_cnt[wave] = incl;
    __syncthreads();
    int off = 0, tot = 0;
    for (int k = 0; k < kW; ++k) {
      if (k < wave) off += s_cnt[k];
      tot += s_cnt[k];
    }
    __syncthreads();
    *total += tot;
    return off + incl - x;
  };
  auto last_le = [&](const int* arr, int n, int key) {   // last index i < n with arr[i] <= key
    int lo = 0, hi = n - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (arr[mid] <= key) lo = mid; else hi = mid - 1;
    }
    return lo;
  };

  // pass 0: request table, q-blocks per request and their offsets
  int G = 0;
  for (int r0 = 0; r0 < B; r0 += kPlanThreads) {
    const int r = r0 + tid;
    int nqb = 0;
    if (r < B) {
      const int q0 = cu_q[r], sq = cu_q[r + 1] - q0;
      s_q0[r] = q0;
      s_sq[r] = sq;
      s_ctx[r] = (cu_k[r + 1] - cu_k[r]) - sq;
      nqb = (sq + qblock - 1) / qblock;
    }
    const int qoff = G + block_scan(nqb, &G);
    if (r < B) s_qbase[r] = qoff;
  }
  __syncthreads();
  G = min(G, kPlanMaxG);
  auto visible = [&](int g, int* b_out, int* qf_out, int* qn_out) {
    const int b = last_le(s_qbase, B, g);
    const int qf = (g - s_qbase[b]) * qblock;
    *b_out = b;
    *qf_out = qf;
    *qn_out = min(s_sq[b] - qf, qblock);
    return (s_ctx[b] + qf + *qn_out - 1) / kPage + 1;
  };

  // pass 1: total and spread of v over all q-blocks; for uneven q-blocks also
  // the chunk count of every candidate item size -> pages per item
  int64_t w = 0;
  int vmin = INT32_MAX, vmax = 0;
  for (int g = tid; g < G; g += kPlanThreads) {
    int b, qf, qn;
    const int v = visible(g, &b, &qf, &qn);
    w += v;
    vmin = min(vmin, v);
    vmax = max(vmax, v);
  }
  w = wave_sum64(w);
  vmin = wave_min(vmin);
  vmax = wave_max(vmax);
  if (lane == 0) { s_w[wave] = w; s_lo[wave] = vmin; s_hi[wave] = vmax; }
  __syncthreads();
  int64_t tw = 0;
  int lo = INT32_MAX, hi = 0;
  for (int k = 0; k < kW; ++k) { tw += s_w[k]; lo = min(lo, s_lo[k]); hi = max(hi, s_hi[k]); }
  int pc = cand_pages(tw, 1, 4);
  if (!plan_uniform(lo, hi)) {
    int cand[kPlanCands], n[kPlanCands] = {};
    plan_candidates(tw, align, cand);
    for (int g = tid; g < G; g += kPlanThreads) {
      int b, qf, qn;
      const int v = visible(g, &b, &qf, &qn);
#pragma unroll
      for (int k = 0; k < kPlanCands; ++k) n[k] += (v + cand[k] - 1) / cand[k];
    }
    block_sum<kW>(n, s_red);
    pc = best_pages(cand, n);
  }

  // pass 2: page chunks per q-block, offsets
  int n_items = 0, maxc = 0;
  for (int base = 0; base < G; base += kPlanThreads) {
    const int g = base + tid;
    int c = 0;
    if (g < G) {
      int b, qf, qn;
      c = (visible(g, &b, &qf, &qn) + pc - 1) / pc;
    }
    const int mx = wave_max(c);
    if (lane == 0) s_mx[wave] = mx;
    const int first = n_items + block_scan(c, &n_items);   // its barriers publish s_mx
#pragma unroll
    for (int k = 0; k < kW; ++k) maxc = max(maxc, s_mx[k]);
    if (g < G) s_first[g] = first;
    __syncthreads();                          // s_mx is rewritten by the next round
  }
  __syncthreads();

  // emit: few chunks per q-block, each q-block's thread writes its own; many,
  // item k goes to the last q-block whose first item is <= k
  const int64_t n_out = min<int64_t>(n_items, max_items);
  if (maxc <= kPlanLoopItems) {
    for (int g = tid; g < G; g += kPlanThreads) {
      int b, qf, qn;
      const int c = (visible(g, &b, &qf, &qn) + pc - 1) / pc;
      const int first = s_first[g];
      for (int k = 0; k < c; ++k)
        if (first + k < n_out) items[first + k] = make_int4(b, s_q0[b] + qf, qn, k * pc);
    }
  } else {
    for (int k = tid; k < n_out; k += kPlanThreads) {
      const int g = last_le(s_first, G, k);
      int b, qf, qn;
      visible(g, &b, &qf, &qn);
      items[k] = make_int4(b, s_q0[b] + qf, qn, (k - s_first[g]) * pc);
    }
  }
  if (tid == 0) {
    hdr->n_items = (int32_t)n_out;
    hdr->pages_per_item = pc;
  }
}

// ---------------------------------------------------------------------------
// Scorer.
// ---------------------------------------------------------------------------

// Index-K page layout in LDS: row t (token) holds its eight 16-byte pieces with
// piece c stored at position c ^ ((t >> 1) & 7).  The direct-to-LDS copy below
// fills whole 1 KiB spans lane by lane, so rows cannot be padded; the swizzle
// makes the fragment reads (16 rows x 32 bytes) free of bank conflicts instead.
struct Swz {
  int off0, off1;   // byte offsets in a row of this lane's two pieces (2 grp, 2 grp + 1)
};
__device__ __forceinline__ Swz lane_swizzle(int col, int grp) {
  const int s = (col >> 1) & 7;                 // rows 16T + col share (row >> 1) & 7
  return Swz{16 * ((2 * grp) ^ s), 16 * ((2 * grp + 1) ^ s)};
}
__device__ __forceinline__ v8i load_frag_swz(const uint8_t* row, const Swz& z) {
  const uint4 x = *reinterpret_cast<const uint4*>(row + z.off0);
  const uint4 y = *reinterpret_cast<const uint4*>(row + z.off1);
  v8i r;
  r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
  r[4] = y.x; r[5] = y.y; r[6] = y.z; r[7] = y.w;
  return r;
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane
// l's bytes land at LDS byte address lds_addr + 16 l (lds_addr wave-uniform,
// passed in M0).  Inline assembly keeps the copy out of the compiler's
// wait-count bookkeeping, which cannot tell the ring slots apart and would
// otherwise wait for every copy in flight before each LDS read; the kernel's own
// vmcnt waits and barriers order copies and reads.  (Counters retire in issue
// order, so copies the compiler does not know of only lengthen the waits it
// places for other loads.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               ::"v"(src), "s"(lds_addr)
               : "m0");
}
#pragma clang diagnostic pop

// MXFP4 keys (E2M1 pairs, element 2i in the low nibble of byte i, and one E8M0
// scale per 32-element block).  A page slot holds 128 rows of 64 bytes, the
// 16-byte piece c of row t (one block) at position c ^ ((t >> 2) & 3) (rows
// 4 apart share banks, so four consecutive row quads take four different
// pieces), then the 512 scale bytes, 4 per row.  The scaled matrix-core op
// (v_mfma_scale_f32_16x16x128_f8f6f4, A = E2M1, B = E4M3) pairs lane group g's
// 32 nibbles (its A block) with query bytes [16g, 16g + 16) and
// [64 + 16g, 80 + 16g) of the B lane group g, and multiplies the lane's A
// products by 2^(scale - 127) (probed on gfx950; the upper four A registers are
// not read).
constexpr int kF4Data = kPage * 64;            // 8 KiB of E2M1 pairs per page
constexpr int kF4Slot = kF4Data + kPage * 4;   // + 512 B of scales
__device__ __forceinline__ int f4_piece(int col, int grp) {   // byte offset of the lane's piece
  return 16 * (grp ^ ((col >> 2) & 3));
}
__device__ __forceinline__ v8i load_frag_f4(const uint8_t* row, int off) {
  const uint4 x = *reinterpret_cast<const uint4*>(row + off);
  v8i r;
  r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
  r[4] = x.x; r[5] = x.y; r[6] = x.z; r[7] = x.w;     // not read by the op
  return r;
}
// Query fragment for MXFP4 keys: bytes [16g, 16g + 16) and [64 + 16g, 80 + 16g).
__device__ __forceinline__ v8i load_qfrag_f4(const uint8_t* q, int grp) {
  const uint4 x = *reinterpret_cast<const uint4*>(q + 16 * grp);
  const uint4 y = *reinterpret_cast<const uint4*>(q + 64 + 16 * grp);
  v8i r;
  r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
  r[4] = y.x; r[5] = y.y; r[6] = y.z; r[7] = y.w;
  return r;
}
__device__ __forceinline__ v4f mfma_f4_e4m3(const v8i& a, const v8i& b, const v4f& c, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, scale_a, 0, 127);
}
// The lane's A fragment and scale of token tile T of an MXFP4 page slot.
__device__ __forceinline__ v8i f4_frag(const uint8_t* pg, int T, int col, int off) {
  return load_frag_f4(pg + (T * 16 + col) * 64, off);
}
__device__ __forceinline__ int f4_scale(const uint8_t* pg, int T, int col, int grp) {
  return pg[kF4Data + (T * 16 + col) * 4 + grp];
}

// Max over one page's 128 tokens for every resident query tile.  A fragments
// (16 tokens x 128 bytes) are read from LDS one tile ahead of their products,
// and the max of each product is taken one product later (after the next one
// is issued), so the wave does not stall on the matrix-core latency.
template <int H, int NQT>
__device__ __forceinline__ void page_max(const uint8_t* __restrict__ pg, const v8i (&qf)[NQT][H],
                                         int col, const Swz& z, v4f (&rmax)[NQT]) {
#pragma unroll
  for (int n = 0; n < NQT; ++n) rmax[n] = v4f{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  v8i a_cur = load_frag_swz(pg + col * kDim, z);
  v4f prev;
#pragma unroll
  for (int T = 0; T < 8; ++T) {
    v8i a_nxt;
    if (T < 7) a_nxt = load_frag_swz(pg + ((T + 1) * 16 + col) * kDim, z);
#pragma unroll
    for (int n = 0; n < NQT; ++n) {
      v4f acc = mfma_e4m3(a_cur, qf[n][0], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int h = 1; h < H; ++h) acc = mfma_e4m3(a_cur, qf[n][h], acc);
      if (T > 0 || n > 0) {
        const int pn = n > 0 ? n - 1 : NQT - 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) rmax[pn][i] = fmax_nan(rmax[pn][i], prev[i]);
      }
      prev = acc;
    }
    if (T < 7) a_cur = a_nxt;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) rmax[NQT - 1][i] = fmax_nan(rmax[NQT - 1][i], prev[i]);
}

// Same with the causal cut: token (16T + 4*grp + i) of the page counts for the
// query in lane column n only if it is <= lim0 + 16n (lim0 = last visible token
// of the lane's query in tile 0; consecutive queries are consecutive
// positions).  L0 (wave-uniform) is the limit of the wave's first query, so the
// limits of tile n span [L0 + 16n, L0 + 16n + 15]: token tiles past all of them
// are skipped, tiles below all of them take the plain max, and only the tiles
// that straddle them are masked element by element.  Used only on the few
// pages that cross a query's position.
template <int H, int NQT>
__device__ __forceinline__ void page_max_causal(const uint8_t* __restrict__ pg,
                                                const v8i (&qf)[NQT][H], int lim0, int L0, int col,
                                                int grp, const Swz& z, v4f (&rmax)[NQT]) {
#pragma unroll
  for (int n = 0; n < NQT; ++n) rmax[n] = v4f{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int T = 0; T < 8; ++T) {
    if (16 * T > L0 + NQT * 16 - 1) break;          // masked for every query of the wave
    const v8i a_cur = load_frag_swz(pg + (T * 16 + col) * kDim, z);
#pragma unroll
    for (int n = 0; n < NQT; ++n) {
      const int lo = L0 + 16 * n;                    // least limit of the tile's queries
      if (16 * T > lo + 15) continue;                // masked for every query of the tile
      v4f acc = mfma_e4m3(a_cur, qf[n][0], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int h = 1; h < H; ++h) acc = mfma_e4m3(a_cur, qf[n][h], acc);
      if (16 * T + 15 <= lo) {                       // visible to every query of the tile
#pragma unroll
        for (int i = 0; i < 4; ++i) rmax[n][i] = fmax_nan(rmax[n][i], acc[i]);
      } else {
        const int lim = lim0 + 16 * n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = (T * 16 + grp * 4 + i > lim) ? -INFINITY : acc[i];
          rmax[n][i] = fmax_nan(rmax[n][i], v);
        }
      }
    }
  }
}

// The same two page maxima over an MXFP4 page slot (scaled matrix-core op).
template <int H, int NQT>
__device__ __forceinline__ void page_max_f4(const uint8_t* __restrict__ pg, const v8i (&qf)[NQT][H],
                                            int col, int grp, int off, v4f (&rmax)[NQT]) {
#pragma unroll
  for (int n = 0; n < NQT; ++n) rmax[n] = v4f{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  v8i a_cur = f4_frag(pg, 0, col, off);
  int s_cur = f4_scale(pg, 0, col, grp);
  v4f prev;
#pragma unroll
  for (int T = 0; T < 8; ++T) {
    v8i a_nxt;
    int s_nxt = 0;
    if (T < 7) {
      a_nxt = f4_frag(pg, T + 1, col, off);
      s_nxt = f4_scale(pg, T + 1, col, grp);
    }
#pragma unroll
    for (int n = 0; n < NQT; ++n) {
      v4f acc = mfma_f4_e4m3(a_cur, qf[n][0], v4f{0.f, 0.f, 0.f, 0.f}, s_cur);
#pragma unroll
      for (int h = 1; h < H; ++h) acc = mfma_f4_e4m3(a_cur, qf[n][h], acc, s_cur);
      if (T > 0 || n > 0) {
        const int pn = n > 0 ? n - 1 : NQT - 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) rmax[pn][i] = fmax_nan(rmax[pn][i], prev[i]);
      }
      prev = acc;
    }
    if (T < 7) {
      a_cur = a_nxt;
      s_cur = s_nxt;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) rmax[NQT - 1][i] = fmax_nan(rmax[NQT - 1][i], prev[i]);
}

template <int H, int NQT>
__device__ __forceinline__ void page_max_causal_f4(const uint8_t* __restrict__ pg,
                                                   const v8i (&qf)[NQT][H], int lim0, int L0,
                                                   int col, int grp, int off, v4f (&rmax)[NQT]) {
#pragma unroll
  for (int n = 0; n < NQT; ++n) rmax[n] = v4f{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int T = 0; T < 8; ++T) {
    if (16 * T > L0 + NQT * 16 - 1) break;
    const v8i a_cur = f4_frag(pg, T, col, off);
    const int s_cur = f4_scale(pg, T, col, grp);
#pragma unroll
    for (int n = 0; n < NQT; ++n) {
      const int lo = L0 + 16 * n;
      if (16 * T > lo + 15) continue;
      v4f acc = mfma_f4_e4m3(a_cur, qf[n][0], v4f{0.f, 0.f, 0.f, 0.f}, s_cur);
#pragma unroll
      for (int h = 1; h < H; ++h) acc = mfma_f4_e4m3(a_cur, qf[n][h], acc, s_cur);
      if (16 * T + 15 <= lo) {
#pragma unroll
        for (int i = 0; i < 4; ++i) rmax[n][i] = fmax_nan(rmax[n][i], acc[i]);
      } else {
        const int lim = lim0 + 16 * n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = (T * 16 + grp * 4 + i > lim) ? -INFINITY : acc[i];
          rmax[n][i] = fmax_nan(rmax[n][i], v);
        }
      }
    }
  }
}

// LDS per block: a ring of four index-K pages (two being scored, two being
// filled), one private partial-max tile per wave ([queries of the wave][8 pages
// x 2 partials], rows padded to kSRowG floats), and the item's physical page ids.
template <int H, int KF>
constexpr size_t score_lds_bytes() {
  return 4 * (KF ? kF4Slot : kLdsPage) +
         (size_t)kScoreWaves * score_qtiles(H) * 16 * kSRowG * sizeof(float) +
         kMaxItemPages * sizeof(int);
}

// One work item of the prefill scorer.  On return no copy into LDS is in
// flight and every wave is past the item's last use of LDS.
// KF: index-K format, 0 = E4M3 rows of 128 bytes, 1 = MXFP4.
template <int H, int KF>
__device__ __forceinline__ void score_item(const ScoreK& a, int4 it, int pc, uint8_t* lds) {
  constexpr int NQT = score_qtiles(H);   // 16-query tiles per wave
  static_assert(NQT >= 1, "at least one query tile per wave");
  constexpr int kSlot = KF ? kF4Slot : kLdsPage;

  const int b = it.x, q_first = it.y, q_count = it.z, p0 = it.w;

  // The lane values below are recomputed per item (the empty asm hides that the
  // thread index is loop-invariant), not kept live across the item loop.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  float* sbuf = reinterpret_cast<float*>(lds + 4 * kSlot) + wave * (NQT * 16 * kSRowG);
  int* s_phys = reinterpret_cast<int*>(lds + 4 * kSlot + kScoreWaves * NQT * 16 * kSRowG * 4);

  const int cq0 = a.cu_q[b];
  const int sq = a.cu_q[b + 1] - cq0;
  const int sk = a.cu_k[b + 1] - a.cu_k[b];
  const int ctx = sk - sq;
  const int pos_first = ctx + (q_first - cq0);
  const int pos_last = pos_first + q_count - 1;
  const int v_block = pos_last / kPage + 1;
  const int p_end = min(min(p0 + pc, v_block), a.max_pages);
  if (p0 >= p_end) return;
  const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;

  // Physical page ids of the item, read once into LDS so that address
  // computation in the page loop never waits on a vector-memory load.
  for (int k = tid; k < p_end - p0; k += kThreads) {
    const int phys = bt[p0 + k];
    s_phys[k] = (phys < 0 || phys >= a.num_pages) ? 0 : phys;
  }
  __syncthreads();

  // Index-K pages (16 KiB) are copied global -> LDS directly (global_load_lds,
  // 16 bytes per lane, one instruction per wave and page: wave w fills rows
  // 8w..8w+7), into a ring of four slots: page p lives in slot p & 3.  While a
  // pair is scored, the next pair is in flight; after the barrier that ends a
  // pair, the pair after next is requested into the slots just freed.  Every
  // slot is requested even past the item's end (page index clamped) so the
  // count of loads in flight is the same on every path.
  static_assert(kThreads == kPage * kDim / 16, "one 16-byte piece per thread and page");
  // MXFP4 pages: waves 0..7 copy the 8 KiB of E2M1 pairs (rows 16w .. 16w + 15),
  // lanes 0..31 of wave 8 the 512 scale bytes; the other waves copy nothing.
  const int ld_row = KF ? wave * 16 + (lane >> 2) : wave * 8 + (lane >> 3);
  const int ld_piece = KF ? (lane & 3) ^ ((ld_row >> 2) & 3) : (lane & 7) ^ ((ld_row >> 1) & 7);
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds + wave * 1024);
  auto issue_page = [&](int p) {
    const int phys = s_phys[min(p, p_end - 1) - p0];
    if constexpr (KF == 0) {
      const uint8_t* src = a.k_cache + (int64_t)phys * (kPage * kDim) + ld_row * kDim + ld_piece * 16;
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(lds + (p & 3) * kLdsPage + wave * 1024),
          16, 0, 0);
    } else {
      if (wave < 8) {
        copy16_to_lds(a.k_cache + (int64_t)phys * kF4Data + ld_row * 64 + ld_piece * 16,
                      lds_wave + (uint32_t)((p & 3) * kSlot));
      } else if (wave == 8 && lane < 32) {
        copy16_to_lds(a.k_scales + (int64_t)phys * (kPage * 4) + lane * 16,
                      lds_wave + (uint32_t)((p & 3) * kSlot + kF4Data - 8 * 1024));
      }
    }
  };
  issue_page(p0);
  issue_page(p0 + 1);
  issue_page(p0 + 2);
  issue_page(p0 + 3);

  // Query fragments (B operand): column = query, K-group = 32-byte slice of D.
  // Loaded after the first index-K pages are requested so the latencies overlap.
  v8i qf[NQT][H];
  const int q_end = q_first + q_count;
  const int wave_q0 = q_first + wave * NQT * 16;
  const bool wave_active = wave_q0 < q_end;
  const int my_q0 = wave_q0 + col;              // query of this lane in tile n: my_q0 + 16n
  const int my_pos0 = ctx + (my_q0 - cq0);      // its position: my_pos0 + 16n
  const int wave_pos0 = ctx + (wave_q0 - cq0);  // position of the wave's first query
#pragma unroll
  for (int n = 0; n < NQT; ++n) {
    const int qi = my_q0 + n * 16;
    const bool ok = qi < q_end;
#pragma unroll
    for (int h = 0; h < H; ++h) {
      if (ok) {
        const uint8_t* qrow = a.q + (int64_t)qi * a.q_stride + h * kDim;
        if constexpr (KF == 0)
          qf[n][h] = load_frag_global(qrow + grp * 32);
        else
          qf[n][h] = load_qfrag_f4(qrow, grp);
      } else {
        qf[n][h] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }
  const float scale = (*a.q_scale) * (*a.k_scale);
  const Swz swz = lane_swizzle(col, grp);
  const int f4off = f4_piece(col, grp);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's page pieces have landed
  __syncthreads();

  // Flush the wave's tile for pages [pg_lo, pg_hi) of the 8-page group that
  // starts at pg0 (a multiple of 8): a lane takes a (query, 4-page) half group,
  // maxes the two half-wave partials of each page, scales and stores the four
  // scores as one 16-byte store when all four are to be written (two lanes
  // cover the 32 contiguous bytes of a query's group).
  auto flush = [&](int pg0, int pg_lo, int pg_hi) {
    constexpr int kTasks = NQT * 16 * 2;
    for (int t = lane; t < kTasks; t += 64) {
      const int ql = t >> 1, h = t & 1;
      const int qi = wave_q0 + ql;
      const int pp = pg0 + 4 * h;
      const v4f g0 = *reinterpret_cast<const v4f*>(sbuf + ql * kSRowG + 8 * h);
      const v4f g1 = *reinterpret_cast<const v4f*>(sbuf + ql * kSRowG + 8 * h + 4);
      const v4f m = v4f{fmax_nan(g0[0], g0[1]), fmax_nan(g0[2], g0[3]), fmax_nan(g1[0], g1[1]),
                        fmax_nan(g1[2], g1[3])} * scale;
      if (qi < q_end) {
        const int pos = ctx + (qi - cq0);
        const int hi = min(pg_hi, pos / kPage + 1);        // pages [pg_lo, hi) are written
        float* dst = a.scores + (int64_t)qi * a.ld + pp;
        if (pp >= pg_lo && pp + 4 <= hi) {
          *reinterpret_cast<v4f*>(dst) = m;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (pp + j >= pg_lo && pp + j < hi) dst[j] = m[j];
        }
      }
    }
  };

  auto score_page = [&](int p) {
    const uint8_t* pg = lds + (p & 3) * kSlot;
    v4f rmax[NQT];
    if constexpr (KF == 0) {
      if ((p + 1) * kPage - 1 > pos_first)
        page_max_causal<H, NQT>(pg, qf, my_pos0 - p * kPage, wave_pos0 - p * kPage, col, grp, swz,
                                rmax);
      else
        page_max<H, NQT>(pg, qf, col, swz, rmax);
    } else {
      if ((p + 1) * kPage - 1 > pos_first)
        page_max_causal_f4<H, NQT>(pg, qf, my_pos0 - p * kPage, wave_pos0 - p * kPage, col, grp,
                                   f4off, rmax);
      else
        page_max_f4<H, NQT>(pg, qf, col, grp, f4off, rmax);
    }
    const int pc = p & 7;                      // slot in the 8-page group
#pragma unroll
    for (int n = 0; n < NQT; ++n) {
      float m = fmax_nan(fmax_nan(rmax[n][0], rmax[n][1]), fmax_nan(rmax[n][2], rmax[n][3]));
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
      m = fmax_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));   // lane groups g and g ^ 2
      if (grp < 2) sbuf[(n * 16 + col) * kSRowG + pc * 2 + grp] = m;
    }
    if (pc == 7 || p == p_end - 1) flush(p - pc, max(p0, p - pc), p + 1);
  };

  // One step: score pages p, p + 1; wait for this wave's pieces of p + 2, p + 3;
  // barrier (pages p + 2, p + 3 complete, slots of p, p + 1 free); request
  // p + 4, p + 5 into those slots.
  for (int p = p0; p < p_end; p += 2) {
    if (wave_active) {
      score_page(p);
      if (p + 1 < p_end) score_page(p + 1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (p + 2 < p_end) {
      issue_page(p + 4);
      issue_page(p + 5);
    }
  }
}

// Persistent blocks (one per compute unit): block i takes items i, i + grid,
// i + 2 grid, ... of the plan's list, so a grid sized for the host's upper bound
// on the item count costs no dispatch rounds of empty blocks.  (Items of one
// plan are about the same size; a shared counter handing out items dynamically
// measured slower, its atomics serialising on one address.)
template <int H, int KF, bool kDecode>
__device__ __forceinline__ void take_items(const ScoreK& a, uint8_t* lds);

template <int H, int KF>
__global__ __launch_bounds__(kThreads) void index_score_kernel(ScoreK a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  take_items<H, KF, false>(a, lds);
}

// ---------------------------------------------------------------------------
// Decode-like batches: every request has at most 64/H queries, so every item
// does and one wave's query tiles hold them all.  The 16 waves then split each
// pair of pages (wave w: page p + w / 8, tokens 16 (w % 8) .. 16 (w % 8) + 15),
// each with all the query tiles, and write per-query partial maxima to LDS;
// wave 0 reduces a pair's 8 + 8 partials one step later (the partials are
// double-buffered across the barrier) and keeps the score tile.
// ---------------------------------------------------------------------------


// LDS: the page ring, wave 0's score tile, the physical page ids and two
// buffers of partial maxima [wave][query].
// MXFP4 pages are half the bytes, so their ring is twice as deep (8 slots) to
// keep as many bytes in flight.
template <int KF>
constexpr int pp_ring() { return KF ? 8 : 4; }

// kSel: the fused selection keeps the item's scores in LDS ([queries, pages])
template <int H, int KF, bool kSel = false>
constexpr size_t score_pp_lds_bytes() {
  return pp_ring<KF>() * (KF ? kF4Slot : kLdsPage) + (size_t)score_qtiles(H) * 16 * kSRow * sizeof(float) +
         kMaxItemPages * sizeof(int) + 2 * kScoreWaves * score_qtiles(H) * 16 * sizeof(float) +
         (kSel ? (size_t)score_qtiles(H) * 16 * kMaxItemPages * sizeof(float) : 0);
}

// Candidate key of (score, page): higher score first, then lower page; 0 is
// "no candidate" (a real key has ~page != 0 in its low half).
__device__ __forceinline__ uint64_t cand_key(float score, int page) {
  return ((uint64_t)float_key(score) << 32) | (uint32_t)(~(uint32_t)page);
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
template <int kCtrl>
__device__ __forceinline__ uint64_t dpp64(uint64_t x) {   // both halves through one DPP pattern
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, kCtrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), kCtrl, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
// Maximum over the wave: within each 16-lane row by DPP (quad_perm xor 1 and
// xor 2, half-row mirror, row mirror), then across the rows with the gfx950
// lane-swap instructions (as in max_across_groups).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  x = umax64(x, dpp64<0xB1>(x));
  x = umax64(x, dpp64<0x4E>(x));
  x = umax64(x, dpp64<0x141>(x));
  x = umax64(x, dpp64<0x140>(x));
  auto l = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  auto h = __builtin_amdgcn_permlane32_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
  x = umax64(((uint64_t)h[0] << 32) | l[0], ((uint64_t)h[1] << 32) | l[1]);
  l = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  h = __builtin_amdgcn_permlane16_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
  return umax64(((uint64_t)h[0] << 32) | l[0], ((uint64_t)h[1] << 32) | l[1]);
}

// Fused selection, end of a decode item: for each of the item's queries, the
// item's 16 best candidate pages (pages below the query's forced recent ones),
// by key, into cand[item, query, 0..15] (0 past the last).  Wave w takes queries
// w, w + 16, ...; lane l holds pages p0 + l + 64 r.  The 16 picks are 16 rounds
// of a wave-wide maximum whose holder drops it.
template <int H>
__device__ __forceinline__ void select_item_candidates(const ScoreK& a, int item, int q_first,
                                                       int q_count, int p0, int p_end, int ctx,
                                                       int cq0, const float* s_isc) {
  constexpr int kQ = score_qtiles(H) * 16;
  constexpr int kPer = kMaxItemPages / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int ql = wave; ql < q_count; ql += kScoreWaves) {
    const int pos = ctx + (q_first + ql - cq0);
    const int v = min(pos / kPage + 1, a.max_pages);
    const int f = min(a.n_local, min(kTopK, v));
    const int c_end = min(p_end, v - f);            // candidate pages of this item: [p0, c_end)
    uint64_t key[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int j = lane + 64 * r;
      key[r] = p0 + j < c_end ? cand_key(s_isc[ql * kMaxItemPages + j], p0 + j) : 0ull;
    }
    uint64_t mine = 0;                              // lane k keeps the k-th pick
#pragma unroll 1
    for (int k = 0; k < kTopK; ++k) {
      uint64_t m = key[0];
#pragma unroll
      for (int r = 1; r < kPer; ++r) m = key[r] > m ? key[r] : m;
      const uint64_t w = wave_max_u64(m);
      if (w == 0) break;                            // wave-uniform: no candidate left
#pragma unroll
      for (int r = 0; r < kPer; ++r) key[r] = key[r] == w ? 0ull : key[r];
      mine = lane == k ? w : mine;
    }
    if (lane < kTopK) a.cand[((int64_t)item * kQ + ql) * kTopK + lane] = mine;
  }
}

// One work item of the decode scorer (same contract as score_item).  kSel: the
// fused selection, which keeps the item's scores in LDS instead of writing them
// and leaves per-item candidate lists.
template <int H, int KF, bool kSel = false>
__device__ __forceinline__ void score_pp_item(const ScoreK& a, int item, int4 it, int pc, uint8_t* lds) {
  constexpr int NQT = score_qtiles(H);
  constexpr int kQ = NQT * 16;                    // query slots
  constexpr int kSlot = KF ? kF4Slot : kLdsPage;
  constexpr int kRingN = pp_ring<KF>();
  constexpr int kReducer = 0;        // the wave that reduces the partials and stores the scores

  const int b = it.x, q_first = it.y, q_count = it.z, p0 = it.w;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  float* sbuf = reinterpret_cast<float*>(lds + kRingN * kSlot);
  int* s_phys = reinterpret_cast<int*>(lds + kRingN * kSlot + kQ * kSRow * 4);
  float* s_part = reinterpret_cast<float*>(s_phys + kMaxItemPages);
  float* s_isc = s_part + 2 * kScoreWaves * kQ;   // kSel: [kQ, kMaxItemPages] item scores

  const int cq0 = a.cu_q[b];
  const int sq = a.cu_q[b + 1] - cq0;
  const int sk = a.cu_k[b + 1] - a.cu_k[b];
  const int ctx = sk - sq;
  const int pos_first = ctx + (q_first - cq0);
  const int pos_last = pos_first + q_count - 1;
  const int v_block = pos_last / kPage + 1;
  const int p_end = min(min(p0 + pc, v_block), a.max_pages);
  if (p0 >= p_end) {
    if constexpr (kSel) {                         // an empty item still leaves (empty) lists
      for (int e = tid; e < q_count * kTopK; e += kThreads)
        a.cand[(int64_t)item * kQ * kTopK + e] = 0ull;
      if (p0 == 0 && tid < q_count) a.first_item[q_first + tid] = make_int2(item, ctx + (q_first + tid - cq0));
    }
    return;
  }
  const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;
  for (int k = tid; k < p_end - p0; k += kThreads) {
    const int phys = bt[p0 + k];
    s_phys[k] = (phys < 0 || phys >= a.num_pages) ? 0 : phys;
  }
  __syncthreads();

  // page ring: as in the prefill kernel, four slots, page p in slot p & 3
  const int ld_row = KF ? wave * 16 + (lane >> 2) : wave * 8 + (lane >> 3);
  const int ld_piece = KF ? (lane & 3) ^ ((ld_row >> 2) & 3) : (lane & 7) ^ ((ld_row >> 1) & 7);
  const uint32_t lds_wave =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds + wave * 1024;
  auto issue_page = [&](int p) {
    const int phys = s_phys[min(p, p_end - 1) - p0];
    if constexpr (KF == 0) {
      const uint8_t* src = a.k_cache + (int64_t)phys * (kPage * kDim) + ld_row * kDim + ld_piece * 16;
      copy16_to_lds(src, lds_wave + (uint32_t)((p & 3) * kLdsPage));
    } else {
      if (wave < 8) {
        copy16_to_lds(a.k_cache + (int64_t)phys * kF4Data + ld_row * 64 + ld_piece * 16,
                      lds_wave + (uint32_t)((p & (kRingN - 1)) * kSlot));
      } else if (wave == 8 && lane < 32) {
        copy16_to_lds(a.k_scales + (int64_t)phys * (kPage * 4) + lane * 16,
                      lds_wave + (uint32_t)((p & (kRingN - 1)) * kSlot + kF4Data - 8 * 1024));
      }
    }
  };
  issue_page(p0);
  issue_page(p0 + 1);
  issue_page(p0 + 2);
  issue_page(p0 + 3);

  // every wave: the fragments of all the item's queries (tiles past them skipped)
  v8i qf[NQT][H];
  const int q_end = q_first + q_count;
  const int nt = (q_count + 15) / 16;
  const int my_q0 = q_first + col;
  const int my_pos0 = ctx + (my_q0 - cq0);
#pragma unroll
  for (int n = 0; n < NQT; ++n) {
    const int qi = my_q0 + n * 16;
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const uint8_t* qrow = a.q + (int64_t)qi * a.q_stride + h * kDim;
      if constexpr (KF == 0)
        qf[n][h] = qi < q_end ? load_frag_global(qrow + grp * 32) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
      else
        qf[n][h] = qi < q_end ? load_qfrag_f4(qrow, grp) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  const float scale = (*a.q_scale) * (*a.k_scale);
  const Swz swz = lane_swizzle(col, grp);
  const int f4off = f4_piece(col, grp);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // a deeper ring fills up once the first four pages are in (the first step
  // waits only for pages it has already waited for)
#pragma unroll
  for (int k = 4; k < kRingN; ++k) issue_page(p0 + k);

  // partial maxima of page pw, tokens 16T .. 16T + 15, into dst[query]
  auto partial = [&](int pw, int T, float* dst) {
    const uint8_t* pg = lds + (pw & (kRingN - 1)) * kSlot;
    const v8i a_t = KF ? f4_frag(pg, T, col, f4off) : load_frag_swz(pg + (T * 16 + col) * kDim, swz);
    const int sa = KF ? f4_scale(pg, T, col, grp) : 0;
    const bool causal = (pw + 1) * kPage - 1 > pos_first;
    const int tok0 = pw * kPage + T * 16 + grp * 4;        // token of acc[0] in this lane
#pragma unroll
    for (int n = 0; n < NQT; ++n) {
      if (n >= nt) break;
      v4f acc = KF ? mfma_f4_e4m3(a_t, qf[n][0], v4f{0.f, 0.f, 0.f, 0.f}, sa)
                   : mfma_e4m3(a_t, qf[n][0], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int h = 1; h < H; ++h) acc = KF ? mfma_f4_e4m3(a_t, qf[n][h], acc, sa) : mfma_e4m3(a_t, qf[n][h], acc);
      float m;
      if (causal) {
        const int lim = my_pos0 + 16 * n;
        m = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmax_nan(m, tok0 + i > lim ? -INFINITY : acc[i]);
      } else {
        m = fmax_nan(fmax_nan(acc[0], acc[1]), fmax_nan(acc[2], acc[3]));
      }
      m = max_across_groups(m);
      if ((n & 3) == grp) dst[n * 16 + col] = m;
    }
  };
  // the reducer wave: score tile flush for pages [pg0, pg_hi), as in the prefill kernel
  auto flush = [&](int pg0, int pg_hi) {
#pragma unroll
    for (int r = 0; r < NQT; ++r) {
      const int ql = r * 16 + (lane >> 2);
      const int c = (lane & 3) * 4;
      const int qi = q_first + ql;
      const int pos = ctx + (qi - cq0);
      const int pp = pg0 + c;
      const float* src = sbuf + ql * kSRow + c;
      const float v0 = src[0], v1 = src[1], v2 = src[2], v3 = src[3];
      if constexpr (kSel) {                      // the item's score row in LDS (pages past
        if (qi < q_end)                          // the visible ones are never read)
          *reinterpret_cast<v4f*>(s_isc + ql * kMaxItemPages + (pp - p0)) = v4f{v0, v1, v2, v3};
        continue;
      }
      if (qi < q_end) {
        float* dst = a.scores + (int64_t)qi * a.ld + pp;
        const int vis_end = min(pg_hi, pos / kPage + 1);
        if (pp + 3 < vis_end) {
          *reinterpret_cast<v4f*>(dst) = v4f{v0, v1, v2, v3};
        } else {
          if (pp + 0 < vis_end) dst[0] = v0;
          if (pp + 1 < vis_end) dst[1] = v1;
          if (pp + 2 < vis_end) dst[2] = v2;
        }
      }
    }
  };
  // the reducer wave: page pr's score from its 8 partials (waves 8j .. 8j + 7 of src)
  auto reduce = [&](int pr, int j, const float* src) {
    const int pc = (pr - p0) & (kFlush - 1);
    if (lane < kQ) {
      float m = -INFINITY;
#pragma unroll
      for (int T = 0; T < 8; ++T) m = fmax_nan(m, src[(j * 8 + T) * kQ + lane]);
      sbuf[lane * kSRow + pc] = m * scale;
    }
    if (pc == kFlush - 1 || pr == p_end - 1) flush(pr - pc, pr + 1);
  };

  // One step: partials of pages p, p + 1 (the reducer also reduces the
  // previous pair); wait for this wave's pieces of p + 2, p + 3 (copies retire
  // in issue order and the kRingN - 4 pages after them were issued later);
  // barrier; request p + kRingN, p + kRingN + 1 into the slots of p, p + 1.
  constexpr int kPartBuf = kScoreWaves * kQ;
  int buf = 0;
  for (int p = p0; p < p_end; p += 2) {
    const int pw = p + (wave >> 3);
    if (pw < p_end) partial(pw, wave & 7, s_part + buf * kPartBuf + wave * kQ);
    if (wave == kReducer && p > p0) {
      reduce(p - 2, 0, s_part + (buf ^ 1) * kPartBuf);
      reduce(p - 1, 1, s_part + (buf ^ 1) * kPartBuf);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kRingN - 4) : "memory");
    __syncthreads();
    if (p + 2 < p_end) {
      issue_page(p + kRingN);
      issue_page(p + kRingN + 1);
    }
    buf ^= 1;
  }
  if (wave == kReducer) {             // the last pair
    const int pl = p0 + (p_end - 1 - p0) / 2 * 2;
    reduce(pl, 0, s_part + (buf ^ 1) * kPartBuf);
    if (pl + 1 < p_end) reduce(pl + 1, 1, s_part + (buf ^ 1) * kPartBuf);
  }
  // copies requested past the item's end (clamped pages) land before the next
  // item reuses the ring, and the reducer's LDS reads finish before its writes
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if constexpr (kSel) {
    select_item_candidates<H>(a, item, q_first, q_count, p0, p_end, ctx, cq0, s_isc);
    if (p0 == 0 && tid < q_count)                 // the query's items start here
      a.first_item[q_first + tid] = make_int2(item, ctx + (q_first + tid - cq0));
    __syncthreads();                              // s_isc is rewritten by the next item
  }
}

template <int H, int KF>
__global__ __launch_bounds__(kThreads) void index_score_pp_kernel(ScoreK a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  take_items<H, KF, true>(a, lds);
}

// The decode scorer with the fused selection (E4M3 keys).
template <int H>
__global__ __launch_bounds__(kThreads) void index_score_sel_kernel(ScoreK a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int n_items = a.hdr->n_items;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x)
    score_pp_item<H, 0, true>(a, item, a.items[item], a.hdr->pages_per_item, lds);
}

// Merge of the per-item candidate lists, one wave per query: the forced recent
// pages first (local page first), then the 16 - forced best candidates over the
// items of the query's request (consecutive in the plan from the one the scorer
// recorded with the query's position, each holding all of the request's
// queries), -1 padding.
constexpr int kMergePer = 16;                // merge candidates per lane per group

struct MergeK {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch;
  int32_t total_q;
  int32_t max_pages;
  int32_t n_local;
  int32_t kq;                       // queries per item list
  const ItemHdr* hdr;
  const int4* items;
  const uint64_t* cand;
  const int2* first_item;
  int32_t* out;
  int64_t out_stride;
};

__global__ __launch_bounds__(256) void topk_merge_kernel(MergeK a) {
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= a.total_q) return;                    // wave-uniform
  const int2 fp = a.first_item[i];               // written by the scorer for every query
  const int lo = fp.x, pos = fp.y;
  const int n_items = a.hdr->n_items;
  const int v = min(pos / kPage + 1, a.max_pages);
  const int k_all = min(kTopK, v);
  const int f = min(a.n_local, k_all);
  const int ksel = k_all - f;
  const int b = a.items[lo].x;
  // the request's item count: consecutive items of request b from lo
  int n_ch = 0;
  for (;;) {
    const int it = lo + n_ch + lane;
    const uint64_t same = __builtin_amdgcn_ballot_w64(it < n_items && a.items[it].x == b);
    const int run = same == ~0ull ? 64 : __builtin_ctzll(~same);
    n_ch += run;
    if (run < 64) break;                          // wave-uniform
  }
  // candidates in groups of kMergePer per lane (kMergePer * 4 items), each
  // group merged with the 16 kept so far by 16 rounds of a wave-wide maximum
  uint64_t keep = 0;                              // lane k < 16: the k-th best so far
  for (int g0 = 0; ksel > 0 && g0 < n_ch * kTopK; g0 += kMergePer * 64) {
    uint64_t c[kMergePer];
#pragma unroll
    for (int r = 0; r < kMergePer; ++r) {
      const int j = g0 + r * 64 + lane;           // candidate j: item lo + j / 16, slot j % 16
      const int it = lo + j / kTopK;
      c[r] = j < n_ch * kTopK
                 ? a.cand[((int64_t)it * a.kq + (i - a.items[it].y)) * kTopK + (j & (kTopK - 1))]
                 : 0ull;
    }
    uint64_t nk = 0;
#pragma unroll 1
    for (int k = 0; k < kTopK; ++k) {
      uint64_t m = keep;
#pragma unroll
      for (int r = 0; r < kMergePer; ++r) m = umax64(m, c[r]);
      const uint64_t w = wave_max_u64(m);
      if (w == 0) break;                          // wave-uniform
#pragma unroll
      for (int r = 0; r < kMergePer; ++r) c[r] = c[r] == w ? 0ull : c[r];
      keep = keep == w ? 0ull : keep;
      nk = lane == k ? w : nk;
    }
    keep = nk;
  }
  const uint64_t pick = (uint64_t)(uint32_t)__shfl((int)(uint32_t)keep, max(lane - f, 0));
  if (lane < kTopK) {
    int page = -1;
    if (lane < f) page = v - 1 - lane;
    else if (lane < k_all) page = (int)~(uint32_t)pick;
    a.out[i * a.out_stride + lane] = page;
  }
}

template <int H, int KF, bool kDecode>
__device__ __forceinline__ void take_items(const ScoreK& a, uint8_t* lds) {
  auto run = [&](int item, int4 it, int pc) {
    if constexpr (kDecode)
      score_pp_item<H, KF>(a, item, it, pc, lds);
    else
      score_item<H, KF>(a, it, pc, lds);
  };
  if (a.direct_items > 0) {
    // Lane l holds the inclusive prefix of the chunk counts of q-blocks l and
    // 64 + l (the host allows at most kDirectMaxQBlocks), so an item's q-block
    // is the number of q-blocks whose items all come before it.
    constexpr int kQB = score_qblock(H);
    const int pc = a.direct_pc, sq = a.direct_sq, ctx = a.direct_ctx;
    const int nqb = (sq + kQB - 1) / kQB;
    const int lane = threadIdx.x & 63;
    auto chunks = [&](int qb) {
      const int qf = qb * kQB;
      return qb < nqb ? (qblock_visible(ctx, qf, plan_min(sq - qf, kQB)) + pc - 1) / pc : 0;
    };
    const int pre0 = wave_inclusive_scan(chunks(lane));
    const int pre1 = wave_inclusive_scan(chunks(64 + lane)) + __builtin_amdgcn_readlane(pre0, 63);
    const int q0 = a.cu_q[0];
    for (int item = blockIdx.x; item < a.direct_items; item += gridDim.x) {
      const int g = (int)__popcll(__ballot(pre0 <= item)) + (int)__popcll(__ballot(pre1 <= item));
      const int base = g == 0 ? 0
                       : g <= 64 ? __builtin_amdgcn_readlane(pre0, g - 1)
                                 : __builtin_amdgcn_readlane(pre1, g - 65);
      const int qf = g * kQB;
      run(item, make_int4(0, q0 + qf, plan_min(sq - qf, kQB), (item - base) * pc), pc);
    }
    return;
  }
  if (a.wave_plan) {
    // Several requests, planned by every wave from cu_seqlens: the plan
    // kernel's sizing and item order, in registers.  Lane b holds request b,
    // lane l q-blocks l and 64 + l.
    constexpr int kQB = score_qblock(H);
    const int lane = threadIdx.x & 63;
    const int B = a.batch;
    const int rb = lane < B ? lane : B - 1;
    const int q0r = a.cu_q[rb];
    const int sqr = lane < B ? a.cu_q[rb + 1] - q0r : 0;
    const int ctxr = (a.cu_k[rb + 1] - a.cu_k[rb]) - sqr;
    const int nqbr = (sqr + kQB - 1) / kQB;                  // q-blocks of request `lane`
    const int preq = wave_inclusive_scan(nqbr);
    const int nqb = __builtin_amdgcn_readlane(preq, 63);
    struct QB { int b, qf, qn, v; };
    auto qblock = [&](int g) {
      int cnt = 0;                                           // requests ending at or before g
      for (int k = 0; k < B; ++k) cnt += __builtin_amdgcn_readlane(preq, k) <= g ? 1 : 0;
      QB r;
      r.b = cnt < B ? cnt : B - 1;
      r.qf = (g - (__shfl(preq, r.b) - __shfl(nqbr, r.b))) * kQB;
      r.qn = plan_min(__shfl(sqr, r.b) - r.qf, kQB);
      // every lane takes part in the shuffle (a lane reading from an inactive
      // one would get 0), so it is not inside the condition
      const int ctx = __shfl(ctxr, r.b);
      r.v = g < nqb ? qblock_visible(ctx, r.qf, r.qn) : 0;
      return r;
    };
    const QB g0 = qblock(lane), g1 = qblock(64 + lane);
    const int64_t w = wave_sum64((int64_t)g0.v + g1.v);
    const int vmin = wave_min(plan_min(lane < nqb ? g0.v : INT32_MAX, 64 + lane < nqb ? g1.v : INT32_MAX));
    const int vmax = wave_max(plan_max(g0.v, g1.v));
    int pc = cand_pages(w, 1, 4);
    if (!plan_uniform(vmin, vmax)) {
      int cand[kPlanCands], n[kPlanCands];
      plan_candidates(w, a.plan_align, cand);
#pragma unroll
      for (int k = 0; k < kPlanCands; ++k)
        n[k] = wave_sum((g0.v + cand[k] - 1) / cand[k] + (g1.v + cand[k] - 1) / cand[k]);
      pc = best_pages(cand, n);
    }
    pc = __builtin_amdgcn_readfirstlane(pc);     // equal in every lane; made known as such
    const int pre0 = wave_inclusive_scan((g0.v + pc - 1) / pc);
    const int pre1 = wave_inclusive_scan((g1.v + pc - 1) / pc) + __builtin_amdgcn_readlane(pre0, 63);
    const int n_items = __builtin_amdgcn_readlane(pre1, 63);
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
      const int g = (int)__popcll(__ballot(pre0 <= item)) + (int)__popcll(__ballot(pre1 <= item));
      const int base = g == 0 ? 0
                       : g <= 64 ? __builtin_amdgcn_readlane(pre0, g - 1)
                                 : __builtin_amdgcn_readlane(pre1, g - 65);
      const int gl = g & 63;
      const bool lo = g < 64;
      const int b = __builtin_amdgcn_readlane(lo ? g0.b : g1.b, gl);
      const int qf = __builtin_amdgcn_readlane(lo ? g0.qf : g1.qf, gl);
      const int qn = __builtin_amdgcn_readlane(lo ? g0.qn : g1.qn, gl);
      run(item, make_int4(b, __builtin_amdgcn_readlane(q0r, b) + qf, qn, (item - base) * pc), pc);
    }
    return;
  }
  const int n_items = a.hdr->n_items;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x)
    run(item, a.items[item], a.hdr->pages_per_item);
}

}  // namespace

template <int H, int KF>
hipError_t launch_scorer(dim3 grid, hipStream_t stream, const ScoreK& k, int max_seqlen_q) {
  if (max_seqlen_q <= score_qtiles(H) * 16) {   // every item fits one wave's query tiles
    constexpr size_t bytes = score_pp_lds_bytes<H, KF>();
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&index_score_pp_kernel<H, KF>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((index_score_pp_kernel<H, KF>), grid, dim3(kThreads), bytes, stream, k);
    return hipGetLastError();
  }
  constexpr size_t bytes = score_lds_bytes<H, KF>();
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&index_score_kernel<H, KF>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((index_score_kernel<H, KF>), grid, dim3(kThreads), bytes, stream, k);
  return hipGetLastError();
}

template <int KF>
hipError_t launch_scorer_h(dim3 grid, hipStream_t stream, const ScoreK& k, int H, int max_seqlen_q) {
  switch (H) {
    case 1: return launch_scorer<1, KF>(grid, stream, k, max_seqlen_q);
    case 2: return launch_scorer<2, KF>(grid, stream, k, max_seqlen_q);
    case 4: return launch_scorer<4, KF>(grid, stream, k, max_seqlen_q);
    default: return hipErrorInvalidValue;
  }
}

ScorePlan score_plan(const msa_varlen_t* vl, int H) {
  ScorePlan p;
  const int qb = score_qblock(H);
  const int64_t qb_bound = ceil_div(vl->total_q, qb) + vl->batch;   // q-blocks, at most
  const int64_t max_pages = std::max<int32_t>(1, vl->max_pages);
  // The device plan picks pages per item pc >= (sum of visible pages) /
  // (kPlanRounds * kPlanCUs), so sum over q-blocks of ceil(v / pc) <=
  // kPlanRounds * kPlanCUs + q-blocks, unless pc hits kMaxItemPages, where it is
  // at most q-blocks * (max_pages / kMaxItemPages + 1).
  p.pages_per_item = 0;   // chosen on the device
  p.max_items = std::max<int64_t>((int64_t)kPlanRounds * kPlanCUs,
                                  qb_bound * ceil_div(max_pages, kMaxItemPages)) +
                qb_bound;
  p.workspace_bytes = sizeof(ItemHdr) + align_up((size_t)p.max_items * sizeof(int4), 256);
  return p;
}

// The device plan (work list of a.H-head q-blocks) into the workspace, then the
// scorer over (q, scores); per-head scoring runs the single-head scorer once per
// head over the same plan.
namespace {
// A one-request batch planned on the host (no plan kernel, no work list).
struct DirectPlan {
  int32_t items = 0, pc = 0, sq = 0, ctx = 0;
  int32_t wave = 0, align = 1;     // planned by the scorer's waves, with this chunk alignment
};
}  // namespace

// The device plan's choice for a single request, made on the host from the
// descriptor's sizes: total_q is the request's query count; its token count is
// known to within one page (total_rows pages, at most max_seqlen_k tokens), so
// the plan takes the largest count that fits, which can only add items that
// find no visible page and end at once.  Items are the same (q-block, chunk)
// list the device plan writes, with q-blocks of up to kDirectMaxQBlocks.
static bool plan_one_request(const msa_varlen_t& vl, int H, DirectPlan* d) {
  if (vl.batch != 1 || vl.total_q <= 0) return false;
  const int qb = score_qblock(H);
  const int64_t sq = vl.total_q;
  const int64_t sk = std::min<int64_t>((int64_t)vl.total_rows * kPage, vl.max_seqlen_k);
  if (sk < sq || ceil_div(sq, qb) > kDirectMaxQBlocks) return false;
  const int ctx = (int)(sk - sq), nqb = (int)ceil_div(sq, qb);
  const int align = vl.max_seqlen_q <= score_qtiles(H) * 16 ? 4 : 1;
  auto vis = [&](int g) { return qblock_visible(ctx, g * qb, (int)std::min<int64_t>(sq - g * qb, qb)); };
  int64_t w = 0;
  int vmin = INT32_MAX, vmax = 0;
  for (int g = 0; g < nqb; ++g) {
    w += vis(g);
    vmin = std::min(vmin, vis(g));
    vmax = std::max(vmax, vis(g));
  }
  int pc = cand_pages(w, 1, 4);
  if (!plan_uniform(vmin, vmax)) {
    int cand[kPlanCands], n[kPlanCands] = {};
    plan_candidates(w, align, cand);
    for (int g = 0; g < nqb; ++g)
      for (int k = 0; k < kPlanCands; ++k) n[k] += (vis(g) + cand[k] - 1) / cand[k];
    pc = best_pages(cand, n);
  }
  int64_t items = 0;
  for (int g = 0; g < nqb; ++g) items += (vis(g) + pc - 1) / pc;
  d->items = (int32_t)items;
  d->pc = pc;
  d->sq = (int32_t)sq;
  d->ctx = ctx;
  return true;
}

// Batches of 2..kWavePlanMaxB requests and at most kDirectMaxQBlocks q-blocks
// are planned by the scorer's waves themselves (the q-block count is bounded
// by ceil(total_q / q-block) + batch).
static bool plan_in_waves(const msa_varlen_t& vl, int H, DirectPlan* d) {
  if (vl.batch < 2 || vl.batch > kWavePlanMaxB ||
      ceil_div(vl.total_q, score_qblock(H)) + vl.batch > kDirectMaxQBlocks)
    return false;
  d->wave = 1;
  d->align = vl.max_seqlen_q <= score_qtiles(H) * 16 ? 4 : 1;   // as the plan kernel's
  return true;
}

static hipError_t launch_plan(const ScoreArgs& a, hipStream_t stream);
static hipError_t launch_scorer_pass(const ScoreArgs& a, const uint8_t* q, float* scores,
                                     const DirectPlan& d, hipStream_t stream);

hipError_t launch_index_score(const ScoreArgs& a, hipStream_t stream) {
  if (a.vl.total_q == 0) return hipSuccess;
  DirectPlan d;
  if (!plan_one_request(a.vl, a.H, &d) && !plan_in_waves(a.vl, a.H, &d)) {
    hipError_t e = launch_plan(a, stream);
    if (e != hipSuccess) return e;
  }
  return launch_scorer_pass(a, a.q, a.scores, d, stream);
}

hipError_t launch_index_score_heads(const ScoreArgs& a, int64_t head_stride, hipStream_t stream) {
  if (a.vl.total_q == 0) return hipSuccess;
  ScoreArgs one = a;
  one.H = 1;                                  // every pass scores one index head
  DirectPlan d;
  if (!plan_one_request(one.vl, 1, &d) && !plan_in_waves(one.vl, 1, &d)) {
    hipError_t e = launch_plan(one, stream);
    if (e != hipSuccess) return e;
  }
  for (int h = 0; h < a.H; ++h) {
    hipError_t e = launch_scorer_pass(one, a.q + (int64_t)h * kDim,
                                      a.scores + (int64_t)h * head_stride, d, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int H>
static hipError_t launch_sel(dim3 grid, hipStream_t stream, const ScoreK& k) {
  constexpr size_t bytes = score_pp_lds_bytes<H, 0, true>();
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&index_score_sel_kernel<H>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((index_score_sel_kernel<H>), grid, dim3(kThreads), bytes, stream, k);
  return hipGetLastError();
}

hipError_t launch_index_score_topk(const ScoreArgs& a, int n_local, int32_t* out,
                                   int64_t out_stride, hipStream_t stream) {
  if (a.vl.total_q == 0) return hipSuccess;
  hipError_t e = launch_plan(a, stream);
  if (e != hipSuccess) return e;
  ItemHdr* hdr = reinterpret_cast<ItemHdr*>(a.workspace);
  int4* items = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(a.workspace) + sizeof(ItemHdr));
  uint64_t* cand = reinterpret_cast<uint64_t*>(reinterpret_cast<uint8_t*>(a.workspace) +
                                               a.plan.workspace_bytes);
  int2* first_item = reinterpret_cast<int2*>(
      reinterpret_cast<uint8_t*>(cand) + index_score_topk_extra_bytes(a.plan, a.H, a.vl.total_q) -
      align_up((size_t)std::max<int64_t>(a.vl.total_q, 1) * sizeof(int2), 256));
  ScoreK k{};
  k.cu_q = a.vl.cu_seqlens_q;
  k.cu_k = a.vl.cu_seqlens_k;
  k.block_table = a.vl.block_table;
  k.bt_stride = a.vl.block_table_stride;
  k.batch = a.vl.batch;
  k.num_pages = a.num_pages;
  k.max_pages = a.vl.max_pages;
  k.q = a.q;
  k.q_stride = a.q_stride;
  k.k_cache = a.k_cache;
  k.q_scale = a.q_scale;
  k.k_scale = a.k_scale;
  k.scores = nullptr;
  k.ld = 0;
  k.hdr = hdr;
  k.items = items;
  k.k_scales = nullptr;
  k.cand = cand;
  k.first_item = first_item;
  k.n_local = n_local;
  k.direct_items = 0;   // the merge reads the plan's list
  k.wave_plan = 0;
  dim3 grid((unsigned)std::min<int64_t>(a.plan.max_items, device_cu_count()));
  switch (a.H) {
    case 1: e = launch_sel<1>(grid, stream, k); break;
    case 2: e = launch_sel<2>(grid, stream, k); break;
    case 4: e = launch_sel<4>(grid, stream, k); break;
    default: e = hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  MergeK m{a.vl.cu_seqlens_q, a.vl.cu_seqlens_k, a.vl.batch, (int32_t)a.vl.total_q,
           a.vl.max_pages, n_local, score_qtiles(a.H) * 16, hdr, items, cand, first_item, out,
           out_stride};
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)ceil_div(a.vl.total_q, 4)), dim3(256), 0,
                     stream, m);
  return hipGetLastError();
}

// Candidate lists [max_items, queries, 16], then (first item, position) per query.
size_t index_score_topk_extra_bytes(const ScorePlan& p, int H, int64_t total_q) {
  return align_up((size_t)p.max_items * score_qtiles(H) * 16 * kTopK * sizeof(uint64_t), 256) +
         align_up((size_t)std::max<int64_t>(total_q, 1) * sizeof(int2), 256);
}

static hipError_t launch_plan(const ScoreArgs& a, hipStream_t stream) {
  ItemHdr* hdr = reinterpret_cast<ItemHdr*>(a.workspace);
  int4* items = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(a.workspace) + sizeof(ItemHdr));
  const int qb = score_qblock(a.H);
  // chunk alignment: 4 pages when the decode kernel runs (see cand_pages)
  const int align = a.vl.max_seqlen_q <= score_qtiles(a.H) * 16 ? 4 : 1;
  // one request: the 256-thread kernel has less to set up; batches: the table kernel
  if (a.vl.batch > 1 && a.vl.batch <= kPlanMaxB &&
      ceil_div(a.vl.total_q, qb) + a.vl.batch <= kPlanMaxG)
    hipLaunchKernelGGL(score_plan_table_kernel, dim3(1), dim3(kPlanThreads), 0, stream,
                       a.vl.cu_seqlens_q, a.vl.cu_seqlens_k, a.vl.batch, qb, align, a.plan.max_items,
                       hdr, items);
  else
    hipLaunchKernelGGL(score_plan_kernel, dim3(1), dim3(256), 0, stream, a.vl.cu_seqlens_q,
                       a.vl.cu_seqlens_k, a.vl.batch, qb, align, a.plan.max_items, hdr, items);
  return hipGetLastError();
}

static hipError_t launch_scorer_pass(const ScoreArgs& a, const uint8_t* q, float* scores,
                                     const DirectPlan& d, hipStream_t stream) {
  ItemHdr* hdr = reinterpret_cast<ItemHdr*>(a.workspace);
  int4* items = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(a.workspace) + sizeof(ItemHdr));
  ScoreK k;
  k.cu_q = a.vl.cu_seqlens_q;
  k.cu_k = a.vl.cu_seqlens_k;
  k.block_table = a.vl.block_table;
  k.bt_stride = a.vl.block_table_stride;
  k.batch = a.vl.batch;
  k.num_pages = a.num_pages;
  k.max_pages = a.vl.max_pages;
  k.q = q;
  k.q_stride = a.q_stride;
  k.k_cache = a.k_cache;
  k.q_scale = a.q_scale;
  k.k_scale = a.k_scale;
  k.scores = scores;
  k.ld = a.ld;
  k.hdr = hdr;
  k.items = items;
  k.k_scales = a.k_scales;
  k.cand = nullptr;
  k.first_item = nullptr;
  k.n_local = 0;
  k.direct_items = d.items;
  k.direct_pc = d.pc;
  k.direct_sq = d.sq;
  k.direct_ctx = d.ctx;
  k.wave_plan = d.wave;
  k.plan_align = d.align;
  // persistent blocks: one per compute unit (the kernels' LDS allows no more)
  const int64_t n_blocks = d.items > 0 ? d.items : a.plan.max_items;
  dim3 grid((unsigned)std::min<int64_t>(n_blocks, device_cu_count()));
  if (a.k_scales) return launch_scorer_h<1>(grid, stream, k, a.H, a.vl.max_seqlen_q);   // MXFP4 keys
  return launch_scorer_h<0>(grid, stream, k, a.H, a.vl.max_seqlen_q);
}

}  // namespace msa
