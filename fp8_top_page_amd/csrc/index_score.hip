// FP8 (E4M3) page indexer for gfx950.
//
// Computes, for every query token and every page it can see, the page score
// q_scale * k_scale * max over the page's visible tokens of sum_h q_h . k
// (vLLM PR 60930, Overview and Details: the FP8 indexer scores every 128-token
// page for each query; the work is planned on the device, with no host sync,
// and the scoring call neither allocates nor synchronises).
//
// Design (MI355X):
//  * Planning: one small kernel turns cu_seqlens_q/k into a list of uniform work
//    items (request, block of queries, chunk of pages), causal-trimmed, in the
//    workspace.  The scorer grid is sized from host-side upper bounds, and
//    blocks past the device-side item count exit.
//  * Scoring: tokens are the MFMA M axis, queries the N axis.  Each wave keeps
//    the E4M3 fragments of 128/H queries (all H heads) in registers for the
//    whole item; the index-K page (16 KiB) is staged once per block in LDS
//    (double-buffered, padded rows) and read by all 8 waves.  The H head
//    products chain into one accumulator (a contraction of length H*128).
//  * Epilogue: each lane holds 4 consecutive tokens of one query per 16-token
//    tile; the max over the page's 8 tiles is taken in registers, then across
//    the 4 lane groups.  Scores of 4 consecutive pages are gathered so each
//    store writes 16 contiguous bytes per query.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kLdsRow = 144;                 // 128 B + 16 B pad against bank conflicts
constexpr int kLdsPage = kPage * kLdsRow;    // 18 KiB
constexpr int kThreads = kScoreWaves * 64;

struct ItemHdr {
  int32_t n_items;
  int32_t pad[63];
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
  const int32_t* n_items;
  const int4* items;
  int32_t pages_per_item;
};

// ---------------------------------------------------------------------------
// Plan: one block.  Items are emitted request by request, q-block by q-block,
// page chunk by page chunk.  item = {b, first global query, query count, first page}.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void score_plan_kernel(const int32_t* __restrict__ cu_q,
                                                         const int32_t* __restrict__ cu_k, int B,
                                                         int qblock, int pc, int64_t max_items,
                                                         int32_t* __restrict__ n_items,
                                                         int4* __restrict__ items) {
  __shared__ int wave_tot[4];
  __shared__ int64_t running;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) running = 0;
  __syncthreads();
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
        const int v = (ctx + qf + qn - 1) / kPage + 1;
        nch = (v + pc - 1) / pc;
      }
      int incl = wave_inclusive_scan(nch);
      if (lane == 63) wave_tot[wave] = incl;
      __syncthreads();
      int wave_off = 0;
      for (int w = 0; w < wave; ++w) wave_off += wave_tot[w];
      const int64_t off = running + wave_off + incl - nch;
      for (int c = 0; c < nch; ++c) {
        const int64_t k = off + c;
        if (k < max_items) items[k] = make_int4(b, q0 + qf, qn, c * pc);
      }
      __syncthreads();
      if (tid == 255) running = off + nch;
      __syncthreads();
    }
  }
  if (tid == 0) *n_items = (int32_t)min<int64_t>(running, max_items);
}

// ---------------------------------------------------------------------------
// Scorer.
// ---------------------------------------------------------------------------
template <int H>
__global__ __launch_bounds__(kThreads) void index_score_kernel(ScoreK a) {
  constexpr int NQT = 8 / H;   // 16-query tiles per wave
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kLdsPage];

  const int item = blockIdx.x;
  if (item >= *a.n_items) return;
  const int4 it = a.items[item];
  const int b = it.x, q_first = it.y, q_count = it.z, p0 = it.w;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;

  const int cq0 = a.cu_q[b];
  const int sq = a.cu_q[b + 1] - cq0;
  const int sk = a.cu_k[b + 1] - a.cu_k[b];
  const int ctx = sk - sq;
  const int pos_first = ctx + (q_first - cq0);
  const int pos_last = pos_first + q_count - 1;
  const int v_block = pos_last / kPage + 1;
  const int p_end = min(min(p0 + a.pages_per_item, v_block), a.max_pages);
  if (p0 >= p_end) return;
  const float scale = (*a.q_scale) * (*a.k_scale);
  const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;

  // Query fragments (B operand): column = query, K-group = 32-byte slice of D.
  v8i qf[NQT][H];
  int qpos[NQT];
  int qrow[NQT];
  const int wave_q0 = q_first + wave * NQT * 16;
  const bool wave_active = wave_q0 < q_first + q_count;
#pragma unroll
  for (int n = 0; n < NQT; ++n) {
    const int qi = wave_q0 + n * 16 + col;
    const bool ok = qi < q_first + q_count;
    qrow[n] = ok ? qi : -1;
    qpos[n] = ok ? ctx + (qi - cq0) : -1;
#pragma unroll
    for (int h = 0; h < H; ++h) {
      if (ok) {
        qf[n][h] = load_frag_global(a.q + (int64_t)qi * a.q_stride + h * kDim + grp * 32);
      } else {
        qf[n][h] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }

  // Stage one page of index-K (16 KiB) into LDS: thread t copies bytes [32t, 32t+32).
  const int st_row = tid >> 2, st_col = (tid & 3) * 32;
  auto page_ptr = [&](int p) -> const uint8_t* {
    int phys = bt[p];
    phys = (phys < 0 || phys >= a.num_pages) ? 0 : phys;
    return a.k_cache + (int64_t)phys * (kPage * kDim) + st_row * kDim + st_col;
  };
  uint4 stage0, stage1;
  {
    const uint8_t* src = page_ptr(p0);
    stage0 = load16_nt(src);
    stage1 = load16_nt(src + 16);
    uint4* dst = reinterpret_cast<uint4*>(lds + st_row * kLdsRow + st_col);
    dst[0] = stage0;
    dst[1] = stage1;
  }
  __syncthreads();

  float stash[NQT];
#pragma unroll
  for (int n = 0; n < NQT; ++n) stash[n] = 0.f;

  int buf = 0;
  for (int p = p0; p < p_end; ++p) {
    const bool has_next = p + 1 < p_end;
    if (has_next) {
      const uint8_t* src = page_ptr(p + 1);
      stage0 = load16_nt(src);
      stage1 = load16_nt(src + 16);
    }
    if (wave_active) {
      const uint8_t* pg = lds + buf * kLdsPage;
      const bool need_mask = (p + 1) * kPage - 1 > pos_first;
      v4f rmax[NQT];
#pragma unroll
      for (int n = 0; n < NQT; ++n) rmax[n] = v4f{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll 2
      for (int T = 0; T < 8; ++T) {
        const v8i ka = load_frag_lds(pg + (T * 16 + col) * kLdsRow + grp * 32);
#pragma unroll
        for (int n = 0; n < NQT; ++n) {
          v4f acc = mfma_e4m3(ka, qf[n][0], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int h = 1; h < H; ++h) acc = mfma_e4m3(ka, qf[n][h], acc);
          if (need_mask) {
            const int lim = qpos[n] - p * kPage;   // last visible token index in this page
            const int t0 = T * 16 + grp * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (t0 + i > lim) acc[i] = -INFINITY;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) rmax[n][i] = fmaxf(rmax[n][i], acc[i]);
        }
      }
#pragma unroll
      for (int n = 0; n < NQT; ++n) {
        float m = fmaxf(fmaxf(rmax[n][0], rmax[n][1]), fmaxf(rmax[n][2], rmax[n][3]));
        m = max_across_groups(m);
        if (grp == (p & 3)) stash[n] = m * scale;
      }
      if ((p & 3) == 3 || p == p_end - 1) {
        const int pp = (p & ~3) + grp;
#pragma unroll
        for (int n = 0; n < NQT; ++n) {
          if (qrow[n] >= 0 && pp >= p0 && pp <= p && pp * kPage <= qpos[n])
            a.scores[(int64_t)qrow[n] * a.ld + pp] = stash[n];
        }
      }
    }
    if (has_next) {
      uint4* dst = reinterpret_cast<uint4*>(lds + (buf ^ 1) * kLdsPage + st_row * kLdsRow + st_col);
      dst[0] = stage0;
      dst[1] = stage1;
    }
    __syncthreads();
    buf ^= 1;
  }
}

}  // namespace

ScorePlan score_plan(const msa_varlen_t* vl, int H) {
  ScorePlan p;
  const int qb = score_qblock(H);
  const int64_t est_qb = std::max<int64_t>(1, ceil_div(vl->total_q, qb));
  const int64_t qb_bound = ceil_div(vl->total_q, qb) + vl->batch;
  const int64_t max_pages = std::max<int32_t>(1, vl->max_pages);
  // about two items per compute unit in total, 4..256 pages per item
  int64_t pc = ceil_div(max_pages * est_qb, 512);
  pc = std::min<int64_t>(256, std::max<int64_t>(4, ceil_div(pc, 4) * 4));
  p.pages_per_item = (int32_t)pc;
  p.max_items = qb_bound * ceil_div(max_pages, pc);
  p.workspace_bytes = sizeof(ItemHdr) + align_up((size_t)p.max_items * sizeof(int4), 256);
  return p;
}

hipError_t launch_index_score(const ScoreArgs& a, hipStream_t stream) {
  if (a.vl.total_q == 0) return hipSuccess;
  ItemHdr* hdr = reinterpret_cast<ItemHdr*>(a.workspace);
  int4* items = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(a.workspace) + sizeof(ItemHdr));
  hipLaunchKernelGGL(score_plan_kernel, dim3(1), dim3(256), 0, stream, a.vl.cu_seqlens_q,
                     a.vl.cu_seqlens_k, a.vl.batch, score_qblock(a.H), a.plan.pages_per_item,
                     a.plan.max_items, &hdr->n_items, items);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ScoreK k;
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
  k.scores = a.scores;
  k.ld = a.ld;
  k.n_items = &hdr->n_items;
  k.items = items;
  k.pages_per_item = a.plan.pages_per_item;
  dim3 grid((unsigned)a.plan.max_items);
  switch (a.H) {
    case 1: hipLaunchKernelGGL(index_score_kernel<1>, grid, dim3(kThreads), 0, stream, k); break;
    case 2: hipLaunchKernelGGL(index_score_kernel<2>, grid, dim3(kThreads), 0, stream, k); break;
    case 4: hipLaunchKernelGGL(index_score_kernel<4>, grid, dim3(kThreads), 0, stream, k); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
