// Causal top-16 page selection for gfx950.
//
// Per query: the local page (and any further forced recent pages) first, then the
// highest-scoring older visible pages, -1 padding (vLLM PR 60684, Validation,
// benchmark script case(): the local page visible-1 is always kept, future pages
// are never chosen, k = min(16, visible)).  Exact-tie order is left open by the
// pages (vLLM PR 64631, Details); here equal scores go to the lower page index,
// which makes the result deterministic.
//
// Rows of up to 512 visible pages: one wave per query, four queries per wave
// (keys in registers, every key >= the wave bound fits the wave's LDS list, so
// no fallback is needed).  Longer rows: one 256-thread block per query:
//  1. each lane takes the max over its strided share of the row;
//  2. within each wave, the ksel-th largest lane maximum is a lower bound tau_w
//     on the ksel-th largest key of the row (ksel distinct elements reach it);
//     tau = max over waves is still such a bound;
//  3. the (few) keys >= tau are collected in LDS and ranked exactly by
//     (key descending, page ascending); ranks < ksel are the selection.
//  If too many keys tie at the top for the LDS list, a bisection over the
//  32-bit key space finds the exact ksel-th key instead and equal keys are
//  admitted in page order by a block scan.
// Rows of 2049..8192 candidates take a leaner form of this (topk_row_kernel:
// raw scores in registers, bound from the top 16 bits of the lane maxima and
// verified by counting) so that a 2048-query batch is resident at once.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kBlock = 256;
constexpr int kCap = 2048;     // LDS candidate list capacity

struct TopkK {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch;
  int32_t total_q;
  int32_t max_pages;
  const float* scores;
  int64_t ld;
  int32_t n_local;
  int32_t* out;
  int64_t out_stride;
};

__device__ __forceinline__ int block_sum(int x, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_sum(x);
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kBlock / 64; ++w) s += red[w];
  return s;
}

// Keys of (score, page) packed so that a larger value is a better candidate:
// higher score first, then lower page.
__device__ __forceinline__ uint64_t pack_key(uint32_t key, int page) {
  return ((uint64_t)key << 32) | (uint32_t)(~(uint32_t)page);
}

// Load KPT keys of this thread for the chunk starting at c0.  Thread t owns
// pages c0 + kBlock*4*k + 4t + {0..3} (k < KPT/4) when KPT >= 4, so each load is
// 16 contiguous bytes; otherwise pages c0 + kBlock*k + t.
template <int KPT>
__device__ __forceinline__ int key_page(int c0, int k, int tid) {
  if constexpr (KPT >= 4) return c0 + (k >> 2) * (kBlock * 4) + tid * 4 + (k & 3);
  else return c0 + k * kBlock + tid;
}
template <int KPT>
__device__ __forceinline__ void load_keys(const float* row, int c0, int ncand, int tid,
                                          uint32_t (&key)[KPT]) {
  if constexpr (KPT >= 4) {
#pragma unroll
    for (int k4 = 0; k4 < KPT / 4; ++k4) {
      const int j = c0 + k4 * (kBlock * 4) + tid * 4;
      if (j + 3 < ncand) {
        const float4 v = *reinterpret_cast<const float4*>(row + j);
        key[4 * k4 + 0] = float_key(v.x);
        key[4 * k4 + 1] = float_key(v.y);
        key[4 * k4 + 2] = float_key(v.z);
        key[4 * k4 + 3] = float_key(v.w);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) key[4 * k4 + e] = (j + e < ncand) ? float_key(row[j + e]) : 0u;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int j = c0 + k * kBlock + tid;
      key[k] = j < ncand ? float_key(row[j]) : 0u;
    }
  }
}

// float_key of the float with bits u, computed without branches; 0 when !valid.
__device__ __forceinline__ uint32_t key_bits(uint32_t u, bool valid) {
  const uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return (valid && (u & 0x7FFFFFFFu) <= 0x7F800000u) ? k : 0u;
}

// Exact rank of c unique packed candidates: the ksel best go to out[f ..].
__device__ __forceinline__ void rank_candidates(const uint64_t* c_pk, int c, int ksel, int f,
                                                int32_t* out) {
  for (int e = threadIdx.x; e < c; e += kBlock) {
    const uint64_t me = c_pk[e];
    int r = 0;
    int o = 0;
    for (; o + 8 <= c; o += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) r += c_pk[o + u] > me ? 1 : 0;
    }
    for (; o < c; ++o) r += c_pk[o] > me ? 1 : 0;
    if (r < ksel) out[f + r] = (int)~(uint32_t)me;
  }
}

// Many keys tie near the top (more candidates than the LDS list holds): find
// the exact ksel-th largest key T by bisection over the 32-bit key space, list
// the keys > T (fewer than ksel) and then the lowest pages with key == T, and
// rank them.  Every thread of the block calls it.
__device__ __noinline__ void exact_select(const TopkK& a, const float* row, int ncand, int ksel,
                                          int f, int32_t* out, uint64_t* c_pk, int* red,
                                          int* n_cand, int* n_eq_taken) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t t = T | (1u << bit);
    int cnt = 0;
    for (int j = tid; j < ncand; j += kBlock) cnt += float_key(row[j]) >= t ? 1 : 0;
    cnt = block_sum(cnt, red);
    if (cnt >= ksel) T = t;
  }
  __syncthreads();
  if (tid == 0) { *n_cand = 0; *n_eq_taken = 0; }
  __syncthreads();
  for (int j = tid; j < ncand; j += kBlock) {
    const uint32_t kj = float_key(row[j]);
    if (kj > T) c_pk[atomicAdd(n_cand, 1)] = pack_key(kj, j);
  }
  __syncthreads();
  const int need = ksel - *n_cand;
  for (int base = 0; base < ncand; base += kBlock) {
    const int j = base + tid;
    const int is_eq = (j < ncand && float_key(row[j]) == T) ? 1 : 0;
    // exclusive prefix of is_eq over the block in page order
    int incl = wave_inclusive_scan(is_eq);
    __syncthreads();
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    int off = *n_eq_taken;
    for (int w = 0; w < wave; ++w) off += red[w];
    const int r = off + incl - is_eq;
    if (is_eq && r < need) c_pk[atomicAdd(n_cand, 1)] = pack_key(T, j);
    __syncthreads();
    if (tid == kBlock - 1) *n_eq_taken = off + incl;
    __syncthreads();
    if (*n_eq_taken >= need) break;
  }
  __syncthreads();
  rank_candidates(c_pk, *n_cand, ksel, f, out);
}

// KPT keys per thread are held in registers: rows of up to kBlock * KPT
// candidates are read once; longer rows are processed in chunks of that size and
// re-read (from cache) by the second pass.
template <int KPT>
__global__ __launch_bounds__(kBlock) void topk_kernel(TopkK a) {
  __shared__ uint64_t c_pk[kCap];
  __shared__ uint32_t wave_tau[kBlock / 64];
  __shared__ int red[kBlock / 64];
  __shared__ int n_cand;
  __shared__ int n_eq_taken;
  constexpr int kChunk = kBlock * KPT;

  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = find_request(a.cu_q, a.batch, i);
  const int cq0 = a.cu_q[b];
  const int sq = a.cu_q[b + 1] - cq0;
  const int sk = a.cu_k[b + 1] - a.cu_k[b];
  const int pos = sk - sq + (int)(i - cq0);
  const int v = min(pos / kPage + 1, a.max_pages);
  const int k_all = min(kTopK, v);
  const int f = min(a.n_local, k_all);
  const int ksel = k_all - f;
  const int ncand = v - f;
  int32_t* out = a.out + i * a.out_stride;
  const float* row = a.scores + i * a.ld;
  const bool vec_ok = (reinterpret_cast<uintptr_t>(row) & 15) == 0;

  if (tid < kTopK) {
    if (tid < f) out[tid] = v - 1 - tid;
    else if (tid >= k_all) out[tid] = -1;
  }
  if (ksel == 0) return;

  // 1. lane maximum (all loads of a chunk are issued together)
  uint32_t key[KPT];
  uint32_t m = 0;
  for (int c0 = 0; c0 < ncand; c0 += kChunk) {
    if (vec_ok) {
      load_keys<KPT>(row, c0, ncand, tid, key);
    } else {
#pragma unroll
      for (int k = 0; k < KPT; ++k) {
        const int j = key_page<KPT>(c0, k, tid);
        key[k] = j < ncand ? float_key(row[j]) : 0u;
      }
    }
#pragma unroll
    for (int k = 0; k < KPT; ++k) m = max(m, key[k]);
  }
  const bool one_chunk = ncand <= kChunk;   // then key[] still holds every key

  // 2. wave bound: the ksel-th largest lane maximum of the wave (bit-by-bit
  //    search with ballots); ksel elements of the row reach it
  uint32_t tw = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t t = tw | (1u << bit);
    if ((int)__popcll(__ballot(m >= t)) >= ksel) tw = t;
  }
  if (lane == 0) wave_tau[wave] = tw;
  if (tid == 0) n_cand = 0;
  __syncthreads();
  uint32_t tau = 0;
#pragma unroll
  for (int w = 0; w < kBlock / 64; ++w) tau = max(tau, wave_tau[w]);

  // 3. collect keys >= tau: one atomic per wave, lanes write at their offsets
  auto collect = [&](int c0, const uint32_t (&kk)[KPT]) {
    int mine = 0;
#pragma unroll
    for (int k = 0; k < KPT; ++k) mine += (key_page<KPT>(c0, k, tid) < ncand && kk[k] >= tau) ? 1 : 0;
    const int incl = wave_inclusive_scan(mine);
    int base = 0;
    if (lane == 63 && incl > 0) base = atomicAdd(&n_cand, incl);
    base = __shfl(base, 63);
    int slot = base + incl - mine;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int j = key_page<KPT>(c0, k, tid);
      if (j < ncand && kk[k] >= tau) {
        if (slot < kCap) c_pk[slot] = pack_key(kk[k], j);
        ++slot;
      }
    }
  };
  if (one_chunk) {
    collect(0, key);
  } else {
    for (int c0 = 0; c0 < ncand; c0 += kChunk) {
#pragma unroll
      for (int k = 0; k < KPT; ++k) {
        const int j = key_page<KPT>(c0, k, tid);
        key[k] = j < ncand ? float_key(row[j]) : 0u;
      }
      collect(c0, key);
    }
  }
  __syncthreads();
  int c = n_cand;

  if (c > kCap) {
    exact_select(a, row, ncand, ksel, f, out, c_pk, red, &n_cand, &n_eq_taken);
    return;
  }
  // 4. exact rank among candidates (packed keys are unique)
  rank_candidates(c_pk, c, ksel, f, out);
}

// Rows of 2,049 .. kBlock * KPT candidates, every score read once and kept as
// loaded (thread t owns pages 256k + t), as dword buffer
// loads over the row's ncand candidates: past them a load returns 0.0, which
// may enter the lane maxima but never the list (the collection below checks
// the page where it could).  So the bound tau taken from the lane maxima is
// checked instead of trusted: every candidate score >= tau is listed, and only
// if at least ksel were found (so the ksel-th best is >= tau, and with it all
// of the top ksel) is the list ranked; otherwise the exact search runs.
// Scores compare as floats up to the list (NaN never reaches it; +0.0 and -0.0
// both do when tau is a zero), and the list is ranked by orderable key and
// page as everywhere.
constexpr int kWaveCap = 64;      // listed candidates per wave

struct RowSmem {
  uint64_t c_pk[kBlock / 64 * kWaveCap];
  int c_j[kBlock / 64 * kWaveCap];          // listed pages before packing
  uint64_t c_all[64];
  uint32_t wave_tau[kBlock / 64];
  int s_cnt[kBlock / 64];
  int red[kBlock / 64];
  int n_cand;
  int n_eq_taken;
};

struct RowQuery {
  const float* row;
  int32_t* out;
  int v, k_all, f, ksel, ncand;
};

__device__ __forceinline__ RowQuery row_query(const TopkK& a, int64_t i) {
  RowQuery q;
  const int b = find_request(a.cu_q, a.batch, i);
  const int cq0 = a.cu_q[b];
  const int sq = a.cu_q[b + 1] - cq0;
  const int sk = a.cu_k[b + 1] - a.cu_k[b];
  const int pos = sk - sq + (int)(i - cq0);
  q.v = min(pos / kPage + 1, a.max_pages);
  q.k_all = min(kTopK, q.v);
  q.f = min(a.n_local, q.k_all);
  q.ksel = q.k_all - q.f;
  q.ncand = q.v - q.f;
  q.row = a.scores + i * a.ld;
  q.out = a.out + i * a.out_stride;
  return q;
}

// Selection for one query whose candidate scores x the block holds (thread t
// pages 256k + t); every thread of the block calls it.
template <int KPT>
__device__ __forceinline__ void select_row(const TopkK& a, const RowQuery& q, const float (&x)[KPT],
                                           RowSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ksel = q.ksel, ncand = q.ncand, f = q.f;
  int32_t* out = q.out;

  // 1. lane maximum (NaN-propagating: a lane holding a NaN drops out of the bound)
  float mf = x[0];
#pragma unroll
  for (int k = 1; k + 1 < KPT; k += 2)
    mf = __builtin_elementwise_maximum(mf, __builtin_elementwise_maximum(x[k], x[k + 1]));
  if constexpr (KPT % 2 == 0) mf = __builtin_elementwise_maximum(mf, x[KPT - 1]);
  const uint32_t m = float_key(mf) >> 16;

  // 2. wave bound: the ksel-th largest top half of the lane maxima; the block
  //    takes the largest, as a float (the least float with that top half)
  uint32_t tw = 0;
  for (int bit = 15; bit >= 0; --bit) {
    const uint32_t t = tw | (1u << bit);
    if ((int)__popcll(__ballot(m >= t)) >= ksel) tw = t;
  }
  if (lane == 0) sm.wave_tau[wave] = tw;
  __syncthreads();
  uint32_t tk = 0;
#pragma unroll
  for (int w = 0; w < kBlock / 64; ++w) tk = max(tk, sm.wave_tau[w]);
  tk <<= 16;
  const float tau = __uint_as_float((tk & 0x80000000u) ? (tk & 0x7FFFFFFFu) : ~tk);

  // 3. list every candidate score >= tau in the wave's part of the list: each
  //    lane first marks its candidate key slots in a bit mask (compares only,
  //    no branches: the scalar unit the CU's waves share is the scarce
  //    resource here), then writes the pages of its set bits.  The listed
  //    scores are read again in full (from cache) by the lane that packs them.
  const int lim = ncand - tid;              // key slot k is a candidate page iff k * kBlock < lim
  const int nvalid = lim <= 0 ? 0 : min(KPT, (lim + kBlock - 1) / kBlock);
  uint32_t cm = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) cm |= (x[k] >= tau ? 1u : 0u) << k;
  cm &= nvalid >= 32 ? 0xFFFFFFFFu : (1u << nvalid) - 1u;
  const int mine = __popc(cm);
  const int incl = wave_inclusive_scan(mine);
  const int n_w = __builtin_amdgcn_readlane(incl, 63);
  int slot = incl - mine;
  while (cm != 0u) {
    const int k = __builtin_ctz(cm);
    cm &= cm - 1u;
    if (slot < kWaveCap) sm.c_j[wave * kWaveCap + slot] = k * kBlock + tid;
    ++slot;
  }
  if (lane < min(n_w, kWaveCap)) {
    const int e = wave * kWaveCap + lane;
    const int j = sm.c_j[e];
    sm.c_pk[e] = pack_key(float_key(q.row[j]), j);
  }
  if (lane == 0) sm.s_cnt[wave] = n_w;
  __syncthreads();
  int c = 0;
  bool over = false;
#pragma unroll
  for (int w = 0; w < kBlock / 64; ++w) {
    c += sm.s_cnt[w];
    over = over || sm.s_cnt[w] > kWaveCap;
  }
  if (over || c < ksel) {
    exact_select(a, q.row, ncand, ksel, f, out, sm.c_pk, sm.red, &sm.n_cand, &sm.n_eq_taken);
  } else if (c <= 64) {
    // 4. exact rank (listed keys are unique).  Up to 64: the four wave lists
    //    are packed into c_all, candidate e = 16w + (lane % 16) of wave w is
    //    compared by the lane's quarter (lane / 16) against entries 16q ..
    //    16q + 15, and the four counts are summed across the quarters.
    //    Entries past c hold 0, below every listed key, so the counts need no
    //    bound check; the store goes through a buffer over the query's 16
    //    outputs and lanes with nothing to write give an offset past it.
    int pre = 0;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) pre += w < wave ? sm.s_cnt[w] : 0;
    if (lane < n_w) sm.c_all[pre + lane] = sm.c_pk[wave * kWaveCap + lane];
    if (wave == 0 && lane >= c) sm.c_all[lane] = 0u;
    __syncthreads();
    const int e = 16 * wave + (lane & 15), qt = lane >> 4;
    const uint64_t me = sm.c_all[min(e, c - 1)];
    int r = 0;
#pragma unroll
    for (int o = 0; o < 16; ++o) r += sm.c_all[16 * qt + o] > me ? 1 : 0;   // all reads in flight together
    r = (int)sum_across_groups((float)r);
    const bool wr = e < c && qt == 0 && r < ksel;
    __builtin_amdgcn_raw_buffer_store_b32((int)~(uint32_t)me, buffer_rsrc(out, kTopK * 4u),
                                          wr ? (f + r) * 4 : 1 << 20, 0, 0);
  } else {
    // more: thread t takes entry t of the four wave lists and counts the
    // larger entries of all four
    const int w = tid / kWaveCap, o = tid % kWaveCap;
    if (o < sm.s_cnt[w]) {
      const uint64_t me = sm.c_pk[tid];
      int r = 0;
#pragma unroll
      for (int w2 = 0; w2 < kBlock / 64; ++w2) {
        const int n2 = sm.s_cnt[w2];
        const uint64_t* l2 = sm.c_pk + w2 * kWaveCap;
        for (int o2 = 0; o2 < n2; ++o2) r += l2[o2] > me ? 1 : 0;
      }
      if (r < ksel) out[f + r] = (int)~(uint32_t)me;
    }
  }
}

// NQ consecutive queries per block: the loads of all NQ rows go out first
// (dword buffer loads over each row's ncand candidates), then the block
// selects for one query after another.  One query per block measured fastest
// on 2048-query batches (all of them resident at once, eight blocks per CU);
// two per block, four blocks per CU, measured 20 % slower.
template <int KPT, int NQ>
__global__ __launch_bounds__(kBlock, 8 / NQ) void topk_row_kernel(TopkK a) {
  __shared__ RowSmem sm;
  const int tid = threadIdx.x;
  const int64_t i0 = (int64_t)blockIdx.x * NQ;
  RowQuery q[NQ];
  float x[NQ][KPT];
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    // a query past the batch repeats the last one; nothing of it is written
    q[qq] = row_query(a, i0 + qq < a.total_q ? i0 + qq : a.total_q - 1);
    const auto rs = buffer_rsrc(q[qq].row, (uint32_t)max(q[qq].ncand, 0) * 4u);
#pragma unroll
    for (int k = 0; k < KPT; ++k)
      x[qq][k] = __builtin_bit_cast(float,
                                    __builtin_amdgcn_raw_buffer_load_b32(rs, (k * kBlock + tid) * 4, 0, 0));
  }
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    if (i0 + qq >= a.total_q) break;
    const RowQuery& r = q[qq];
    if (tid < kTopK) {
      if (tid < r.f) r.out[tid] = r.v - 1 - tid;
      else if (tid >= r.k_all) r.out[tid] = -1;
    }
    if (r.ksel == 0) continue;
    select_row<KPT>(a, r, x[qq], sm);
    __syncthreads();                        // the lists are reused by the next query
  }
}

// One wave per query for rows of at most 64 * KPT candidates, NQ consecutive
// queries per wave: the loads of all NQ rows go out first (lane l owns pages
// 64k + l, one dword buffer load each over the row's first min(ld, max_pages)
// entries; keys past the candidates are masked), so the wave waits for memory
// once and then selects for its queries one after another.  Per query the
// bound is the ksel-th largest lane maximum of the keys' top 16 bits (ksel
// keys reach it, so every key of the top ksel does too); every key whose top
// half reaches it (at most 64 * KPT) is ranked exactly from the wave's LDS list.
template <int KPT, int NQ>
__global__ __launch_bounds__(kBlock) void topk_wave_kernel(TopkK a) {
  constexpr int kWaves = kBlock / 64;
  constexpr int kList = 64 * KPT;
  __shared__ uint64_t c_pk[kWaves][kList + 64];   // the list, then one discard entry per lane
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t i0 = ((int64_t)blockIdx.x * kWaves + wave) * NQ;
  if (i0 >= a.total_q) return;
  const int row_len = a.ld < (int64_t)a.max_pages ? (int)a.ld : a.max_pages;
  // the first query's request, looked up before the rows are requested (vector
  // loads complete in order, so a lookup issued after them would wait for them)
  int b = find_request(a.cu_q, a.batch, i0);
  int cq0 = a.cu_q[b], cq1 = a.cu_q[b + 1];
  int sk = a.cu_k[b + 1] - a.cu_k[b];
  __builtin_amdgcn_sched_barrier(0);        // keep those loads ahead of the rows'

  uint32_t x[NQ][KPT];
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    // queries past the batch re-read the last row; their results are not written
    const int64_t i = i0 + qq < a.total_q ? i0 + qq : a.total_q - 1;
    const auto rs = buffer_rsrc(a.scores + i * a.ld, (uint32_t)row_len * 4u);
#pragma unroll
    for (int k = 0; k < KPT; ++k) x[qq][k] = __builtin_amdgcn_raw_buffer_load_b32(rs, (k * 64 + lane) * 4, 0, 0);
  }
  // the empty asm keeps every load unconditional
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq)
#pragma unroll
    for (int k = 0; k < KPT; ++k) asm volatile("" : "+v"(x[qq][k]));

#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    const int64_t i = i0 + qq;
    if (i >= a.total_q) break;
    if (i >= cq1) {                         // the wave's queries cross into a later request
      b = find_request(a.cu_q, a.batch, i);
      cq0 = a.cu_q[b];
      cq1 = a.cu_q[b + 1];
      sk = a.cu_k[b + 1] - a.cu_k[b];
    }
    const int pos = sk - (cq1 - cq0) + (int)(i - cq0);
    const int v = min(pos / kPage + 1, a.max_pages);
    const int k_all = min(kTopK, v);
    const int f = min(a.n_local, k_all);
    const int ksel = k_all - f;
    const int ncand = v - f;
    // stores go through a buffer over the query's 16 output slots, so a lane
    // with nothing to write gives an offset past them and its store is
    // dropped: no branches (each one costs scalar instructions, which limit
    // this kernel with eight waves per SIMD)
    const auto rs_out = buffer_rsrc(a.out + i * a.out_stride, kTopK * 4u);
    constexpr int kDrop = 1 << 20;
    {
      const bool w = lane < kTopK && (lane < f || lane >= k_all);
      __builtin_amdgcn_raw_buffer_store_b32(lane < f ? v - 1 - lane : -1, rs_out, w ? lane * 4 : kDrop, 0, 0);
    }
    if (ksel == 0) continue;

    const int lim = ncand - lane;           // page 64k + lane is a candidate iff 64k < lim
    uint32_t key[KPT];
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      key[k] = key_bits(x[qq][k], k * 64 < lim);
      m = max(m, key[k]);
    }
    // the ksel-th largest lane maximum of the top halves
    uint32_t t16 = 0;
    m >>= 16;
#pragma unroll
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t t = t16 | (1u << bit);
      if ((int)__popcll(__ballot(m >= t)) >= ksel) t16 = t;
    }
    const uint32_t tau = t16 << 16;

    // every candidate key >= tau goes to the list; the others to the lane's
    // discard entry.  The first 64 entries start at 0, below every listed key,
    // so the rank below needs no count check.  Keys past the candidates are 0,
    // so with tau > 0 the key alone decides (only tau == 0 checks the page).
    c_pk[wave][lane] = 0u;
    bool cand[KPT];
    int mine = 0;
    const bool any_key = tau == 0u;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      cand[k] = any_key ? k * 64 < lim : key[k] >= tau;
      mine += (int)cand[k];
    }
    const int incl = wave_inclusive_scan(mine);
    const int c = __builtin_amdgcn_readlane(incl, 63);
    int slot = incl - mine;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      c_pk[wave][cand[k] ? slot : kList + lane] = pack_key(key[k], k * 64 + lane);
      slot += (int)cand[k];
    }
    // a wave's LDS operations complete in order: only the compiler is held here
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");

    // exact rank among the candidates (packed keys are unique): in registers
    // for up to 64 of them, else from the list
    if (c <= 64) {
      // candidates 16 at a time, lane l taking candidate e0 + l % 16 and
      // comparing it with every fourth entry from l / 16 on (all 16 reads in
      // flight together); the four quarter counts are summed across lanes
      const int qt = lane >> 4;
      for (int e0 = 0; e0 < c; e0 += 16) {
        const int e = e0 + (lane & 15);
        const uint64_t me = c_pk[wave][min(e, c - 1)];
        int r = 0;
#pragma unroll
        for (int o = 0; o < 16; ++o) r += c_pk[wave][4 * o + qt] > me ? 1 : 0;
        r = (int)sum_across_groups((float)r);
        const bool w = e < c && qt == 0 && r < ksel;
        __builtin_amdgcn_raw_buffer_store_b32((int)~(uint32_t)me, rs_out, w ? (f + r) * 4 : kDrop, 0, 0);
      }
    } else {
      for (int e = lane; e < c; e += 64) {
        const uint64_t me = c_pk[wave][e];
        int r = 0;
        for (int o = 0; o < c; ++o) r += c_pk[wave][o] > me ? 1 : 0;
        if (r < ksel) a.out[i * a.out_stride + f + r] = (int)~(uint32_t)me;
      }
    }
    // the list is rewritten for the next query
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.vl.total_q == 0) return hipSuccess;
  TopkK k;
  k.cu_q = a.vl.cu_seqlens_q;
  k.cu_k = a.vl.cu_seqlens_k;
  k.batch = a.vl.batch;
  k.total_q = a.vl.total_q;
  k.max_pages = a.vl.max_pages;
  k.scores = a.scores;
  k.ld = a.ld;
  k.n_local = a.n_local;
  k.out = a.out;
  k.out_stride = a.out_stride;
  const int need = std::max(1, a.vl.max_pages);   // candidates per query, at most
  if (need <= 512) {
    constexpr int kNQ = 4;                        // queries per wave
    const dim3 wgrid((unsigned)ceil_div(a.vl.total_q, (int64_t)(kBlock / 64) * kNQ));
    if (need <= 256) hipLaunchKernelGGL((topk_wave_kernel<4, kNQ>), wgrid, dim3(kBlock), 0, stream, k);
    else hipLaunchKernelGGL((topk_wave_kernel<8, kNQ>), wgrid, dim3(kBlock), 0, stream, k);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)a.vl.total_q);
  if (need <= kBlock * 1) hipLaunchKernelGGL(topk_kernel<1>, grid, dim3(kBlock), 0, stream, k);
  else if (need <= kBlock * 2) hipLaunchKernelGGL(topk_kernel<2>, grid, dim3(kBlock), 0, stream, k);
  else if (need <= kBlock * 4) hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(kBlock), 0, stream, k);
  else if (need <= kBlock * 8) hipLaunchKernelGGL(topk_kernel<8>, grid, dim3(kBlock), 0, stream, k);
  else if (need <= kBlock * 16) hipLaunchKernelGGL((topk_row_kernel<16, 1>), grid, dim3(kBlock), 0, stream, k);
  else if (need <= kBlock * 32) hipLaunchKernelGGL((topk_row_kernel<32, 1>), grid, dim3(kBlock), 0, stream, k);
  else hipLaunchKernelGGL(topk_kernel<32>, grid, dim3(kBlock), 0, stream, k);
  return hipGetLastError();
}

}  // namespace msa
