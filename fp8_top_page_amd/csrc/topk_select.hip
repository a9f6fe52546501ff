// Causal top-16 page selection for gfx950.
//
// Per query: the local page (and any further forced recent pages) first, then the
// highest-scoring older visible pages, -1 padding (vLLM PR 60684, Validation,
// benchmark script case(): the local page visible-1 is always kept, future pages
// are never chosen, k = min(16, visible)).  Exact-tie order is left open by the
// pages (vLLM PR 64631, Details); here equal scores go to the lower page index,
// which makes the result deterministic.
//
// Rows of up to 512 visible pages: one wave per query (keys in registers, every
// key >= the wave bound fits the wave's LDS list, so no fallback is needed).
// Longer rows: one 256-thread block per query:
//  1. each lane takes the max orderable key over its strided share of the row;
//  2. within each wave, the ksel-th largest lane maximum is a lower bound tau_w
//     on the ksel-th largest key of the row (ksel distinct elements reach it);
//     tau = max over waves is still such a bound;
//  3. the (few) keys >= tau are collected in LDS and ranked exactly by
//     (key descending, page ascending); ranks < ksel are the selection.
//  If too many keys tie at the top for the LDS list, a bisection over the
//  32-bit key space finds the exact ksel-th key instead and equal keys are
//  admitted in page order by a block scan.
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
    // Many keys tie near the top: find the exact ksel-th largest key T.
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t t = T | (1u << bit);
      int cnt = 0;
      for (int j = tid; j < ncand; j += kBlock) cnt += float_key(row[j]) >= t ? 1 : 0;
      cnt = block_sum(cnt, red);
      if (cnt >= ksel) T = t;
    }
    // keys > T (fewer than ksel), then the lowest pages with key == T
    if (tid == 0) { n_cand = 0; n_eq_taken = 0; }
    __syncthreads();
    for (int j = tid; j < ncand; j += kBlock) {
      const uint32_t kj = float_key(row[j]);
      if (kj > T) c_pk[atomicAdd(&n_cand, 1)] = pack_key(kj, j);
    }
    __syncthreads();
    const int need = ksel - n_cand;
    for (int base = 0; base < ncand; base += kBlock) {
      const int j = base + tid;
      const int is_eq = (j < ncand && float_key(row[j]) == T) ? 1 : 0;
      // exclusive prefix of is_eq over the block in page order
      int incl = wave_inclusive_scan(is_eq);
      __syncthreads();
      if (lane == 63) red[wave] = incl;
      __syncthreads();
      int off = n_eq_taken;
      for (int w = 0; w < wave; ++w) off += red[w];
      const int r = off + incl - is_eq;
      if (is_eq && r < need) c_pk[atomicAdd(&n_cand, 1)] = pack_key(T, j);
      __syncthreads();
      if (tid == kBlock - 1) n_eq_taken = off + incl;
      __syncthreads();
      if (n_eq_taken >= need) break;
    }
    __syncthreads();
    c = n_cand;
  }

  // 4. exact rank among candidates (packed keys are unique)
  for (int e = tid; e < c; e += kBlock) {
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

// One wave per query for rows of at most 64 * KPT candidates.  Lane l owns pages
// 256k + 4l + {0..3} (16-byte loads); the wave bound is taken as in the block
// kernel and every key >= it (at most 64 * KPT) is ranked from the wave's LDS list.
template <int KPT>
__global__ __launch_bounds__(kBlock) void topk_wave_kernel(TopkK a) {
  static_assert(KPT % 4 == 0, "four keys per 16-byte load");
  constexpr int kWaves = kBlock / 64;
  constexpr int kList = 64 * KPT;
  __shared__ uint64_t c_pk[kWaves][kList];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t i = (int64_t)blockIdx.x * kWaves + wave;
  if (i >= a.total_q) return;
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

  if (lane < kTopK) {
    if (lane < f) out[lane] = v - 1 - lane;
    else if (lane >= k_all) out[lane] = -1;
  }
  if (ksel == 0) return;

  uint32_t key[KPT];
#pragma unroll
  for (int k4 = 0; k4 < KPT / 4; ++k4) {
    const int j = k4 * 256 + lane * 4;
    if (vec_ok && j + 3 < ncand) {
      const float4 x = *reinterpret_cast<const float4*>(row + j);
      key[4 * k4 + 0] = float_key(x.x);
      key[4 * k4 + 1] = float_key(x.y);
      key[4 * k4 + 2] = float_key(x.z);
      key[4 * k4 + 3] = float_key(x.w);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) key[4 * k4 + e] = (j + e < ncand) ? float_key(row[j + e]) : 0u;
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) m = max(m, key[k]);

  // the ksel-th largest lane maximum: ksel keys of the row reach it
  uint32_t tau = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t t = tau | (1u << bit);
    if ((int)__popcll(__ballot(m >= t)) >= ksel) tau = t;
  }

  // every candidate key >= tau goes to the list (at most 64 * KPT of them);
  // slots past ncand are skipped by their page index
  int mine = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int j = (k >> 2) * 256 + lane * 4 + (k & 3);
    mine += (j < ncand && key[k] >= tau) ? 1 : 0;
  }
  const int incl = wave_inclusive_scan(mine);
  const int c = __shfl(incl, 63);
  int slot = incl - mine;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int j = (k >> 2) * 256 + lane * 4 + (k & 3);
    if (j < ncand && key[k] >= tau) c_pk[wave][slot++] = pack_key(key[k], j);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

  // exact rank among the candidates (packed keys are unique)
  for (int e = lane; e < c; e += 64) {
    const uint64_t me = c_pk[wave][e];
    int r = 0;
    for (int o = 0; o < c; ++o) r += c_pk[wave][o] > me ? 1 : 0;
    if (r < ksel) out[f + r] = (int)~(uint32_t)me;
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
    const dim3 wgrid((unsigned)ceil_div(a.vl.total_q, kBlock / 64));
    if (need <= 256) hipLaunchKernelGGL(topk_wave_kernel<4>, wgrid, dim3(kBlock), 0, stream, k);
    else hipLaunchKernelGGL(topk_wave_kernel<8>, wgrid, dim3(kBlock), 0, stream, k);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)a.vl.total_q);
  if (need <= kBlock * 1) hipLaunchKernelGGL(topk_kernel<1>, grid, dim3(kBlock), 0, stream, k);
  else if (need <= kBlock * 2) hipLaunchKernelGGL(topk_kernel<2>, grid, dim3(kBlock), 0, stream, k);
  else if (need <= kBlock * 4) hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(kBlock), 0, stream, k);
  else if (need <= kBlock * 8) hipLaunchKernelGGL(topk_kernel<8>, grid, dim3(kBlock), 0, stream, k);
  else if (need <= kBlock * 16) hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(kBlock), 0, stream, k);
  else hipLaunchKernelGGL(topk_kernel<32>, grid, dim3(kBlock), 0, stream, k);
  return hipGetLastError();
}

}  // namespace msa
