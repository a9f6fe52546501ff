// Causal top-16 page selection for gfx950.
//
// Per query: the local page (and any further forced recent pages) first, then the
// highest-scoring older visible pages, -1 padding (vLLM PR 60684, Validation,
// benchmark script case(): the local page visible-1 is always kept, future pages
// are never chosen, k = min(16, visible)).  Exact-tie order is left open by the
// pages (vLLM PR 64631, Details); here equal scores go to the lower page index,
// which makes the result deterministic.
//
// One 256-thread block per query:
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

__global__ __launch_bounds__(kBlock) void topk_kernel(TopkK a) {
  __shared__ uint32_t c_key[kCap];
  __shared__ int32_t c_page[kCap];
  __shared__ uint32_t wave_tau[kBlock / 64];
  __shared__ int red[kBlock / 64];
  __shared__ int n_cand;
  __shared__ int n_eq_taken;

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

  if (tid < kTopK) {
    if (tid < f) out[tid] = v - 1 - tid;
    else if (tid >= k_all) out[tid] = -1;
  }
  if (ksel == 0) return;

  // 1. lane maximum
  uint32_t m = 0;
  for (int j = tid; j < ncand; j += kBlock) m = max(m, float_key(row[j]));
  // 2. wave bound: key of the lane with rank ksel-1 by (key desc, lane asc)
  int rank = 0;
  for (int l = 0; l < 64; ++l) {
    const uint32_t o = __builtin_amdgcn_readlane(m, l);
    rank += (o > m || (o == m && l < lane)) ? 1 : 0;
  }
  const unsigned long long sel = __ballot(rank == ksel - 1);
  const uint32_t tau_w = __builtin_amdgcn_readlane(m, __builtin_ctzll(sel));
  if (lane == 0) wave_tau[wave] = tau_w;
  if (tid == 0) n_cand = 0;
  __syncthreads();
  uint32_t tau = 0;
#pragma unroll
  for (int w = 0; w < kBlock / 64; ++w) tau = max(tau, wave_tau[w]);

  // 3. collect keys >= tau
  for (int j = tid; j < ncand; j += kBlock) {
    const uint32_t key = float_key(row[j]);
    if (key >= tau) {
      const int slot = atomicAdd(&n_cand, 1);
      if (slot < kCap) {
        c_key[slot] = key;
        c_page[slot] = j;
      }
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
      const uint32_t key = float_key(row[j]);
      if (key > T) {
        const int slot = atomicAdd(&n_cand, 1);
        c_key[slot] = key;
        c_page[slot] = j;
      }
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
      if (is_eq && r < need) {
        const int slot = atomicAdd(&n_cand, 1);
        c_key[slot] = T;
        c_page[slot] = j;
      }
      __syncthreads();
      if (tid == kBlock - 1) n_eq_taken = off + incl;
      __syncthreads();
      if (n_eq_taken >= need) break;
    }
    __syncthreads();
    c = n_cand;
  }

  // 4. exact rank among candidates
  for (int e = tid; e < c; e += kBlock) {
    const uint32_t key = c_key[e];
    const int page = c_page[e];
    int r = 0;
    for (int o = 0; o < c; ++o) {
      const uint32_t ko = c_key[o];
      r += (ko > key || (ko == key && c_page[o] < page)) ? 1 : 0;
    }
    if (r < ksel) out[f + r] = page;
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
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.vl.total_q), dim3(kBlock), 0, stream, k);
  return hipGetLastError();
}

}  // namespace msa
