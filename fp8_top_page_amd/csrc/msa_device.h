// Device helpers for the gfx950 kernels: fp8 matrix-core op, wave reductions,
// orderable float keys, E4M3 packing, bfloat16 rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace msa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// D = A * B + C on one 16x16x128 E4M3 tile (v_mfma_f32_16x16x128_f8f6f4, no block
// scales).  Lane l holds row (l % 16) of A and column (l % 16) of B, each with the
// 32 K-elements of K-group (l / 16); C/D lane l holds column (l % 16), rows
// 4 * (l / 16) + {0,1,2,3}.  Both operands use the same lane -> K mapping, so a
// contraction is correct for any fixed assignment of the 128 K indices to
// (K-group, byte) slots, as long as A and B use the same one.
__device__ __forceinline__ v4f mfma_e4m3(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// 16-byte streaming load (nontemporal: data read once per block).
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ v8i load_frag_global(const uint8_t* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 x = q[0];
  uint4 y = q[1];
  v8i r;
  r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
  r[4] = y.x; r[5] = y.y; r[6] = y.z; r[7] = y.w;
  return r;
}

__device__ __forceinline__ v8i load_frag_lds(const uint8_t* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 x = q[0];
  uint4 y = q[1];
  v8i r;
  r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
  r[4] = y.x; r[5] = y.y; r[6] = y.z; r[7] = y.w;
  return r;
}

// Reductions across the four 16-lane groups (lanes l, l^16, l^32, l^48), on the
// VALU with the gfx950 lane-swap instructions: permlane32_swap exchanges the two
// 32-lane halves between its two operands and permlane16_swap the odd/even
// 16-lane rows, so with both operands equal to x the pair it returns holds x and
// x's partner (in some order) and a symmetric max/sum of the two completes one
// butterfly step.
// (The maximum is IEEE 754-2019 maximum: a NaN in any lane gives NaN.)
__device__ __forceinline__ float max_across_groups(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_groups(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// r differs from the values of the lanes 1 .. 15 places down this lane's
// 16-lane row (row_shr by D + 1; a lane whose source lies before the row start
// sees -2, which no caller uses as a value).  Every lane of the row must be
// active.
template <int... D>
__device__ __forceinline__ bool first_in_row(int r, std::integer_sequence<int, D...>) {
  return ((__builtin_amdgcn_update_dpp(-2, r, 0x111 + D, 0xF, 0xF, false) != r) && ...);
}
__device__ __forceinline__ bool first_in_row16(int r) {
  return first_in_row(r, std::make_integer_sequence<int, 15>{});
}

// A block barrier that orders LDS only: the waves' LDS operations complete,
// then all waves meet.  __syncthreads also waits for every global memory
// operation in flight (stores included: on gfx950 loads and stores share one
// counter), which a barrier that only hands LDS between waves does not need.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Raw buffer resource over `bytes` bytes at p: buffer loads past the end return
// zero instead of reading memory, and stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// Monotone map float -> uint32 (larger float, larger key).  NaN maps to 0, below
// every number (-inf maps to 0x007FFFFF).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Four floats in [0, 448] -> one dword of E4M3 codes (byte k = value k), hardware
// round-to-nearest-even conversion (gfx950 converts to OCP E4M3).
__device__ __forceinline__ int pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return w;
}

// float -> bfloat16 bits, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Inclusive scan over a 64-lane wave on the VALU, through DPP lane moves
// instead of LDS permutes: a Hillis-Steele scan inside each 16-lane row
// (row_shr by 1, 2, 4 and 8, zero where the source lies before the row), then
// rows 1 and 3 add lane 15 of the row before them (row_bcast:15) and rows 2 and
// 3 add lane 31 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return x;
}

// Sum over the wave, the same in every lane.
__device__ __forceinline__ int wave_sum(int x) {
  return __builtin_amdgcn_readlane(wave_inclusive_scan(x), 63);
}

// Reductions over the whole wave, the result in every lane: the same butterfly
// as group_sum below, each step combining a lane with its partner.
template <class Op>
__device__ __forceinline__ int wave_reduce(int x, Op op) {
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));
  auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  x = op((int)r[0], (int)r[1]);
  r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return op((int)r[0], (int)r[1]);
}
__device__ __forceinline__ int wave_min(int x) {
  return wave_reduce(x, [](int a, int b) { return a < b ? a : b; });
}
__device__ __forceinline__ int wave_max(int x) {
  return wave_reduce(x, [](int a, int b) { return a > b ? a : b; });
}
// 64-bit sum: both halves of the partner's value move through the same lane
// pattern, then a 64-bit add.
__device__ __forceinline__ int64_t wave_sum64(int64_t x) {
  auto mv = [](int64_t v, auto move) -> int64_t {
    const uint32_t lo = move((uint32_t)v), hi = move((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };
  x += mv(x, [](uint32_t u) { return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, false); });
  x += mv(x, [](uint32_t u) { return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, false); });
  x += mv(x, [](uint32_t u) { return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x141, 0xF, 0xF, false); });
  x += mv(x, [](uint32_t u) { return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x140, 0xF, 0xF, false); });
  // row swaps: the pair holds this lane's value and its partner's, in some
  // order, so their sum is the same whichever it is
  auto sw = [](int64_t v, bool wide) -> int64_t {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)((uint64_t)v >> 32);
    const auto a = wide ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                        : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto b = wide ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                        : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    return (int64_t)(((uint64_t)b[0] << 32) | a[0]) + (int64_t)(((uint64_t)b[1] << 32) | a[1]);
  };
  x = sw(x, false);
  return sw(x, true);
}

// Sum over aligned groups of G lanes (G a power of two up to 64), in every lane
// of the group: a butterfly of symmetric lane exchanges (quad permutes, the
// 8- and 16-lane mirrors, then the 16- and 32-lane row swaps).
__device__ __forceinline__ int group_sum(int x, int G) {
  if (G >= 2) x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);
  if (G >= 4) x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
  if (G >= 8) x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);
  if (G >= 16) x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);
  if (G >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    x = (int)(r[0] + r[1]);
  }
  if (G >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    x = (int)(r[0] + r[1]);
  }
  return x;
}

// Request owning global query i: largest b with cu_q[b] <= i (cu_q has B+1 entries).
__device__ __forceinline__ int find_request(const int32_t* cu, int B, int64_t i) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace msa
