// E4M3 quantisation and the paged cache write for gfx950: the step just before
// the path, where new tokens' keys and values enter the paged caches and the
// queries become E4M3 (vLLM PR 60684, Overview: a fused insert kernel writes the
// query in E4M3 and the new K|V into the packed cache pages; Details: the FP8
// cache is written with unit scales; the benchmark script and the MiniMax-M3
// forward pass give each token one int64 cache slot, slot_mapping).
//
// One kernel serves every case: a row is 128 consecutive source elements (one
// head of one token); 16 lanes take a row, 8 elements each (one 16- or 32-byte
// load, one 8-byte store), and each lane takes four rows with all loads in
// flight together, so a 256-thread block moves 64 rows.  A row's
// destination is either linear (queries) or page slot_mapping[t] / 128, row
// slot_mapping[t] % 128 of a paged cache; grid y selects one of up to two
// source/destination parts (K and V of the packed cache).  HBM-bound: bytes =
// rows * 128 * (source element size + 1) + 8 per token for the slot.
//
// Conversion: x / scale in fp32 (one correctly rounded division), NaN -> 0x7F,
// otherwise clamped to +-448 and converted by the hardware (v_cvt_pk_fp8_f32,
// round to nearest even, OCP E4M3).
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kGroups = kThreads / 16;           // 16-lane groups, one row each per round
constexpr int kRowsPerGroup = 4;                 // rounds: rows per group
constexpr int kRowsPerBlock = kGroups * kRowsPerGroup;

struct Part {
  const void* src;
  const float* scale;
  int64_t col_off;           // destination byte offset inside a row
  int64_t src_tok_stride;    // elements
};

struct QuantK {
  Part part[2];
  int dtype;                 // MSA_DTYPE_BF16 / MSA_DTYPE_F32
  int64_t n_tokens;
  int heads;
  int64_t src_head_stride;   // elements
  const int64_t* slots;      // nullptr: linear destination
  int64_t max_slot;          // num_pages * 128 (paged destination)
  uint8_t* dst;
  int64_t dst_tok_stride;    // bytes, linear destination
  int64_t dst_page_stride;   // bytes, paged destination
  int64_t dst_head_stride;   // bytes
  int64_t dst_row_stride;    // bytes between tokens of one page (paged)
};

// Source element e of a row as fp32 (bf16 widens exactly).
__device__ __forceinline__ void load8(int dtype, const void* src, int64_t src_off, float (&x)[8]) {
  if (dtype == MSA_DTYPE_BF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(src) + src_off);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else {
    const float* f = reinterpret_cast<const float*>(src) + src_off;
    const float4 u = *reinterpret_cast<const float4*>(f);
    const float4 v = *reinterpret_cast<const float4*>(f + 4);
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
  }
}

// Eight E4M3 codes of x / s: clamped to +-448 for the saturating conversion;
// NaN is set apart (the clamp would turn it into a number) and written as 0x7F.
// When s is a normal power of two (unit scales, the pages' FP8 cache), 1/s is
// exact and x * (1/s) is the same real number as x / s, rounded once the same
// way, so the multiply replaces the division sequence.
template <bool kPow2>
__device__ __forceinline__ uint2 encode8(const float (&x)[8], float s, float inv_s) {
  float y[8];
  uint32_t nan_mask = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float q = kPow2 ? x[e] * inv_s : x[e] / s;
    nan_mask |= (q != q) ? (1u << e) : 0u;
    y[e] = fminf(fmaxf(q, -448.f), 448.f);
  }
  uint32_t w[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * k], y[4 * k + 1], 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * k + 2], y[4 * k + 3], v, true);
    w[k] = (uint32_t)v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((nan_mask >> (4 * k + e)) & 1u) w[k] = (w[k] & ~(0xFFu << (8 * e))) | (0x7Fu << (8 * e));
  }
  return make_uint2(w[0], w[1]);
}

// Block b, 16-lane group g, round r: row (b * kRowsPerGroup + r) * 16 + g; all
// of a lane's loads are issued before its conversions and stores.
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(QuantK a) {
  const Part p = a.part[blockIdx.y];
  const int64_t n_rows = a.n_tokens * a.heads;
  const int g = threadIdx.x >> 4;
  const int c0 = (threadIdx.x & 15) * 8;             // first element of this lane
  int64_t dst_off[kRowsPerGroup];
  float x[kRowsPerGroup][8];
#pragma unroll
  for (int r = 0; r < kRowsPerGroup; ++r) {
    const int64_t row = ((int64_t)blockIdx.x * kRowsPerGroup + r) * kGroups + g;
    dst_off[r] = -1;
    if (row >= n_rows) continue;
    const int64_t t = row / a.heads;
    const int h = (int)(row - t * a.heads);
    int64_t off;
    if (a.slots) {
      const int64_t s = a.slots[t];
      if (s < 0 || s >= a.max_slot) continue;        // padding token (or out of range): skipped
      off = (s / kPage) * a.dst_page_stride + (s % kPage) * a.dst_row_stride;
    } else {
      off = t * a.dst_tok_stride;
    }
    dst_off[r] = off + h * a.dst_head_stride + p.col_off + c0;
    load8(a.dtype, p.src, t * p.src_tok_stride + h * a.src_head_stride + c0, x[r]);
  }
  const float s = *p.scale;
  const uint32_t sb = __float_as_uint(s);
  const uint32_t ex = (sb >> 23) & 0xFFu;
  if ((sb & 0x7FFFFFu) == 0u && ex != 0u && ex != 0xFFu) {   // +-2^k, normal
    const float inv_s = 1.0f / s;
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r)
      if (dst_off[r] >= 0) *reinterpret_cast<uint2*>(a.dst + dst_off[r]) = encode8<true>(x[r], s, inv_s);
  } else {
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r)
      if (dst_off[r] >= 0) *reinterpret_cast<uint2*>(a.dst + dst_off[r]) = encode8<false>(x[r], s, 0.f);
  }
}

// ---- MXFP4 index keys --------------------------------------------------------
// Row of 128 elements -> 4 blocks of 32 E2M1 codes sharing one E8M0 scale
// (OCP Microscaling conversion): exponent = floor(log2(max |x|)) - 2, clamped
// to [-127, 127] (-127 for a block of zeros); elements = nearest E2M1 of
// x * 2^-exponent, ties to the even code, saturating at 6.  A block holding NaN
// or an infinity gets scale 0xFF and zero elements.  A block is 4 lanes of the
// row's 16; each lane writes its 8 codes as 4 bytes (element 2i low nibble),
// the block's first lane its scale byte.
struct Mx4K {
  const void* src;
  int dtype;
  int64_t n_tokens;
  int64_t src_tok_stride;    // elements
  const int64_t* slots;
  int64_t max_slot;
  uint8_t* data;             // [num_pages, 128, 64]
  uint8_t* scales;           // [num_pages, 128, 4]
};

__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.f ? 6u : 7u;
  return c | (signbit(v) ? 8u : 0u);
}

__global__ __launch_bounds__(kThreads) void insert_mxfp4_kernel(Mx4K a) {
  const int g = threadIdx.x >> 4, l16 = threadIdx.x & 15;
  const int c0 = l16 * 8;
#pragma unroll
  for (int r = 0; r < kRowsPerGroup; ++r) {
    const int64_t t = ((int64_t)blockIdx.x * kRowsPerGroup + r) * kGroups + g;   // group-uniform
    if (t >= a.n_tokens) break;
    const int64_t s = a.slots[t];
    if (s < 0 || s >= a.max_slot) continue;          // padding token (or out of range): skipped
    float x[8];
    load8(a.dtype, a.src, t * a.src_tok_stride + c0, x);
    float amax = 0.f;
    bool bad = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bad |= !isfinite(x[e]);
      amax = fmaxf(amax, fabsf(x[e]));
    }
    // the block's 4 lanes (aligned within the 16-lane row)
#pragma unroll
    for (int m = 1; m < 4; m <<= 1) {
      amax = fmaxf(amax, __shfl_xor(amax, m));
      bad |= __shfl_xor((int)bad, m) != 0;
    }
    const int ex = amax == 0.f ? -127 : min(127, max(-127, ilogbf(amax) - 2));
    uint32_t w = 0;
    if (!bad) {
#pragma unroll
      for (int e = 0; e < 8; ++e) w |= e2m1_code(ldexpf(x[e], -ex)) << (4 * e);
    }
    // slot s is row s % 128 of page s / 128, i.e. row s of the [pages * 128] rows
    *reinterpret_cast<uint32_t*>(a.data + s * 64 + l16 * 4) = w;
    if ((l16 & 3) == 0) a.scales[s * 4 + (l16 >> 2)] = bad ? (uint8_t)0xFF : (uint8_t)(ex + 127);
  }
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& q, hipStream_t stream) {
  const int64_t n_rows = q.n_tokens * q.heads;
  if (n_rows == 0) return hipSuccess;
  QuantK k;
  for (int i = 0; i < 2; ++i) k.part[i] = Part{q.src[i], q.scale[i], q.col_off[i], q.src_tok_stride[i]};
  k.dtype = q.dtype;
  k.n_tokens = q.n_tokens;
  k.heads = q.heads;
  k.src_head_stride = q.src_head_stride;
  k.slots = q.slots;
  k.max_slot = q.max_slot;
  k.dst = q.dst;
  k.dst_tok_stride = q.dst_tok_stride;
  k.dst_page_stride = q.dst_page_stride;
  k.dst_head_stride = q.dst_head_stride;
  k.dst_row_stride = q.dst_row_stride;
  const dim3 grid((unsigned)ceil_div(n_rows, kRowsPerBlock), (unsigned)q.n_parts);
  hipLaunchKernelGGL(quantize_rows_kernel, grid, dim3(kThreads), 0, stream, k);
  return hipGetLastError();
}

hipError_t launch_insert_mxfp4(const Mx4Args& q, hipStream_t stream) {
  if (q.n_tokens == 0) return hipSuccess;
  Mx4K k{q.src, q.dtype, q.n_tokens, q.src_tok_stride, q.slots, q.max_slot, q.data, q.scales};
  const dim3 grid((unsigned)ceil_div(q.n_tokens, kRowsPerBlock));
  hipLaunchKernelGGL(insert_mxfp4_kernel, grid, dim3(kThreads), 0, stream, k);
  return hipGetLastError();
}

}  // namespace msa
