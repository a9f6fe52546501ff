// Block-sparse prefill attention over a paged E4M3 K|V cache, for gfx950.
//
// vLLM API docs, sparse_attention_msa, MiniMaxM3SparseMSAImpl.forward:
// sparse_atten_func(q, k, v, row_ptr, q_indices, topK=16, blk_kv=128,
// causal=True, softmax_scale, ..., page_table=block_table, schedule, out), with
// k, v = kv_cache.split(128, -1).  vLLM PR 60684 (Overview, Details): the
// query is E4M3, QK and PV products are FP8, softmax probabilities are rounded
// to E4M3, q_scale folds into the softmax scale, the K scale applies to the
// scores and the V scale to the output; per-split partials are merged by a
// combine.
//
// Page-major (k2q) design: a work item is (CSR row = one logical page of one
// request, up to 32 or 64 of the queries that selected it, one KV head).  The
// block stages the page's K (token-major) and V (transposed, d-major) in LDS
// once and every wave runs 16-row tiles of (query, q-head) rows against it:
//   S^T = K Q^T           8 MFMA 16x16x128 (tokens on M, rows on N)
//   softmax over the page's 128 tokens (causal mask only on a query's own page)
//   O^T = V^T P^T         8 MFMA, P^T packed to E4M3 straight from S^T's lanes
//   l   = 1^T P^T         1 MFMA against a constant all-ones operand
// Because S^T leaves each lane with tokens {16T + 4g + i} of one row, V^T is
// stored with its token axis permuted to the same order, so no shuffles are
// needed between the two products.  (A form that runs two tiles per fragment
// read is kept in the source, switched off.)  Blocks are persistent: while one
// item is computed, the next item's page and query list are already being
// fetched into registers.
//
// Each (query, q-head, page) split writes its unnormalised output row as int8
// codes with one power-of-two scale per 16 values, staged in LDS so that whole
// rows go out as 16-byte stores, with the pair (running max m in the log2
// domain, probability sum l) in the same 144-byte row.  Split rows are laid
// out query-major, (query, selection head, slot of the page in the query's
// selection, head), so the combine reads a query's (at most 16) splits as one
// contiguous run; a small pass before the partials maps every CSR position to
// its (query, selection head, slot) entry.
#include <type_traits>

#include <utility>

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowB = 144;          // LDS row stride (bytes)
// Blocks per CU: the wide kernel (items of many rows, two-tile sets) needs about
// 240 registers per lane; the narrow one (one-tile sets) fits three blocks.
constexpr int kBlocksWide = 2;
constexpr int kBlocksNarrow = 3;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kOnesE4M3 = 0x38383838;   // four E4M3 1.0 codes
constexpr int kMaxKvHeads = 64;         // selection heads per query, at most (Hq <= 64)

struct AttnK {
  const uint8_t* q;
  int64_t q_stride;
  int32_t G, n_sel, HP, GY;        // GY: KV heads per schedule item (Hkv if shared selection)
  uint32_t g_magic;                // ceil(2^20 / G): row / G == (row * g_magic) >> 20 for rows < 64 G
  const uint8_t* kv;               // E4M3 K|V rows, or MXFP4 K|V codes (kv_scales != nullptr)
  const uint8_t* kv_scales;        // MXFP4 E8M0 block scales [num_pages, Hkv, 128, 8], or nullptr
  int32_t num_pages, Hkv;
  const int32_t* q_indices;
  const int32_t* q_slot;           // [nnz]: (query, selection head, slot) entry of each CSR position
  const int4* items;
  const int32_t* perm;             // order in which the items are taken, or nullptr: list order
  const int32_t* n_items;
  float logit_scale_log2;          // softmax_scale * log2(e)
  const float* q_scale;
  const float* k_scale;
  uint8_t* part_o;                 // [entries * HP + 1] rows: int8 (144 B), or f12 (192 B) when chunked
  float2* part_ml;                 // chunked kernel: [entries * HP + 1] (max in log2 units, probability sum)
  int32_t trash;                   // partial row written by rows past an item's end
  uint32_t part_o_bytes, part_ml_bytes;   // chunked kernel: ring sizes (buffer-op bounds)
};

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int k) { return (w >> (8 * k)) & 0xFFu; }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two floats -> two bf16 (round to nearest even, gfx950 v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Compact partials ("f12"): a float rounded to fp16, then to the fp16's top 12
// bits (sign, 5 exponent and 6 mantissa bits) by adding half of the dropped
// range before dropping it: round to nearest, ties away from zero, relative
// error <= 2^-7.  Unnormalised split outputs stay below 128 * 448 = 57344,
// inside fp16's range, so the rounding never carries out of a half.  Eight
// values v0..v7 pack into three dwords: the high bytes of v0..v3, the high bytes
// of v4..v7, and the eight low nibbles (fp16 bits 7:4), placed so that packing
// and unpacking are byte permutes and masks.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t round_f16x2(float a, float b) {
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  return h + 0x00080008u;
}
__device__ __forceinline__ uint3 pack8_f12(float v0, float v1, float v2, float v3, float v4,
                                           float v5, float v6, float v7) {
  const uint32_t h01 = round_f16x2(v0, v1), h23 = round_f16x2(v2, v3);
  const uint32_t h45 = round_f16x2(v4, v5), h67 = round_f16x2(v6, v7);
  // v_perm_b32 selector bytes: 0-3 pick bytes of the second operand, 4-7 of the first
  const uint32_t hi0 = __builtin_amdgcn_perm(h23, h01, 0x07050301u);   // high bytes v0 v1 v2 v3
  const uint32_t hi1 = __builtin_amdgcn_perm(h67, h45, 0x07050301u);   // high bytes v4 v5 v6 v7
  // byte 0: v0 nibble | v2 nibble, byte 2: v1 | v3 (and v4..v7 likewise)
  const uint32_t n0 = (h01 & 0x00F000F0u) | ((h23 >> 4) & 0x000F000Fu);
  const uint32_t n1 = (h45 & 0x00F000F0u) | ((h67 >> 4) & 0x000F000Fu);
  return make_uint3(hi0, hi1, __builtin_amdgcn_perm(n1, n0, 0x06040200u));
}
__device__ __forceinline__ float2 f16x2_to_f32(uint32_t p) {
  const f32x2 f = __builtin_convertvector(__builtin_bit_cast(f16x2, p), f32x2);
  return make_float2(f[0], f[1]);
}
__device__ __forceinline__ void unpack8_f12(uint3 w, float (&v)[8]) {
  const uint32_t n = w.z, n4 = w.z << 4;      // n4: the low nibbles moved up
  const float2 a = f16x2_to_f32(__builtin_amdgcn_perm(w.x, n, 0x05010400u) & 0xFFF0FFF0u);
  const float2 b = f16x2_to_f32(__builtin_amdgcn_perm(w.x, n4, 0x07010600u) & 0xFFF0FFF0u);
  const float2 c = f16x2_to_f32(__builtin_amdgcn_perm(w.y, n, 0x05030402u) & 0xFFF0FFF0u);
  const float2 d = f16x2_to_f32(__builtin_amdgcn_perm(w.y, n4, 0x07030602u) & 0xFFF0FFF0u);
  v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
  v[4] = c.x; v[5] = c.y; v[6] = d.x; v[7] = d.y;
}
constexpr int kRowBytes = kDim * 3 / 2;   // 192 bytes per f12 partial row (chunked kernel)

// Block-scaled int8 partials (the split rows of the default kernels): each
// group of 16 values is stored as 8-bit integer codes with one power-of-two
// scale, as in the OCP Microscaling MXINT8 format (blocks of 16 here).  With
// e = floor(log2(max |x|)) - 6, the codes are the nearest integers of x 2^-e,
// saturated to [-128, 127], and a value decodes as code * 2^e: the error is at
// most 2^e <= max |x| / 64 for a saturated code and 2^(e-1) otherwise, i.e.
// within 1/127 of the group's largest magnitude.  e = -128 marks a group that
// held a NaN (it decodes as NaN); smaller scales than 2^-127 are not used.
// A row is 144 bytes: 128 codes (value j at byte j), the split's (max, sum)
// as two floats, and the 8 group exponents as signed bytes.
constexpr int kRowBytesI8 = kDim + 16;
constexpr int kI8Meta = kDim;             // byte offset of (max, sum, exponents)
__device__ __forceinline__ int quant16_i8(const float (&x)[16], uint4& q) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = __builtin_elementwise_maximum(amax, __builtin_fabsf(x[i]));
  const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  const int e = ex == 0xFF ? -128 : (ex - 133 < -127 ? -127 : ex - 133);
  const float sc = __uint_as_float((uint32_t)(127 - e) << 23);    // 2^-e (inf for the NaN mark)
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // x 2^-e + 128 lies in (0, 256); v_cvt_pk_u8_f32 rounds it to the nearest
    // integer (ties to even), saturates to [0, 255] and writes it as byte i of
    // the word; flipping bit 7 of each byte turns code + 128 into the
    // two's-complement code.  (The fma's own rounding is 2^-16 of a step.)
    uint32_t b = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) b = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(x[4 * k + i], sc, 128.f), i, b);
    w[k] = b ^ 0x80808080u;
  }
  q = make_uint4(w[0], w[1], w[2], w[3]);
  return e;
}
// 2^e for a group exponent byte (NaN for the NaN mark).
__device__ __forceinline__ float i8_scale(int e) {
  return e == -128 ? __builtin_nanf("") : __builtin_ldexpf(1.f, e);
}

// IEEE 754-2019 maximum (v_maximum_f32 / v_maximum3_f32): NaN-propagating, so
// unlike fmaxf it needs no quieting moves on operands the compiler cannot prove
// canonical (MFMA results, lane swaps).  A NaN score (a NaN code in q or K)
// spoils its row with either max.
__device__ __forceinline__ float fmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
__device__ __forceinline__ float max4_groups(float x) {   // max over lanes l, l^16, l^32, l^48
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// One work item as the kernel uses it (wave-uniform values).
struct Work {
  int start, count, g, lim_base, n_valid;
  int64_t kvp;                     // physical page * Hkv + KV head g: the page's K|V rows
};

__device__ __forceinline__ Work decode_work(const AttnK& a, int64_t w, int4 x, int4 y) {
  Work r;
  const int64_t item = w / a.GY;
  r.start = __builtin_amdgcn_readfirstlane(x.x);
  r.count = __builtin_amdgcn_readfirstlane(x.y);
  int phys = __builtin_amdgcn_readfirstlane(x.z);
  r.g = a.n_sel == 1 ? (int)(w - item * a.GY) : __builtin_amdgcn_readfirstlane(x.w);
  phys = (phys < 0 || phys >= a.num_pages) ? 0 : phys;
  r.kvp = (int64_t)phys * a.Hkv + r.g;
  r.lim_base = __builtin_amdgcn_readfirstlane(y.x);
  r.n_valid = min(__builtin_amdgcn_readfirstlane(y.y), kPage);
  return r;
}

// A page in flight: thread t holds 64 bytes of K (token t/2, half t%2) and the
// V bytes 16*(t%8).. of tokens 4*(t/8)..+3.
struct PageRegs {
  v4u k[4];
  v4u v[4];
  int qi;                          // q_indices[start + t] for t < count
  int sl;                          // q_slot[start + t]
};

__device__ __forceinline__ void fetch_page(PageRegs& r, const AttnK& a, const Work& w, int tid) {
  const uint8_t* page = a.kv + w.kvp * (kPage * 2 * kDim);
  const int t = tid >> 1, h = tid & 1;
  const v4u* ks = reinterpret_cast<const v4u*>(page + t * (2 * kDim) + h * 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) r.k[i] = ks[i];
  const int m = tid >> 3, dc = tid & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r.v[i] = *reinterpret_cast<const v4u*>(page + (4 * m + i) * (2 * kDim) + kDim + 16 * dc);
  r.qi = a.q_indices[w.start + min(tid, w.count - 1)];
  r.sl = a.q_slot[w.start + min(tid, w.count - 1)];
}

// An MXFP4 page in flight (the E4M3-staged reading of a 4-bit K|V page: every
// code times its block scale becomes an E4M3 value before the FP8 products).
// Rows are 128 code bytes (K elements in bytes 0..63, V in 64..127, element 2i
// in the low nibble of byte i) with 8 E8M0 scales (K blocks 0..3, V 4..7).
// Thread t holds the same K and V elements as PageRegs: K elements
// 64 (t%2) .. +63 of token t/2 (blocks 2 (t%2) and 2 (t%2) + 1), and V elements
// 16 (t%8) .. +15 (block (t%8)/2) of tokens 4 (t/8) .. +3.
struct PageRegs4 {
  v4u k[2];
  uint32_t ks;                     // the two K block scales, bytes 0 and 1
  uint2 v[4];
  uint32_t vs;                     // each token's V block scale, one byte per token
  int qi, sl;
};

__device__ __forceinline__ void fetch_page(PageRegs4& r, const AttnK& a, const Work& w, int tid) {
  const uint8_t* page = a.kv + w.kvp * (kPage * kDim);
  const uint8_t* sc = a.kv_scales + w.kvp * (kPage * 8);
  const int t = tid >> 1, h = tid & 1;
  const v4u* ks = reinterpret_cast<const v4u*>(page + t * kDim + h * 32);
  r.k[0] = ks[0];
  r.k[1] = ks[1];
  r.ks = *reinterpret_cast<const uint16_t*>(sc + t * 8 + 2 * h);
  const int m = tid >> 3, dc = tid & 7;
  uint32_t vs = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.v[i] = *reinterpret_cast<const uint2*>(page + (4 * m + i) * kDim + 64 + 8 * dc);
    vs |= (uint32_t)sc[(4 * m + i) * 8 + 4 + (dc >> 1)] << (8 * i);
  }
  r.vs = vs;
  r.qi = a.q_indices[w.start + min(tid, w.count - 1)];
  r.sl = a.q_slot[w.start + min(tid, w.count - 1)];
}

// E4M3 code of (1 + m3/8) * 2^(E - 7), m3 in {0, 4}: nearest, ties to even,
// saturating at 448.  Below the normal range the value is (8 + m3) * 2^(E - 1)
// units of the subnormal step 2^-9.
__device__ uint32_t e4m3_code(int E, int m3) {
  if (E >= 16) return 0x7Eu;
  if (E >= 1) return (uint32_t)((E << 3) | m3);        // E = 15 with m3 <= 4 stays <= 384
  const int sh = 1 - E;
  if (sh > 4) return 0u;                               // below half a step
  const int num = 8 + m3, q = num >> sh, rem = num & ((1 << sh) - 1), half = 1 << (sh - 1);
  return (uint32_t)(q + ((rem > half || (rem == half && (q & 1))) ? 1 : 0));
}

// The E4M3 codes of the E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 times
// 2^(s - 127), one byte each (magnitude k in byte k); the NaN scale 0xFF gives
// NaN codes.
__device__ uint2 staged_magnitudes(int s) {
  if (s == 0xFF) return make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
  const int e = s - 127;
  const uint32_t b1 = e4m3_code(e + 6, 0);                       // 0.5 = 2^-1
  const uint32_t b2 = e4m3_code(e + 7, 0), b3 = e4m3_code(e + 7, 4);   // 1, 1.5
  const uint32_t b4 = e4m3_code(e + 8, 0), b5 = e4m3_code(e + 8, 4);   // 2, 3
  const uint32_t b6 = e4m3_code(e + 9, 0), b7 = e4m3_code(e + 9, 4);   // 4, 6
  return make_uint2((b1 << 8) | (b2 << 16) | (b3 << 24), b4 | (b5 << 8) | (b6 << 16) | (b7 << 24));
}

// Eight codes (one dword, element 2k in the low nibble of byte k) to eight E4M3
// bytes through the block's magnitude table: byte permutes look the magnitudes
// up, the sign bits are ORed in, and the even and odd elements are interleaved.
__device__ __forceinline__ uint2 fp4x8_to_e4m3(uint32_t w, uint2 tab) {
  const uint32_t ev = __builtin_amdgcn_perm(tab.y, tab.x, w & 0x07070707u) | ((w & 0x08080808u) << 4);
  const uint32_t od = __builtin_amdgcn_perm(tab.y, tab.x, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
  return make_uint2(__builtin_amdgcn_perm(od, ev, 0x05010400u), __builtin_amdgcn_perm(od, ev, 0x07030602u));
}

__device__ __forceinline__ PageRegs to_e4m3(const PageRegs4& r, const uint2* s_tab) {
  PageRegs o;
#pragma unroll
  for (int b = 0; b < 2; ++b) {                        // K blocks: 16 code bytes -> 32 E4M3 bytes
    const uint2 tab = s_tab[(r.ks >> (8 * b)) & 0xFFu];
    const v4u c = r.k[b];
    const uint2 x0 = fp4x8_to_e4m3(c[0], tab), x1 = fp4x8_to_e4m3(c[1], tab);
    const uint2 x2 = fp4x8_to_e4m3(c[2], tab), x3 = fp4x8_to_e4m3(c[3], tab);
    o.k[2 * b] = v4u{x0.x, x0.y, x1.x, x1.y};
    o.k[2 * b + 1] = v4u{x2.x, x2.y, x3.x, x3.y};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {                        // V: 8 code bytes of token i -> 16 E4M3 bytes
    const uint2 tab = s_tab[(r.vs >> (8 * i)) & 0xFFu];
    const uint2 x0 = fp4x8_to_e4m3(r.v[i].x, tab), x1 = fp4x8_to_e4m3(r.v[i].y, tab);
    o.v[i] = v4u{x0.x, x0.y, x1.x, x1.y};
  }
  o.qi = r.qi;
  o.sl = r.sl;
  return o;
}

__device__ __forceinline__ void stage_page(const PageRegs& r, const Work& w, uint8_t* k_lds,
                                           uint8_t* vt_lds, int* s_qi, int tid) {
  {
    const int t = tid >> 1, h = tid & 1;
    v4u* dst = reinterpret_cast<v4u*>(k_lds + t * kRowB + h * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = r.k[i];
  }
  {
    // token group m = tokens 4m..4m+3 -> permuted positions 32*(m&3) + 4*(m>>2) + {0..3}.
    // Tokens past the end of the sequence hold no data (the page tail may be
    // anything, even NaN); their probability is exactly 0, so V is zeroed there
    // to keep 0 * V finite.
    const int m = tid >> 3, dc = tid & 7;
    const v4u zero = v4u{0u, 0u, 0u, 0u};
    const v4u v0 = (4 * m + 0 < w.n_valid) ? r.v[0] : zero;
    const v4u v1 = (4 * m + 1 < w.n_valid) ? r.v[1] : zero;
    const v4u v2 = (4 * m + 2 < w.n_valid) ? r.v[2] : zero;
    const v4u v3 = (4 * m + 3 < w.n_valid) ? r.v[3] : zero;
    const int kpos = 32 * (m & 3) + 4 * (m >> 2);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w0 = v0[e], w1 = v1[e], w2 = v2[e], w3 = v3[e];
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const uint32_t c = byte_of(w0, dd) | (byte_of(w1, dd) << 8) | (byte_of(w2, dd) << 16) |
                           (byte_of(w3, dd) << 24);
        const int d = 16 * dc + 4 * e + dd;
        *reinterpret_cast<uint32_t*>(vt_lds + d * kRowB + kpos) = c;
      }
    }
  }
  if (tid < kAttnQCMax) {
    s_qi[tid] = r.qi;
    s_qi[kAttnQCMax + tid] = r.sl;   // the entries' split slots follow their queries
  }
}

// The rows of NT consecutive 16-row tiles on one wave: lane (col, grp) of tile
// u holds row (tile0 + u) * 16 + col.  Rows past the item's end alias its first
// row for loading (their results go to the trash row), so every load and store
// below is unconditional and the compiler can count outstanding memory
// operations exactly instead of draining them.
template <int NT>
struct RowSet {
  v8i qb[NT];
  int lim[NT];
  int32_t pidx[NT];
};

template <int NT>
__device__ __forceinline__ RowSet<NT> load_rows(const AttnK& a, const Work& w, int tile0,
                                                int n_rows, const int* s_qi, int lane) {
  const int col = lane & 15, grp = lane >> 4;
  RowSet<NT> r;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int rid = (tile0 + u) * 16 + col;
    const bool valid = rid < n_rows;
    // branch-free: rows past the end are clamped after the division (exact for
    // rid < n_rows <= 64 G; past the end the product may wrap, unused)
    const int q0 = (int)(__umul24((uint32_t)rid, a.g_magic) >> 20);
    const int ql = valid ? q0 : 0;
    const int h = valid ? rid - q0 * a.G : 0;
    const int hq = w.g * a.G + h;
    const int qi = s_qi[ql];
    r.lim[u] = valid ? qi + w.lim_base : kPage;
    r.pidx[u] = valid ? s_qi[kAttnQCMax + ql] * a.HP + (a.n_sel == 1 ? hq : h) : a.trash;
    r.qb[u] = load_frag_global(a.q + (int64_t)qi * a.q_stride + hq * kDim + grp * 32);
  }
  return r;
}

// S^T, softmax and O^T of one row set, written to its partial rows.
// kWt: the split rows go out as write-through (device-coherent, sc1) buffer
// stores, readable by blocks on other dies once the writer has waited for them.
typedef unsigned v3u __attribute__((ext_vector_type(3)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
constexpr int kSc1 = 16;                  // buffer-op cache policy: device-scope coherence

template <int NT, bool kWt = false, bool kStage = true>
__device__ __forceinline__ void compute_set(const AttnK& a, const RowSet<NT>& r,
                                            const uint8_t* k_lds, const uint8_t* vt_lds,
                                            uint8_t* stage, float zscale, int lane) {
  const int col = lane & 15, grp = lane >> 4;
  // The page fragments are re-read from LDS for every set rather than kept
  // live across sets (128 registers); the laundered zero offset stops the
  // compiler from hoisting the reads out of the caller's loop (laundering the
  // pointers themselves would turn them into generic pointers).
  int zero = 0;
  asm volatile("" : "+v"(zero));
  k_lds += zero;
  vt_lds += zero;

  // S^T: every K fragment read from LDS feeds NT products
  v4f s[NT][8];
#pragma unroll
  for (int T = 0; T < 8; ++T) {
    const v8i ka = load_frag_lds(k_lds + (T * 16 + col) * kRowB + grp * 32);
#pragma unroll
    for (int u = 0; u < NT; ++u) s[u][T] = mfma_e4m3(ka, r.qb[u], v4f{0.f, 0.f, 0.f, 0.f});
  }

  // Only the rows of queries whose own page this is see a causal boundary.
  bool need_mask = false;
#pragma unroll
  for (int u = 0; u < NT; ++u) need_mask |= r.lim[u] < kPage - 1;
  const bool masked = __builtin_amdgcn_ballot_w64(need_mask) != 0;

  v8i pb[NT];
  float mz[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    if (masked) {
#pragma unroll
      for (int T = 0; T < 8; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = T * 16 + grp * 4 + i;
          s[u][T][i] = (t > r.lim[u]) ? -INFINITY : s[u][T][i];
        }
    }
    // IEEE maximum (v_maximum3_f32): unlike fmaxf it needs no quieting of the
    // MFMA results first; masked lanes are -inf, never NaN
    float mx = -INFINITY;
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      mx = fmax3(mx, s[u][T][0], s[u][T][1]);
      mx = fmax3(mx, s[u][T][2], s[u][T][3]);
    }
    mx = max4_groups(mx);
    // scales are positive, so the max of the raw products gives the max logit
    mz[u] = (mx == -INFINITY) ? 0.f : mx * zscale;
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u][T][0], zscale, -mz[u]));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u][T][1], zscale, -mz[u]));
      const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u][T][2], zscale, -mz[u]));
      const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u][T][3], zscale, -mz[u]));
      pb[u][T] = pack4_e4m3(p0, p1, p2, p3);
    }
  }

  // l = sum of the E4M3 probabilities (the same values the PV product uses)
  const v8i ones = v8i{kOnesE4M3, kOnesE4M3, kOnesE4M3, kOnesE4M3,
                       kOnesE4M3, kOnesE4M3, kOnesE4M3, kOnesE4M3};
  float l[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) l[u] = mfma_e4m3(ones, pb[u], v4f{0.f, 0.f, 0.f, 0.f})[0];

  uint32_t ex[NT] = {};              // unstaged rows: the lane's two group exponents
  // O^T = V^T P^T in two halves of 64 output dims.  Lane (row, group g) holds
  // d = 16 dt + 4 g + i; in the partial row those 32 values sit at
  // 32 g + 4 dt + i, so a half is 32 contiguous bytes (24 packed).  The packed
  // rows are staged in the wave's LDS area and then written out whole (below).
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    v4f o[NT][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const v8i va = load_frag_lds(vt_lds + ((half * 4 + k) * 16 + col) * kRowB + grp * 32);
#pragma unroll
      for (int u = 0; u < NT; ++u) o[u][k] = mfma_e4m3(va, pb[u], v4f{0.f, 0.f, 0.f, 0.f});
    }
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      if constexpr (kWt) {
        const uint3 p0 = pack8_f12(o[u][0][0], o[u][0][1], o[u][0][2], o[u][0][3], o[u][1][0],
                                   o[u][1][1], o[u][1][2], o[u][1][3]);
        const uint3 p1 = pack8_f12(o[u][2][0], o[u][2][1], o[u][2][2], o[u][2][3], o[u][3][0],
                                   o[u][3][1], o[u][3][2], o[u][3][3]);
        const auto rs = buffer_rsrc(a.part_o, a.part_o_bytes);
        const int off = r.pidx[u] * kRowBytes + grp * 48 + half * 24;
        __builtin_amdgcn_raw_buffer_store_b96(v3u{p0.x, p0.y, p0.z}, rs, off, 0, kSc1);
        __builtin_amdgcn_raw_buffer_store_b96(v3u{p1.x, p1.y, p1.z}, rs, off + 12, 0, kSc1);
      } else {
        // values 32 grp + 16 half + j (j = 4 k + i of o[u][k][i]) as one group
        const float x[16] = {o[u][0][0], o[u][0][1], o[u][0][2], o[u][0][3],
                             o[u][1][0], o[u][1][1], o[u][1][2], o[u][1][3],
                             o[u][2][0], o[u][2][1], o[u][2][2], o[u][2][3],
                             o[u][3][0], o[u][3][1], o[u][3][2], o[u][3][3]};
        uint4 q;
        const int e = quant16_i8(x, q);
        if constexpr (kStage) {
          uint8_t* row = stage + (u * 16 + col) * kRowBytesI8;
          *reinterpret_cast<uint4*>(row + grp * 32 + half * 16) = q;
          row[kI8Meta + 8 + 2 * grp + half] = (uint8_t)e;
        } else {
          *reinterpret_cast<uint4*>(a.part_o + (int64_t)r.pidx[u] * kRowBytesI8 + grp * 32 +
                                    half * 16) = q;
          ex[u] |= (uint32_t)(e & 0xFF) << (8 * half);
        }
      }
    }
  }
  if constexpr (kWt) {
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const auto rs = buffer_rsrc(a.part_ml, a.part_ml_bytes);
      __builtin_amdgcn_raw_buffer_store_b64(v2u{__float_as_uint(mz[u]), __float_as_uint(l[u])}, rs,
                                            r.pidx[u] * 8, 0, kSc1);
    }
  } else if constexpr (!kStage) {
    // each lane's two group exponents (its 16-bit piece of the row's 8), and
    // the row's (max, sum) from one lane of the row
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      uint8_t* row = a.part_o + (int64_t)r.pidx[u] * kRowBytesI8;
      *reinterpret_cast<uint16_t*>(row + kI8Meta + 8 + 2 * grp) = (uint16_t)ex[u];
      if (grp == 0) *reinterpret_cast<float2*>(row + kI8Meta) = make_float2(mz[u], l[u]);
    }
  } else {
    // the row's (max, sum) beside its codes (every lane of a row holds them)
#pragma unroll
    for (int u = 0; u < NT; ++u)
      if (grp == 0)
        *reinterpret_cast<float2*>(stage + (u * 16 + col) * kRowBytesI8 + kI8Meta) =
            make_float2(mz[u], l[u]);
    // Whole rows out as 16-byte stores, lane c of the 144 pieces of a tile
    // taking row c / 9, bytes 16 (c % 9): the rows of one query (its q-heads
    // of this KV head) are consecutive in the split buffer, so a store
    // instruction covers whole cache lines.  A wave's LDS operations complete
    // in order: only the compiler is held here.
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    constexpr int kPieces = 16 * kRowBytesI8 / 16;
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int k = 0; k < (kPieces + 63) / 64; ++k) {
        const int c = k * 64 + lane;
        const int row = c / 9, off = (c - row * 9) * 16;
        const int prow = __shfl(r.pidx[u], row & 15);    // lane `row` holds that row's index
        if (k * 64 + 64 <= kPieces || c < kPieces) {
          const uint4 v = *reinterpret_cast<const uint4*>(stage + (u * 16 + row) * kRowBytesI8 + off);
          *reinterpret_cast<uint4*>(a.part_o + (int64_t)prow * kRowBytesI8 + off) = v;
        }
      }
    asm volatile("" ::: "memory");                      // the next set's staging stays behind
  }
}

// All sets of one item on this wave.  Query rows are requested two sets ahead,
// and the first two sets' rows before `prefetch` issues the next item's loads:
// memory operations complete in issue order, so a wait for a row requested
// after the prefetch would also wait for the next page.
template <int NT, bool kWt = false, class Prefetch>
__device__ __forceinline__ void run_item(const AttnK& a, const Work& w, const uint8_t* k_lds,
                                         const uint8_t* vt_lds, uint8_t* stage, const int* s_qi,
                                         float zscale, int wave, int lane, Prefetch&& prefetch) {
  constexpr int kStep = NT * kWaves;
  const int n_rows = w.count * a.G;
  const int n_tiles = (n_rows + 15) >> 4;
  int t = NT * wave;
  // two row sets alternate roles (unrolled by two), so no loop-carried copy of
  // a loaded set forces an early wait for its loads
  RowSet<NT> ra = load_rows<NT>(a, w, t, n_rows, s_qi, lane);
  RowSet<NT> rb = load_rows<NT>(a, w, t + kStep, n_rows, s_qi, lane);
  __builtin_amdgcn_sched_barrier(0);        // keep the row loads ahead of the prefetch
  prefetch();
  __builtin_amdgcn_sched_barrier(0);
  for (;;) {
    if (t >= n_tiles) break;
    compute_set<NT, kWt>(a, ra, k_lds, vt_lds, stage, zscale, lane);
    ra = load_rows<NT>(a, w, t + 2 * kStep, n_rows, s_qi, lane);
    t += kStep;
    if (t >= n_tiles) break;
    compute_set<NT, kWt>(a, rb, k_lds, vt_lds, stage, zscale, lane);
    rb = load_rows<NT>(a, w, t + 2 * kStep, n_rows, s_qi, lane);
    t += kStep;
  }
}

// Items of a few rows: one-tile sets, rows requested one set ahead only (a wave
// rarely has a second set), which keeps the register count at three blocks per CU.
template <bool kStage, bool kPeel, class Prefetch>
__device__ __forceinline__ void run_item_narrow(const AttnK& a, const Work& w,
                                                const uint8_t* k_lds, const uint8_t* vt_lds,
                                                uint8_t* stage, const int* s_qi, float zscale,
                                                int wave, int lane, Prefetch&& prefetch) {
  const int n_rows = w.count * a.G;
  const int n_tiles = (n_rows + 15) >> 4;
  int t = wave;
  RowSet<1> r = load_rows<1>(a, w, t, n_rows, s_qi, lane);
  __builtin_amdgcn_sched_barrier(0);        // keep the row loads ahead of the prefetch
  prefetch();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kPeel) {
    // Items of one or two tiles: the first set is computed outside the loop.
    // On this path the compiler knows how many loads (the prefetch) follow its
    // rows and waits for the rows alone; at a loop header shared with the back
    // edge it would wait for every load in flight, i.e. for the next item's
    // page as well.  (Items of many tiles keep the loop: there the page wait
    // is spread over many sets, and a second copy of the set's code would
    // not fit the registers; nor does it with MXFP4 pages.)
    if (t >= n_tiles) return;
    compute_set<1, false, kStage>(a, r, k_lds, vt_lds, stage, zscale, lane);
    for (t += kWaves; t < n_tiles; t += kWaves) {
      r = load_rows<1>(a, w, t, n_rows, s_qi, lane);
      compute_set<1, false, kStage>(a, r, k_lds, vt_lds, stage, zscale, lane);
    }
  } else {
    while (t < n_tiles) {
      compute_set<1, false, kStage>(a, r, k_lds, vt_lds, stage, zscale, lane);
      t += kWaves;
      if (t >= n_tiles) break;
      r = load_rows<1>(a, w, t, n_rows, s_qi, lane);
    }
  }
}

// kFp4: MXFP4 K|V pages, turned into E4M3 while they are staged in LDS.
template <bool kWide, bool kFp4, bool kStage>
__global__ __launch_bounds__(kThreads, kWide ? kBlocksWide : kBlocksNarrow) void attn_partial_kernel(
    AttnK a) {
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kPage * kRowB];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[kDim * kRowB];
  __shared__ int s_qi[2 * kAttnQCMax];     // the item's queries, then their split slots
  __shared__ uint2 s_tab[kFp4 ? 256 : 1];  // E4M3 codes of the E2M1 magnitudes, per E8M0 scale
  constexpr int kStageTiles = kWide ? 2 : 1;   // 16-row tiles per set
  __shared__ __attribute__((aligned(16)))
  uint8_t s_stage[kStage || kWide ? kWaves * kStageTiles * 16 * kRowBytesI8 : 16];

  const int n_items = *a.n_items;
  const int64_t n_work = (int64_t)n_items * a.GY;
  int64_t w = blockIdx.x;
  if (w >= n_work) return;
  const int tid = threadIdx.x, lane = tid & 63;
  if constexpr (kFp4) {
    static_assert(kThreads == 256, "one magnitude table entry per thread");
    s_tab[tid] = staged_magnitudes(tid);   // read after the first barrier of the item loop
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: loops below do not diverge
  uint8_t* const stage = s_stage + wave * (kStageTiles * 16 * kRowBytesI8);   // the wave's staging rows
  const float zscale = a.logit_scale_log2 * (a.q_scale ? *a.q_scale : 1.f) *
                       (a.k_scale ? *a.k_scale : 1.f);
  // item of work index x (clamped to the last item, so the loads are always
  // valid), through the order table when there is one
  // (32-bit: item counts are checked against INT32_MAX, and a 64-bit index
  // would be sign-extended right after the table load, i.e. waited for there)
  auto item_of = [&](int64_t x) -> int {
    const int64_t it = x / a.GY;
    const int c = (int)(it < n_items - 1 ? it : (int64_t)(n_items - 1));
    if (a.perm) return a.perm[c];   // only long rows are ordered
    return c;
  };

  // prologue: the first item's page in registers, the second item's metadata in
  // flight, and the index of the item after that (an order-table lookup, when
  // there is one) known: a table lookup is made one work step before the
  // item's metadata is requested, so neither waits on a load issued after a
  // page fetch (memory operations complete in issue order).
  Work cur;
  typename std::conditional<kFp4, PageRegs4, PageRegs>::type pr;
  int4 mx, my;
  int i_nn;
  {
    const int i0 = item_of(w), i1 = item_of(w + gridDim.x);
    i_nn = item_of(w + 2 * (int64_t)gridDim.x);
    cur = decode_work(a, w, a.items[2 * i0], a.items[2 * i0 + 1]);
    mx = a.items[2 * i1];
    my = a.items[2 * i1 + 1];
    fetch_page(pr, a, cur, tid);
  }

  for (;;) {
    lds_barrier();                           // the previous item is done with LDS
    if constexpr (kFp4)
      stage_page(to_e4m3(pr, s_tab), cur, k_lds, vt_lds, s_qi, tid);
    else
      stage_page(pr, cur, k_lds, vt_lds, s_qi, tid);
    lds_barrier();
    const int64_t wn = w + gridDim.x;
    const bool has_next = wn < n_work;
    // past the last item the "next" item is the current one again: its loads
    // are issued all the same and their data is never used
    const Work nxt = has_next ? decode_work(a, wn, mx, my) : cur;
    auto prefetch = [&]() {
      fetch_page(pr, a, nxt, tid);
      mx = a.items[2 * i_nn];
      my = a.items[2 * i_nn + 1];
      i_nn = item_of(wn + 2 * (int64_t)gridDim.x);
    };
    const int n_tiles = (cur.count * a.G + 15) >> 4;
    if (!kWide)
      run_item_narrow<kStage, !kStage && !kFp4>(a, cur, k_lds, vt_lds, stage, s_qi, zscale, wave,
                                                lane, prefetch);
    else if (n_tiles >= 2 * kWaves)
      run_item<2>(a, cur, k_lds, vt_lds, stage, s_qi, zscale, wave, lane, prefetch);
    else
      run_item<1>(a, cur, k_lds, vt_lds, stage, s_qi, zscale, wave, lane, prefetch);
    if (!has_next) break;
    cur = nxt;
    w = wn;
  }
}

// Chunked attention only (the CSR build writes these otherwise).  Split slots
// of every CSR position, one thread per (query, selection head, slot): the
// position of (query i, slot s) is the first position of i's bitmap
// word in the slot's row plus the row's set bits below i in that word.  Writes
// q_slot[position] = (i * n_sel + head) * 16 + s for the first listing of each
// selected page, and per (query, selection head) the 16-bit mask of those slots,
// which the combine merges (the 16 slots of one (query, head) are 16
// consecutive lanes, so the mask is a slice of one ballot).
struct SlotK {
  int64_t n;                      // total_q * n_sel * 16
  int32_t n_sel;
  const int32_t* cu_q;
  int32_t batch;
  const int32_t* rowsel;          // [total_q, n_sel, 16] CSR row of each selected page, or -1
  const int32_t* wbase;           // [rows, words] CSR position of each bitmap word's first entry
  const uint32_t* bitmap;         // [rows, words] the rows' query-slot bitmaps
  int64_t words;
  int64_t max_pos;                // q_slot entries (positions at or past it are skipped)
  int32_t* q_slot;
  uint32_t* mask;                 // [total_q, n_sel]
  int32_t ring;                   // chunked kernel: entries go to ring slot (query chunk % ring)
};

constexpr int kRingSlots = 3;     // chunks whose split rows are live at once
constexpr int kChunkQ = 1 << kChunkShift;

// Split-row entry of (query i, selection head sel, slot s): query-major over the
// whole batch, or, in the chunked kernel, inside the ring slot of i's chunk.
__device__ __forceinline__ int64_t split_entry(int64_t i, int sel, int s, int n_sel, bool ring) {
  if (!ring) return (i * n_sel + sel) * kTopK + s;
  const int64_t slot = (i >> kChunkShift) % kRingSlots;
  return ((slot * kChunkQ + (i & (kChunkQ - 1))) * n_sel + sel) * kTopK + s;
}

__global__ __launch_bounds__(256) void attn_slot_kernel(SlotK a) {
  // entries number fewer than 2^31 (the call checks total_q * n_sel * 16)
  const int e = (int)blockIdx.x * 256 + (int)threadIdx.x;
  const int lane = threadIdx.x & 63;
  const bool in = e < a.n;
  const int s = e & (kTopK - 1);
  const int r = a.rowsel[in ? e : (int)a.n - 1];
  // a page listed twice counts at its first slot: the 16 slots of one (query,
  // selection head) are one 16-lane row, so the slots below s are the lanes
  // 1 .. s places down the row (row_shr; past the row start the old value, -2,
  // stays)
  bool ok = in && r >= 0 && first_in_row16(r);
  if (ok) {
    const int qs = e >> 4;                              // query * n_sel + head
    const int64_t i = a.n_sel == 1 ? qs : qs / a.n_sel;
    const int b = find_request(a.cu_q, a.batch, i);
    const int local = (int)(i - a.cu_q[b]);
    const int64_t wi = (int64_t)r * a.words + (local >> 5);
    const int64_t p = (int64_t)a.wbase[wi] + __popc(a.bitmap[wi] & ((1u << (local & 31)) - 1u));
    ok = p >= 0 && p < a.max_pos;
    if (ok)
      a.q_slot[p] = a.ring ? (int32_t)split_entry(i, qs - (int)i * a.n_sel, s, a.n_sel, true) : e;
  }
  const uint64_t bal = __builtin_amdgcn_ballot_w64(ok);
  if (in && s == 0) a.mask[e / kTopK] = (uint32_t)(bal >> (lane & ~(kTopK - 1))) & 0xFFFFu;
}

struct CombineK {
  int64_t total_q;
  int32_t Hq, G, n_sel, HP;
  const uint32_t* mask;           // [total_q, n_sel] slots holding a split
  const uint8_t* part_o;
  const float2* part_ml;
  const float* v_scale;
  uint16_t* out;
  int64_t out_stride;
};

// One block per query, Hq * 16 threads: thread t owns q-head t / 16 and the 8
// codes at 8 * (t % 16) of each split row, i.e. eight of the row's values, with
// the row's (max, sum) and group exponents (the split rows of one (query,
// selection head) are contiguous, slot-major, with the heads of each slot
// together).
__global__ __launch_bounds__(1024) void attn_combine_kernel(CombineK a) {
  const int64_t i = blockIdx.x;
  const int t = threadIdx.x;
  const int hq = t >> 4, c = t & 15;
  const int sel = a.n_sel == 1 ? 0 : hq / a.G;
  const int hp = a.n_sel == 1 ? hq : hq % a.G;
  const int64_t e0 = (i * a.n_sel + sel) * kTopK;
  const uint32_t m = a.mask[i * a.n_sel + sel];
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (m != 0u) {
    // all split rows are loaded together; a slot without a split reads the
    // first slot's (finite) row and gets weight 0
    const int first = __builtin_ctz(m);
    uint4 meta[kTopK];              // (max, sum, exponents 0..3, exponents 4..7)
    uint2 v[kTopK];
#pragma unroll
    for (int s = 0; s < kTopK; ++s) {
      const int64_t r = (e0 + (((m >> s) & 1u) ? s : first)) * a.HP + hp;
      meta[s] = *reinterpret_cast<const uint4*>(a.part_o + r * kRowBytesI8 + kI8Meta);
      v[s] = *reinterpret_cast<const uint2*>(a.part_o + r * kRowBytesI8 + 8 * c);
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kTopK; ++s)
      M = ((m >> s) & 1u) ? __builtin_elementwise_maximum(M, __uint_as_float(meta[s].x)) : M;
    float L = 0.f;
    const int eshift = 8 * ((c >> 1) & 3);   // this thread's group exponent: byte c / 2
#pragma unroll
    for (int s = 0; s < kTopK; ++s) {
      const float wgt = ((m >> s) & 1u) ? __builtin_amdgcn_exp2f(__uint_as_float(meta[s].x) - M) : 0.f;
      const uint32_t ew = (c >> 3) ? meta[s].w : meta[s].z;
      const float ws = wgt * i8_scale((int)(int8_t)(ew >> eshift));
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t word = k < 4 ? v[s].x : v[s].y;
        o[k] += ws * (float)(int8_t)(word >> (8 * (k & 3)));
      }
      L += wgt * __uint_as_float(meta[s].y);
    }
    const float f = L > 0.f ? (a.v_scale ? *a.v_scale : 1.f) / L : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] *= f;
  }
  uint16_t* dst = a.out + i * a.out_stride + hq * kDim + 32 * (c & 3) + 4 * (c >> 2);
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3]));
  *reinterpret_cast<uint2*>(dst + 16) = make_uint2(pack2_bf16(o[4], o[5]), pack2_bf16(o[6], o[7]));
}

// ---------------------------------------------------------------------------
// Chunked persistent attention (one long request).  Work items never cross a
// chunk of kChunkQ queries and are ordered by chunk.  The split rows of chunk c
// go to ring slot c % kRingSlots through write-through stores, so that the
// memory-side cache (256 MiB), not HBM, holds them until they are merged; the
// chunk's combine tasks run in the same kernel.  Tasks are dealt to kQueues
// queues (block b takes from queue b % kQueues, one atomic per task), each in
// the order
//   items(0), items(1), combine(0), items(2), combine(1), ..., combine(C - 1)
// (chunk c's items and combine tasks spread round robin over the queues).  A
// combine task of chunk c waits until all of c's items are done; an item of
// chunk c >= kRingSlots waits until chunk c - kRingSlots is merged (its ring
// slot is free).  Every wait is on tasks that precede the waiting one in every
// queue, so the kernel completes whatever subset of its blocks is resident.
// ---------------------------------------------------------------------------
constexpr int kQueues = 8;
constexpr int kCombQ = 16;                       // queries per combine task
constexpr int kCombPerChunk = kChunkQ / kCombQ;

struct QueueK {
  const int32_t* kstart;          // [chunks + 1] first perm position of each chunk's items
  int32_t n_chunks;
  int64_t total_q;
  int2* queues;                   // [kQueues, qcap] (perm position or -1 - combine task, chunk)
  int64_t qcap;
  int32_t* qlen;                  // [kQueues]
  int32_t* qhead;                 // [kQueues]
  int32_t* chunk_done;            // [chunks] items finished
  int32_t* comb_done;             // [chunks] combine tasks finished
  int32_t* give_up;               // set once a wait ran out (later waits then return at once)
};

__device__ __forceinline__ int comb_tasks(int64_t total_q, int c) {
  const int64_t q = min<int64_t>(kChunkQ, total_q - (int64_t)c * kChunkQ);
  return q > 0 ? (int)((q + kCombQ - 1) / kCombQ) : 0;
}
__device__ __forceinline__ int share(int n, int x) {   // members m < n with m % kQueues == x
  return n > x ? (n - x + kQueues - 1) / kQueues : 0;
}

__global__ __launch_bounds__(1024) void attn_queue_kernel(QueueK a) {
  __shared__ int s_wave[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int C = a.n_chunks;
  const int c = tid;                              // one chunk per thread (C <= 1024)
  const int n_c = c < C ? a.kstart[c + 1] - a.kstart[c] : 0;
  const int ct_prev = (c >= 1 && c < C) ? comb_tasks(a.total_q, c - 1) : 0;
  const int ct_last = (c == C - 1) ? comb_tasks(a.total_q, c) : 0;
  // the counters are cleared by write-through stores: they are then changed and
  // read only by device-scope atomics, from every die
  if (c < C) {
    __hip_atomic_store(a.chunk_done + c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.comb_done + c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid < kQueues) __hip_atomic_store(a.qhead + tid, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) __hip_atomic_store(a.give_up, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int x = 0; x < kQueues; ++x) {
    const int len = share(n_c, x) + share(ct_prev, x) + share(ct_last, x);
    const int incl = wave_inclusive_scan(len);
    __syncthreads();
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int off = incl - len;
    for (int w = 0; w < wave; ++w) off += s_wave[w];
    if (tid == 1023) a.qlen[x] = off + len;
    int2* q = a.queues + (int64_t)x * a.qcap + off;
    if (c < C) {
      int k = 0;
      for (int m = x; m < n_c; m += kQueues) q[k++] = make_int2(a.kstart[c] + m, c);
      for (int t = x; t < ct_prev; t += kQueues) q[k++] = make_int2(-1 - t, c - 1);
      for (int t = x; t < ct_last; t += kQueues) q[k++] = make_int2(-1 - t, c);
    }
  }
}

struct FusedK {
  AttnK a;
  const int32_t* kstart;
  const int2* queues;
  int64_t qcap;
  const int32_t* qlen;
  int32_t* qhead;
  int32_t* chunk_done;
  int32_t* comb_done;
  int32_t* give_up;
  int64_t total_q;
  int32_t Hq;
  const uint32_t* mask;
  const float* v_scale;
  uint16_t* out;
  int64_t out_stride;
};

// Wait until a device-scope counter reaches target, reading it by atomic
// read-modify-writes (adding 0), the same coherence path as its increments.
// The wait is bounded in time (s_memrealtime, 100 MHz) and in polls: past
// kWaitTicks or 2^18 polls the block goes on and sets give_up, after which every wait returns at once, so
// a broken schedule gives wrong results in a fraction of a second, never a hang.
constexpr uint64_t kWaitTicks = 20000000;        // 0.2 s
// Atomic add of 0 that stays an add: a literal 0 lets the compiler turn the
// read-modify-write into a plain load (an idempotent operation).
__device__ __forceinline__ int32_t rmw_read(int32_t* p) {
  int zero = 0;
  asm volatile("" : "+v"(zero));
  return __hip_atomic_fetch_add(p, zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_count(int32_t* c, int target, int32_t* give_up) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (int spin = 0;; ++spin) {
    if (rmw_read(c) >= target) return;
    if ((spin & 15) == 15) {
      if (rmw_read(give_up) != 0) return;
      if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks || spin >= (1 << 18)) {
        __hip_atomic_fetch_or(give_up, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

// Merge of queries [i0, i0 + n) of a chunk: as attn_combine_kernel, with the
// split rows read from the chunk's ring slot by device-coherent loads.
__device__ __forceinline__ void combine_task(const FusedK& f, int64_t i0, int n, int tid) {
  const AttnK& a = f.a;
  const auto ro = buffer_rsrc(a.part_o, a.part_o_bytes);
  const auto rm = buffer_rsrc(a.part_ml, a.part_ml_bytes);
  const int per_q = f.Hq * 16;
  for (int u = tid; u < n * per_q; u += kThreads) {
    const int ql = u / per_q, t = u - ql * per_q;
    const int64_t i = i0 + ql;
    const int hq = t >> 4, c = t & 15;
    const int sel = a.n_sel == 1 ? 0 : hq / a.G;
    const int hp = a.n_sel == 1 ? hq : hq % a.G;
    const uint32_t m = f.mask[i * a.n_sel + sel];
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (m != 0u) {
      const int first = __builtin_ctz(m);
      const int64_t e0 = split_entry(i, sel, 0, a.n_sel, true);
      float2 ml[kTopK];
      uint3 v[kTopK];
#pragma unroll
      for (int s = 0; s < kTopK; ++s) {
        const int r = (int)((e0 + (((m >> s) & 1u) ? s : first)) * a.HP + hp);
        const v2u x = __builtin_amdgcn_raw_buffer_load_b64(rm, r * 8, 0, kSc1);
        ml[s] = make_float2(__uint_as_float(x.x), __uint_as_float(x.y));
        const v3u y = __builtin_amdgcn_raw_buffer_load_b96(ro, r * kRowBytes + 12 * c, 0, kSc1);
        v[s] = make_uint3(y.x, y.y, y.z);
      }
      float M = -INFINITY;
#pragma unroll
      for (int s = 0; s < kTopK; ++s)
        M = ((m >> s) & 1u) ? __builtin_elementwise_maximum(M, ml[s].x) : M;
      float L = 0.f;
#pragma unroll
      for (int s = 0; s < kTopK; ++s) {
        const float wgt = ((m >> s) & 1u) ? __builtin_amdgcn_exp2f(ml[s].x - M) : 0.f;
        float x[8];
        unpack8_f12(v[s], x);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] += wgt * x[k];
        L += wgt * ml[s].y;
      }
      const float fs = L > 0.f ? (f.v_scale ? *f.v_scale : 1.f) / L : 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] *= fs;
    }
    uint16_t* dst = f.out + i * f.out_stride + hq * kDim + 32 * (c & 3) + 4 * (c >> 2);
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3]));
    *reinterpret_cast<uint2*>(dst + 16) = make_uint2(pack2_bf16(o[4], o[5]), pack2_bf16(o[6], o[7]));
  }
}

template <bool kFp4>
__global__ __launch_bounds__(kThreads, kBlocksWide) void attn_fused_kernel(FusedK f) {
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kPage * kRowB];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[kDim * kRowB];
  __shared__ int s_qi[2 * kAttnQCMax];
  __shared__ uint2 s_tab[kFp4 ? 256 : 1];
  __shared__ int2 s_task;
  const AttnK& a = f.a;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int queue = blockIdx.x % kQueues;
  const float zscale = a.logit_scale_log2 * (a.q_scale ? *a.q_scale : 1.f) *
                       (a.k_scale ? *a.k_scale : 1.f);
  if constexpr (kFp4) s_tab[tid] = staged_magnitudes(tid);
  typename std::conditional<kFp4, PageRegs4, PageRegs>::type pr;
  const int qlen = __builtin_amdgcn_readfirstlane(f.qlen[queue]);
  for (;;) {
    if (tid == 0) {
      const int t = atomicAdd(&f.qhead[queue], 1);
      s_task = t < qlen ? f.queues[(int64_t)queue * f.qcap + t] : make_int2(0, -1);
    }
    __syncthreads();
    // wave-uniform by construction; readfirstlane makes it so for the compiler
    // too, so every branch below (each holding barriers) is a scalar branch
    const int2 task = make_int2(__builtin_amdgcn_readfirstlane(s_task.x),
                                __builtin_amdgcn_readfirstlane(s_task.y));
    __syncthreads();                              // s_task is rewritten next round
    if (task.y < 0) break;
    const int chunk = task.y;
    if (task.x < 0) {                             // combine task
      if (tid == 0) wait_count(f.chunk_done + chunk, f.kstart[chunk + 1] - f.kstart[chunk], f.give_up);
      __syncthreads();
      const int64_t i0 = (int64_t)chunk * kChunkQ + (int64_t)(-1 - task.x) * kCombQ;
      combine_task(f, i0, (int)min<int64_t>(kCombQ, f.total_q - i0), tid);
      __syncthreads();                            // every load of the task has returned
      if (tid == 0) __hip_atomic_fetch_add(f.comb_done + chunk, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      continue;
    }
    // work item: the (page, queries) item at perm position task.x, every KV head
    const int item = __builtin_amdgcn_readfirstlane(a.perm[task.x]);
    const int4 mx = a.items[2 * item], my = a.items[2 * item + 1];
    if (chunk >= kRingSlots) {                    // the chunk's ring slot must be merged
      if (tid == 0)
        wait_count(f.comb_done + (chunk - kRingSlots), comb_tasks(f.total_q, chunk - kRingSlots),
                   f.give_up);
      __syncthreads();
    }
    Work cur = decode_work(a, (int64_t)item * a.GY, mx, my);
    fetch_page(pr, a, cur, tid);
    for (int g = 0; g < a.GY; ++g) {
      __syncthreads();                            // the previous head is done with LDS
      if constexpr (kFp4)
        stage_page(to_e4m3(pr, s_tab), cur, k_lds, vt_lds, s_qi, tid);
      else
        stage_page(pr, cur, k_lds, vt_lds, s_qi, tid);
      __syncthreads();
      const bool more = g + 1 < a.GY;
      const Work nxt = more ? decode_work(a, (int64_t)item * a.GY + g + 1, mx, my) : cur;
      auto prefetch = [&]() {
        if (more) fetch_page(pr, a, nxt, tid);
      };
      const int n_tiles = (cur.count * a.G + 15) >> 4;
      if (n_tiles >= 2 * kWaves)
        run_item<2, true>(a, cur, k_lds, vt_lds, nullptr, s_qi, zscale, wave, lane, prefetch);
      else
        run_item<1, true>(a, cur, k_lds, vt_lds, nullptr, s_qi, zscale, wave, lane, prefetch);
      cur = nxt;
    }
    // the item's split rows are written through before it counts as done
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) __hip_atomic_fetch_add(f.chunk_done + chunk, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev] = n;
  return n;
}

// Split rows: one per ((query, selection head, slot), head of that selection),
// plus one trash row.
static int64_t partial_rows(const msa_varlen_t* vl, int Hq, int n_sel, int topk) {
  return (int64_t)n_sel * vl->total_q * topk * (Hq / n_sel) + 1;
}

struct AttnWs {
  int64_t rows;                   // split rows (the last one is the trash row)
  int32_t fused, n_chunks;
  int64_t qcap;                   // chunked kernel: tasks per queue, at most
  size_t o, ml, slot, mask, queues, qlen, qhead, chunk_done, comb_done, give_up, total;
};
static AttnWs attn_ws(const msa_varlen_t* vl, int Hq, int n_sel, int topk) {
  const SchedLayout L = sched_layout(vl, n_sel, topk);
  const int64_t entries = (int64_t)n_sel * vl->total_q * topk;
  AttnWs w;
  w.fused = L.fused;
  w.n_chunks = L.fused ? L.order_keys : 0;
  // chunked: a ring of kRingSlots chunks of split rows; else every query's
  w.rows = L.fused ? (int64_t)std::min<int64_t>(kRingSlots, w.n_chunks) * kChunkQ * n_sel * topk *
                             (Hq / n_sel) + 1
                   : partial_rows(vl, Hq, n_sel, topk);
  w.qcap = L.fused ? ceil_div(L.max_items, kQueues) + 6 * (int64_t)w.n_chunks + 8 : 0;
  size_t off = 0;
  // f12 rows and a (max, sum) array in the chunked kernel; 144-byte int8 rows
  // that hold their (max, sum) otherwise
  w.o = off;    off += align_up((size_t)(w.rows * (L.fused ? kRowBytes : kRowBytesI8)), 256);
  w.ml = off;   off += L.fused ? align_up((size_t)(w.rows * sizeof(float2)), 256) : 256;
  // chunked: split slots and masks found by the slot kernel (the CSR build
  // writes them into the schedule otherwise)
  const int64_t slots = L.fused ? std::max<int64_t>(entries, 1) : 1;
  w.slot = off; off += align_up((size_t)(slots * sizeof(int32_t)), 256);
  w.mask = off; off += align_up((size_t)(std::max<int64_t>(slots / topk, 1) * sizeof(uint32_t)), 256);
  w.queues = off;     off += align_up((size_t)(kQueues * w.qcap * sizeof(int2)), 256);
  w.qlen = off;       off += 256;
  w.qhead = off;      off += 256;
  w.chunk_done = off; off += align_up((size_t)std::max(w.n_chunks, 1) * sizeof(int32_t), 256);
  w.comb_done = off;  off += align_up((size_t)std::max(w.n_chunks, 1) * sizeof(int32_t), 256);
  w.give_up = off;    off += 256;
  w.total = off;
  return w;
}

size_t attn_workspace_bytes(const msa_varlen_t* vl, int Hq, int Hkv, int n_sel, int topk) {
  (void)Hkv;
  return attn_ws(vl, Hq, n_sel, topk).total;
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.vl.total_q == 0) return hipSuccess;
  const SchedLayout& L = a.L;
  const AttnWs ws = attn_ws(&a.vl, a.Hq, a.n_sel, kTopK);
  const int64_t rows = ws.rows;
  if (rows > (int64_t)INT32_MAX) return hipErrorInvalidValue;   // split rows are indexed in 32 bits
  if (ws.fused && rows * kRowBytes > (int64_t)INT32_MAX) return hipErrorInvalidValue;   // buffer offsets
  uint8_t* wsb = reinterpret_cast<uint8_t*>(a.workspace);
  const int HP = a.Hq / a.n_sel;

  // split slot of each CSR position and the combine's masks: written by the
  // CSR build, or (chunked) by the slot kernel from its row table
  const int32_t* q_slot = reinterpret_cast<const int32_t*>(a.sched + L.qslot);
  const uint32_t* smask = reinterpret_cast<const uint32_t*>(a.sched + L.smask);
  SlotK sk;
  sk.n = (int64_t)a.vl.total_q * a.n_sel * kTopK;
  sk.n_sel = a.n_sel;
  sk.cu_q = a.vl.cu_seqlens_q;
  sk.batch = a.vl.batch;
  sk.rowsel = reinterpret_cast<const int32_t*>(a.sched + L.rowsel);
  sk.wbase = reinterpret_cast<const int32_t*>(a.sched + L.wbase);
  sk.bitmap = reinterpret_cast<const uint32_t*>(a.sched + L.bitmap);
  sk.words = L.words_per_row;
  sk.max_pos = L.inv_len;
  sk.q_slot = reinterpret_cast<int32_t*>(wsb + ws.slot);
  sk.mask = reinterpret_cast<uint32_t*>(wsb + ws.mask);
  sk.ring = ws.fused;
  if (ws.fused) {
    hipLaunchKernelGGL(attn_slot_kernel, dim3((unsigned)ceil_div(sk.n, 256)), dim3(256), 0, stream, sk);
    q_slot = sk.q_slot;
    smask = sk.mask;
  }

  AttnK k;
  k.q = a.q;
  k.q_stride = a.q_stride;
  k.G = a.Hq / a.Hkv;
  k.n_sel = a.n_sel;
  k.HP = HP;
  k.GY = a.n_sel == 1 ? a.Hkv : 1;
  k.g_magic = (uint32_t)(((1u << 20) + k.G - 1) / k.G);
  k.kv = a.kv;
  k.kv_scales = a.kv_scales;
  k.num_pages = a.num_pages;
  k.Hkv = a.Hkv;
  k.q_indices = a.q_indices;
  k.q_slot = q_slot;
  k.items = reinterpret_cast<const int4*>(a.sched + L.items);
  k.perm = L.order_shift > 0 ? reinterpret_cast<const int32_t*>(a.sched + L.perm) : nullptr;
  k.n_items = reinterpret_cast<const int32_t*>(a.sched + L.hdr);
  k.logit_scale_log2 = a.softmax_scale * kLog2e;
  k.q_scale = a.q_scale;
  k.k_scale = a.k_scale;
  k.part_o = wsb + ws.o;
  k.part_ml = reinterpret_cast<float2*>(wsb + ws.ml);
  k.trash = (int32_t)(rows - 1);
  k.part_o_bytes = (uint32_t)std::min<int64_t>(rows * kRowBytes, INT32_MAX);
  k.part_ml_bytes = (uint32_t)std::min<int64_t>(rows * (int64_t)sizeof(float2), INT32_MAX);
  if (ws.fused) {
    QueueK qk;
    qk.kstart = reinterpret_cast<const int32_t*>(a.sched + L.kstart);
    qk.n_chunks = ws.n_chunks;
    qk.total_q = a.vl.total_q;
    qk.queues = reinterpret_cast<int2*>(wsb + ws.queues);
    qk.qcap = ws.qcap;
    qk.qlen = reinterpret_cast<int32_t*>(wsb + ws.qlen);
    qk.qhead = reinterpret_cast<int32_t*>(wsb + ws.qhead);
    qk.chunk_done = reinterpret_cast<int32_t*>(wsb + ws.chunk_done);
    qk.comb_done = reinterpret_cast<int32_t*>(wsb + ws.comb_done);
    qk.give_up = reinterpret_cast<int32_t*>(wsb + ws.give_up);
    hipLaunchKernelGGL(attn_queue_kernel, dim3(1), dim3(1024), 0, stream, qk);
    FusedK f;
    f.a = k;
    f.kstart = qk.kstart;
    f.queues = qk.queues;
    f.qcap = qk.qcap;
    f.qlen = qk.qlen;
    f.qhead = qk.qhead;
    f.chunk_done = qk.chunk_done;
    f.comb_done = qk.comb_done;
    f.give_up = qk.give_up;
    f.total_q = a.vl.total_q;
    f.Hq = a.Hq;
    f.mask = sk.mask;
    f.v_scale = a.v_scale;
    f.out = a.out;
    f.out_stride = a.out_stride;
    const dim3 grid((unsigned)(device_cu_count() * kBlocksWide));
    if (a.kv_scales)
      hipLaunchKernelGGL((attn_fused_kernel<true>), grid, dim3(kThreads), 0, stream, f);
    else
      hipLaunchKernelGGL((attn_fused_kernel<false>), grid, dim3(kThreads), 0, stream, f);
    return hipGetLastError();
  }
  const int64_t max_work = L.max_items * k.GY;
  if (max_work > 0) {
    // Every batch takes the one-tile kernel at three blocks per CU: the
    // two-tile kernel (two blocks per CU, each K/V fragment read serving two
    // 16-row tiles) measured 1 to 5 % slower on items of many rows too, whose
    // time goes to the split rows' memory traffic rather than to LDS reads.
    const bool wide = false;
    const int per_cu = wide ? kBlocksWide : kBlocksNarrow;
    const int64_t grid = std::min<int64_t>(max_work, (int64_t)device_cu_count() * per_cu);
    const bool fp4 = a.kv_scales != nullptr;
    const bool stage = attn_stage_rows(&a.vl);
    const dim3 g((unsigned)grid), b(kThreads);
    if (wide && fp4)
      hipLaunchKernelGGL((attn_partial_kernel<true, true, true>), g, b, 0, stream, k);
    else if (wide)
      hipLaunchKernelGGL((attn_partial_kernel<true, false, true>), g, b, 0, stream, k);
    else if (fp4 && stage)
      hipLaunchKernelGGL((attn_partial_kernel<false, true, true>), g, b, 0, stream, k);
    else if (fp4)
      hipLaunchKernelGGL((attn_partial_kernel<false, true, false>), g, b, 0, stream, k);
    else if (stage)
      hipLaunchKernelGGL((attn_partial_kernel<false, false, true>), g, b, 0, stream, k);
    else
      hipLaunchKernelGGL((attn_partial_kernel<false, false, false>), g, b, 0, stream, k);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CombineK c;
  c.total_q = a.vl.total_q;
  c.Hq = a.Hq;
  c.G = a.Hq / a.Hkv;
  c.n_sel = a.n_sel;
  c.HP = HP;
  c.mask = smask;
  c.part_o = k.part_o;
  c.part_ml = k.part_ml;
  c.v_scale = a.v_scale;
  c.out = a.out;
  c.out_stride = a.out_stride;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)a.vl.total_q), dim3(a.Hq * 16), 0, stream,
                     c);
  return hipGetLastError();
}

}  // namespace msa
