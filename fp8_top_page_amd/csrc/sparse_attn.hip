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
// request, up to kAttnQC of the queries that selected it, one KV head).  The
// block stages the page's K (token-major) and V (transposed, d-major) in LDS
// once and every wave runs 16-row tiles of (query, q-head) rows against it:
//   S^T = K Q^T           8 MFMA 16x16x128 (tokens on M, rows on N)
//   softmax over the page's 128 tokens (causal mask on tokens > pos)
//   O^T = V^T P^T         8 MFMA, P^T packed to E4M3 straight from S^T's lanes
// Because S^T leaves each lane with tokens {16T + 4g + i} of one row, V^T is
// stored with its token axis permuted to the same order, so no shuffles are
// needed between the two products.  Each (query, q-head, page) split writes a
// normalised bf16 output row and its log2-sum-exp; the combine merges a
// query's (at most 16) splits in slot order.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kRowB = 144;          // LDS row stride (bytes)
constexpr float kLog2e = 1.4426950408889634f;

struct SchedHdr {
  int32_t n_items;
  int32_t nnz;
  int32_t pad[62];
};

struct AttnK {
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* block_table;
  int64_t bt_stride;
  int32_t batch;
  int32_t num_pages;
  int32_t total_rows;
  const uint8_t* q;
  int64_t q_stride;
  int32_t Hq, Hkv, G, n_sel, HP;
  const uint8_t* kv;
  const int32_t* row_base;
  const int32_t* row_ptr;
  const int32_t* q_indices;
  const int4* items;
  const int32_t* n_items;
  float logit_scale_log2;          // softmax_scale * log2(e)
  const float* q_scale;
  const float* k_scale;
  uint16_t* part_o;                // [nnz, HP, 128] bf16, normalised
  float* part_lse;                 // [nnz, HP] log2-sum-exp
};

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int k) { return (w >> (8 * k)) & 0xFFu; }

__global__ __launch_bounds__(kThreads, 4) void attn_partial_kernel(AttnK a) {
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kPage * kRowB];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[kDim * kRowB];

  const int item = blockIdx.x;
  if (item >= *a.n_items) return;
  // work item: {row, first entry, count, request} {page, cu_seqlens_q[b], context, seqlen_k}
  const int4 it = a.items[2 * item];
  const int4 it2 = a.items[2 * item + 1];
  const int row = it.x, start = it.y, count = it.z, b = it.w;
  const int j = it2.x, cq0 = it2.y, ctx = it2.z, sk = it2.w;
  if (count <= 0) return;
  const int g = (a.n_sel == 1) ? (int)blockIdx.y : row / a.total_rows;
  int phys = a.block_table[(int64_t)b * a.bt_stride + j];
  phys = (phys < 0 || phys >= a.num_pages) ? 0 : phys;
  const uint8_t* page = a.kv + ((int64_t)phys * a.Hkv + g) * (kPage * 2 * kDim);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int n_rows = count * a.G;
  const int n_tiles = (n_rows + 15) >> 4;

  // Row rid = (query ql of the item, head h): its query index, its last visible
  // token in this page, and its Q fragment (B operand).  The first tile's rows
  // are fetched before the page is staged so the two latencies overlap.
  struct TileRow {
    bool valid;
    int ql, hq, h, lim;
    v8i qb;
  };
  auto tile_row = [&](int tile) {
    TileRow r;
    const int rid = tile * 16 + col;
    r.valid = tile < n_tiles && rid < n_rows;
    r.ql = r.valid ? rid / a.G : 0;
    r.h = r.valid ? rid - r.ql * a.G : 0;
    r.hq = g * a.G + r.h;
    const int qi = r.valid ? a.q_indices[start + r.ql] : 0;
    r.lim = r.valid ? ctx + (qi - cq0) - j * kPage : -1;
    if (r.valid) r.qb = load_frag_global(a.q + (int64_t)qi * a.q_stride + r.hq * kDim + grp * 32);
    else r.qb = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    return r;
  };
  TileRow cur = tile_row(wave);

  // ---- stage K (token-major) and V^T (d-major, token axis permuted) in LDS
  {
    const int t = tid >> 1, h = tid & 1;
    const uint4* src = reinterpret_cast<const uint4*>(page + t * (2 * kDim) + h * 64);
    uint4 x0 = src[0], x1 = src[1], x2 = src[2], x3 = src[3];
    uint4* dst = reinterpret_cast<uint4*>(k_lds + t * kRowB + h * 64);
    dst[0] = x0; dst[1] = x1; dst[2] = x2; dst[3] = x3;
  }
  {
    // token group m = tokens 4m..4m+3 -> permuted positions 32*(m&3) + 4*(m>>2) + {0..3}.
    // Tokens past the end of the sequence hold no data (the page tail may be
    // anything, even NaN); their probability is exactly 0, so V is zeroed there
    // to keep 0 * V finite.
    const int n_valid = sk - j * kPage;
    const int m = tid >> 3, dc = tid & 7;
    uint4 r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = *reinterpret_cast<const uint4*>(page + (4 * m + i) * (2 * kDim) + kDim + 16 * dc);
      if (4 * m + i >= n_valid) r[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    const int kpos = 32 * (m & 3) + 4 * (m >> 2);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w0 = (&r[0].x)[e], w1 = (&r[1].x)[e], w2 = (&r[2].x)[e], w3 = (&r[3].x)[e];
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const uint32_t c = byte_of(w0, dd) | (byte_of(w1, dd) << 8) | (byte_of(w2, dd) << 16) |
                           (byte_of(w3, dd) << 24);
        const int d = 16 * dc + 4 * e + dd;
        *reinterpret_cast<uint32_t*>(vt_lds + d * kRowB + kpos) = c;
      }
    }
  }
  __syncthreads();

  const float qs = a.q_scale ? *a.q_scale : 1.f;
  const float ks = a.k_scale ? *a.k_scale : 1.f;
  const float zscale = a.logit_scale_log2 * qs * ks;
  for (int tile = wave; tile < n_tiles; tile += kThreads / 64) {
    // Re-read the page fragments from LDS for every tile instead of keeping all
    // 16 of them (128 registers) live across tiles: the launder stops the
    // compiler from hoisting the loads out of the loop.
    const uint8_t* k_base = k_lds;
    const uint8_t* v_base = vt_lds;
    asm volatile("" : "+v"(k_base), "+v"(v_base));
    const bool valid = cur.valid;
    const int ql = cur.ql, h = cur.h, hq = cur.hq, lim = cur.lim;
    const v8i qb = cur.qb;
    cur = tile_row(tile + kThreads / 64);   // next tile's rows, in flight meanwhile

    v4f s[8];
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      const v8i ka = load_frag_lds(k_base + (T * 16 + col) * kRowB + grp * 32);
      s[T] = mfma_e4m3(ka, qb, v4f{0.f, 0.f, 0.f, 0.f});
    }
    float mx = -INFINITY;
#pragma unroll
    for (int T = 0; T < 8; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = T * 16 + grp * 4 + i;
        float z = s[T][i] * zscale;
        z = (t > lim) ? -INFINITY : z;
        s[T][i] = z;
        mx = fmaxf(mx, z);
      }
    mx = max_across_groups(mx);
    const float mref = (mx == -INFINITY) ? 0.f : mx;
    float l = 0.f;
    v8i pb;
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      float p0 = __builtin_amdgcn_exp2f(s[T][0] - mref);
      float p1 = __builtin_amdgcn_exp2f(s[T][1] - mref);
      float p2 = __builtin_amdgcn_exp2f(s[T][2] - mref);
      float p3 = __builtin_amdgcn_exp2f(s[T][3] - mref);
      l += (p0 + p1) + (p2 + p3);
      pb[T] = pack4_e4m3(p0, p1, p2, p3);
    }
    l = sum_across_groups(l);

    // O^T = V^T P^T in two halves of 64 output dims, each stored as soon as it
    // is done (keeps the live accumulators to 16 registers).
    const int64_t pidx = (int64_t)(start + ql) * a.HP + (a.n_sel == 1 ? hq : h);
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
    uint16_t* dst = a.part_o + pidx * kDim + grp * 4;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      v4f o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int dt = half * 4 + k;
        const v8i va = load_frag_lds(v_base + (dt * 16 + col) * kRowB + grp * 32);
        o[k] = mfma_e4m3(va, pb, v4f{0.f, 0.f, 0.f, 0.f});
      }
      if (valid) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int dt = half * 4 + k;
          const uint32_t lo = (uint32_t)f32_to_bf16(o[k][0] * inv_l) |
                              ((uint32_t)f32_to_bf16(o[k][1] * inv_l) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16(o[k][2] * inv_l) |
                              ((uint32_t)f32_to_bf16(o[k][3] * inv_l) << 16);
          *reinterpret_cast<uint2*>(dst + dt * 16) = make_uint2(lo, hi);
        }
      }
    }
    if (valid) {
      if (grp == 0) a.part_lse[pidx] = (l > 0.f) ? mx + __log2f(l) : -INFINITY;
    }
  }
}

struct CombineK {
  int64_t total_q;
  int32_t Hq, G, n_sel, HP;
  const int32_t* inv;             // [total_q, n_sel, 16] CSR position or -1
  const uint16_t* part_o;
  const float* part_lse;
  const float* v_scale;
  uint16_t* out;
  int64_t out_stride;
};

// One block per query, Hq * 16 threads: thread t owns q-head t / 16 and output
// dims 8 * (t % 16) .. + 7, so each split row (all heads of one (query, page)
// pair, contiguous) is read with 16-byte loads.
__global__ __launch_bounds__(1024) void attn_combine_kernel(CombineK a) {
  const int64_t i = blockIdx.x;
  const int t = threadIdx.x;
  const int hq = t >> 4, d0 = (t & 15) * 8;
  const int sel = a.n_sel == 1 ? 0 : hq / a.G;
  const int hp = a.n_sel == 1 ? hq : hq % a.G;
  const int32_t* pos = a.inv + (i * a.n_sel + sel) * kTopK;
  int32_t pi[kTopK];
  float ls[kTopK];
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kTopK; ++s) {
    pi[s] = pos[s];
    ls[s] = pi[s] >= 0 ? a.part_lse[(int64_t)pi[s] * a.HP + hp] : -INFINITY;
    M = fmaxf(M, ls[s]);
  }
  // all 16 split rows are loaded together (a missing split reads row 0 with
  // weight 0) so their latencies overlap
  uint4 v[kTopK];
#pragma unroll
  for (int s = 0; s < kTopK; ++s)
    v[s] = *reinterpret_cast<const uint4*>(a.part_o + ((int64_t)max(pi[s], 0) * a.HP + hp) * kDim + d0);
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    float W = 0.f;
#pragma unroll
    for (int s = 0; s < kTopK; ++s) {
      const float w = (ls[s] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ls[s] - M);
      const uint32_t wv[4] = {v[s].x, v[s].y, v[s].z, v[s].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[2 * k] += w * bf16_to_f32((uint16_t)(wv[k] & 0xFFFFu));
        o[2 * k + 1] += w * bf16_to_f32((uint16_t)(wv[k] >> 16));
      }
      W += w;
    }
    const float f = (a.v_scale ? *a.v_scale : 1.f) / W;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] *= f;
  }
  uint4 packed;
  packed.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
  packed.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
  packed.z = (uint32_t)f32_to_bf16(o[4]) | ((uint32_t)f32_to_bf16(o[5]) << 16);
  packed.w = (uint32_t)f32_to_bf16(o[6]) | ((uint32_t)f32_to_bf16(o[7]) << 16);
  *reinterpret_cast<uint4*>(a.out + i * a.out_stride + hq * kDim + d0) = packed;
}

}  // namespace

size_t attn_workspace_bytes(const msa_varlen_t* vl, int Hq, int Hkv, int n_sel, int topk) {
  (void)Hkv;
  const int64_t nnz_max = (int64_t)n_sel * vl->total_q * topk;
  const int64_t hp = Hq / n_sel;
  return align_up((size_t)(nnz_max * hp * kDim * sizeof(uint16_t)), 256) +
         align_up((size_t)(nnz_max * hp * sizeof(float)), 256);
}

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.vl.total_q == 0) return hipSuccess;
  const SchedLayout& L = a.L;
  const int64_t nnz_max = (int64_t)a.n_sel * a.vl.total_q * kTopK;
  const int HP = a.Hq / a.n_sel;
  AttnK k;
  k.cu_q = a.vl.cu_seqlens_q;
  k.cu_k = a.vl.cu_seqlens_k;
  k.block_table = a.vl.block_table;
  k.bt_stride = a.vl.block_table_stride;
  k.batch = a.vl.batch;
  k.num_pages = a.num_pages;
  k.total_rows = a.vl.total_rows;
  k.q = a.q;
  k.q_stride = a.q_stride;
  k.Hq = a.Hq;
  k.Hkv = a.Hkv;
  k.G = a.Hq / a.Hkv;
  k.n_sel = a.n_sel;
  k.HP = HP;
  k.kv = a.kv;
  k.row_base = reinterpret_cast<const int32_t*>(a.sched + L.row_base);
  k.row_ptr = a.row_ptr;
  k.q_indices = a.q_indices;
  k.items = reinterpret_cast<const int4*>(a.sched + L.items);
  k.n_items = reinterpret_cast<const int32_t*>(a.sched + L.hdr);
  k.logit_scale_log2 = a.softmax_scale * kLog2e;
  k.q_scale = a.q_scale;
  k.k_scale = a.k_scale;
  k.part_o = reinterpret_cast<uint16_t*>(a.workspace);
  k.part_lse = reinterpret_cast<float*>(
      reinterpret_cast<uint8_t*>(a.workspace) +
      align_up((size_t)(nnz_max * HP * kDim * sizeof(uint16_t)), 256));
  if (L.max_items > 0) {
    dim3 grid((unsigned)L.max_items, a.n_sel == 1 ? a.Hkv : 1);
    hipLaunchKernelGGL(attn_partial_kernel, grid, dim3(kThreads), 0, stream, k);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  CombineK c;
  c.total_q = a.vl.total_q;
  c.Hq = a.Hq;
  c.G = a.Hq / a.Hkv;
  c.n_sel = a.n_sel;
  c.HP = HP;
  c.inv = reinterpret_cast<const int32_t*>(a.sched + L.inv);
  c.part_o = k.part_o;
  c.part_lse = k.part_lse;
  c.v_scale = a.v_scale;
  c.out = a.out;
  c.out_stride = a.out_stride;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)a.vl.total_q), dim3(a.Hq * 16), 0, stream,
                     c);
  return hipGetLastError();
}

}  // namespace msa
