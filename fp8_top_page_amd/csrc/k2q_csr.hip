// KV-page -> query CSR and the attention work list for gfx950.
//
// Transposes each query's selected pages into rows of (request, logical page)
// listing the queries that chose them, ascending (vLLM API docs,
// sparse_attention_msa, MiniMaxM3SparseMSAImpl.forward: build_k2q_csr(topk,
// cu_seqlens_q, cu_seqlens_k, 128, ..., total_rows=total_kv_blocks, ...,
// return_schedule=True) returns row_ptr, q_indices and a schedule).
//
// Deterministic without sorting: every row owns a bitmap over its request's
// query slots, walked in order, so each row comes out ascending.  A row's bitmap
// is cut into units of 64 words (2048 query slots); units are the grain of the
// count, scan and fill passes, so long rows (a page chosen by thousands of
// queries) are spread over many waves.
//
// Three launches on the caller's stream, no host sync:
//   words  -- one block per (request, 32 query slots): sets the bits of those
//             slots for every row of the request in LDS and writes the word
//             column out (so the bitmap needs no clearing and no global
//             atomics); also row_base[b] (page rows of earlier requests) and
//             the (query, slot) -> CSR row table (-1 for empty slots)
//   count  -- one wave per unit: entries and attention items of the unit, and
//             per-block totals
//   fill   -- per block: base offsets from the totals of earlier blocks, scan of
//             its units, then one wave per unit (one lane per bitmap word)
//             writes q_indices (ascending), each word's first CSR position,
//             row_ptr and the work items of at most kAttnQC entries each:
//               {first entry, count, physical page, selection head}
//               {context - cu_seqlens_q[b] - 128 j, valid tokens of the page, row, request}
//             (a query i of the item sees the page's tokens up to i + the first
//             value; the physical page comes from the block table)
// The CSR position of (query i, slot s) is then the first position of i's word
// in its row plus the set bits below i in that word; the attention's combine
// computes it from the row table, the word positions and the bitmap.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kUnitWords = 64;                 // bitmap words per unit (one per lane)
constexpr int kUnitsPerBlock = 4;              // units per count/fill block (one per wave)
constexpr int kUnitsPerWave = kUnitsPerBlock / (256 / 64);
constexpr int kThreads = 256;

struct Hdr {
  int32_t n_items;
  int32_t nnz;
  int32_t pad[62];
};

constexpr int kWordRows = 1024;               // rows per words-kernel block

struct WordsK {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch;
  const int32_t* topk;
  int64_t tq, th;
  int32_t n_sel;
  int32_t total_rows;
  int32_t* row_base;
  uint32_t* bitmap;
  int64_t words;          // per row
  int32_t* rowsel;        // [total_q, n_sel, 16]: CSR row of each selected page, or -1
  int32_t n_chunks;       // blocks per (request, word): ceil(n_sel * max_pages / kWordRows)
};

__device__ __forceinline__ int request_pages(const int32_t* cu_k, int b) {
  return (cu_k[b + 1] - cu_k[b] + kPage - 1) / kPage;
}

// Block ((b * words) + w) * n_chunks + c: query slots 32w .. 32w+31 of request b,
// rows c * kWordRows .. of the request (g-major: r = g * pages + j).
__global__ __launch_bounds__(kThreads) void csr_words_kernel(WordsK a) {
  __shared__ uint32_t s_bits[kWordRows];
  __shared__ int s_red[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bw = blockIdx.x / a.n_chunks;
  const int c = (int)(blockIdx.x % a.n_chunks);
  const int b = (int)(bw / a.words), w = (int)(bw % a.words);
  const int pages = request_pages(a.cu_k, b);
  const int rows = a.n_sel * pages;
  const int r0 = c * kWordRows;
  if (r0 >= rows && c > 0) return;

  // rows of earlier requests
  int part = 0;
  for (int k = tid; k < b; k += kThreads) part += request_pages(a.cu_k, k);
  part = wave_sum(part);
  if (lane == 0) s_red[wave] = part;
  __syncthreads();
  int base = 0;
  for (int k = 0; k < kThreads / 64; ++k) base += s_red[k];

  const int q0 = a.cu_q[b], sq = a.cu_q[b + 1] - q0;
  const int per_q = a.n_sel * kTopK;
  const int n_e = 32 * per_q;                       // (query, selection head, slot) entries
  if (c == 0) {
    if (w == 0 && tid == 0) {
      a.row_base[b] = base;
      if (b == a.batch - 1) a.row_base[a.batch] = base + pages;
    }
    // the CSR row of every selection slot of this block's queries
    for (int e = tid; e < n_e; e += kThreads) {
      const int local = 32 * w + e / per_q;
      if (local >= sq) continue;
      const int g = (e % per_q) / kTopK, sl = e % kTopK;
      const int j = a.topk[(int64_t)(q0 + local) * a.tq + (int64_t)g * a.th + sl];
      a.rowsel[(int64_t)(q0 + local) * per_q + e % per_q] =
          (j < 0 || j >= pages) ? -1 : g * a.total_rows + base + j;
    }
    // the last request's blocks also clear any rows past the requests' pages
    if (b == a.batch - 1) {
      const int end = base + pages;
      for (int g = 0; g < a.n_sel; ++g)
        for (int rr = end + tid; rr < a.total_rows; rr += kThreads)
          a.bitmap[((int64_t)g * a.total_rows + rr) * a.words + w] = 0u;
    }
  }
  const int n_r = min(kWordRows, rows - r0);
  if (n_r <= 0) return;
  for (int k = tid; k < n_r; k += kThreads) s_bits[k] = 0u;
  __syncthreads();
  for (int e = tid; e < n_e; e += kThreads) {
    const int ql = e / per_q, g = (e % per_q) / kTopK, sl = e % kTopK;
    const int local = 32 * w + ql;
    if (local >= sq) continue;
    const int j = a.topk[(int64_t)(q0 + local) * a.tq + (int64_t)g * a.th + sl];
    if (j < 0 || j >= pages) continue;
    const int r = g * pages + j - r0;
    if (r >= 0 && r < n_r) atomicOr(&s_bits[r], 1u << ql);
  }
  __syncthreads();
  for (int k = tid; k < n_r; k += kThreads) {
    const int r = r0 + k, g = r / pages, j = r - g * pages;
    a.bitmap[((int64_t)g * a.total_rows + base + j) * a.words + w] = s_bits[k];
  }
}

struct CountK {
  const uint32_t* bitmap;
  int64_t words;          // per row
  int32_t units_per_row;
  int64_t n_units;
  int32_t* unit_cnt;
  int32_t* blk_tot;       // [n_blocks]: entries
  int32_t* blk_items;     // [n_blocks]: attention items
};

__device__ __forceinline__ int unit_popcount(const uint32_t* bitmap, int64_t words, int upr,
                                             int64_t u, int lane, uint32_t* bits_out) {
  const int64_t row = u / upr;
  const int64_t w = (u % upr) * kUnitWords + lane;
  const uint32_t bits = w < words ? bitmap[row * words + w] : 0u;
  *bits_out = bits;
  return __popc(bits);
}

__global__ __launch_bounds__(kThreads) void csr_count_kernel(CountK a) {
  __shared__ int s_tot[kThreads / 64], s_it[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t u0 = (int64_t)blockIdx.x * kUnitsPerBlock + wave * kUnitsPerWave;
  uint32_t bits[kUnitsPerWave];
#pragma unroll
  for (int k = 0; k < kUnitsPerWave; ++k) {   // all loads in flight together
    const int64_t u = u0 + k;
    bits[k] = 0u;
    if (u < a.n_units) unit_popcount(a.bitmap, a.words, a.units_per_row, u, lane, &bits[k]);
  }
  int tot = 0, its = 0;
#pragma unroll
  for (int k = 0; k < kUnitsPerWave; ++k) {
    const int64_t u = u0 + k;
    const int c = wave_sum(__popc(bits[k]));
    if (u < a.n_units && lane == 0) a.unit_cnt[u] = c;
    tot += c;
    its += (c + kAttnQC - 1) / kAttnQC;
  }
  if (lane == 0) { s_tot[wave] = tot; s_it[wave] = its; }
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0, i = 0;
    for (int w = 0; w < kThreads / 64; ++w) { t += s_tot[w]; i += s_it[w]; }
    a.blk_tot[blockIdx.x] = t;
    a.blk_items[blockIdx.x] = i;
  }
}

struct FillK {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch;
  const int32_t* block_table;
  int64_t bt_stride;
  const int32_t* topk;
  int64_t tq, th;
  int32_t n_sel;
  int32_t total_rows;
  const int32_t* row_base;
  const uint32_t* bitmap;
  int64_t words;
  int32_t units_per_row;
  int64_t n_units;
  int64_t n_rows;
  int32_t n_blocks;
  const int32_t* unit_cnt;
  const int32_t* blk_tot;
  const int32_t* blk_items;
  int32_t* row_ptr;
  int32_t* q_indices;
  int32_t* wbase;      // [n_rows, words]: CSR position of each word's first entry
  int4* items;
  int64_t max_items;
  Hdr* hdr;
};

__global__ __launch_bounds__(kThreads) void csr_fill_kernel(FillK a) {
  __shared__ int s_red[2][kThreads / 64];
  __shared__ int s_pos[kUnitsPerBlock];     // first CSR position of each unit
  __shared__ int s_item[kUnitsPerBlock];    // first item index of each unit
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blk = blockIdx.x;
  const int64_t u0 = (int64_t)blk * kUnitsPerBlock;

  // entries and items of all earlier blocks
  int base_e = 0, base_i = 0;
  for (int j = tid; j < blk; j += kThreads) {
    base_e += a.blk_tot[j];
    base_i += a.blk_items[j];
  }
  base_e = wave_sum(base_e);
  base_i = wave_sum(base_i);
  if (lane == 0) { s_red[0][wave] = base_e; s_red[1][wave] = base_i; }
  __syncthreads();
  base_e = 0;
  base_i = 0;
  for (int w = 0; w < kThreads / 64; ++w) { base_e += s_red[0][w]; base_i += s_red[1][w]; }

  // scan of this block's units (one lane per unit)
  static_assert(kUnitsPerBlock <= 64, "one lane per unit in the block scan");
  if (wave == 0) {
    const int64_t u = u0 + lane;
    const bool mine = lane < kUnitsPerBlock && u < a.n_units;
    const int c = mine ? a.unit_cnt[u] : 0;
    const int it = (c + kAttnQC - 1) / kAttnQC;
    const int ie = wave_inclusive_scan(c);
    const int ii = wave_inclusive_scan(it);
    if (lane < kUnitsPerBlock) {
      s_pos[lane] = base_e + ie - c;
      s_item[lane] = base_i + ii - it;
    }
    if (mine && u % a.units_per_row == 0) a.row_ptr[u / a.units_per_row] = base_e + ie - c;
    if (blk == a.n_blocks - 1 && lane == 63) {
      a.row_ptr[a.n_rows] = base_e + ie;
      a.hdr->nnz = base_e + ie;
      a.hdr->n_items = (int)min<int64_t>(base_i + ii, a.max_items);
    }
  }
  __syncthreads();

  uint32_t ubits[kUnitsPerWave];
#pragma unroll
  for (int k = 0; k < kUnitsPerWave; ++k) {   // all loads in flight together
    const int64_t u = u0 + wave * kUnitsPerWave + k;
    ubits[k] = 0u;
    if (u < a.n_units) unit_popcount(a.bitmap, a.words, a.units_per_row, u, lane, &ubits[k]);
  }
#pragma unroll
  for (int k = 0; k < kUnitsPerWave; ++k) {
    const int ku = wave * kUnitsPerWave + k;
    const int64_t u = u0 + ku;
    if (u >= a.n_units) break;
    const int64_t row = u / a.units_per_row;
    const int g = (int)(row / a.total_rows);
    const int64_t rr = row % a.total_rows;
    const int b = find_request(a.row_base, a.batch, rr);
    const int j = (int)(rr - a.row_base[b]);
    const int64_t q_base = a.cu_q[b] + (u % a.units_per_row) * (kUnitWords * 32);
    const int sk = a.cu_k[b + 1] - a.cu_k[b];
    const int ctx = sk - (a.cu_q[b + 1] - a.cu_q[b]);
    // One lane per bitmap word: the word's first CSR position is the unit's
    // plus the bits of earlier words; the lane then writes the word's entries
    // in bit order (a wave-uniform loop as long as any lane has bits left).
    const uint32_t bits = ubits[k];
    const int c = __popc(bits);
    const int incl = wave_inclusive_scan(c);
    const int n = __shfl(incl, 63);
    int pos = s_pos[ku] + incl - c;
    const int64_t wi = row * a.words + (u % a.units_per_row) * kUnitWords + lane;
    if ((u % a.units_per_row) * kUnitWords + lane < a.words) a.wbase[wi] = pos;
    uint32_t x = bits;
    const int64_t q_word = q_base + lane * 32;
    while (__builtin_amdgcn_ballot_w64(x != 0u) != 0) {
      if (x != 0u) {
        a.q_indices[pos++] = (int32_t)(q_word + __builtin_ctz(x));
        x &= x - 1u;
      }
    }
    // work items of the unit: (row, first entry, count)
    const int n_it = (n + kAttnQC - 1) / kAttnQC;
    const int phys = n_it > 0 ? a.block_table[(int64_t)b * a.bt_stride + j] : 0;
    for (int t = lane; t < n_it; t += 64) {
      const int64_t idx = (int64_t)s_item[ku] + t;
      if (idx < a.max_items) {
        a.items[2 * idx] = make_int4(s_pos[ku] + t * kAttnQC, min(kAttnQC, n - t * kAttnQC), phys, g);
        a.items[2 * idx + 1] = make_int4(ctx - a.cu_q[b] - j * kPage, sk - j * kPage, (int)row, b);
      }
    }
  }
}

}  // namespace

SchedLayout sched_layout(const msa_varlen_t* vl, int n_sel, int topk) {
  SchedLayout L;
  L.n_rows = (int64_t)n_sel * vl->total_rows;
  L.words_per_row = std::max<int64_t>(1, ceil_div(std::max(vl->max_seqlen_q, 1), 32));
  L.units_per_row = ceil_div(L.words_per_row, kUnitWords);
  L.n_units = L.n_rows * L.units_per_row;
  L.n_blocks = std::max<int64_t>(1, ceil_div(L.n_units, kUnitsPerBlock));
  L.inv_len = (int64_t)vl->total_q * n_sel * topk;
  L.word_chunks = std::max<int64_t>(1, ceil_div((int64_t)n_sel * std::max(vl->max_pages, 1), kWordRows));
  L.word_blocks = L.words_per_row * std::max(vl->batch, 0) * L.word_chunks;
  // every unit holding c entries yields ceil(c / kAttnQC) items
  L.max_items = ceil_div((int64_t)n_sel * vl->total_q * topk, kAttnQC) + L.n_units;
  size_t off = 0;
  L.hdr = off;        off += sizeof(Hdr);
  L.row_base = off;   off += align_up(sizeof(int32_t) * (vl->batch + 1), 256);
  L.unit_cnt = off;   off += align_up(sizeof(int32_t) * std::max<int64_t>(1, L.n_units), 256);
  L.blk_tot = off;    off += align_up(sizeof(int32_t) * 2 * L.n_blocks, 256);
  L.items = off;      off += align_up(2 * sizeof(int4) * std::max<int64_t>(1, L.max_items), 256);
  L.rowsel = off;     off += align_up(sizeof(int32_t) * std::max<int64_t>(1, L.inv_len), 256);
  L.wbase = off;      off += align_up(sizeof(int32_t) * L.n_rows * L.words_per_row, 256);
  L.bitmap = off;     off += align_up(sizeof(uint32_t) * L.n_rows * L.words_per_row, 256);
  L.total = off;
  return L;
}

hipError_t launch_k2q_csr(const CsrArgs& a, hipStream_t stream) {
  const SchedLayout& L = a.L;
  Hdr* hdr = reinterpret_cast<Hdr*>(a.sched + L.hdr);
  int32_t* row_base = reinterpret_cast<int32_t*>(a.sched + L.row_base);
  int32_t* unit_cnt = reinterpret_cast<int32_t*>(a.sched + L.unit_cnt);
  int32_t* blk_tot = reinterpret_cast<int32_t*>(a.sched + L.blk_tot);
  int32_t* blk_items = blk_tot + L.n_blocks;
  int4* items = reinterpret_cast<int4*>(a.sched + L.items);
  int32_t* rowsel = reinterpret_cast<int32_t*>(a.sched + L.rowsel);
  int32_t* wbase = reinterpret_cast<int32_t*>(a.sched + L.wbase);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(a.sched + L.bitmap);

  if (a.vl.batch > 0 && L.words_per_row > 0) {
    WordsK wk{a.vl.cu_seqlens_q, a.vl.cu_seqlens_k, a.vl.batch, a.topk, a.tq_stride, a.th_stride,
              a.n_sel, a.vl.total_rows, row_base, bitmap, L.words_per_row, rowsel,
              (int32_t)L.word_chunks};
    hipLaunchKernelGGL(csr_words_kernel, dim3((unsigned)L.word_blocks), dim3(kThreads), 0, stream,
                       wk);
  }

  CountK cnt{bitmap, L.words_per_row, (int32_t)L.units_per_row, L.n_units, unit_cnt, blk_tot,
             blk_items};
  hipLaunchKernelGGL(csr_count_kernel, dim3((unsigned)L.n_blocks), dim3(kThreads), 0, stream, cnt);

  FillK fk{a.vl.cu_seqlens_q, a.vl.cu_seqlens_k, a.vl.batch, a.vl.block_table,
           a.vl.block_table_stride, a.topk, a.tq_stride, a.th_stride, a.n_sel,
           a.vl.total_rows, row_base, bitmap, L.words_per_row, (int32_t)L.units_per_row,
           L.n_units, L.n_rows, (int32_t)L.n_blocks, unit_cnt, blk_tot, blk_items, a.row_ptr,
           a.q_indices, wbase, items, L.max_items, hdr};
  hipLaunchKernelGGL(csr_fill_kernel, dim3((unsigned)L.n_blocks), dim3(kThreads), 0, stream, fk);
  return hipGetLastError();
}

}  // namespace msa
