// KV-page -> query CSR and the attention work list for gfx950.
//
// Transposes each query's selected pages into rows of (request, logical page)
// listing the queries that chose them, ascending (vLLM API docs,
// sparse_attention_msa, MiniMaxM3SparseMSAImpl.forward: build_k2q_csr(topk,
// cu_seqlens_q, cu_seqlens_k, 128, ..., total_rows=total_kv_blocks, ...,
// return_schedule=True) returns row_ptr, q_indices and a schedule).
//
// Deterministic without sorting: every row owns a bitmap over its request's
// query slots, walked in order, so each row comes out ascending.  The row-major
// bitmap is cut into units of 64 consecutive words (one per lane); rows are
// padded so a unit holds whole short rows (decode: one word per row, 64 rows per
// unit) or one 2048-slot piece of a long row (a page chosen by thousands of
// queries is spread over many waves).  Units are the grain of the count, scan
// and fill passes.
//
// Three launches on the caller's stream (four for large grids, one more for
// very long rows), no host sync:
//   words  -- one block per (request, 32 query slots): sets the bits of those
//             slots for every row of the request in LDS and writes the word
//             column out (so the bitmap needs no clearing and no global
//             atomics); also row_base[b] (page rows of earlier requests), per
//             (query, selection head) the mask of slots holding a page's first
//             listing, and per bitmap word with bits set the first-listing slot
//             of each of its queries (4 bits each)
//   count  -- one wave per unit: entries and attention items of the unit, and
//             per-block totals
//   (scan) -- large grids only: exclusive prefix sums of the block totals
//   fill   -- per block: base offsets from the totals of earlier blocks, scan of
//             its units, then one wave per unit (one lane per bitmap word)
//             writes q_indices (ascending) and beside each entry its split
//             slot ((query, selection head, slot): where the attention puts the
//             entry's partial), row_ptr and the work items of at most 32 or 64
//             entries each
//             (64 when the rows average at least 64 queries):
//               {first entry, count, physical page, selection head}
//               {context - cu_seqlens_q[b] - 128 j, valid tokens of the page, row, request}
//             (a query i of the item sees the page's tokens up to i + the first
//             value; the physical page comes from the block table)
//   (order) -- rows of >= 512 queries on average only: the items' order for
//             the attention, sorted by the query range of their piece (a key
//             the fill writes per item)
// For the chunked attention (switched off) the words kernel writes the
// (query, slot) -> CSR row table instead and the fill each word's first CSR
// position, from which that attention's slot kernel finds the split slots.
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
  int32_t* rowsel;        // chunked attention: [total_q, n_sel, 16] CSR row of each selected
                          // page, or -1; else null
  uint32_t* mask;         // else: [total_q, n_sel] slots holding a page's first listing
  uint4* nib;             // else: [rows, words] first-listing slot of each query bit, 4 bits
                          // per query slot (words with no bits set are not written)
  int32_t n_chunks;       // blocks per (request, word): ceil(n_sel * max_pages / kWordRows)
  int32_t max_pages;
};

// Pages of request b, clamped to max_pages (device data contradicting the
// host-side sizes must not move a write past the bitmap or a read past the
// request's block-table row).
__device__ __forceinline__ int request_pages(const int32_t* cu_k, int b, int max_pages) {
  return min(max((cu_k[b + 1] - cu_k[b] + kPage - 1) / kPage, 0), max_pages);
}

// Block ((b * words) + w) * n_chunks + c: query slots 32w .. 32w+31 of request b,
// rows c * kWordRows .. of the request (g-major: r = g * pages + j).
__global__ __launch_bounds__(kThreads) void csr_words_kernel(WordsK a) {
  __shared__ uint32_t s_bits[kWordRows];
  __shared__ __align__(16) uint32_t s_nib[kWordRows][4];
  __shared__ int s_red[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bw = blockIdx.x / a.n_chunks;
  const int c = (int)(blockIdx.x % a.n_chunks);
  const int b = (int)(bw / a.words), w = (int)(bw % a.words);
  const int pages = request_pages(a.cu_k, b, a.max_pages);
  const int rows = a.n_sel * pages;
  const int r0 = c * kWordRows;
  if (r0 >= rows && c > 0) return;

  // rows of earlier requests
  int part = 0;
  for (int k = tid; k < b; k += kThreads) part += request_pages(a.cu_k, k, a.max_pages);
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
    // the last request's blocks also clear any rows past the requests' pages
    if (b == a.batch - 1) {
      const int end = base + pages;
      for (int g = 0; g < a.n_sel; ++g)
        for (int rr = end + tid; rr < a.total_rows; rr += kThreads)
          a.bitmap[((int64_t)g * a.total_rows + rr) * a.words + w] = 0u;
    }
  }
  const int n_r = max(min(kWordRows, rows - r0), 0);
  for (int k = tid; k < n_r; k += kThreads) {
    s_bits[k] = 0u;
    if (!a.rowsel) *reinterpret_cast<uint4*>(s_nib[k]) = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  // each selection entry of the block's queries once, its bit set in its row.
  // A page listed twice counts at its first slot (the one the attention writes
  // a split row for).  Both listings then set the same bit of the same row, so
  // the bit's old value shows a repeat among the block's rows; the 16 slots of
  // one (query, selection head) are one 16-lane row (kThreads and n_sel * 16
  // are multiples of 16, and a row's lanes skip or run together), and a wave
  // with a repeat, or a block that writes masks without holding all of its
  // queries' rows, finds the first listings by comparing with the lanes below.
  // The first row-chunk block writes the (query, selection head) masks of those
  // slots (or, for the chunked attention, the (query, slot) -> row table); each
  // block records the first slot of each of its rows' bits.
  const bool all_rows = c > 0 || a.n_chunks == 1;
  for (int e = tid; e < n_e; e += kThreads) {
    const int ql = e / per_q;
    const int local = 32 * w + ql;
    if (local >= sq) continue;
    const int g = (e % per_q) / kTopK, sl = e % kTopK;
    const int j = a.topk[(int64_t)(q0 + local) * a.tq + (int64_t)g * a.th + sl];
    const bool ok = !(j < 0 || j >= pages || base + j >= a.total_rows);
    const int r = g * pages + j - r0;
    const bool here = ok && r >= 0 && r < n_r;
    uint32_t old = 0u;
    if (here) old = atomicOr(&s_bits[r], 1u << ql);
    if (a.rowsel) {
      if (c == 0) a.rowsel[(int64_t)(q0 + local) * per_q + e % per_q] = ok ? g * a.total_rows + base + j : -1;
    } else {
      bool first = ok;
      if (!all_rows || __builtin_amdgcn_ballot_w64(here && ((old >> ql) & 1u)) != 0)
        first = ok && first_in_row16(ok ? j : -1);
      const uint64_t bal = __builtin_amdgcn_ballot_w64(first);
      if (c == 0 && sl == 0)
        a.mask[(int64_t)(q0 + local) * a.n_sel + g] = (uint32_t)(bal >> (lane & ~(kTopK - 1))) & 0xFFFFu;
      if (first && here) atomicOr(&s_nib[r][ql >> 3], (uint32_t)sl << (4 * (ql & 7)));
    }
  }
  __syncthreads();
  for (int k = tid; k < n_r; k += kThreads) {
    const int r = r0 + k, g = r / pages, j = r - g * pages;
    if (base + j < a.total_rows) {
      const int64_t wi = ((int64_t)g * a.total_rows + base + j) * a.words + w;
      const uint32_t bits = s_bits[k];
      a.bitmap[wi] = bits;
      if (!a.rowsel && bits != 0u) a.nib[wi] = *reinterpret_cast<const uint4*>(s_nib[k]);
    }
  }
}

// A unit is 64 consecutive words (one per lane) of the row-major bitmap
// [n_rows, words].  Rows hold a power of two of words up to 64, else a multiple
// of 64, so a unit covers whole rows (64 / words of them) or a 64-word piece of
// one row; a "piece" is the part of one row inside one unit, G = min(words, 64)
// lanes.  Work items never cross pieces.
__device__ __forceinline__ int piece_sum(int x, int G) {   // sum over aligned groups of G lanes
  return group_sum(x, G);
}

struct CountK {
  const uint32_t* bitmap;
  int64_t n_words;        // n_rows * words
  int32_t G;              // lanes per piece
  int32_t* blk_tot;       // [n_blocks]: entries
  int32_t* blk_items;     // [n_blocks]: attention items
  int32_t qc;             // queries per attention item, at most
};

__global__ __launch_bounds__(kThreads) void csr_count_kernel(CountK a) {
  __shared__ int s_tot[kThreads / 64], s_it[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t u0 = (int64_t)blockIdx.x * kUnitsPerBlock + wave * kUnitsPerWave;
  uint32_t bits[kUnitsPerWave];
#pragma unroll
  for (int k = 0; k < kUnitsPerWave; ++k) {   // all loads in flight together
    const int64_t fw = (u0 + k) * kUnitWords + lane;
    bits[k] = fw < a.n_words ? a.bitmap[fw] : 0u;
  }
  int tot = 0, its = 0;
#pragma unroll
  for (int k = 0; k < kUnitsPerWave; ++k) {
    const int c = __popc(bits[k]);
    const int n = piece_sum(c, a.G);
    tot += c;
    its += (lane & (a.G - 1)) == 0 ? (n + a.qc - 1) / a.qc : 0;
  }
  tot = wave_sum(tot);
  its = wave_sum(its);
  if (lane == 0) { s_tot[wave] = tot; s_it[wave] = its; }
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0, i = 0;
    for (int w = 0; w < kThreads / 64; ++w) { t += s_tot[w]; i += s_it[w]; }
    a.blk_tot[blockIdx.x] = t;
    a.blk_items[blockIdx.x] = i;
  }
}

// Exclusive prefix sums of the count blocks' totals, in place: one block of
// 1024 threads walks tiles of 1024 x kScanPer entries; thread t loads its
// kScanPer consecutive entries together, the per-thread sums are scanned across
// the block and each thread writes its entries' prefixes.  Used when the grid
// is large enough that every fill block summing its predecessors would cost
// more than this launch.
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 16;
constexpr int kScanFrom = 8192;               // count/fill blocks from which the scan runs

__global__ __launch_bounds__(kScanThreads) void csr_scan_kernel(int32_t* tot, int32_t* items,
                                                                int64_t n) {
  __shared__ int s_a[kScanThreads / 64], s_b[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry_a = 0, carry_b = 0;
  for (int64_t t0 = 0; t0 < n; t0 += (int64_t)kScanThreads * kScanPer) {
    const int64_t j0 = t0 + (int64_t)tid * kScanPer;
    int va[kScanPer], vb[kScanPer];
    int sa = 0, sb = 0;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      const bool ok = j0 + k < n;
      va[k] = ok ? tot[j0 + k] : 0;
      vb[k] = ok ? items[j0 + k] : 0;
    }
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) { sa += va[k]; sb += vb[k]; }
    const int ia = wave_inclusive_scan(sa), ib = wave_inclusive_scan(sb);
    if (lane == 63) { s_a[wave] = ia; s_b[wave] = ib; }
    __syncthreads();
    int ra = carry_a + ia - sa, rb = carry_b + ib - sb;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      if (w < wave) { ra += s_a[w]; rb += s_b[w]; }
      carry_a += s_a[w];
      carry_b += s_b[w];
    }
    __syncthreads();                          // s_a / s_b are rewritten by the next tile
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      if (j0 + k < n) { tot[j0 + k] = ra; items[j0 + k] = rb; }
      ra += va[k];
      rb += vb[k];
    }
  }
}

constexpr int kLdsBatch = 1024;               // requests whose offsets the fill keeps in LDS

struct FillK {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch;
  const int32_t* block_table;
  int64_t bt_stride;
  int32_t total_rows;
  const int32_t* row_base;
  const uint32_t* bitmap;
  int64_t words;           // per row
  int32_t G;               // lanes per piece
  int64_t n_words;         // n_rows * words
  int64_t n_rows;
  int32_t n_blocks;
  const int32_t* blk_tot;  // per-block totals, or (prefixed) their exclusive prefix sums
  const int32_t* blk_items;
  int32_t prefixed;
  int32_t* row_ptr;
  int32_t* q_indices;
  int32_t* wbase;          // chunked attention: [n_rows, words] CSR position of each word's
                           // first entry; else null
  const uint4* nib;        // else: [n_rows, words] first-listing slot of each query bit
  int32_t* q_slot;         // else: [nnz] split-row entry (query, selection head, slot) of each
                           // CSR position
  int32_t n_sel;
  int4* items;
  int64_t max_items;
  Hdr* hdr;
  int32_t qc;              // queries per attention item, at most
  int32_t order_shift;     // > 0: write each item's order key (query range of its piece)
  int32_t* okey;
  int32_t max_pages;
};

__global__ __launch_bounds__(kThreads) void csr_fill_kernel(FillK a) {
  __shared__ int s_red[2][kThreads / 64];
  __shared__ int s_cnt[kUnitsPerBlock], s_itc[kUnitsPerBlock];
  __shared__ int s_pos[kUnitsPerBlock];     // first CSR position of each unit
  __shared__ int s_item[kUnitsPerBlock];    // first item index of each unit
  __shared__ int s_rb[kLdsBatch + 1], s_cq[kLdsBatch + 1], s_ck[kLdsBatch + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blk = blockIdx.x;
  const bool lds_req = a.batch <= kLdsBatch;
  const int G = a.G;

  uint32_t bits[kUnitsPerWave];
#pragma unroll
  for (int k = 0; k < kUnitsPerWave; ++k) {   // all loads in flight together
    const int64_t fw = ((int64_t)blk * kUnitsPerBlock + wave * kUnitsPerWave + k) * kUnitWords + lane;
    bits[k] = fw < a.n_words ? a.bitmap[fw] : 0u;
  }
  if (lds_req)
    for (int i = tid; i <= a.batch; i += kThreads) {
      s_rb[i] = a.row_base[i];
      s_cq[i] = a.cu_q[i];
      s_ck[i] = a.cu_k[i];
    }

  // entries and items of all earlier blocks (summed here for small grids)
  int base_e = 0, base_i = 0;
  if (a.prefixed) {
    base_e = a.blk_tot[blk];
    base_i = a.blk_items[blk];
  } else {
    // eight loads per thread in flight together; buffer loads past blk return 0
    const auto rt = buffer_rsrc(a.blk_tot, (uint32_t)blk * 4u);
    const auto ri = buffer_rsrc(a.blk_items, (uint32_t)blk * 4u);
    for (int j0 = 0; j0 < blk; j0 += kThreads * 8) {
      int te[8], ti[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int off = (j0 + u * kThreads + tid) * 4;
        te[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(rt, off, 0, 0);
        ti[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(ri, off, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) { base_e += te[u]; base_i += ti[u]; }
    }
    base_e = wave_sum(base_e);
    base_i = wave_sum(base_i);
    if (lane == 0) { s_red[0][wave] = base_e; s_red[1][wave] = base_i; }
  }
  // entries and items of this block's units
#pragma unroll
  for (int k = 0; k < kUnitsPerWave; ++k) {
    const int c = __popc(bits[k]);
    const int n = piece_sum(c, G);
    const int it = (lane & (G - 1)) == 0 ? (n + a.qc - 1) / a.qc : 0;
    const int tc = wave_sum(c), ti = wave_sum(it);
    if (lane == 0) { s_cnt[wave * kUnitsPerWave + k] = tc; s_itc[wave * kUnitsPerWave + k] = ti; }
  }
  __syncthreads();
  if (!a.prefixed) {
    base_e = 0;
    base_i = 0;
    for (int w = 0; w < kThreads / 64; ++w) { base_e += s_red[0][w]; base_i += s_red[1][w]; }
  }

  // request, page and physical page of each lane's word, the block-table load
  // in flight during the block scan below
  const int32_t* rbase = lds_req ? s_rb : a.row_base;
  int req_k[kUnitsPerWave], page_k[kUnitsPerWave], phys_k[kUnitsPerWave];
  uint4 nib_k[kUnitsPerWave];
#pragma unroll
  for (int k = 0; k < kUnitsPerWave; ++k) {
    const int64_t fw = ((int64_t)blk * kUnitsPerBlock + wave * kUnitsPerWave + k) * kUnitWords + lane;
    const bool valid = fw < a.n_words;
    const int64_t row = fw / a.words;
    const int64_t rr = row - (int64_t)(row / a.total_rows) * a.total_rows;
    req_k[k] = valid ? find_request(rbase, a.batch, rr) : 0;
    page_k[k] = min(max((int)(rr - rbase[req_k[k]]), 0), a.max_pages - 1);
    phys_k[k] = valid ? a.block_table[(int64_t)req_k[k] * a.bt_stride + page_k[k]] : 0;
    // the words kernel writes slot nibbles only for words with bits set
    nib_k[k] = make_uint4(0u, 0u, 0u, 0u);
    if (a.nib && bits[k] != 0u) nib_k[k] = a.nib[fw];
  }

  // scan of this block's units (one lane per unit)
  static_assert(kUnitsPerBlock <= 64, "one lane per unit in the block scan");
  if (wave == 0) {
    const int c = lane < kUnitsPerBlock ? s_cnt[lane] : 0;
    const int it = lane < kUnitsPerBlock ? s_itc[lane] : 0;
    const int ie = wave_inclusive_scan(c);
    const int ii = wave_inclusive_scan(it);
    if (lane < kUnitsPerBlock) {
      s_pos[lane] = base_e + ie - c;
      s_item[lane] = base_i + ii - it;
    }
    if (blk == a.n_blocks - 1 && lane == 63) {
      a.row_ptr[a.n_rows] = base_e + ie;
      a.hdr->nnz = base_e + ie;
      a.hdr->n_items = (int)min<int64_t>(base_i + ii, a.max_items);
    }
  }
  __syncthreads();

  const int32_t* cq = lds_req ? s_cq : a.cu_q;
  const int32_t* ck = lds_req ? s_ck : a.cu_k;
  const int lead = lane & ~(G - 1);
#pragma unroll
  for (int k = 0; k < kUnitsPerWave; ++k) {
    const int ku = wave * kUnitsPerWave + k;
    const int64_t fw = ((int64_t)blk * kUnitsPerBlock + ku) * kUnitWords + lane;
    if (fw - lane >= a.n_words) break;
    const bool valid = fw < a.n_words;
    const int64_t row = fw / a.words;
    const int64_t word = fw - row * a.words;
    const int g = (int)(row / a.total_rows);
    const int64_t rr = row - (int64_t)g * a.total_rows;
    const int b = req_k[k];
    const int j = page_k[k];
    // One lane per bitmap word: the word's first CSR position is the unit's
    // plus the bits of earlier words; the lane then writes the word's entries
    // in bit order (a wave-uniform loop as long as any lane has bits left).
    const uint32_t bits_k = bits[k];
    const int c = __popc(bits_k);
    const int incl = wave_inclusive_scan(c);
    int pos = s_pos[ku] + incl - c;
    if (valid) {
      if (a.wbase) a.wbase[fw] = pos;
      if (word == 0) a.row_ptr[row] = pos;
    }
    // work items of the lane's piece: (row, first entry, count), lane t of the
    // piece writing item t (a piece of G words yields at most G items)
    const int n = piece_sum(c, G);
    const int n_it = (n + a.qc - 1) / a.qc;
    const int it = lane == lead ? n_it : 0;
    const int iincl = wave_inclusive_scan(it);
    const int p_pos = __shfl(pos, lead);
    const int p_item = s_item[ku] + __shfl(iincl - it, lead);
    uint32_t x = bits_k;
    const int64_t q_word = cq[b] + word * 32;
    const uint4 nb = nib_k[k];
    while (__builtin_amdgcn_ballot_w64(x != 0u) != 0) {
      if (x != 0u) {
        const int bit = __builtin_ctz(x);
        const int64_t i = q_word + bit;
        const uint32_t nw = bit < 16 ? (bit < 8 ? nb.x : nb.y) : (bit < 24 ? nb.z : nb.w);
        if (a.q_slot)
          a.q_slot[pos] = (int32_t)((i * a.n_sel + g) * kTopK + ((nw >> (4 * (bit & 7))) & 15u));
        a.q_indices[pos++] = (int32_t)i;
        x &= x - 1u;
      }
    }
    const int t = lane - lead;
    const int64_t q_piece = __shfl(q_word, lead);   // first query slot of the piece
    if (valid && t < n_it) {
      const int64_t idx = (int64_t)p_item + t;
      if (idx < a.max_items) {
        const int sk = ck[b + 1] - ck[b];
        const int ctx = sk - (cq[b + 1] - cq[b]);
        a.items[2 * idx] = make_int4(p_pos + t * a.qc, min(a.qc, n - t * a.qc), phys_k[k], g);
        a.items[2 * idx + 1] = make_int4(ctx - cq[b] - j * kPage, sk - j * kPage, (int)row, b);
        if (a.order_shift > 0) a.okey[idx] = (int32_t)(q_piece >> a.order_shift);
      }
    }
  }
}

// Attention item order for very long rows: items sorted by the query range of
// their piece (key = first query slot of the piece >> shift, written by the
// fill), so that the attention's resident blocks work on one range of queries
// at a time and that range's query rows stay in cache while every page that
// any of them selected is visited; within a bucket items keep about their list
// order (rows ascending).  One block: histogram, scan, scatter of item indices.
constexpr int kOrderThreads = 1024;
constexpr int kOrderKeys = 1024;

__global__ __launch_bounds__(kOrderThreads) void item_order_kernel(const Hdr* __restrict__ hdr,
                                                                   const int32_t* __restrict__ okey,
                                                                   int n_keys, int64_t max_items,
                                                                   int32_t* __restrict__ perm,
                                                                   int32_t* __restrict__ kstart) {
  __shared__ int s_cnt[kOrderKeys];
  __shared__ int s_wave[kOrderThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = (int)min<int64_t>(hdr->n_items, max_items);
  for (int k = tid; k < kOrderKeys; k += kOrderThreads) s_cnt[k] = 0;
  __syncthreads();
  auto key_of = [&](int i) { return min(n_keys - 1, max(0, okey[i])); };
  for (int i = tid; i < n; i += kOrderThreads) atomicAdd(&s_cnt[key_of(i)], 1);
  __syncthreads();
  // exclusive scan over the keys (one per thread)
  const int c = s_cnt[tid];
  const int incl = wave_inclusive_scan(c);
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int off = 0;
  for (int k = 0; k < wave; ++k) off += s_wave[k];
  __syncthreads();
  s_cnt[tid] = off + incl - c;
  if (tid < n_keys) kstart[tid] = off + incl - c;   // first perm position of each key
  if (tid == kOrderThreads - 1) kstart[n_keys] = off + incl;
  __syncthreads();
  for (int i = tid; i < n; i += kOrderThreads) perm[atomicAdd(&s_cnt[key_of(i)], 1)] = i;
}

}  // namespace

SchedLayout sched_layout(const msa_varlen_t* vl, int n_sel, int topk) {
  SchedLayout L;
  L.n_rows = (int64_t)n_sel * vl->total_rows;
  // one bit per query slot; rows padded to a power of two of words up to 64,
  // else to a multiple of 64, so bitmap units align with rows
  const int64_t w = std::max<int64_t>(1, ceil_div(std::max(vl->max_seqlen_q, 1), 32));
  int64_t wp = 1;
  while (wp < w && wp < kUnitWords) wp <<= 1;
  L.words_per_row = w <= kUnitWords ? wp : ceil_div(w, kUnitWords) * kUnitWords;
  L.n_units = ceil_div(L.n_rows * L.words_per_row, kUnitWords);
  L.n_blocks = std::max<int64_t>(1, ceil_div(L.n_units, kUnitsPerBlock));
  L.inv_len = (int64_t)vl->total_q * n_sel * topk;
  L.word_chunks = std::max<int64_t>(1, ceil_div((int64_t)n_sel * std::max(vl->max_pages, 1), kWordRows));
  L.word_blocks = L.words_per_row * std::max(vl->batch, 0) * L.word_chunks;
  // a piece (a row's words inside one unit) holding c entries yields
  // ceil(c / item_q) items; only pieces with entries yield any
  L.item_q = attn_item_queries(vl);
  const int64_t entries = (int64_t)n_sel * vl->total_q * topk;
  const int64_t per_row =
      ceil_div((int64_t)vl->total_q * topk, std::max<int64_t>(1, vl->total_rows));
  // one long request (a fresh prefill or a long chunk): the chunked persistent
  // attention, whose items must not cross a chunk of 2^kChunkShift queries, so
  // pieces are cut to that many query slots
  // Switched off: its first GPU runs (1536 queries, three chunks) did not
  // finish, for a reason not yet found; every batch takes the split path.
  L.fused = (kChunkedAttention && vl->batch == 1 && L.item_q == kAttnQCMax && per_row >= 512 &&
             L.words_per_row % kUnitWords == 0 && vl->total_q < ((int64_t)1 << 19))
                ? 1 : 0;
  L.piece_words = (int32_t)std::min<int64_t>(L.words_per_row,
                                             L.fused ? (1 << kChunkShift) / 32 : kUnitWords);
  const int64_t pieces = L.n_rows * std::max<int64_t>(1, L.words_per_row / L.piece_words);
  L.max_items = ceil_div(entries, L.item_q) + std::min(entries, pieces);
  // rows of at least 512 queries on average (a long fresh prefill): items in
  // query-range order, ranges of 2048 queries (wider if there would be more
  // than kOrderKeys); shorter rows lose more page reuse than they gain
  L.order_shift = 0;
  L.order_keys = 1;
  if (L.fused && L.max_items <= (int64_t)INT32_MAX) {   // items in chunk order
    L.order_shift = kChunkShift;
    L.order_keys = (int32_t)((std::max<int64_t>(vl->total_q, 1) >> kChunkShift) + 1);
  } else if (L.item_q == kAttnQCMax && per_row >= 512 && L.max_items <= (int64_t)INT32_MAX) {
    L.fused = 0;
    int shift = 11;
    while ((std::max<int64_t>(vl->total_q, 1) >> shift) + 1 > kOrderKeys) ++shift;
    L.order_shift = shift;
    L.order_keys = (int32_t)((std::max<int64_t>(vl->total_q, 1) >> shift) + 1);
  }
  if (L.order_shift != kChunkShift) L.fused = 0;
  size_t off = 0;
  L.hdr = off;        off += sizeof(Hdr);
  L.row_base = off;   off += align_up(sizeof(int32_t) * (vl->batch + 1), 256);
  L.blk_tot = off;    off += align_up(sizeof(int32_t) * 2 * L.n_blocks, 256);
  L.items = off;      off += align_up(2 * sizeof(int4) * std::max<int64_t>(1, L.max_items), 256);
  L.okey = off;       off += align_up(sizeof(int32_t) * std::max<int64_t>(1, L.max_items), 256);
  L.perm = off;       off += align_up(sizeof(int32_t) * std::max<int64_t>(1, L.max_items), 256);
  L.kstart = off;     off += align_up(sizeof(int32_t) * (L.order_keys + 1), 256);
  // the chunked attention finds each CSR position's split slot itself, from
  // the (query, slot) -> row table and the words' first positions; otherwise the
  // fill writes it (from the words kernel's slot nibbles) with the combine's
  // first-listing masks
  const int64_t n_words = L.n_rows * L.words_per_row;
  const int64_t chunked = L.fused ? 1 : 0;
  L.rowsel = off;     off += align_up(sizeof(int32_t) * (chunked ? std::max<int64_t>(1, L.inv_len) : 1), 256);
  L.wbase = off;      off += align_up(sizeof(int32_t) * (chunked ? n_words : 1), 256);
  L.bitmap = off;     off += align_up(sizeof(uint32_t) * n_words, 256);
  L.qslot = off;      off += align_up(sizeof(int32_t) * (chunked ? 1 : std::max<int64_t>(1, L.inv_len)), 256);
  L.smask = off;
  off += align_up(sizeof(uint32_t) * (chunked ? 1 : std::max<int64_t>(1, (int64_t)vl->total_q * n_sel)), 256);
  L.nib = off;        off += align_up(16 * (chunked ? 1 : std::max<int64_t>(1, n_words)), 256);
  L.total = off;
  return L;
}

hipError_t launch_k2q_csr(const CsrArgs& a, hipStream_t stream) {
  const SchedLayout& L = a.L;
  Hdr* hdr = reinterpret_cast<Hdr*>(a.sched + L.hdr);
  int32_t* row_base = reinterpret_cast<int32_t*>(a.sched + L.row_base);
  int32_t* blk_tot = reinterpret_cast<int32_t*>(a.sched + L.blk_tot);
  int32_t* blk_items = blk_tot + L.n_blocks;
  int4* items = reinterpret_cast<int4*>(a.sched + L.items);
  const bool chunked = L.fused != 0;
  int32_t* rowsel = chunked ? reinterpret_cast<int32_t*>(a.sched + L.rowsel) : nullptr;
  int32_t* wbase = chunked ? reinterpret_cast<int32_t*>(a.sched + L.wbase) : nullptr;
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(a.sched + L.bitmap);
  int32_t* q_slot = chunked ? nullptr : reinterpret_cast<int32_t*>(a.sched + L.qslot);
  uint32_t* smask = chunked ? nullptr : reinterpret_cast<uint32_t*>(a.sched + L.smask);
  uint4* nib = chunked ? nullptr : reinterpret_cast<uint4*>(a.sched + L.nib);

  if (a.vl.batch > 0 && L.words_per_row > 0) {
    WordsK wk{a.vl.cu_seqlens_q, a.vl.cu_seqlens_k, a.vl.batch, a.topk, a.tq_stride, a.th_stride,
              a.n_sel, a.vl.total_rows, row_base, bitmap, L.words_per_row, rowsel, smask, nib,
              (int32_t)L.word_chunks, std::max(a.vl.max_pages, 1)};
    hipLaunchKernelGGL(csr_words_kernel, dim3((unsigned)L.word_blocks), dim3(kThreads), 0, stream,
                       wk);
  }

  const int32_t G = L.piece_words;
  const int64_t n_words = L.n_rows * L.words_per_row;
  CountK cnt{bitmap, n_words, G, blk_tot, blk_items, L.item_q};
  hipLaunchKernelGGL(csr_count_kernel, dim3((unsigned)L.n_blocks), dim3(kThreads), 0, stream, cnt);

  const int32_t prefixed = L.n_blocks >= kScanFrom ? 1 : 0;
  if (prefixed)
    hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, blk_tot, blk_items,
                       L.n_blocks);
  FillK fk{a.vl.cu_seqlens_q, a.vl.cu_seqlens_k, a.vl.batch, a.vl.block_table,
           a.vl.block_table_stride, a.vl.total_rows, row_base, bitmap, L.words_per_row, G,
           n_words, L.n_rows, (int32_t)L.n_blocks, blk_tot, blk_items, prefixed, a.row_ptr,
           a.q_indices, wbase, nib, q_slot, a.n_sel, items, L.max_items, hdr, L.item_q, L.order_shift,
           reinterpret_cast<int32_t*>(a.sched + L.okey), std::max(a.vl.max_pages, 1)};
  hipLaunchKernelGGL(csr_fill_kernel, dim3((unsigned)L.n_blocks), dim3(kThreads), 0, stream, fk);
  if (L.order_shift > 0)
    hipLaunchKernelGGL(item_order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, hdr,
                       reinterpret_cast<const int32_t*>(a.sched + L.okey), L.order_keys,
                       L.max_items, reinterpret_cast<int32_t*>(a.sched + L.perm),
                       reinterpret_cast<int32_t*>(a.sched + L.kstart));
  return hipGetLastError();
}

}  // namespace msa
