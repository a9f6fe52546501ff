// KV-page -> query CSR and the attention work list for gfx950.
//
// Transposes each query's selected pages into rows of (request, logical page)
// listing the queries that chose them, ascending (vLLM API docs,
// sparse_attention_msa, MiniMaxM3SparseMSAImpl.forward: build_k2q_csr(topk,
// cu_seqlens_q, cu_seqlens_k, 128, ..., total_rows=total_kv_blocks, ...,
// return_schedule=True) returns row_ptr, q_indices and a schedule).
//
// Deterministic without sorting: every row owns a bitmap over its request's
// query slots.  Marking sets bits with atomic OR; a row's popcount is its
// length; the fill walks the bitmap in order, so each row comes out ascending.
// The fill also records, for every (query, selection head, slot), the CSR
// position of that entry (the combine uses it to find a query's partials in
// slot order) and emits the attention work items: (row, first entry) for
// chunks of kAttnQC entries.
//
// Kernels (all on the caller's stream, no host sync):
//   prep   -- row_base[b] = sum of page counts of earlier requests; zero header
//   zero   -- clear the bitmap
//   mark   -- one thread per (query, head, slot)
//   count  -- one wave per row: popcount
//   scan   -- one block: row_ptr and per-row item offsets (exclusive scans)
//   fill   -- one wave per row: q_indices, positions, work items
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

struct Hdr {
  int32_t n_items;
  int32_t nnz;
  int32_t pad[62];
};

__global__ __launch_bounds__(256) void csr_prep_kernel(const int32_t* __restrict__ cu_k, int B,
                                                       int32_t* __restrict__ row_base,
                                                       Hdr* __restrict__ hdr) {
  // single block: exclusive scan of ceil(seqlen_k / 128) over requests
  __shared__ int wave_tot[4];
  __shared__ int running;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) { running = 0; hdr->n_items = 0; hdr->nnz = 0; }
  __syncthreads();
  for (int base = 0; base <= B; base += 256) {
    const int b = base + tid;
    int pages = 0;
    if (b < B) pages = (cu_k[b + 1] - cu_k[b] + kPage - 1) / kPage;
    const int incl = wave_inclusive_scan(pages);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int off = running;
    for (int w = 0; w < wave; ++w) off += wave_tot[w];
    if (b <= B) row_base[b] = off + incl - pages;
    __syncthreads();
    if (tid == 255) running = off + incl;
    __syncthreads();
  }
}

__global__ void fill_words_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t value) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += stride) p[k] = value;
}

struct MarkK {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch;
  int64_t total_q;
  const int32_t* topk;
  int64_t tq, th;
  int32_t n_sel;
  int32_t total_rows;
  const int32_t* row_base;
  uint32_t* bitmap;
  int64_t words;
};

__global__ __launch_bounds__(256) void csr_mark_kernel(MarkK a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (query, head, slot)
  const int64_t per_q = (int64_t)a.n_sel * kTopK;
  if (e >= a.total_q * per_q) return;
  const int64_t i = e / per_q;
  const int g = (int)((e % per_q) / kTopK);
  const int s = (int)(e % kTopK);
  const int j = a.topk[i * a.tq + g * a.th + s];
  if (j < 0) return;
  const int b = find_request(a.cu_q, a.batch, i);
  const int pages = (a.cu_k[b + 1] - a.cu_k[b] + kPage - 1) / kPage;
  if (j >= pages) return;
  const int64_t rr = a.row_base[b] + j;
  if (rr >= a.total_rows) return;
  const int64_t row = (int64_t)g * a.total_rows + rr;
  const int64_t local = i - a.cu_q[b];
  if (local >= a.words * 32) return;
  atomicOr(&a.bitmap[row * a.words + (local >> 5)], 1u << (local & 31));
}

__global__ __launch_bounds__(256) void csr_count_kernel(const uint32_t* __restrict__ bitmap,
                                                        int64_t words, int64_t n_rows,
                                                        int32_t* __restrict__ counts) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  const uint32_t* w = bitmap + row * words;
  int c = 0;
  for (int64_t k = lane; k < words; k += 64) c += __popc(w[k]);
  c = wave_sum(c);
  if (lane == 0) counts[row] = c;
}

// Single block of 1024: row_ptr = exclusive scan of counts (counts live in
// row_ptr[1..n]); row_items = exclusive scan of ceil(count / kAttnQC).
__global__ __launch_bounds__(1024) void csr_scan_kernel(int32_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ row_items,
                                                        int64_t n_rows, Hdr* __restrict__ hdr) {
  __shared__ int wt_a[16], wt_b[16];
  __shared__ int run_a, run_b;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) { run_a = 0; run_b = 0; }
  __syncthreads();
  for (int64_t base = 0; base < n_rows; base += 1024) {
    const int64_t r = base + tid;
    const int c = r < n_rows ? row_ptr[r + 1] : 0;
    const int it = (c + kAttnQC - 1) / kAttnQC;
    const int ia = wave_inclusive_scan(c);
    const int ib = wave_inclusive_scan(it);
    if (lane == 63) { wt_a[wave] = ia; wt_b[wave] = ib; }
    __syncthreads();
    int oa = run_a, ob = run_b;
    for (int w = 0; w < wave; ++w) { oa += wt_a[w]; ob += wt_b[w]; }
    __syncthreads();   // all reads of row_ptr[r+1] in this chunk precede the writes below
    if (r < n_rows) {
      row_ptr[r] = oa + ia - c;
      row_items[r] = ob + ib - it;
    }
    if (tid == 1023) { run_a = oa + ia; run_b = ob + ib; }
    __syncthreads();
  }
  if (tid == 0) {
    row_ptr[n_rows] = run_a;
    row_items[n_rows] = run_b;
    hdr->nnz = run_a;
    hdr->n_items = run_b;
  }
}

struct FillK {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch;
  const int32_t* topk;
  int64_t tq, th;
  int32_t n_sel;
  int32_t total_rows;
  const int32_t* row_base;
  const uint32_t* bitmap;
  int64_t words;
  int64_t n_rows;
  const int32_t* row_ptr;
  const int32_t* row_items;
  int32_t* q_indices;
  int32_t* inv;       // [total_q, n_sel, 16]
  int2* items;
  int64_t max_items;
};

__global__ __launch_bounds__(256) void csr_fill_kernel(FillK a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.n_rows) return;
  const int g = (int)(row / a.total_rows);
  const int64_t rr = row % a.total_rows;
  const int b = find_request(a.row_base, a.batch, rr);
  const int j = (int)(rr - a.row_base[b]);
  const int cq0 = a.cu_q[b];
  const int32_t start = a.row_ptr[row];
  const uint32_t* w = a.bitmap + row * a.words;
  int base = 0;
  for (int64_t k0 = 0; k0 < a.words; k0 += 64) {
    const int64_t k = k0 + lane;
    uint32_t bits = k < a.words ? w[k] : 0u;
    const int c = __popc(bits);
    const int incl = wave_inclusive_scan(c);
    int p = start + base + incl - c;
    while (bits) {
      const int bit = __builtin_ctz(bits);
      bits &= bits - 1;
      const int64_t qi = cq0 + k * 32 + bit;
      a.q_indices[p] = (int32_t)qi;
      const int32_t* sel = a.topk + qi * a.tq + (int64_t)g * a.th;
      for (int s = 0; s < kTopK; ++s) {
        if (sel[s] == j) {
          a.inv[(qi * a.n_sel + g) * kTopK + s] = p;
          break;
        }
      }
      ++p;
    }
    base += __shfl(incl, 63);
  }
  // work items of this row
  const int32_t len = a.row_ptr[row + 1] - start;
  const int32_t i0 = a.row_items[row];
  const int n_it = (len + kAttnQC - 1) / kAttnQC;
  for (int t = lane; t < n_it; t += 64) {
    const int64_t idx = (int64_t)i0 + t;
    if (idx < a.max_items) a.items[idx] = make_int2((int)row, start + t * kAttnQC);
  }
}

}  // namespace

SchedLayout sched_layout(const msa_varlen_t* vl, int n_sel, int topk) {
  SchedLayout L;
  L.n_rows = (int64_t)n_sel * vl->total_rows;
  L.words_per_row = std::max<int64_t>(1, ceil_div(std::max(vl->max_seqlen_q, 1), 32));
  L.inv_len = (int64_t)vl->total_q * n_sel * topk;
  L.max_items = ceil_div((int64_t)n_sel * vl->total_q * topk, kAttnQC) + L.n_rows;
  size_t off = 0;
  L.hdr = off;        off += sizeof(Hdr);
  L.row_base = off;   off += align_up(sizeof(int32_t) * (vl->batch + 1), 256);
  L.row_items = off;  off += align_up(sizeof(int32_t) * (L.n_rows + 1), 256);
  L.items = off;      off += align_up(sizeof(int2) * L.max_items, 256);
  L.inv = off;        off += align_up(sizeof(int32_t) * std::max<int64_t>(1, L.inv_len), 256);
  L.bitmap = off;     off += align_up(sizeof(uint32_t) * L.n_rows * L.words_per_row, 256);
  L.total = off;
  return L;
}

hipError_t launch_k2q_csr(const CsrArgs& a, hipStream_t stream) {
  const SchedLayout& L = a.L;
  Hdr* hdr = reinterpret_cast<Hdr*>(a.sched + L.hdr);
  int32_t* row_base = reinterpret_cast<int32_t*>(a.sched + L.row_base);
  int32_t* row_items = reinterpret_cast<int32_t*>(a.sched + L.row_items);
  int2* items = reinterpret_cast<int2*>(a.sched + L.items);
  int32_t* inv = reinterpret_cast<int32_t*>(a.sched + L.inv);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(a.sched + L.bitmap);
  const int64_t n_words = L.n_rows * L.words_per_row;

  hipLaunchKernelGGL(csr_prep_kernel, dim3(1), dim3(256), 0, stream, a.vl.cu_seqlens_k,
                     a.vl.batch, row_base, hdr);
  auto fill = [&](void* p, int64_t n, uint32_t value) {
    if (n <= 0) return;
    const int64_t blocks = std::min<int64_t>(8192, ceil_div(n, 256));
    hipLaunchKernelGGL(fill_words_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t*>(p), n, value);
  };
  fill(bitmap, n_words, 0u);
  fill(inv, L.inv_len, 0xFFFFFFFFu);   // -1: no entry

  MarkK mk;
  mk.cu_q = a.vl.cu_seqlens_q;
  mk.cu_k = a.vl.cu_seqlens_k;
  mk.batch = a.vl.batch;
  mk.total_q = a.vl.total_q;
  mk.topk = a.topk;
  mk.tq = a.tq_stride;
  mk.th = a.th_stride;
  mk.n_sel = a.n_sel;
  mk.total_rows = a.vl.total_rows;
  mk.row_base = row_base;
  mk.bitmap = bitmap;
  mk.words = L.words_per_row;
  const int64_t n_mark = (int64_t)a.vl.total_q * a.n_sel * kTopK;
  if (n_mark > 0)
    hipLaunchKernelGGL(csr_mark_kernel, dim3((unsigned)ceil_div(n_mark, 256)), dim3(256), 0,
                       stream, mk);
  if (L.n_rows > 0)
    hipLaunchKernelGGL(csr_count_kernel, dim3((unsigned)ceil_div(L.n_rows, 4)), dim3(256), 0,
                       stream, bitmap, L.words_per_row, L.n_rows, a.row_ptr + 1);
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, stream, a.row_ptr, row_items,
                     L.n_rows, hdr);
  FillK fk;
  fk.cu_q = a.vl.cu_seqlens_q;
  fk.cu_k = a.vl.cu_seqlens_k;
  fk.batch = a.vl.batch;
  fk.topk = a.topk;
  fk.tq = a.tq_stride;
  fk.th = a.th_stride;
  fk.n_sel = a.n_sel;
  fk.total_rows = a.vl.total_rows;
  fk.row_base = row_base;
  fk.bitmap = bitmap;
  fk.words = L.words_per_row;
  fk.n_rows = L.n_rows;
  fk.row_ptr = a.row_ptr;
  fk.row_items = row_items;
  fk.q_indices = a.q_indices;
  fk.inv = inv;
  fk.items = items;
  fk.max_items = L.max_items;
  if (L.n_rows > 0)
    hipLaunchKernelGGL(csr_fill_kernel, dim3((unsigned)ceil_div(L.n_rows, 4)), dim3(256), 0,
                       stream, fk);
  return hipGetLastError();
}

}  // namespace msa
