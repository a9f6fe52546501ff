// C-ABI entry points: host-side validation, workspace sizing and launches.
// Every check runs before any HIP call, so each error path can be exercised
// without a GPU.  Unsupported configurations return MSA_ERR_UNSUPPORTED, the
// analogue of the indexer's admission rule (vLLM PR 60930, Details: the CuTe
// scorer is admitted only for E4M3, D128, page 128, H in {1,2,4} per rank and
// sparse_local_block >= 1; otherwise the caller keeps another backend).
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>

#include "msa_internal.h"

using namespace msa;

namespace {

thread_local char g_last_error[512] = "";

msa_status_t fail(msa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

msa_status_t hip_fail(hipError_t e, const char* where) {
  return fail(MSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define MSA_CHECK(cond, st, ...) \
  do {                           \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

msa_status_t check_varlen(const msa_varlen_t* vl) {
  MSA_CHECK(vl != nullptr, MSA_ERR_INVALID_ARGUMENT, "varlen descriptor is NULL");
  MSA_CHECK(vl->batch >= 1, MSA_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", vl->batch);
  MSA_CHECK(vl->total_q >= 0 && vl->max_seqlen_q >= 0 && vl->max_seqlen_k >= 0 &&
                vl->total_rows >= 0 && vl->max_pages >= 0,
            MSA_ERR_INVALID_ARGUMENT, "negative size in varlen descriptor");
  MSA_CHECK(vl->max_seqlen_q <= vl->max_seqlen_k, MSA_ERR_INVALID_ARGUMENT,
            "max_seqlen_q (%d) exceeds max_seqlen_k (%d)", vl->max_seqlen_q, vl->max_seqlen_k);
  MSA_CHECK(vl->total_q == 0 || vl->max_seqlen_q >= 1, MSA_ERR_INVALID_ARGUMENT,
            "total_q > 0 needs max_seqlen_q >= 1");
  MSA_CHECK((int64_t)vl->max_pages * kPage >= vl->max_seqlen_k, MSA_ERR_INVALID_ARGUMENT,
            "max_pages (%d) cannot hold max_seqlen_k (%d)", vl->max_pages, vl->max_seqlen_k);
  MSA_CHECK((int64_t)vl->total_q <= (int64_t)vl->batch * vl->max_seqlen_q,
            MSA_ERR_INVALID_ARGUMENT, "total_q exceeds batch * max_seqlen_q");
  MSA_CHECK((int64_t)vl->total_rows <= (int64_t)vl->batch * vl->max_pages,
            MSA_ERR_INVALID_ARGUMENT, "total_rows exceeds batch * max_pages");
  MSA_CHECK(vl->cu_seqlens_q && vl->cu_seqlens_k && vl->block_table, MSA_ERR_INVALID_ARGUMENT,
            "cu_seqlens_q, cu_seqlens_k and block_table must be non-NULL");
  MSA_CHECK(vl->block_table_stride >= vl->max_pages, MSA_ERR_INVALID_ARGUMENT,
            "block_table_stride (%lld) < max_pages (%d)", (long long)vl->block_table_stride,
            vl->max_pages);
  return MSA_OK;
}

msa_status_t check_device() {
  static const int n_dev = [] {
    int n = 0;
    return hipGetDeviceCount(&n) == hipSuccess ? n : 0;
  }();
  if (n_dev == 0) return fail(MSA_ERR_NO_DEVICE, "no HIP device available");
  return MSA_OK;
}

}  // namespace

extern "C" {

const char* msa_status_string(msa_status_t st) {
  switch (st) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARGUMENT: return "MSA_ERR_INVALID_ARGUMENT";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "MSA_ERR_WORKSPACE_TOO_SMALL";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
    case MSA_ERR_NO_DEVICE: return "MSA_ERR_NO_DEVICE";
  }
  return "MSA_ERR_UNKNOWN";
}

const char* msa_last_error(void) { return g_last_error; }

int32_t msa_abi_version(void) { return MSA_ABI_VERSION; }

// ---------------------------------------------------------------------------
size_t msa_index_score_workspace_size(const msa_varlen_t* vl, int32_t num_index_heads) {
  if (!vl || vl->batch < 1 || vl->total_q < 0 || vl->max_pages < 0) return 0;
  if (num_index_heads != 1 && num_index_heads != 2 && num_index_heads != 4) return 0;
  return score_plan(vl, num_index_heads).workspace_bytes;
}

size_t msa_index_score_topk_workspace_size(const msa_varlen_t* vl, int32_t num_index_heads) {
  if (!vl || vl->batch < 1 || vl->total_q < 0 || vl->max_pages < 0) return 0;
  if (num_index_heads != 1 && num_index_heads != 2 && num_index_heads != 4) return 0;
  const ScorePlan p = score_plan(vl, num_index_heads);
  return p.workspace_bytes + index_score_topk_extra_bytes(p, num_index_heads, vl->total_q);
}

}  // extern "C"

namespace {

// Shared by both key formats: k_scales == nullptr means E4M3 keys.
// head_stride < 0: scores summed over the index heads (one row per query);
// otherwise one row per (query, head), head h's row at h * head_stride.
msa_status_t index_score_impl(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                              int32_t num_index_heads, const uint8_t* k_cache,
                              const uint8_t* k_scales, int32_t num_pages, const float* q_scale,
                              const float* k_scale, float* scores, int64_t ld_scores,
                              void* workspace, size_t workspace_bytes, void* stream,
                              const char* name, int64_t head_stride = -1) {
  msa_status_t st = check_varlen(vl);
  if (st != MSA_OK) return st;
  const int H = num_index_heads;
  MSA_CHECK(H == 1 || H == 2 || H == 4, MSA_ERR_UNSUPPORTED,
            "num_index_heads must be 1, 2 or 4 (got %d)", H);
  if (vl->total_q == 0) return MSA_OK;   // nothing to score
  MSA_CHECK(q && k_cache && q_scale && k_scale && scores && workspace, MSA_ERR_INVALID_ARGUMENT,
            "NULL pointer argument");
  MSA_CHECK(q_stride >= (int64_t)H * kDim && q_stride % 16 == 0, MSA_ERR_INVALID_ARGUMENT,
            "q_stride must be >= H*128 and a multiple of 16 (got %lld)", (long long)q_stride);
  MSA_CHECK(aligned(q, 16) && aligned(k_cache, 16), MSA_ERR_INVALID_ARGUMENT,
            "q and k_cache must be 16-byte aligned");
  MSA_CHECK(!k_scales || aligned(k_scales, 16), MSA_ERR_INVALID_ARGUMENT,
            "k_scales must be 16-byte aligned");
  MSA_CHECK(num_pages >= 1, MSA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
  MSA_CHECK(ld_scores >= vl->max_pages && ld_scores >= 1, MSA_ERR_INVALID_ARGUMENT,
            "ld_scores (%lld) < max_pages (%d)", (long long)ld_scores, vl->max_pages);
  MSA_CHECK(ld_scores % 4 == 0 && aligned(scores, 16), MSA_ERR_INVALID_ARGUMENT,
            "ld_scores must be a multiple of 4 and scores 16-byte aligned");
  MSA_CHECK(aligned(workspace, 16), MSA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  if (head_stride >= 0) {
    MSA_CHECK(head_stride >= vl->max_pages && head_stride % 4 == 0, MSA_ERR_INVALID_ARGUMENT,
              "head_stride (%lld) must be >= max_pages (%d) and a multiple of 4",
              (long long)head_stride, vl->max_pages);
    MSA_CHECK(ld_scores >= (int64_t)(H - 1) * head_stride + vl->max_pages, MSA_ERR_INVALID_ARGUMENT,
              "ld_scores (%lld) cannot hold %d head rows of stride %lld", (long long)ld_scores, H,
              (long long)head_stride);
  }
  const ScorePlan plan = score_plan(vl, head_stride >= 0 ? 1 : H);
  MSA_CHECK(workspace_bytes >= plan.workspace_bytes, MSA_ERR_WORKSPACE_TOO_SMALL,
            "workspace has %zu bytes, needs %zu", workspace_bytes, plan.workspace_bytes);
  MSA_CHECK(plan.max_items < (int64_t)INT32_MAX, MSA_ERR_UNSUPPORTED, "batch too large");
  st = check_device();
  if (st != MSA_OK) return st;
  ScoreArgs a{*vl, q, q_stride, H, k_cache, num_pages, q_scale, k_scale,
              scores, ld_scores, workspace, plan, k_scales};
  hipError_t e = head_stride >= 0
                     ? launch_index_score_heads(a, head_stride, reinterpret_cast<hipStream_t>(stream))
                     : launch_index_score(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, name);
  return MSA_OK;
}

}  // namespace

extern "C" {

msa_status_t msa_index_score(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                             int32_t num_index_heads, const uint8_t* k_cache, int32_t num_pages,
                             const float* q_scale, const float* k_scale, float* scores,
                             int64_t ld_scores, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return index_score_impl(vl, q, q_stride, num_index_heads, k_cache, nullptr, num_pages, q_scale,
                          k_scale, scores, ld_scores, workspace, workspace_bytes, stream,
                          "msa_index_score");
}

// ---- index scoring without allocation ---------------------------------------
// The scorer's work list (a header and one 16-byte item per planned work item)
// lives in this file-scope device array instead of a caller workspace.  Each
// GPU holds its own copy until the process ends.  Host code never uses the
// array's name as an address: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and kept per device.
}  // extern "C"

namespace {

constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

msa_status_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "msa_index_score_noalloc: hipGetDevice");
  MSA_CHECK(dev >= 0 && dev < kMaxDevices, MSA_ERR_UNSUPPORTED,
            "msa_index_score_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "msa_index_score_noalloc: hipGetSymbolAddress(scratch)");
    MSA_CHECK(p != nullptr, MSA_ERR_HIP, "msa_index_score_noalloc: scratch has no device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

msa_status_t msa_index_score_noalloc(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                                     int32_t num_index_heads, const uint8_t* k_cache,
                                     int32_t num_pages, const float* q_scale,
                                     const float* k_scale, float* scores, int64_t ld_scores,
                                     void* stream) {
  msa_status_t st = check_varlen(vl);
  if (st != MSA_OK) return st;
  const int H = num_index_heads;
  MSA_CHECK(H == 1 || H == 2 || H == 4, MSA_ERR_UNSUPPORTED,
            "num_index_heads must be 1, 2 or 4 (got %d)", H);
  if (vl->total_q == 0) return MSA_OK;
  const size_t need = score_plan(vl, H).workspace_bytes;
  MSA_CHECK(need <= kNoAllocScratchBytes, MSA_ERR_UNSUPPORTED,
            "msa_index_score_noalloc: the batch needs %zu bytes of work list, the built-in scratch "
            "holds %zu; use msa_index_score with a workspace", need, kNoAllocScratchBytes);
  st = check_device();
  if (st != MSA_OK) return st;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != MSA_OK) return st;
  return index_score_impl(vl, q, q_stride, num_index_heads, k_cache, nullptr, num_pages, q_scale,
                          k_scale, scores, ld_scores, ws, kNoAllocScratchBytes, stream,
                          "msa_index_score_noalloc");
}

msa_status_t msa_index_score_per_head(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                                      int32_t num_index_heads, const uint8_t* k_cache,
                                      int32_t num_pages, const float* q_scale,
                                      const float* k_scale, float* scores, int64_t ld_scores,
                                      int64_t head_stride, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  return index_score_impl(vl, q, q_stride, num_index_heads, k_cache, nullptr, num_pages, q_scale,
                          k_scale, scores, ld_scores, workspace, workspace_bytes, stream,
                          "msa_index_score_per_head", head_stride);
}

msa_status_t msa_index_score_mxfp4(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                                   int32_t num_index_heads, const uint8_t* k_data,
                                   const uint8_t* k_scales, int32_t num_pages,
                                   const float* q_scale, const float* k_scale, float* scores,
                                   int64_t ld_scores, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  MSA_CHECK(k_scales != nullptr || !vl || vl->total_q == 0, MSA_ERR_INVALID_ARGUMENT,
            "msa_index_score_mxfp4: k_scales is NULL");
  return index_score_impl(vl, q, q_stride, num_index_heads, k_data, k_scales, num_pages, q_scale,
                          k_scale, scores, ld_scores, workspace, workspace_bytes, stream,
                          "msa_index_score_mxfp4");
}

msa_status_t msa_index_score_topk(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                                  int32_t num_index_heads, const uint8_t* k_cache,
                                  int32_t num_pages, const float* q_scale, const float* k_scale,
                                  int32_t topk, int32_t n_local, int32_t* topk_idx,
                                  int64_t topk_stride, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  msa_status_t st = check_varlen(vl);
  if (st != MSA_OK) return st;
  const int H = num_index_heads;
  MSA_CHECK(H == 1 || H == 2 || H == 4, MSA_ERR_UNSUPPORTED,
            "num_index_heads must be 1, 2 or 4 (got %d)", H);
  MSA_CHECK(topk == kTopK, MSA_ERR_UNSUPPORTED, "topk must be 16 (got %d)", topk);
  MSA_CHECK(n_local >= 1 && n_local <= kTopK, MSA_ERR_UNSUPPORTED,
            "n_local must be in [1, 16] (got %d)", n_local);
  MSA_CHECK(vl->max_seqlen_q <= kScoreQueriesPerWave / H, MSA_ERR_UNSUPPORTED,
            "the fused selection takes decode-like batches: max_seqlen_q (%d) > %d / H",
            vl->max_seqlen_q, kScoreQueriesPerWave);
  if (vl->total_q == 0) return MSA_OK;
  MSA_CHECK(q && k_cache && q_scale && k_scale && topk_idx && workspace,
            MSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  MSA_CHECK(q_stride >= (int64_t)H * kDim && q_stride % 16 == 0, MSA_ERR_INVALID_ARGUMENT,
            "q_stride must be >= H*128 and a multiple of 16 (got %lld)", (long long)q_stride);
  MSA_CHECK(aligned(q, 16) && aligned(k_cache, 16) && aligned(workspace, 16),
            MSA_ERR_INVALID_ARGUMENT, "q, k_cache and workspace must be 16-byte aligned");
  MSA_CHECK(num_pages >= 1, MSA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
  MSA_CHECK(topk_stride >= kTopK, MSA_ERR_INVALID_ARGUMENT, "topk_stride must be >= 16");
  const ScorePlan plan = score_plan(vl, H);
  const size_t need = plan.workspace_bytes + index_score_topk_extra_bytes(plan, H, vl->total_q);
  MSA_CHECK(workspace_bytes >= need, MSA_ERR_WORKSPACE_TOO_SMALL,
            "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  MSA_CHECK(plan.max_items < (int64_t)INT32_MAX, MSA_ERR_UNSUPPORTED, "batch too large");
  st = check_device();
  if (st != MSA_OK) return st;
  ScoreArgs a{*vl, q, q_stride, H, k_cache, num_pages, q_scale, k_scale,
              nullptr, 0, workspace, plan, nullptr};
  hipError_t e = launch_index_score_topk(a, n_local, topk_idx, topk_stride,
                                         reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "msa_index_score_topk");
  return MSA_OK;
}

// ---------------------------------------------------------------------------
msa_status_t msa_topk_select(const msa_varlen_t* vl, const float* scores, int64_t ld_scores,
                             int32_t topk, int32_t n_local, int32_t* topk_idx,
                             int64_t topk_stride, void* stream) {
  msa_status_t st = check_varlen(vl);
  if (st != MSA_OK) return st;
  MSA_CHECK(topk == kTopK, MSA_ERR_UNSUPPORTED, "topk must be 16 (got %d)", topk);
  MSA_CHECK(n_local >= 1 && n_local <= kTopK, MSA_ERR_UNSUPPORTED,
            "n_local must be in [1, 16] (got %d)", n_local);
  if (vl->total_q == 0) return MSA_OK;   // nothing to select
  MSA_CHECK(scores && topk_idx, MSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  MSA_CHECK(ld_scores >= vl->max_pages && ld_scores >= 1, MSA_ERR_INVALID_ARGUMENT,
            "ld_scores (%lld) < max_pages (%d)", (long long)ld_scores, vl->max_pages);
  MSA_CHECK(topk_stride >= kTopK, MSA_ERR_INVALID_ARGUMENT, "topk_stride must be >= 16");
  st = check_device();
  if (st != MSA_OK) return st;
  TopkArgs a{*vl, scores, ld_scores, n_local, topk_idx, topk_stride};
  hipError_t e = launch_topk(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "msa_topk_select");
  return MSA_OK;
}

// ---------------------------------------------------------------------------
size_t msa_k2q_schedule_size(const msa_varlen_t* vl, int32_t n_sel_heads, int32_t topk) {
  if (!vl || vl->batch < 1 || vl->total_q < 0 || vl->total_rows < 0 || n_sel_heads < 1 ||
      topk != kTopK)
    return 0;
  return sched_layout(vl, n_sel_heads, topk).total;
}

msa_status_t msa_build_k2q_csr(const msa_varlen_t* vl, const int32_t* topk_idx,
                               int64_t topk_q_stride, int64_t topk_h_stride, int32_t n_sel_heads,
                               int32_t topk, int32_t* row_ptr, int32_t* q_indices, void* schedule,
                               size_t schedule_bytes, void* stream) {
  msa_status_t st = check_varlen(vl);
  if (st != MSA_OK) return st;
  MSA_CHECK(topk == kTopK, MSA_ERR_UNSUPPORTED, "topk must be 16 (got %d)", topk);
  MSA_CHECK(n_sel_heads >= 1, MSA_ERR_INVALID_ARGUMENT, "n_sel_heads must be >= 1");
  MSA_CHECK(row_ptr && schedule, MSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  MSA_CHECK(vl->total_q == 0 || (topk_idx && q_indices), MSA_ERR_INVALID_ARGUMENT,
            "NULL pointer argument");
  MSA_CHECK(topk_h_stride >= 0 && topk_q_stride >= 0, MSA_ERR_INVALID_ARGUMENT,
            "negative top-k stride");
  MSA_CHECK(n_sel_heads == 1 || topk_h_stride >= kTopK, MSA_ERR_INVALID_ARGUMENT,
            "topk_h_stride must be >= 16 with several selection heads");
  MSA_CHECK(topk_q_stride >= (int64_t)(n_sel_heads - 1) * topk_h_stride + kTopK,
            MSA_ERR_INVALID_ARGUMENT, "topk_q_stride too small for the head layout");
  MSA_CHECK(aligned(schedule, 16), MSA_ERR_INVALID_ARGUMENT, "schedule must be 16-byte aligned");
  const SchedLayout L = sched_layout(vl, n_sel_heads, topk);
  MSA_CHECK(schedule_bytes >= L.total, MSA_ERR_WORKSPACE_TOO_SMALL,
            "schedule has %zu bytes, needs %zu", schedule_bytes, L.total);
  MSA_CHECK(L.max_items < (int64_t)INT32_MAX && L.n_rows < (int64_t)INT32_MAX / 4 &&
                L.word_blocks < (int64_t)INT32_MAX,
            MSA_ERR_UNSUPPORTED, "batch too large");
  st = check_device();
  if (st != MSA_OK) return st;
  CsrArgs a{*vl, topk_idx, topk_q_stride, topk_h_stride, n_sel_heads, row_ptr, q_indices,
            reinterpret_cast<uint8_t*>(schedule), L};
  hipError_t e = launch_k2q_csr(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "msa_build_k2q_csr");
  return MSA_OK;
}

// ---------------------------------------------------------------------------
size_t msa_sparse_attn_workspace_size(const msa_varlen_t* vl, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t n_sel_heads, int32_t topk) {
  if (!vl || vl->batch < 1 || vl->total_q < 0 || num_kv_heads < 1 || num_q_heads < 1 ||
      num_q_heads % num_kv_heads != 0 || topk != kTopK ||
      (n_sel_heads != 1 && n_sel_heads != num_kv_heads))
    return 0;
  return attn_workspace_bytes(vl, num_q_heads, num_kv_heads, n_sel_heads, topk);
}

namespace {
// Both cache formats: kv_scales == nullptr reads E4M3 K|V rows, else MXFP4 codes
// with their block scales (the same checks, one more pointer).
msa_status_t sparse_attn_impl(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                              int32_t num_q_heads, const uint8_t* kv_cache,
                              const uint8_t* kv_scales, int32_t num_pages, int32_t num_kv_heads,
                              const int32_t* row_ptr, const int32_t* q_indices,
                              int32_t n_sel_heads, const void* schedule, size_t schedule_bytes,
                              int32_t topk, float softmax_scale, const float* q_scale,
                              const float* k_scale, const float* v_scale, uint16_t* out,
                              int64_t out_stride, void* workspace, size_t workspace_bytes,
                              void* stream, const char* name) {
  msa_status_t st = check_varlen(vl);
  if (st != MSA_OK) return st;
  const int Hq = num_q_heads, Hkv = num_kv_heads;
  MSA_CHECK(Hq >= 1 && Hkv >= 1, MSA_ERR_INVALID_ARGUMENT, "head counts must be >= 1");
  MSA_CHECK(Hq % Hkv == 0, MSA_ERR_UNSUPPORTED, "num_q_heads (%d) %% num_kv_heads (%d) != 0", Hq,
            Hkv);
  MSA_CHECK(topk == kTopK, MSA_ERR_UNSUPPORTED, "topk must be 16 (got %d)", topk);
  MSA_CHECK(n_sel_heads == 1 || n_sel_heads == Hkv, MSA_ERR_UNSUPPORTED,
            "n_sel_heads must be 1 or num_kv_heads (got %d)", n_sel_heads);
  if (vl->total_q == 0) return MSA_OK;   // no query, no output
  MSA_CHECK(q && kv_cache && row_ptr && q_indices && schedule && out && workspace,
            MSA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  MSA_CHECK(q_stride >= (int64_t)Hq * kDim && q_stride % 16 == 0, MSA_ERR_INVALID_ARGUMENT,
            "q_stride must be >= Hq*128 and a multiple of 16");
  MSA_CHECK(out_stride >= (int64_t)Hq * kDim && out_stride % 8 == 0, MSA_ERR_INVALID_ARGUMENT,
            "out_stride must be >= Hq*128 and a multiple of 8");
  MSA_CHECK(aligned(q, 16) && aligned(kv_cache, 16) && aligned(out, 16), MSA_ERR_INVALID_ARGUMENT,
            "q, kv_cache and out must be 16-byte aligned");
  MSA_CHECK(Hq <= 64, MSA_ERR_UNSUPPORTED, "num_q_heads must be <= 64 (got %d)", Hq);
  MSA_CHECK(num_pages >= 1, MSA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
  MSA_CHECK(softmax_scale > 0.f, MSA_ERR_INVALID_ARGUMENT, "softmax_scale must be > 0");
  MSA_CHECK(aligned(schedule, 16) && aligned(workspace, 16), MSA_ERR_INVALID_ARGUMENT,
            "schedule and workspace must be 16-byte aligned");
  const SchedLayout L = sched_layout(vl, n_sel_heads, topk);
  MSA_CHECK(schedule_bytes >= L.total, MSA_ERR_WORKSPACE_TOO_SMALL,
            "schedule has %zu bytes, needs %zu", schedule_bytes, L.total);
  const size_t need = attn_workspace_bytes(vl, Hq, Hkv, n_sel_heads, topk);
  MSA_CHECK(workspace_bytes >= need, MSA_ERR_WORKSPACE_TOO_SMALL,
            "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  MSA_CHECK(Hkv <= 65535 && L.max_items < (int64_t)INT32_MAX, MSA_ERR_UNSUPPORTED,
            "batch or head count too large");
  MSA_CHECK((int64_t)vl->total_q * topk * Hq < (int64_t)INT32_MAX, MSA_ERR_UNSUPPORTED,
            "total_q * topk * num_q_heads must be < 2^31 (split rows are indexed in 32 bits)");
  st = check_device();
  if (st != MSA_OK) return st;
  AttnArgs a{*vl, q, q_stride, Hq, Hkv, n_sel_heads, kv_cache, num_pages, row_ptr, q_indices,
             reinterpret_cast<const uint8_t*>(schedule), L, softmax_scale, q_scale, k_scale,
             v_scale, out, out_stride, workspace, kv_scales};
  hipError_t e = launch_sparse_attn(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, name);
  return MSA_OK;
}
}  // namespace

msa_status_t msa_sparse_attn_prefill(const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride,
                                     int32_t num_q_heads, const uint8_t* kv_cache,
                                     int32_t num_pages, int32_t num_kv_heads,
                                     const int32_t* row_ptr, const int32_t* q_indices,
                                     int32_t n_sel_heads, const void* schedule,
                                     size_t schedule_bytes, int32_t topk, float softmax_scale,
                                     const float* q_scale, const float* k_scale,
                                     const float* v_scale, uint16_t* out, int64_t out_stride,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_attn_impl(vl, q, q_stride, num_q_heads, kv_cache, nullptr, num_pages, num_kv_heads,
                          row_ptr, q_indices, n_sel_heads, schedule, schedule_bytes, topk,
                          softmax_scale, q_scale, k_scale, v_scale, out, out_stride, workspace,
                          workspace_bytes, stream, "msa_sparse_attn_prefill");
}

msa_status_t msa_sparse_attn_prefill_mxfp4(
    const msa_varlen_t* vl, const uint8_t* q, int64_t q_stride, int32_t num_q_heads,
    const uint8_t* kv_data, const uint8_t* kv_scales, int32_t num_pages, int32_t num_kv_heads,
    const int32_t* row_ptr, const int32_t* q_indices, int32_t n_sel_heads, const void* schedule,
    size_t schedule_bytes, int32_t topk, float softmax_scale, const float* q_scale,
    const float* k_scale, const float* v_scale, uint16_t* out, int64_t out_stride,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (vl && vl->total_q > 0)
    MSA_CHECK(kv_scales && aligned(kv_scales, 8), MSA_ERR_INVALID_ARGUMENT,
              "kv_scales must be non-NULL and 8-byte aligned");
  return sparse_attn_impl(vl, q, q_stride, num_q_heads, kv_data, kv_scales, num_pages,
                          num_kv_heads, row_ptr, q_indices, n_sel_heads, schedule, schedule_bytes,
                          topk, softmax_scale, q_scale, k_scale, v_scale, out, out_stride,
                          workspace, workspace_bytes, stream, "msa_sparse_attn_prefill_mxfp4");
}


// ---- E4M3 quantisation and the paged cache write ---------------------------

namespace {

msa_status_t check_src(const void* p, int32_t dtype, int64_t stride, int64_t min_stride,
                       const char* name) {
  MSA_CHECK(dtype == MSA_DTYPE_BF16 || dtype == MSA_DTYPE_F32, MSA_ERR_UNSUPPORTED,
            "%s: src_dtype must be MSA_DTYPE_BF16 or MSA_DTYPE_F32 (got %d)", name, dtype);
  MSA_CHECK(p != nullptr, MSA_ERR_INVALID_ARGUMENT, "%s: NULL source", name);
  MSA_CHECK(aligned(p, 16), MSA_ERR_INVALID_ARGUMENT, "%s: source must be 16-byte aligned", name);
  MSA_CHECK(stride >= min_stride && stride % 8 == 0, MSA_ERR_INVALID_ARGUMENT,
            "%s: stride (%lld) must be >= %lld elements and a multiple of 8", name,
            (long long)stride, (long long)min_stride);
  return MSA_OK;
}

msa_status_t run_quantize(const QuantArgs& q, void* stream, const char* name) {
  msa_status_t st = check_device();
  if (st != MSA_OK) return st;
  hipError_t e = launch_quantize(q, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, name);
  return MSA_OK;
}

constexpr int64_t kMaxQuantRows = (int64_t)UINT32_MAX * 16;   // grid x limit of the row kernel

}  // namespace

msa_status_t msa_quantize_e4m3(const void* src, int32_t src_dtype, int64_t n_rows, int32_t heads,
                               int64_t src_stride, const float* scale, uint8_t* dst,
                               int64_t dst_stride, void* stream) {
  MSA_CHECK(n_rows >= 0 && heads >= 1, MSA_ERR_INVALID_ARGUMENT,
            "msa_quantize_e4m3: n_rows must be >= 0 and heads >= 1");
  MSA_CHECK(n_rows * heads <= kMaxQuantRows, MSA_ERR_UNSUPPORTED, "msa_quantize_e4m3: too many rows");
  if (n_rows == 0) return MSA_OK;
  msa_status_t st = check_src(src, src_dtype, src_stride, (int64_t)heads * kDim, "msa_quantize_e4m3");
  if (st != MSA_OK) return st;
  MSA_CHECK(scale && dst, MSA_ERR_INVALID_ARGUMENT, "msa_quantize_e4m3: NULL scale or dst");
  MSA_CHECK(aligned(dst, 8) && dst_stride >= (int64_t)heads * kDim && dst_stride % 8 == 0,
            MSA_ERR_INVALID_ARGUMENT,
            "msa_quantize_e4m3: dst must be 8-byte aligned, dst_stride >= heads*128 and a multiple of 8");
  QuantArgs q{};
  q.n_parts = 1;
  q.src[0] = q.src[1] = src;
  q.scale[0] = q.scale[1] = scale;
  q.dtype = src_dtype;
  q.n_tokens = n_rows;
  q.heads = heads;
  q.src_tok_stride[0] = q.src_tok_stride[1] = src_stride;
  q.src_head_stride = kDim;
  q.dst = dst;
  q.dst_tok_stride = dst_stride;
  q.dst_head_stride = kDim;
  return run_quantize(q, stream, "msa_quantize_e4m3");
}

msa_status_t msa_insert_index_k(const void* k, int32_t src_dtype, int64_t n_tokens,
                                int64_t k_stride, const int64_t* slot_mapping, const float* scale,
                                uint8_t* k_cache, int32_t num_pages, void* stream) {
  MSA_CHECK(n_tokens >= 0, MSA_ERR_INVALID_ARGUMENT, "msa_insert_index_k: n_tokens must be >= 0");
  MSA_CHECK(n_tokens <= kMaxQuantRows, MSA_ERR_UNSUPPORTED, "msa_insert_index_k: too many tokens");
  if (n_tokens == 0) return MSA_OK;
  msa_status_t st = check_src(k, src_dtype, k_stride, kDim, "msa_insert_index_k");
  if (st != MSA_OK) return st;
  MSA_CHECK(slot_mapping && scale && k_cache, MSA_ERR_INVALID_ARGUMENT,
            "msa_insert_index_k: NULL slot_mapping, scale or k_cache");
  MSA_CHECK(aligned(k_cache, 8) && num_pages >= 1, MSA_ERR_INVALID_ARGUMENT,
            "msa_insert_index_k: k_cache must be 8-byte aligned and num_pages >= 1");
  QuantArgs q{};
  q.n_parts = 1;
  q.src[0] = q.src[1] = k;
  q.scale[0] = q.scale[1] = scale;
  q.dtype = src_dtype;
  q.n_tokens = n_tokens;
  q.heads = 1;
  q.src_tok_stride[0] = q.src_tok_stride[1] = k_stride;
  q.src_head_stride = kDim;
  q.slots = slot_mapping;
  q.max_slot = (int64_t)num_pages * kPage;
  q.dst = k_cache;
  q.dst_page_stride = (int64_t)kPage * kDim;
  q.dst_row_stride = kDim;
  return run_quantize(q, stream, "msa_insert_index_k");
}

msa_status_t msa_insert_kv(const void* k, const void* v, int32_t src_dtype, int64_t n_tokens,
                           int32_t num_kv_heads, int64_t k_stride, int64_t v_stride,
                           const int64_t* slot_mapping, const float* k_scale,
                           const float* v_scale, uint8_t* kv_cache, int32_t num_pages,
                           void* stream) {
  MSA_CHECK(n_tokens >= 0 && num_kv_heads >= 1, MSA_ERR_INVALID_ARGUMENT,
            "msa_insert_kv: n_tokens must be >= 0 and num_kv_heads >= 1");
  MSA_CHECK(n_tokens * num_kv_heads <= kMaxQuantRows, MSA_ERR_UNSUPPORTED,
            "msa_insert_kv: too many rows");
  if (n_tokens == 0) return MSA_OK;
  const int64_t min_stride = (int64_t)num_kv_heads * kDim;
  msa_status_t st = check_src(k, src_dtype, k_stride, min_stride, "msa_insert_kv (k)");
  if (st != MSA_OK) return st;
  st = check_src(v, src_dtype, v_stride, min_stride, "msa_insert_kv (v)");
  if (st != MSA_OK) return st;
  MSA_CHECK(slot_mapping && k_scale && v_scale && kv_cache, MSA_ERR_INVALID_ARGUMENT,
            "msa_insert_kv: NULL slot_mapping, scale or kv_cache");
  MSA_CHECK(aligned(kv_cache, 8) && num_pages >= 1, MSA_ERR_INVALID_ARGUMENT,
            "msa_insert_kv: kv_cache must be 8-byte aligned and num_pages >= 1");
  QuantArgs q{};
  q.n_parts = 2;
  q.src[0] = k;
  q.src[1] = v;
  q.scale[0] = k_scale;
  q.scale[1] = v_scale;
  q.col_off[0] = 0;
  q.col_off[1] = kDim;
  q.dtype = src_dtype;
  q.n_tokens = n_tokens;
  q.heads = num_kv_heads;
  q.src_tok_stride[0] = k_stride;
  q.src_tok_stride[1] = v_stride;
  q.src_head_stride = kDim;
  q.slots = slot_mapping;
  q.max_slot = (int64_t)num_pages * kPage;
  q.dst = kv_cache;
  q.dst_page_stride = (int64_t)num_kv_heads * kPage * 2 * kDim;
  q.dst_head_stride = (int64_t)kPage * 2 * kDim;
  q.dst_row_stride = 2 * kDim;
  return run_quantize(q, stream, "msa_insert_kv");
}

msa_status_t msa_insert_index_k_mxfp4(const void* k, int32_t src_dtype, int64_t n_tokens,
                                      int64_t k_stride, const int64_t* slot_mapping,
                                      uint8_t* k_data, uint8_t* k_scales, int32_t num_pages,
                                      void* stream) {
  MSA_CHECK(n_tokens >= 0, MSA_ERR_INVALID_ARGUMENT, "msa_insert_index_k_mxfp4: n_tokens must be >= 0");
  MSA_CHECK(n_tokens <= kMaxQuantRows, MSA_ERR_UNSUPPORTED, "msa_insert_index_k_mxfp4: too many tokens");
  if (n_tokens == 0) return MSA_OK;
  msa_status_t st = check_src(k, src_dtype, k_stride, kDim, "msa_insert_index_k_mxfp4");
  if (st != MSA_OK) return st;
  MSA_CHECK(slot_mapping && k_data && k_scales, MSA_ERR_INVALID_ARGUMENT,
            "msa_insert_index_k_mxfp4: NULL slot_mapping, k_data or k_scales");
  MSA_CHECK(aligned(k_data, 4) && num_pages >= 1, MSA_ERR_INVALID_ARGUMENT,
            "msa_insert_index_k_mxfp4: k_data must be 4-byte aligned and num_pages >= 1");
  st = check_device();
  if (st != MSA_OK) return st;
  Mx4Args q{k, src_dtype, n_tokens, k_stride, slot_mapping, (int64_t)num_pages * kPage, k_data,
            k_scales};
  hipError_t e = launch_insert_mxfp4(q, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "msa_insert_index_k_mxfp4");
  return MSA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Device-side check of a batch's metadata against its host-side sizes: one
// block; thread b takes request b's bounds, then all threads take each
// request's block-table entries in turn.  Every read stays inside the arrays
// the host-side sizes describe (block-table columns below min(pages,
// max_pages)), whatever the device data holds.
namespace {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void varlen_check_kernel(msa_varlen_t vl, int32_t num_pages,
                                                                      int32_t* flags) {
  __shared__ int s_or[kCheckThreads / 64];
  __shared__ long long s_rows[kCheckThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int f = 0;
  long long rows = 0;
  for (int b = tid; b < vl.batch; b += kCheckThreads) {
    const int q0 = vl.cu_seqlens_q[b], q1 = vl.cu_seqlens_q[b + 1];
    const int k0 = vl.cu_seqlens_k[b], k1 = vl.cu_seqlens_k[b + 1];
    if ((b == 0 && q0 != 0) || q1 < q0 || q1 > vl.total_q) f |= MSA_BAD_CU_Q;
    if ((b == 0 && k0 != 0) || k1 < k0) f |= MSA_BAD_CU_K;
    const int sq = q1 - q0, sk = k1 - k0;
    if (sq > sk) f |= MSA_BAD_CU_K;
    if (sq > vl.max_seqlen_q) f |= MSA_BAD_MAX_Q;
    if (sk > vl.max_seqlen_k) f |= MSA_BAD_MAX_K;
    const long long pages = sk > 0 ? ((long long)sk + kPage - 1) / kPage : 0;
    if (pages > vl.max_pages) f |= MSA_BAD_PAGES;
    rows += pages;
  }
  if (tid == 0 && vl.cu_seqlens_q[vl.batch] != vl.total_q) f |= MSA_BAD_CU_Q;
  for (int b = 0; b < vl.batch; ++b) {
    const int sk = vl.cu_seqlens_k[b + 1] - vl.cu_seqlens_k[b];
    const int np = sk > 0 ? min((int)(((long long)sk + kPage - 1) / kPage), vl.max_pages) : 0;
    const int32_t* row = vl.block_table + (int64_t)b * vl.block_table_stride;
    for (int j = tid; j < np; j += kCheckThreads) {
      const int p = row[j];
      if (p < 0 || p >= num_pages) f |= MSA_BAD_BLOCK;
    }
  }
  // block-wide OR of the flags and sum of the page counts
  for (int o = 32; o > 0; o >>= 1) {
    f |= __shfl_xor(f, o);
    rows += __shfl_xor(rows, o);
  }
  if (lane == 0) { s_or[wave] = f; s_rows[wave] = rows; }
  __syncthreads();
  if (tid == 0) {
    int all = 0;
    long long total = 0;
    for (int k = 0; k < kCheckThreads / 64; ++k) { all |= s_or[k]; total += s_rows[k]; }
    if (total != vl.total_rows) all |= MSA_BAD_ROWS;
    flags[0] = all;
  }
}

}  // namespace

extern "C" {

msa_status_t msa_check_varlen(const msa_varlen_t* vl, int32_t num_pages, int32_t* flags,
                              void* stream) {
  msa_status_t st = check_varlen(vl);
  if (st != MSA_OK) return st;
  MSA_CHECK(num_pages >= 1, MSA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1 (got %d)", num_pages);
  MSA_CHECK(flags != nullptr, MSA_ERR_INVALID_ARGUMENT, "flags is NULL");
  st = check_device();
  if (st != MSA_OK) return st;
  hipLaunchKernelGGL(varlen_check_kernel, dim3(1), dim3(kCheckThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), *vl, num_pages, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "msa_check_varlen");
  return MSA_OK;
}

}  // extern "C"
