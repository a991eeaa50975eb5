// C ABI of the library: host-side checks, then kernel launches on the
// caller's stream.  No device allocation and no synchronisation; this layer
// keeps no state besides the per-thread error text (the prefill path's
// second stream per device lives beside its kernels).
#include <hip/hip_runtime_api.h>

#include <cmath>

#include "fp2.h"
#include "fp2_internal.h"

namespace fp2 {
hipError_t launch_block_stats(const fp2_batch* b, const fp2_kv* kv, const BatchInfo& info,
                              float* kbar, float* vbar, hipStream_t stream);
hipError_t launch_block_stats_cached(const fp2_batch* b, const fp2_kv* kv, const BatchInfo& info, float* kcache,
                                     float* vcache, int refresh, hipStream_t stream);
hipError_t launch_gather_stats(const fp2_batch* b, const fp2_kv* kv, const BatchInfo& info, const float* kcache,
                               const float* vcache, float* kbar, float* vbar, hipStream_t stream);
hipError_t launch_plan(const fp2_batch* b, const fp2_q* q, int hkv, const BatchInfo& info,
                       const float* kbar, float tau, int32_t* row_ptr, int32_t* col_idx,
                       int32_t* nnz, float* scores, void* workspace, hipStream_t stream);
hipError_t launch_zero_plan(int32_t* row_ptr, int32_t* nnz, hipStream_t stream);
hipError_t launch_stage1(const fp2_batch* b, const fp2_q* q, const fp2_kv* kv, const BatchInfo& info, float tau,
                         float* kbar, float* vbar, int32_t* row_ptr, int32_t* col_idx, int32_t* nnz, float* scores,
                         void* workspace, hipStream_t stream);
hipError_t scratch_address(void** out);
hipError_t launch_prefill(const fp2_batch* b, const fp2_q* q, const fp2_kv* kv, const BatchInfo& info,
                          const int32_t* row_ptr, const int32_t* col_idx, const float* kbar,
                          const float* vbar, int correction, float softmax_scale, int out_f32,
                          void* out, int max_chunk_tiles, void* workspace, hipStream_t stream);

static fp2_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FP2_OK;
  return fail(FP2_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Kernels run on the device of the stream they are enqueued on, while the
// library's per-device state (the prefill call's second stream and events,
// the allocation-free call's scratch array, the bounds word) is taken for
// the current device: a stream of another device is refused.  The NULL
// stream is the current device's.  A handle the runtime cannot place (a
// special stream handle) is left to the launch itself.
static fp2_status check_stream(void* stream, const char* what) {
  if (!stream) return FP2_OK;
  int cur = 0;
  hipDevice_t sdev = 0;
  if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess)
    return FP2_OK;
  if (sdev != cur)
    return fail(FP2_ERR_INVALID, std::string(what) + ": the stream belongs to device " + std::to_string(sdev) +
                                     " but the current device is " + std::to_string(cur));
  return FP2_OK;
}
}  // namespace fp2

using namespace fp2;

extern "C" {

fp2_status fp2_block_stats(const fp2_batch* batch, const fp2_kv* kv, float* kbar, float* vbar,
                           void* stream) {
  BatchInfo info;
  fp2_status st = check_batch(batch, &info);
  if (st != FP2_OK) return st;
  if ((st = check_kv(kv, batch, info)) != FP2_OK) return st;
  if (info.total_kblocks > 0 && (!kbar || !vbar)) return fail(FP2_ERR_INVALID, "kbar/vbar is NULL");
  if ((st = check_stream(stream, "fp2_block_stats")) != FP2_OK) return st;
  if (hipError_t e = launch_check_pages(batch, kv, (hipStream_t)stream); e != hipSuccess)
    return hip_status(e, "fp2_block_stats bounds check");
  return hip_status(launch_block_stats(batch, kv, info, kbar, vbar, (hipStream_t)stream),
                    "fp2_block_stats launch");
}

int64_t fp2_block_stats_cache_rows(const fp2_batch* batch, const fp2_kv* kv) {
  BatchInfo info;
  if (check_batch(batch, &info) != FP2_OK || check_kv(kv, batch, info) != FP2_OK) return 0;
  const int ps = kv->page_size, B = info.kvblock;
  if (ps % B != 0 && B % ps != 0) return 0;
  return (int64_t)kv->num_pages * (ps >= B ? ps / B : 1);
}

fp2_status fp2_block_stats_cached(const fp2_batch* batch, const fp2_kv* kv, float* kbar_cache, float* vbar_cache,
                                  int32_t refresh_prefix, void* stream) {
  BatchInfo info;
  fp2_status st = check_batch(batch, &info);
  if (st != FP2_OK) return st;
  if ((st = check_kv(kv, batch, info)) != FP2_OK) return st;
  if (kv->page_size % info.kvblock != 0 && info.kvblock % kv->page_size != 0)
    return fail(FP2_ERR_UNSUPPORTED, "the block stats cache needs page_size and the KV block to divide one another");
  if (refresh_prefix != 0 && refresh_prefix != 1) return fail(FP2_ERR_INVALID, "refresh_prefix must be 0 or 1");
  if (info.total_kblocks > 0 && (!kbar_cache || !vbar_cache))
    return fail(FP2_ERR_INVALID, "kbar_cache/vbar_cache is NULL");
  if ((st = check_stream(stream, "fp2_block_stats_cached")) != FP2_OK) return st;
  if (hipError_t e = launch_check_pages(batch, kv, (hipStream_t)stream); e != hipSuccess)
    return hip_status(e, "fp2_block_stats_cached bounds check");
  return hip_status(launch_block_stats_cached(batch, kv, info, kbar_cache, vbar_cache, refresh_prefix,
                                              (hipStream_t)stream),
                    "fp2_block_stats_cached launch");
}

fp2_status fp2_gather_block_stats(const fp2_batch* batch, const fp2_kv* kv, const float* kbar_cache,
                                  const float* vbar_cache, float* kbar, float* vbar, void* stream) {
  BatchInfo info;
  fp2_status st = check_batch(batch, &info);
  if (st != FP2_OK) return st;
  if ((st = check_kv(kv, batch, info)) != FP2_OK) return st;
  if (kv->page_size % info.kvblock != 0 && info.kvblock % kv->page_size != 0)
    return fail(FP2_ERR_UNSUPPORTED, "the block stats cache needs page_size and the KV block to divide one another");
  if (info.total_kblocks > 0 && (!kbar_cache || !vbar_cache || !kbar || !vbar))
    return fail(FP2_ERR_INVALID, "a cache or output pointer is NULL");
  if ((st = check_stream(stream, "fp2_gather_block_stats")) != FP2_OK) return st;
  if (hipError_t e = launch_check_pages(batch, kv, (hipStream_t)stream); e != hipSuccess)
    return hip_status(e, "fp2_gather_block_stats bounds check");
  return hip_status(launch_gather_stats(batch, kv, info, kbar_cache, vbar_cache, kbar, vbar, (hipStream_t)stream),
                    "fp2_gather_block_stats launch");
}

size_t fp2_plan_workspace_bytes(const fp2_batch* batch, int32_t num_kv_heads) {
  BatchInfo info;
  if (check_batch(batch, &info) != FP2_OK || num_kv_heads < 1) return 0;
  return plan_workspace_bytes(info, num_kv_heads);
}

int64_t fp2_plan_max_nnz(const fp2_batch* batch, int32_t num_kv_heads) {
  BatchInfo info;
  if (check_batch(batch, &info) != FP2_OK || num_kv_heads < 1) return -1;
  return info.causal_pairs * num_kv_heads;
}

// Checks shared by fp2_plan_mask and fp2_plan_mask_noalloc (everything but
// the workspace).
static fp2_status check_plan(const fp2_batch* batch, const fp2_q* q, int32_t num_kv_heads, const float* kbar,
                             float tau, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, int32_t* nnz,
                             BatchInfo* info) {
  fp2_status st = check_batch(batch, info);
  if (st != FP2_OK) return st;
  if ((st = check_q(q, num_kv_heads, *info, batch->block)) != FP2_OK) return st;
  if ((st = check_index_range(*info, num_kv_heads)) != FP2_OK) return st;
  if (std::isnan(tau)) return fail(FP2_ERR_INVALID, "tau is NaN");
  if (!nnz) return fail(FP2_ERR_INVALID, "nnz is NULL");
  if (info->total_qblocks > 0) {
    if (!kbar || !row_ptr || !col_idx) return fail(FP2_ERR_INVALID, "kbar/row_ptr/col_idx is NULL");
  } else if (!row_ptr) {
    return fail(FP2_ERR_INVALID, "row_ptr is NULL");
  }
  const int64_t need = info->causal_pairs * num_kv_heads;
  if (col_capacity < need)
    return fail(FP2_ERR_CAPACITY, "col_capacity " + std::to_string(col_capacity) + " < " +
                                      std::to_string(need) + " (fp2_plan_max_nnz)");
  return FP2_OK;
}

fp2_status fp2_plan_mask(const fp2_batch* batch, const fp2_q* q, int32_t num_kv_heads,
                         const float* kbar, float tau, int32_t* row_ptr, int32_t* col_idx,
                         int64_t col_capacity, int32_t* nnz, float* scores, void* workspace,
                         size_t workspace_bytes, void* stream) {
  BatchInfo info;
  fp2_status st = check_plan(batch, q, num_kv_heads, kbar, tau, row_ptr, col_idx, col_capacity, nnz, &info);
  if (st != FP2_OK) return st;
  if (info.total_qblocks > 0 && !workspace) return fail(FP2_ERR_INVALID, "workspace is NULL");
  const size_t wneed = plan_workspace_bytes(info, num_kv_heads);
  if (workspace_bytes < wneed)
    return fail(FP2_ERR_CAPACITY, "plan workspace " + std::to_string(workspace_bytes) + " < " +
                                      std::to_string(wneed) + " bytes");
  if ((st = check_stream(stream, "fp2_plan_mask")) != FP2_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (info.total_qblocks == 0) return hip_status(launch_zero_plan(row_ptr, nnz, s), "fp2_plan_mask");
  return hip_status(launch_plan(batch, q, num_kv_heads, info, kbar, tau, row_ptr, col_idx, nnz,
                                scores, workspace, s),
                    "fp2_plan_mask launch");
}

fp2_status fp2_plan_mask_noalloc(const fp2_batch* batch, const fp2_q* q, int32_t num_kv_heads,
                                 const float* kbar, float tau, int32_t* row_ptr, int32_t* col_idx,
                                 int64_t col_capacity, int32_t* nnz, float* scores, void* stream) {
  BatchInfo info;
  fp2_status st = check_plan(batch, q, num_kv_heads, kbar, tau, row_ptr, col_idx, col_capacity, nnz, &info);
  if (st != FP2_OK) return st;
  const size_t wneed = plan_workspace_bytes(info, num_kv_heads);
  if (wneed > kPlanScratchBytes)
    return fail(FP2_ERR_CAPACITY, "this batch needs " + std::to_string(wneed) +
                                      " bytes of plan workspace; the allocation-free call holds at most " +
                                      std::to_string(kPlanScratchBytes) + " (use fp2_plan_mask)");
  if ((st = check_stream(stream, "fp2_plan_mask_noalloc")) != FP2_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (info.total_qblocks == 0) return hip_status(launch_zero_plan(row_ptr, nnz, s), "fp2_plan_mask_noalloc");
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_status(e, "fp2_plan_mask_noalloc: scratch address");
  return hip_status(launch_plan(batch, q, num_kv_heads, info, kbar, tau, row_ptr, col_idx, nnz,
                                scores, ws, s),
                    "fp2_plan_mask_noalloc launch");
}

size_t fp2_stage1_workspace_bytes(const fp2_batch* batch, int32_t num_kv_heads, int32_t head_dim) {
  BatchInfo info;
  if (check_batch(batch, &info) != FP2_OK || num_kv_heads < 1 || head_dim < 1) return 0;
  return stage1_workspace_bytes(info, num_kv_heads, head_dim);
}

fp2_status fp2_stage1(const fp2_batch* batch, const fp2_q* q, const fp2_kv* kv, float tau, float* kbar, float* vbar,
                      int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, int32_t* nnz, float* scores,
                      void* workspace, size_t workspace_bytes, void* stream) {
  BatchInfo info;
  fp2_status st = check_batch(batch, &info);
  if (st != FP2_OK) return st;
  if ((st = check_kv(kv, batch, info)) != FP2_OK) return st;
  if ((st = check_plan(batch, q, kv->num_kv_heads, kbar, tau, row_ptr, col_idx, col_capacity, nnz, &info)) != FP2_OK)
    return st;
  if (q->dtype != kv->dtype) return fail(FP2_ERR_UNSUPPORTED, "q and kv dtypes differ");
  if (q->head_dim != kv->head_dim) return fail(FP2_ERR_INVALID, "q and kv head_dim differ");
  if (info.total_kblocks > 0 && (!kbar || !vbar)) return fail(FP2_ERR_INVALID, "kbar/vbar is NULL");
  const size_t wneed = stage1_workspace_bytes(info, kv->num_kv_heads, kv->head_dim);
  if (wneed > 0 && !workspace) return fail(FP2_ERR_INVALID, "workspace is NULL");
  if (workspace_bytes < wneed)
    return fail(FP2_ERR_CAPACITY, "stage-1 workspace " + std::to_string(workspace_bytes) + " < " +
                                      std::to_string(wneed) + " bytes");
  if ((st = check_stream(stream, "fp2_stage1")) != FP2_OK) return st;
  if (hipError_t e = launch_check_pages(batch, kv, (hipStream_t)stream); e != hipSuccess)
    return hip_status(e, "fp2_stage1 bounds check");
  return hip_status(launch_stage1(batch, q, kv, info, tau, kbar, vbar, row_ptr, col_idx, nnz, scores, workspace,
                                  (hipStream_t)stream),
                    "fp2_stage1 launch");
}

size_t fp2_run_workspace_bytes(const fp2_batch* batch, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, fp2_dtype dtype) {
  BatchInfo info;
  if (check_batch(batch, &info) != FP2_OK || num_kv_heads < 1 || num_q_heads < num_kv_heads || head_dim < 1)
    return 0;
  return run_layout(info, batch->num_seqs, num_q_heads, num_kv_heads, head_dim, dtype).total;
}

fp2_status fp2_prefill_run(const fp2_batch* batch, const fp2_q* q, const fp2_kv* kv,
                           const int32_t* row_ptr, const int32_t* col_idx, const float* kbar,
                           const float* vbar, int32_t mean_correction, float softmax_scale,
                           fp2_out_dtype out_dtype, void* out, int32_t max_chunk_tiles, void* workspace,
                           size_t workspace_bytes, void* stream) {
  BatchInfo info;
  fp2_status st = check_batch(batch, &info);
  if (st != FP2_OK) return st;
  if ((st = check_kv(kv, batch, info)) != FP2_OK) return st;
  if ((st = check_q(q, kv->num_kv_heads, info, batch->block)) != FP2_OK) return st;
  if ((st = check_index_range(info, kv->num_kv_heads)) != FP2_OK) return st;
  if (q->dtype != kv->dtype) return fail(FP2_ERR_UNSUPPORTED, "q and kv dtypes differ");
  if (q->head_dim != kv->head_dim) return fail(FP2_ERR_INVALID, "q and kv head_dim differ");
  if (mean_correction != 0 && mean_correction != 1)
    return fail(FP2_ERR_INVALID, "mean_correction must be 0 or 1");
  if (out_dtype != FP2_OUT_BF16 && out_dtype != FP2_OUT_F32)
    return fail(FP2_ERR_INVALID, "unknown out_dtype");
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(FP2_ERR_INVALID, "softmax_scale must be finite and > 0");
  if (info.total_qblocks == 0) return FP2_OK;
  if (!row_ptr || !col_idx || !out) return fail(FP2_ERR_INVALID, "row_ptr/col_idx/out is NULL");
  if (mean_correction && (!kbar || !vbar)) return fail(FP2_ERR_INVALID, "mean correction needs kbar and vbar");
  if (mean_correction || vt_path(q->dtype, q->head_dim, info)) {
    const size_t wneed =
        run_layout(info, batch->num_seqs, q->num_q_heads, kv->num_kv_heads, kv->head_dim, kv->dtype).total;
    if (!workspace || workspace_bytes < wneed)
      return fail(FP2_ERR_CAPACITY, "run workspace " + std::to_string(workspace_bytes) + " < " +
                                        std::to_string(wneed) + " bytes");
  }
  if ((st = check_stream(stream, "fp2_prefill_run")) != FP2_OK) return st;
  if (hipError_t e = launch_check_pages(batch, kv, (hipStream_t)stream); e != hipSuccess)
    return hip_status(e, "fp2_prefill_run bounds check");
  if (hipError_t e = launch_check_csr(batch, info, kv->num_kv_heads, row_ptr, col_idx, (hipStream_t)stream);
      e != hipSuccess)
    return hip_status(e, "fp2_prefill_run bounds check");
  return hip_status(launch_prefill(batch, q, kv, info, row_ptr, col_idx, kbar, vbar,
                                   mean_correction, softmax_scale, out_dtype == FP2_OUT_F32, out, max_chunk_tiles,
                                   workspace, (hipStream_t)stream),
                    "fp2_prefill_run launch");
}

fp2_status fp2_debug_bounds_word(uint32_t* word) {
  if (!word) return fail(FP2_ERR_INVALID, "word is NULL");
  return read_bounds_word(word);
}

const char* fp2_last_error(void) { return fp2::last_error(); }

}  // extern "C"
