// Host-side internals shared by the C ABI (fp2_api.cpp), the argument checks
// (fp2_validate.cpp, plain C++ with no HIP dependency) and the kernel
// launchers (*.hip).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include <hip/hip_runtime_api.h>

#include "fp2.h"

namespace fp2 {

// Limits of the kernels (checked on the host; beyond them a call returns
// FP2_ERR_UNSUPPORTED).
constexpr int kMaxKBlocks = 16384;   // kept-block bitmask and score row held in LDS
constexpr int kPoolRowBytes = 4096;  // G*d*elem_size of one token of a KV group
constexpr int kRowsPerWG = 128;      // packed (head, token) query rows per attention workgroup

// Sizes derived from the host mirrors of a batch.
struct BatchInfo {
  int64_t total_q = 0;
  int64_t total_qblocks = 0;
  int64_t total_kblocks = 0;
  int64_t max_kblocks = 0;
  int64_t causal_pairs = 0;  // sum over query blocks of (last diagonal KV block + 1), one KV head
  int qblock = 0;            // B: query block tokens
  int kvblock = 0;           // KV block tokens (B, or 64 with B = 128)
};

// Sets the calling thread's error text and returns `st`.
fp2_status fail(fp2_status st, const std::string& msg);
const char* last_error();

fp2_status check_batch(const fp2_batch* b, BatchInfo* info);
fp2_status check_q(const fp2_q* q, int num_kv_heads, const BatchInfo& info, int block);
fp2_status check_kv(const fp2_kv* kv, const fp2_batch* b, const BatchInfo& info);
// The CSR's row_ptr, col_idx and nnz are int32: rows and entries (the causal
// pair count, reached at tau = +inf) must stay below 2^31.
fp2_status check_index_range(const BatchInfo& info, int num_kv_heads);

size_t plan_workspace_bytes(const BatchInfo& info, int num_kv_heads);
// fp2_stage1: the plan workspace followed by the pooled query means
// (float32 [Hkv, total_qblocks, d])
// the fused stage 1's workspace: the plan workspace, the pooled query means
// (256-byte aligned) and the select pass's claim counter (its own 256 bytes)
constexpr size_t kStage1TicketBytes = 256;
size_t stage1_workspace_bytes(const BatchInfo& info, int num_kv_heads, int head_dim);
// fp2_prefill_run runs the DMA kernel on V^T tiles for d = 128 and query
// blocks of 128 over KV blocks of 128 or of 64 (two to a tile), bf16 or e4m3,
// and the register-staged kernel otherwise.
inline bool vt_path(int dtype, int head_dim, const BatchInfo& info) {
  return (dtype == FP2_BF16 || dtype == FP2_FP8_E4M3) && head_dim == 128 && info.qblock == 128 &&
         (info.kvblock == 128 || info.kvblock == 64);
}

// Byte offsets of the parts of the fp2_prefill_run workspace.
struct RunLayout {
  size_t k16 = 0;      // bf16 kbar rows [Hkv, total_kblocks, d]
  size_t v16 = 0;      // fp16 vbar rows (register-staged path) or vbar^T tiles (V^T path)
  size_t vt = 0;       // V^T tiles of every KV block (V^T path; 64 keys a tile with 64-token blocks)
  size_t items = 0;    // V^T path: work items in launch order, int4 [rows + extra_cap]
  size_t splits = 0;   // V^T path: rows split into chunks, int4 [extra_cap]
  size_t rank_slot = 0;  // V^T path: per row {exact tiles, mean tiles, first partial slot, 0}, int4 [rows]
  size_t counters = 0;   // V^T path: item and split-row counts, int32 [4]
  size_t part = 0;       // V^T path: partial results of the chunks of split rows
  size_t info = 0;       // V^T path: per work item, the values its workgroup starts from, int32 [items, kInfoInts]
  size_t skip = 0;       // V^T path with correction: per CSR row, the skipped-block bitmask, u32 [rows, wskip]
  size_t mlist = 0;      // V^T path with correction: per CSR row, the first mean token of each mean tile, [rows, mtmax]
  size_t mcount = 0;     // V^T path with correction: per CSR row, its number of mean tiles, int32 [rows]
  int wskip = 0, mtmax = 0;
  int64_t extra_cap = 0;  // most work items beyond one per row (chunks of split rows)
  size_t total = 0;
  int64_t mt_cap = 0;  // vbar^T tiles per KV head (V^T path)
};
RunLayout run_layout(const BatchInfo& info, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                     int dtype);
// Work items beyond one per CSR row that the d = 128, B = 128 path may create
// by splitting the exact tiles of heavy rows (at most 256; fewer for small
// batches), and the floats of one partial result (per slot, slice and wave:
// O as 16 float4 per lane, then the reference max and row sum per lane).
constexpr int64_t kMaxExtraItems = 256;
// Size of the device array that serves as fp2_plan_mask_noalloc's workspace.
constexpr size_t kPlanScratchBytes = FP2_PLAN_NOALLOC_MAX_BYTES;
constexpr int64_t kPartFloatsPerWave = 64 * 64 + 2 * 64;
constexpr int kInfoInts = 48;  // a work item's record: see item_info_kernel
inline int plan_words(const BatchInfo& info) { return int((info.max_kblocks + 31) / 32); }

// Bounds-checking builds (FP2_DEBUG_BOUNDS, see fp2_device.h; csrc/debug_bounds.hip):
// the device address of the error word on the current device (nullptr in
// release builds), the check kernels (no-ops in release builds), and the
// word's read-and-clear (FP2_ERR_UNSUPPORTED in release builds).
const uint32_t* bounds_word();
hipError_t launch_check_pages(const fp2_batch* b, const fp2_kv* kv, hipStream_t stream);
hipError_t launch_check_csr(const fp2_batch* b, const BatchInfo& info, int num_kv_heads, const int32_t* row_ptr,
                            const int32_t* col_idx, hipStream_t stream);
fp2_status read_bounds_word(uint32_t* word);

}  // namespace fp2
