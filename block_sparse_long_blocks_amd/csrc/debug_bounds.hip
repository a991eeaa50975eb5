// Bounds-checking builds (FP2_DEBUG_BOUNDS): the check kernels that run ahead
// of a call's kernels and the error word they set (see fp2_device.h).  Page
// ids and CSR contents are device data the host checks cannot see; the
// release library trusts them (include/fp2.h), a build with FP2_DEBUG_BOUNDS
// verifies them on the device and reports a violation through
// fp2_debug_bounds_word() instead of reading past a buffer.
//
// Checked, per call: every page id a sequence's tokens use lies in
// [0, num_pages) (calls that read the KV cache); and for fp2_prefill_run
// every CSR row pointer lies in order within the causal pair count, and
// every row's entries are strictly ascending KV blocks of the row's own
// sequence from block 0 through its last diagonal block (the contract of
// include/fp2.h).
#include "fp2_device.h"
#include "fp2_internal.h"

namespace fp2 {

#ifdef FP2_DEBUG_BOUNDS

namespace {

__device__ uint32_t g_bounds_word;

// (s, page index p): grid (pages / 256, sequences)
__global__ __launch_bounds__(256) void check_pages_kernel(const int32_t* seqlens_k, const int32_t* page_table,
                                                          int max_pages, int page_size, int num_pages,
                                                          uint32_t* word) {
  const int s = blockIdx.y;
  const int p = blockIdx.x * 256 + threadIdx.x;
  const int T = seqlens_k[s];
  if (p >= (T + page_size - 1) / page_size) return;
  const int v = page_table[(int64_t)s * max_pages + p];
  if (v < 0 || v >= num_pages) atomicOr(word, 1u);
}

// one thread per CSR row r = g * total_qblocks + global query block
__global__ __launch_bounds__(256) void check_csr_kernel(const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                                                        const int32_t* cu_qblocks, int num_seqs, int block,
                                                        int kvblock, int total_qblocks, int rows, int64_t max_nnz,
                                                        const int32_t* row_ptr, const int32_t* col_idx,
                                                        uint32_t* word) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int qb = r % total_qblocks;
  const int s = find_seq(cu_qblocks, num_seqs, qb);
  const int I = qb - cu_qblocks[s];
  const int n = cu_seqlens_q[s + 1] - cu_seqlens_q[s];
  const int P = seqlens_k[s] - n;
  const int diag = (P + min((I + 1) * block, n) - 1) / kvblock;  // the row's last diagonal KV block
  const int b = row_ptr[r], e = row_ptr[r + 1];
  if ((r == 0 && b != 0) || b > e || e > max_nnz || e - b > diag + 1) {
    atomicOr(word, 4u);
    return;
  }
  int prev = -1;
  for (int k = b; k < e; ++k) {
    const int c = col_idx[k];
    if (c <= prev || c > diag) {
      atomicOr(word, 2u);
      return;
    }
    prev = c;
  }
  if (e == b || col_idx[b] != 0 || prev != diag) atomicOr(word, 2u);
}

}  // namespace

const uint32_t* bounds_word() {
  static void* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (!addr[dev] && hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(g_bounds_word)) != hipSuccess) return nullptr;
  return static_cast<const uint32_t*>(addr[dev]);
}

hipError_t launch_check_pages(const fp2_batch* b, const fp2_kv* kv, hipStream_t stream) {
  uint32_t* w = const_cast<uint32_t*>(bounds_word());
  if (!w) return hipErrorInvalidSymbol;
  if (b->num_seqs <= 0 || kv->max_pages_per_seq <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_pages_kernel, dim3((unsigned)((kv->max_pages_per_seq + 255) / 256), (unsigned)b->num_seqs),
                     dim3(256), 0, stream, b->seqlens_k, kv->page_table, kv->max_pages_per_seq, kv->page_size,
                     kv->num_pages, w);
  return hipGetLastError();
}

hipError_t launch_check_csr(const fp2_batch* b, const BatchInfo& info, int num_kv_heads, const int32_t* row_ptr,
                            const int32_t* col_idx, hipStream_t stream) {
  uint32_t* w = const_cast<uint32_t*>(bounds_word());
  if (!w) return hipErrorInvalidSymbol;
  const int64_t rows = (int64_t)num_kv_heads * info.total_qblocks;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_csr_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, b->cu_seqlens_q,
                     b->seqlens_k, b->cu_qblocks, b->num_seqs, b->block, info.kvblock, (int)info.total_qblocks,
                     (int)rows, info.causal_pairs * num_kv_heads, row_ptr, col_idx, w);
  return hipGetLastError();
}

fp2_status read_bounds_word(uint32_t* word) {
  uint32_t v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_bounds_word), sizeof(v), 0, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(FP2_ERR_HIP, "fp2_debug_bounds_word: reading the error word failed");
  const uint32_t zero = 0;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_bounds_word), &zero, sizeof(zero), 0, hipMemcpyHostToDevice) != hipSuccess)
    return fail(FP2_ERR_HIP, "fp2_debug_bounds_word: clearing the error word failed");
  *word = v;
  return FP2_OK;
}

#else  // release build: nothing is checked on the device

const uint32_t* bounds_word() { return nullptr; }
hipError_t launch_check_pages(const fp2_batch*, const fp2_kv*, hipStream_t) { return hipSuccess; }
hipError_t launch_check_csr(const fp2_batch*, const BatchInfo&, int, const int32_t*, const int32_t*, hipStream_t) {
  return hipSuccess;
}
fp2_status read_bounds_word(uint32_t*) {
  return fail(FP2_ERR_UNSUPPORTED, "fp2_debug_bounds_word: this library was built without FP2_DEBUG_BOUNDS");
}

#endif

}  // namespace fp2
