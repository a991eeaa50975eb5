// Stage 1a: per-block key/value means over a paged KV cache.
//
// FlashPrefill V2 (metallab.ai paper page), Figure 3 ("pools block-mean
// statistics") and Figure 4 (kbar_J, vbar_J of every block).
//
// One workgroup per global KV block.  A token's keys for all KV heads are one
// contiguous row of Hkv*d elements; the workgroup streams the block's rows
// with 16-byte loads (CH chunks per row, R token lanes side by side), sums in
// float32 per thread, then reduces the R token lanes through LDS in a fixed
// order.  HBM-bound: every K/V byte is read exactly once.
//
// The same kernel also writes a cache kept alongside the KV pages (chunked
// prefill: the blocks of a cached prefix keep their means from the call that
// computed them, so only the blocks holding new tokens are read again); a
// gather then lays the cache rows out as the dense [Hkv, total_kblocks, d]
// arrays the plan and the attention take, bit for bit the same values.
#include "fp2_device.h"
#include "fp2_internal.h"
#include "pool_device.h"

namespace fp2 {

namespace {

constexpr int kThreads = kPoolThreads;

template <int ESZ>
__global__ __launch_bounds__(kThreads) void block_stats_kernel(StatsArgs a) {
  constexpr int N = Chunk<ESZ>::N;
  __shared__ float red_k[kThreads][N + 1];
  __shared__ float red_v[kThreads][N + 1];
  __shared__ int s_pg[kPoolMaxPages];
  FP2_BOUNDS_GUARD(a.dbg);
  kv_block_stats<ESZ>(a, blockIdx.x, red_k, red_v, s_pg);
}

// kbar / vbar [g, kb, :] <- the cache rows of block kb (one workgroup per
// global KV block, float4 copies).
__global__ __launch_bounds__(kThreads) void gather_stats_kernel(StatsArgs a, const float* kc, const float* vc) {
  FP2_BOUNDS_GUARD(a.dbg);
  const int kb = blockIdx.x;
  const int s = find_seq(a.cu_kblocks, a.num_seqs, kb);
  const int J = kb - a.cu_kblocks[s];
  const int64_t crow = cache_row(a, a.page_table + (int64_t)s * a.max_pages, J);
  const int n4 = a.hkv * a.d / 4;
  for (int i = threadIdx.x; i < n4; i += kThreads) {
    const int g = (4 * i) / a.d, dim = (4 * i) % a.d;
    const int64_t src = (crow * a.hkv + g) * a.d + dim;
    const int64_t dst = ((int64_t)g * a.total_kblocks + kb) * a.d + dim;
    *reinterpret_cast<f32x4*>(a.kbar + dst) = *reinterpret_cast<const f32x4*>(kc + src);
    *reinterpret_cast<f32x4*>(a.vbar + dst) = *reinterpret_cast<const f32x4*>(vc + src);
  }
}

hipError_t launch_stats(const StatsArgs& a, int dtype, int64_t total_kblocks, hipStream_t stream) {
  dim3 grid((unsigned)total_kblocks);
  if (dtype == FP2_BF16)
    hipLaunchKernelGGL(block_stats_kernel<2>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(block_stats_kernel<1>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_stats_cached(const fp2_batch* b, const fp2_kv* kv, const BatchInfo& info, float* kcache,
                                     float* vcache, int refresh, hipStream_t stream) {
  if (info.total_kblocks == 0) return hipSuccess;
  StatsArgs a = stats_args(b, kv, info, kcache, vcache);
  a.cached = 1;
  a.refresh = refresh;
  return launch_stats(a, kv->dtype, info.total_kblocks, stream);
}

hipError_t launch_gather_stats(const fp2_batch* b, const fp2_kv* kv, const BatchInfo& info, const float* kcache,
                               const float* vcache, float* kbar, float* vbar, hipStream_t stream) {
  if (info.total_kblocks == 0) return hipSuccess;
  StatsArgs a = stats_args(b, kv, info, kbar, vbar);
  hipLaunchKernelGGL(gather_stats_kernel, dim3((unsigned)info.total_kblocks), dim3(kThreads), 0, stream, a, kcache,
                     vcache);
  return hipGetLastError();
}

hipError_t launch_block_stats(const fp2_batch* b, const fp2_kv* kv, const BatchInfo& info,
                              float* kbar, float* vbar, hipStream_t stream) {
  if (info.total_kblocks == 0) return hipSuccess;
  return launch_stats(stats_args(b, kv, info, kbar, vbar), kv->dtype, info.total_kblocks, stream);
}

}  // namespace fp2
