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

namespace fp2 {

namespace {

constexpr int kThreads = 256;

template <int ESZ>
struct Chunk;  // 16 bytes of elements -> floats
template <>
struct Chunk<2> {
  static constexpr int N = 8;
  __device__ static void add(float* acc, uint4 w) {
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16lo(v[i]);
      acc[2 * i + 1] += bf16hi(v[i]);
    }
  }
};
template <>
struct Chunk<1> {
  static constexpr int N = 16;
  __device__ static void add(float* acc, uint4 w) {
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 f = e4m3x4_to_f32(v[i]);
      acc[4 * i + 0] += f[0];
      acc[4 * i + 1] += f[1];
      acc[4 * i + 2] += f[2];
      acc[4 * i + 3] += f[3];
    }
  }
};

struct StatsArgs {
  const int32_t* cu_kblocks;
  const int32_t* seqlens_k;
  const int32_t* page_table;
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const float* k_scale;
  const float* v_scale;
  float* kbar;
  float* vbar;
  const int32_t* cu_seqlens_q;
  PageMap pm;
  int num_seqs, max_pages, page_size, hkv, d, block, total_kblocks;
  int cached;   // 1: kbar / vbar are the paged caches [cache rows, Hkv, d]
  int refresh;  // cached: 1 also recomputes the blocks of the cached prefix
  int bpp;      // cached: KV blocks per page, max(1, page_size / block)
};

// Cache row of block J of a sequence with page table pt: the block's first
// page, times the blocks a page holds, plus the block's place in its page.
__device__ __forceinline__ int64_t cache_row(const StatsArgs& a, const int32_t* pt, int J) {
  return (int64_t)pt[(int64_t)J * a.block / a.page_size] * a.bpp + J % a.bpp;
}

template <int ESZ>
__global__ __launch_bounds__(kThreads) void block_stats_kernel(StatsArgs a) {
  using C = Chunk<ESZ>;
  constexpr int N = C::N;
  __shared__ float red_k[kThreads][N + 1];
  __shared__ float red_v[kThreads][N + 1];

  const int kb = blockIdx.x;
  const int s = find_seq(a.cu_kblocks, a.num_seqs, kb);
  const int J = kb - a.cu_kblocks[s];
  const int T = a.seqlens_k[s];
  if (a.cached && !a.refresh) {
    const int n = a.cu_seqlens_q[s + 1] - a.cu_seqlens_q[s];
    if (J < (T - n) / a.block) return;  // a block of the cached prefix: its cache row stands
  }
  const int count = min(a.block, T - J * a.block);
  const int row_bytes = a.hkv * a.d * ESZ;
  const int CH = row_bytes / 16;                  // 16-byte chunks per token row
  const int R = CH >= kThreads ? 1 : kThreads / CH;  // token lanes
  const int t = threadIdx.x;
  const int32_t* pt = a.page_table + (int64_t)s * a.max_pages;

  for (int cbase = 0; cbase < CH; cbase += kThreads) {
    const int c = cbase + (t % min(CH, kThreads));
    const int r = t / min(CH, kThreads);
    const bool active = r < R && c < CH;
    float acck[N], accv[N];
#pragma unroll
    for (int e = 0; e < N; ++e) acck[e] = accv[e] = 0.f;
    if (active) {
      constexpr int U = 4;  // tokens in flight per thread
      int tok = r;
      for (; tok + (U - 1) * R < count; tok += U * R) {
        uint4 wk[U], wv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int pos = J * a.block + tok + u * R;
          int pi, slot;
          a.pm.split(pos, pi, slot);
          const int64_t off = (((int64_t)pt[pi] * a.page_size + slot) * row_bytes) + c * 16;
          wk[u] = *reinterpret_cast<const uint4*>(a.k_pages + off);
          wv[u] = *reinterpret_cast<const uint4*>(a.v_pages + off);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          C::add(acck, wk[u]);
          C::add(accv, wv[u]);
        }
      }
      for (; tok < count; tok += R) {
        const int pos = J * a.block + tok;
        int pi, slot;
        a.pm.split(pos, pi, slot);
        const int64_t off = (((int64_t)pt[pi] * a.page_size + slot) * row_bytes) + c * 16;
        C::add(acck, *reinterpret_cast<const uint4*>(a.k_pages + off));
        C::add(accv, *reinterpret_cast<const uint4*>(a.v_pages + off));
      }
    }
#pragma unroll
    for (int e = 0; e < N; ++e) {
      red_k[t][e] = acck[e];
      red_v[t][e] = accv[e];
    }
    __syncthreads();
    const int cw = min(CH, kThreads);
    if (t < cw && cbase + t < CH) {
      const int cc = cbase + t;
      float sk[N], sv[N];
#pragma unroll
      for (int e = 0; e < N; ++e) sk[e] = sv[e] = 0.f;
      for (int rr = 0; rr < R; ++rr) {
#pragma unroll
        for (int e = 0; e < N; ++e) {
          sk[e] += red_k[rr * cw + t][e];
          sv[e] += red_v[rr * cw + t][e];
        }
      }
      const int elem0 = cc * N;       // first element of this chunk within the row
      const int g = elem0 / a.d;      // a chunk never straddles two heads (d % N == 0)
      const int dim = elem0 % a.d;
      float mk = 1.f, mv = 1.f;
      if (ESZ == 1) {  // e4m3: one scale per (page, head); page_size == KV block
        const int64_t page = pt[J];
        mk = a.k_scale[page * a.hkv + g];
        mv = a.v_scale[page * a.hkv + g];
      }
      const float inv = (float)count;
      const int64_t orow = a.cached ? cache_row(a, pt, J) * a.hkv + g : (int64_t)g * a.total_kblocks + kb;
      float* ok = a.kbar + orow * a.d + dim;
      float* ov = a.vbar + orow * a.d + dim;
#pragma unroll
      for (int e = 0; e < N; e += 4) {
        f32x4 vk, vv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          vk[q] = (sk[e + q] * mk) / inv;
          vv[q] = (sv[e + q] * mv) / inv;
        }
        *reinterpret_cast<f32x4*>(ok + e) = vk;
        *reinterpret_cast<f32x4*>(ov + e) = vv;
      }
    }
    __syncthreads();
  }
}

// kbar / vbar [g, kb, :] <- the cache rows of block kb (one workgroup per
// global KV block, float4 copies).
__global__ __launch_bounds__(kThreads) void gather_stats_kernel(StatsArgs a, const float* kc, const float* vc) {
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

StatsArgs stats_args(const fp2_batch* b, const fp2_kv* kv, const BatchInfo& info, float* kbar, float* vbar) {
  StatsArgs a;
  a.cu_kblocks = b->cu_kblocks;
  a.seqlens_k = b->seqlens_k;
  a.cu_seqlens_q = b->cu_seqlens_q;
  a.page_table = kv->page_table;
  a.k_pages = static_cast<const uint8_t*>(kv->k_pages);
  a.v_pages = static_cast<const uint8_t*>(kv->v_pages);
  a.k_scale = kv->k_scale;
  a.v_scale = kv->v_scale;
  a.kbar = kbar;
  a.vbar = vbar;
  a.num_seqs = b->num_seqs;
  a.max_pages = kv->max_pages_per_seq;
  a.page_size = kv->page_size;
  a.pm = PageMap::make(kv->page_size);
  a.hkv = kv->num_kv_heads;
  a.d = kv->head_dim;
  a.block = info.kvblock;
  a.total_kblocks = (int)info.total_kblocks;
  a.cached = 0;
  a.refresh = 1;
  a.bpp = kv->page_size >= info.kvblock ? kv->page_size / info.kvblock : 1;
  return a;
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
