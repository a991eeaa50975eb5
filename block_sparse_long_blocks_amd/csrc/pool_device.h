// Block-mean pooling shared by the stage-1 kernels: the KV block means
// (fp2_block_stats, and the fused stage-1 pass) and the pooled query means
// (fp2_plan_mask's pooling phase, and the fused pass).  One definition, so
// that every path sums the same elements in the same order.
//
// FlashPrefill V2 (metallab.ai paper page), Figure 3 (PackGQA packing and
// block-mean pooling in Stage 1) and Figure 4 (kbar_J, vbar_J).
#pragma once

#include "fp2_device.h"
#include "fp2_internal.h"

namespace fp2 {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kPoolMaxPages = 132;  // page entries of one KV block (<= 128 tokens, pages of >= 1 token)

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
  const uint32_t* dbg;  // bounds-checking builds: the error word (see fp2_device.h), else nullptr
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

// Means of K and V over the tokens of global KV block kb, all KV heads
// (one workgroup of kPoolThreads threads; red_k, red_v: LDS of kPoolThreads x (N+1)
// floats each).  A token's keys for all KV heads are one contiguous row of
// Hkv*d elements; the workgroup streams the block's rows with 16-byte loads
// (CH chunks per row, R token lanes side by side), sums in float32 per
// thread, then reduces the R token lanes through LDS in a fixed order.
template <int ESZ>
__device__ __forceinline__ void kv_block_stats(const StatsArgs& a, int kb, float (*red_k)[Chunk<ESZ>::N + 1],
                                               float (*red_v)[Chunk<ESZ>::N + 1], int* s_pg) {
  using C = Chunk<ESZ>;
  constexpr int N = C::N;
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
  const int R = CH >= kPoolThreads ? 1 : kPoolThreads / CH;  // token lanes
  const int t = threadIdx.x;
  const int32_t* pt = a.page_table + (int64_t)s * a.max_pages;
  // the page entries of the block's tokens, loaded once into LDS (s_pg:
  // kPoolMaxPages ints), so that the streaming loads below do not each wait
  // on a page-table load
  int pi0, slot0, pi1, slot1;
  a.pm.split(J * a.block, pi0, slot0);
  a.pm.split(J * a.block + count - 1, pi1, slot1);
  for (int i = t; i <= pi1 - pi0; i += kPoolThreads) s_pg[i] = pt[pi0 + i];
  __syncthreads();

  for (int cbase = 0; cbase < CH; cbase += kPoolThreads) {
    const int c = cbase + (t % min(CH, kPoolThreads));
    const int r = t / min(CH, kPoolThreads);
    const bool active = r < R && c < CH;
    float acck[N], accv[N];
#pragma unroll
    for (int e = 0; e < N; ++e) acck[e] = accv[e] = 0.f;
    if (active) {
      constexpr int U = 8;  // tokens in flight per thread
      int tok = r;
      for (; tok + (U - 1) * R < count; tok += U * R) {
        uint4 wk[U], wv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int pos = J * a.block + tok + u * R;
          int pi, slot;
          a.pm.split(pos, pi, slot);
          const int64_t off = (((int64_t)s_pg[pi - pi0] * a.page_size + slot) * row_bytes) + c * 16;
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
        const int64_t off = (((int64_t)s_pg[pi - pi0] * a.page_size + slot) * row_bytes) + c * 16;
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
    const int cw = min(CH, kPoolThreads);
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
      if (ESZ == 1) {  // e4m3: one scale per (page, head); page_size == KV block, so the block's page is s_pg[0]
        const int64_t page = s_pg[0];
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

inline StatsArgs stats_args(const fp2_batch* b, const fp2_kv* kv, const BatchInfo& info, float* kbar, float* vbar) {
  StatsArgs a;
  a.dbg = bounds_word();
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

struct PlanArgs {
  const int32_t* cu_seqlens_q;
  const int32_t* seqlens_k;
  const int32_t* cu_qblocks;
  const int32_t* cu_kblocks;
  const uint8_t* q;
  const float* q_scale;
  const float* kbar;
  uint32_t* bits;       // [rows, W]
  int32_t* counts;      // [rows]
  float* scores_out;    // optional [rows, max_kblocks]
  float* qbar;          // fused stage 1: pooled query means [Hkv, total_qblocks, d]
  int32_t* ticket;      // fused stage 1: the select pass's work-item claim counter
  float tau, scale;
  int num_seqs, hq, hkv, d, total_qblocks, total_kblocks, W, max_kblocks;
  int qblock, kvblock;  // query block and KV block tokens (kvblock divides qblock)
};

template <int ESZ>
__device__ __forceinline__ void add_chunk(float* acc, uint4 w, float mul) {
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
  if (ESZ == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16lo(v[i]);
      acc[2 * i + 1] += bf16hi(v[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 f = e4m3x4_to_f32(v[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[4 * i + q] += f[q] * mul;
    }
  }
}

// qbar of query block qb (global) and KV head g: the mean of Q over the
// block's ntok tokens and the G query heads of the group (adjacent in a
// token's row), float32 in a fixed order, into s_qbar[0..d).  One workgroup
// of kPoolThreads threads; red: LDS of kPoolThreads x (N+1) floats.
template <int ESZ>
__device__ __forceinline__ void pool_qbar(const PlanArgs& a, int qb, int g, float (*red)[16 / ESZ + 1],
                                          float* s_qbar) {
  constexpr int N = 16 / ESZ;  // elements per 16-byte chunk
  const int t = threadIdx.x;
  const int s = find_seq(a.cu_qblocks, a.num_seqs, qb);
  const int I = qb - a.cu_qblocks[s];
  const int q0 = a.cu_seqlens_q[s];
  const int n = a.cu_seqlens_q[s + 1] - q0;
  const int ntok = min(a.qblock, n - I * a.qblock);
  const int G = a.hq / a.hkv;
  const int row_bytes = G * a.d * ESZ;  // <= 4096: CH <= 256
  const int CH = row_bytes / 16;
  const int R = kPoolThreads / CH;
  const int c = t % CH, r = t / CH;
  float acc[N];
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = 0.f;
  if (r < R) {
    const int elem0 = c * N;
    const int h = g * G + elem0 / a.d;  // a chunk stays within one head
    float mul = 1.f;
    if (ESZ == 1) mul = a.q_scale[(int64_t)qb * a.hq + h];
    const uint8_t* base = a.q + ((int64_t)(q0 + I * a.qblock) * a.hq + g * G) * a.d * ESZ + c * 16;
    const int64_t tok_stride = (int64_t)a.hq * a.d * ESZ;
    constexpr int U = 8;
    int tok = r;
    for (; tok + (U - 1) * R < ntok; tok += U * R) {
      uint4 w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) w[u] = *reinterpret_cast<const uint4*>(base + (tok + u * R) * tok_stride);
#pragma unroll
      for (int u = 0; u < U; ++u) add_chunk<ESZ>(acc, w[u], mul);
    }
    for (; tok < ntok; tok += R) add_chunk<ESZ>(acc, *reinterpret_cast<const uint4*>(base + tok * tok_stride), mul);
  }
#pragma unroll
  for (int e = 0; e < N; ++e) red[t][e] = acc[e];
  __syncthreads();
  if (t < a.d) {
    // element t of qbar: sum over heads hh and token lanes rr of chunk (hh*d + t)/N
    float sum = 0.f;
    for (int hh = 0; hh < G; ++hh) {
      const int el = hh * a.d + t;
      const int cc = el / N, ee = el % N;
      float part = 0.f;
      for (int rr = 0; rr < R; ++rr) part += red[rr * CH + cc][ee];
      sum += part;
    }
    s_qbar[t] = sum / (float)(G * ntok);
  }
  __syncthreads();

}

}  // namespace
}  // namespace fp2
