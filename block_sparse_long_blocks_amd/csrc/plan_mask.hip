// Stage 1b: pattern discovery (PackGQA query pooling + pooled block scores)
// and max-based dynamic thresholding, emitting a CSR of kept blocks per
// (query block, KV head).
//
// FlashPrefill V2 (metallab.ai paper page): Figure 3 (pack queries with
// PackGQA, pool block means, CSR index of selected blocks), the abstract
// ("instantaneous pattern discovery and max-based dynamic thresholding") and
// Table 7 (CSR per KV head).  Block 0 and the diagonal block are always kept
// (with 64-token KV blocks under 128-token query blocks, Table 7's pairing,
// the diagonal is the run of KV blocks holding the query block's positions).
//
// Three launches, no host synchronisation:
//   score_select : one workgroup per CSR row (query block I, KV head g).
//                  Pools qbar over the block's tokens and the G heads of the
//                  group (float32, fixed order), scores every causal KV block
//                  against kbar (float32 dot products, d/8 lanes per kbar
//                  row so that the loads coalesce), reduces the row
//                  maximum, applies s >= max - tau and writes a keep bitmask
//                  and the row's kept count.
//   scan_counts  : one workgroup; exclusive scan of the counts -> row_ptr, nnz.
//   fill_cols    : one workgroup per row; expands the bitmask into ascending
//                  KV-block indices at row_ptr[row].
#include <mutex>

#include "fp2_device.h"
#include "fp2_internal.h"

namespace fp2 {

// Workspace of fp2_plan_mask_noalloc (callers that cannot allocate): the
// keep bitmask and kept counts live in this array, one copy per GPU, held
// until the process ends.  Host code never uses its name as an address:
// scratch_address() looks the device address up once per device.
static __device__ __align__(256) uint8_t scratch[kPlanScratchBytes];

namespace {

constexpr int kThreads = 256;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

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

template <int ESZ>
__global__ __launch_bounds__(kThreads) void score_select_kernel(PlanArgs a) {
  constexpr int N = 16 / ESZ;  // elements per 16-byte chunk
  extern __shared__ float s_scores[];  // [max_kblocks]
  __shared__ float red[kThreads][N + 1];
  __shared__ float s_qbar[128];
  __shared__ float s_wmax[kThreads / 64];
  __shared__ int s_wcnt[kThreads / 64];

  const int qb = blockIdx.x;  // global query block
  const int g = blockIdx.y;   // KV head
  const int t = threadIdx.x;
  const int s = find_seq(a.cu_qblocks, a.num_seqs, qb);
  const int I = qb - a.cu_qblocks[s];
  const int q0 = a.cu_seqlens_q[s];
  const int n = a.cu_seqlens_q[s + 1] - q0;
  const int T = a.seqlens_k[s];
  const int P = T - n;
  const int ntok = min(a.qblock, n - I * a.qblock);
  // the diagonal: the KV blocks holding one of the query block's positions
  const int dlo = (P + I * a.qblock) / a.kvblock;
  const int diag = (P + I * a.qblock + ntok - 1) / a.kvblock;  // the last causal KV block
  const int G = a.hq / a.hkv;

  // ---- pool qbar over ntok tokens x G heads (the group's heads are adjacent)
  const int row_bytes = G * a.d * ESZ;  // <= 4096: CH <= 256
  const int CH = row_bytes / 16;
  const int R = kThreads / CH;
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

  // ---- scores for J = 0..diag: float32 dot(qbar, kbar_J) * scale.  LPB =
  // d/8 lanes share a kbar row (8 floats each, so a wave's loads cover
  // 64/LPB whole rows), then sum their partials across the lanes.
  const float* kb = a.kbar + ((int64_t)g * a.total_kblocks + a.cu_kblocks[s]) * a.d;
  const int lpb = a.d / 8;           // 16 (d = 128) or 8 (d = 64)
  const int bpw = 64 / lpb;          // rows per wave and load
  const int lane = t & 63, sub = lane % lpb;
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = s_qbar[8 * sub + e];
  float lmax = -INFINITY;
  constexpr int UJ = 4;  // row groups whose loads are in flight together
  const int jstep = (kThreads / 64) * bpw;
  for (int J0 = (t >> 6) * bpw; J0 <= diag; J0 += UJ * jstep) {
    f32x4 k0[UJ], k1[UJ];
#pragma unroll
    for (int u = 0; u < UJ; ++u) {
      const int J = J0 + u * jstep + lane / lpb;
      k0[u] = k1[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (J <= diag) {
        const f32x4* kr = reinterpret_cast<const f32x4*>(kb + (int64_t)J * a.d + 8 * sub);
        k0[u] = kr[0];
        k1[u] = kr[1];
      }
    }
#pragma unroll
    for (int u = 0; u < UJ; ++u) {
      const int J = J0 + u * jstep + lane / lpb;
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p0 = fmaf(qv[e], k0[u][e], p0);
        p1 = fmaf(qv[4 + e], k1[u][e], p1);
      }
      float p = p0 + p1;
      for (int m = lpb >> 1; m > 0; m >>= 1) p += __shfl_xor(p, m);
      if (J <= diag) {
        const float sc = p * a.scale;
        if (sub == 0) s_scores[J] = sc;
        lmax = fmaxf(lmax, sc);
      }
    }
  }
  lmax = wave_max(lmax);
  if ((t & 63) == 0) s_wmax[t >> 6] = lmax;
  __syncthreads();
  float rmax = s_wmax[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) rmax = fmaxf(rmax, s_wmax[w]);
  const float thr = rmax - a.tau;

  // ---- keep bitmask (forced: block 0 and the diagonal run) and kept count
  const int row = g * a.total_qblocks + qb;
  int cnt = 0;
  for (int w = t; w < a.W; w += kThreads) {
    uint32_t word = 0;
    const int j0 = w * 32;
    for (int b = 0; b < 32; ++b) {
      const int J = j0 + b;
      if (J <= diag && (s_scores[J] >= thr || J == 0 || J >= dlo)) word |= 1u << b;
    }
    a.bits[(int64_t)row * a.W + w] = word;
    cnt += __popc(word);
  }
  if (a.scores_out) {
    float* so = a.scores_out + (int64_t)row * a.max_kblocks;
    for (int J = t; J < a.max_kblocks; J += kThreads) so[J] = J <= diag ? s_scores[J] : -INFINITY;
  }
  cnt = wave_sum_i(cnt);
  if ((t & 63) == 0) s_wcnt[t >> 6] = cnt;
  __syncthreads();
  if (t == 0) {
    int tot = 0;
    for (int w = 0; w < kThreads / 64; ++w) tot += s_wcnt[w];
    a.counts[row] = tot;
  }
}

// Exclusive scan of counts[0..rows) -> row_ptr[0..rows], nnz = row_ptr[rows].
__global__ __launch_bounds__(1024) void scan_counts_kernel(const int32_t* __restrict__ counts,
                                                           int rows, int32_t* __restrict__ row_ptr,
                                                           int32_t* __restrict__ nnz) {
  __shared__ int s_part[1024];
  const int t = threadIdx.x;
  const int per = (rows + 1023) / 1024;
  const int lo = min(rows, t * per), hi = min(rows, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += counts[i];
  s_part[t] = sum;
  __syncthreads();
  // Hillis-Steele inclusive scan over 1024 partials
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = t >= o ? s_part[t - o] : 0;
    __syncthreads();
    s_part[t] += v;
    __syncthreads();
  }
  int run = s_part[t] - sum;  // exclusive prefix of this thread's chunk
  for (int i = lo; i < hi; ++i) {
    row_ptr[i] = run;
    run += counts[i];
  }
  if (t == 1023) {
    row_ptr[rows] = s_part[1023];
    nnz[0] = s_part[1023];
  }
}

// Expand each row's bitmask into ascending column indices.
__global__ __launch_bounds__(kThreads) void fill_cols_kernel(const uint32_t* __restrict__ bits, int W,
                                                             const int32_t* __restrict__ row_ptr,
                                                             int32_t* __restrict__ col_idx) {
  __shared__ int s_wsum[kThreads / 64];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  int base = row_ptr[row];
  for (int w0 = 0; w0 < W; w0 += kThreads) {
    const int w = w0 + t;
    const uint32_t word = w < W ? bits[(int64_t)row * W + w] : 0u;
    const int c = __popc(word);
    // exclusive scan of c across the workgroup
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if ((t & 63) >= o) incl += v;
    }
    if ((t & 63) == 63) s_wsum[t >> 6] = incl;
    __syncthreads();
    int wave_off = 0, total = 0;
    for (int i = 0; i < kThreads / 64; ++i) {
      if (i < (t >> 6)) wave_off += s_wsum[i];
      total += s_wsum[i];
    }
    int pos = base + wave_off + incl - c;
    uint32_t m = word;
    while (m) {
      const int b = __ffs(m) - 1;
      col_idx[pos++] = w * 32 + b;
      m &= m - 1;
    }
    base += total;
    __syncthreads();
  }
}

// An empty plan: row_ptr = {0}, nnz = 0 (a kernel, not a memset, so that the
// call can be captured into a HIP graph).
__global__ void zero_plan_kernel(int32_t* row_ptr, int32_t* nnz) {
  if (threadIdx.x == 0) {
    row_ptr[0] = 0;
    nnz[0] = 0;
  }
}

}  // namespace

hipError_t launch_zero_plan(int32_t* row_ptr, int32_t* nnz, hipStream_t stream) {
  hipLaunchKernelGGL(zero_plan_kernel, dim3(1), dim3(64), 0, stream, row_ptr, nnz);
  return hipGetLastError();
}

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with this device current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_plan(const fp2_batch* b, const fp2_q* q, int hkv, const BatchInfo& info,
                       const float* kbar, float tau, int32_t* row_ptr, int32_t* col_idx,
                       int32_t* nnz, float* scores, void* workspace, hipStream_t stream) {
  const int rows = (int)(info.total_qblocks * hkv);
  const int W = plan_words(info);
  uint32_t* bits = static_cast<uint32_t*>(workspace);
  size_t off = ((size_t)rows * W * 4 + 255) & ~size_t(255);
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + off);

  PlanArgs a;
  a.cu_seqlens_q = b->cu_seqlens_q;
  a.seqlens_k = b->seqlens_k;
  a.cu_qblocks = b->cu_qblocks;
  a.cu_kblocks = b->cu_kblocks;
  a.q = static_cast<const uint8_t*>(q->q);
  a.q_scale = q->q_scale;
  a.kbar = kbar;
  a.bits = bits;
  a.counts = counts;
  a.scores_out = scores;
  a.tau = tau;
  a.scale = 1.0f / sqrtf((float)q->head_dim);
  a.num_seqs = b->num_seqs;
  a.hq = q->num_q_heads;
  a.hkv = hkv;
  a.d = q->head_dim;
  a.qblock = info.qblock;
  a.kvblock = info.kvblock;
  a.total_qblocks = (int)info.total_qblocks;
  a.total_kblocks = (int)info.total_kblocks;
  a.W = W;
  a.max_kblocks = (int)info.max_kblocks;
  const size_t lds = (size_t)info.max_kblocks * sizeof(float);
  dim3 grid((unsigned)info.total_qblocks, (unsigned)hkv);
  if (q->dtype == FP2_BF16)
    hipLaunchKernelGGL(score_select_kernel<2>, grid, dim3(kThreads), lds, stream, a);
  else
    hipLaunchKernelGGL(score_select_kernel<1>, grid, dim3(kThreads), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_counts_kernel, dim3(1), dim3(1024), 0, stream, counts, rows, row_ptr, nnz);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fill_cols_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, bits, W,
                     row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace fp2
