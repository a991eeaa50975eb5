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
#include "pool_device.h"

namespace fp2 {

// Workspace of fp2_plan_mask_noalloc (callers that cannot allocate): the
// keep bitmask and kept counts live in this array, one copy per GPU, held
// until the process ends.  Host code never uses its name as an address:
// scratch_address() looks the device address up once per device.
static __device__ __align__(256) uint8_t scratch[kPlanScratchBytes];

namespace {

constexpr int kThreads = kPoolThreads;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Sum of p over the lpb lanes that share a kbar row (lpb = d/8: 16 or 8),
// lane 0 of the group holding the tree ((p0 + p8) + (p4 + p12)) + ...: with
// 16 lanes by DPP row rotations (one vector add each, no LDS traffic), with
// 8 by cross-lane shuffles in the same order.
__device__ __forceinline__ float row_sum(float p, int lpb) {
  if (lpb == 16) {
    p += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(p), 0x128, 0xf, 0xf, false));  // row_ror:8
    p += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(p), 0x124, 0xf, 0xf, false));  // row_ror:4
    p += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(p), 0x122, 0xf, 0xf, false));  // row_ror:2
    p += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(p), 0x121, 0xf, 0xf, false));  // row_ror:1
    return p;
  }
  for (int m = lpb >> 1; m > 0; m >>= 1) p += __shfl_xor(p, m);
  return p;
}

template <int ESZ, bool POOLED>
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

  // ---- qbar: pooled here, or (fused stage 1) read back from the pooling pass
  if constexpr (POOLED) {
    if (t < a.d) s_qbar[t] = a.qbar[((int64_t)g * a.total_qblocks + qb) * a.d + t];
    __syncthreads();
  } else {
    pool_qbar<ESZ>(a, qb, g, red, s_qbar);
  }

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
      const float p = row_sum(p0 + p1, lpb);
      if (J <= diag && sub == 0) {  // the row maximum is the maximum of the stored scores
        const float sc = p * a.scale;
        s_scores[J] = sc;
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

  // ---- keep bitmask (forced: block 0 and the diagonal run) and kept count:
  // one ballot per 64 KV blocks, lane l deciding block J0 + l, lanes 0 and 1
  // storing the two 32-bit words
  const int row = g * a.total_qblocks + qb;
  int cnt = 0;
  uint32_t* brow = a.bits + (int64_t)row * a.W;
  for (int J0 = 64 * (t >> 6); J0 < 32 * a.W; J0 += kThreads) {
    const int J = J0 + lane;
    const bool keep = J <= diag && (s_scores[J] >= thr || J == 0 || J >= dlo);
    const uint64_t m = __ballot(keep);
    const int w = (J0 >> 5) + lane;
    if (lane < 2 && w < a.W) brow[w] = (uint32_t)(m >> (32 * lane));
    cnt += __popcll(m);
  }
  if (a.scores_out) {
    float* so = a.scores_out + (int64_t)row * a.max_kblocks;
    for (int J = t; J < a.max_kblocks; J += kThreads) so[J] = J <= diag ? s_scores[J] : -INFINITY;
  }
  if ((t & 63) == 0) s_wcnt[t >> 6] = cnt;
  __syncthreads();
  if (t == 0) {
    int tot = 0;
    for (int w = 0; w < kThreads / 64; ++w) tot += s_wcnt[w];
    a.counts[row] = tot;
  }
}

// Fused stage 1, selection pass: work items of up to QT (<= kMaxQT)
// consecutive query blocks of one KV head, their pooled means scored against
// the sequence's kbar rows with each kbar row read once for all of them (the
// scores of one (query block, KV block) pair are summed exactly as
// score_select_kernel sums them, so the CSR is the same bit for bit), then
// each row's maximum, threshold, keep bitmask and count as there.  A grid of
// at most kSelectMaxWorkgroups claims the items, latest query blocks first.
#ifndef FP2_MAX_QT
#define FP2_MAX_QT 8
#endif
constexpr int kMaxQT = FP2_MAX_QT;
constexpr int kSelectMaxWorkgroups = 2048;  // 8 per CU of a 256-CU part
__global__ __launch_bounds__(kThreads) void select_tiled_kernel(PlanArgs a, int QT) {
  extern __shared__ float s_sc[];  // [QT][max_kblocks]
  __shared__ int s_seq[kMaxQT], s_diag[kMaxQT], s_dlo[kMaxQT];
  __shared__ float s_q[kMaxQT][128];
  __shared__ float s_wmax[kMaxQT][kThreads / 64];
  __shared__ int s_wcnt[kMaxQT][kThreads / 64];
  __shared__ int s_item;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // Work items (query tile, KV head) in descending tile order, claimed
  // through a counter until none is left: rows late in a sequence score many
  // more KV blocks than early ones, so the heaviest go first and every
  // workgroup keeps claiming until the list is done, however the hardware
  // placed the workgroups on the CUs.
  const int ntiles = (a.total_qblocks + QT - 1) / QT;
  const int nitems = ntiles * a.hkv;
  for (;;) {
    __syncthreads();  // the previous item's LDS reads are done
    if (t == 0) s_item = atomicAdd(a.ticket, 1);
    __syncthreads();
    const int item = s_item;
    if (item >= nitems) break;
    const int g = item % a.hkv;
    const int qb0 = (ntiles - 1 - item / a.hkv) * QT;
    const int nrows = min(QT, a.total_qblocks - qb0);
    if (t < nrows) {
      const int qb = qb0 + t;
      const int s = find_seq(a.cu_qblocks, a.num_seqs, qb);
      const int I = qb - a.cu_qblocks[s];
      const int n = a.cu_seqlens_q[s + 1] - a.cu_seqlens_q[s];
      const int P = a.seqlens_k[s] - n;
      const int ntok = min(a.qblock, n - I * a.qblock);
      s_seq[t] = s;
      s_dlo[t] = (P + I * a.qblock) / a.kvblock;
      s_diag[t] = (P + I * a.qblock + ntok - 1) / a.kvblock;
    }
    for (int i = t; i < nrows * a.d; i += kThreads)
      s_q[i / a.d][i % a.d] = a.qbar[((int64_t)g * a.total_qblocks + qb0 + i / a.d) * a.d + i % a.d];
    __syncthreads();

    const int lpb = a.d / 8;  // lanes sharing a kbar row, 8 floats each
    const int bpw = 64 / lpb;
    const int sub = lane % lpb;
    constexpr int UJ = 4;
    const int jstep = (kThreads / 64) * bpw;
    // runs of rows from one sequence (a tile crosses a sequence boundary rarely)
    for (int i0 = 0; i0 < nrows;) {
      const int s = s_seq[i0];
      int i1 = i0, jmax = 0;
      while (i1 < nrows && s_seq[i1] == s) jmax = max(jmax, s_diag[i1++]);
      float qv[kMaxQT][8];
      #pragma unroll
      for (int i = 0; i < kMaxQT; ++i)
        #pragma unroll
        for (int e = 0; e < 8; ++e) qv[i][e] = i0 + i < i1 ? s_q[i0 + i][8 * sub + e] : 0.f;
      const float* kb = a.kbar + ((int64_t)g * a.total_kblocks + a.cu_kblocks[s]) * a.d;
      for (int J0 = wave * bpw; J0 <= jmax; J0 += UJ * jstep) {
        f32x4 k0[UJ], k1[UJ];
        #pragma unroll
        for (int u = 0; u < UJ; ++u) {
          const int J = J0 + u * jstep + lane / lpb;
          k0[u] = k1[u] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (J <= jmax) {
            const f32x4* kr = reinterpret_cast<const f32x4*>(kb + (int64_t)J * a.d + 8 * sub);
            k0[u] = kr[0];
            k1[u] = kr[1];
          }
        }
        #pragma unroll
        for (int u = 0; u < UJ; ++u) {
          const int J = J0 + u * jstep + lane / lpb;
          #pragma unroll
          for (int i = 0; i < kMaxQT; ++i) {
            if (i0 + i >= i1) break;
            float p0 = 0.f, p1 = 0.f;
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
              p0 = fmaf(qv[i][e], k0[u][e], p0);
              p1 = fmaf(qv[i][4 + e], k1[u][e], p1);
            }
            const float p = row_sum(p0 + p1, lpb);
            if (sub == 0 && J <= s_diag[i0 + i]) s_sc[(i0 + i) * a.max_kblocks + J] = p * a.scale;
          }
        }
      }
      i0 = i1;
    }
    __syncthreads();

    // per row: maximum, threshold, keep bitmask (forced: block 0 and the
    // diagonal run), kept count; all waves on each row in turn
    for (int i = 0; i < nrows; ++i) {
      const int diag = s_diag[i];
      const float* sc = s_sc + i * a.max_kblocks;
      float lmax = -INFINITY;
      for (int J = t; J <= diag; J += kThreads) lmax = fmaxf(lmax, sc[J]);
      lmax = wave_max(lmax);
      if (lane == 0) s_wmax[i][wave] = lmax;
    }
    __syncthreads();
    for (int i = 0; i < nrows; ++i) {
      const int diag = s_diag[i], dlo = s_dlo[i];
      const float* sc = s_sc + i * a.max_kblocks;
      float rmax = s_wmax[i][0];
      #pragma unroll
      for (int w = 1; w < kThreads / 64; ++w) rmax = fmaxf(rmax, s_wmax[i][w]);
      const float thr = rmax - a.tau;
      const int row = g * a.total_qblocks + qb0 + i;
      // one ballot per 64 KV blocks: lane l decides block J0 + l, lanes 0 and
      // 1 store the two 32-bit words
      int cnt = 0;
      uint32_t* brow = a.bits + (int64_t)row * a.W;
      for (int J0 = 64 * wave; J0 < 32 * a.W; J0 += kThreads) {
        const int J = J0 + lane;
        const bool keep = J <= diag && (sc[J] >= thr || J == 0 || J >= dlo);
        const uint64_t m = __ballot(keep);
        const int w = (J0 >> 5) + lane;
        if (lane < 2 && w < a.W) brow[w] = (uint32_t)(m >> (32 * lane));
        cnt += __popcll(m);
      }
      if (a.scores_out) {
        float* so = a.scores_out + (int64_t)row * a.max_kblocks;
        for (int J = t; J < a.max_kblocks; J += kThreads) so[J] = J <= diag ? sc[J] : -INFINITY;
      }
      if (lane == 0) s_wcnt[i][wave] = cnt;
    }
    __syncthreads();
    if (t < nrows) {
      int tot = 0;
      for (int w = 0; w < kThreads / 64; ++w) tot += s_wcnt[t][w];
      a.counts[g * a.total_qblocks + qb0 + t] = tot;
    }
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

// Fused stage 1, first pass: every K, V and Q byte of the batch read once in
// one launch.  Workgroups [0, total_kblocks) write the KV block means (as
// fp2_block_stats), the rest one pooled query mean each (query block qb,
// KV head g: as fp2_plan_mask's pooling phase) into a.qbar, which the
// select pass then scores against kbar from L2.
template <int ESZ>
__global__ __launch_bounds__(kThreads) void pool_kernel(StatsArgs sa, PlanArgs a) {
  constexpr int N = 16 / ESZ;
  __shared__ float red_k[kThreads][N + 1];
  __shared__ float red_v[kThreads][N + 1];
  __shared__ float s_qbar[128];
  __shared__ int s_pg[kPoolMaxPages];
  // the select pass's claim counter (it runs after this launch), cleared
  // ahead of the bounds guard so that the select pass always runs whole
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.ticket = 0;
  FP2_BOUNDS_GUARD(sa.dbg);
  const int b = blockIdx.x;
  if (b < sa.total_kblocks) {
    kv_block_stats<ESZ>(sa, b, red_k, red_v, s_pg);
    return;
  }
  const int idx = b - sa.total_kblocks;
  const int qb = idx / a.hkv, g = idx % a.hkv;
  pool_qbar<ESZ>(a, qb, g, red_k, s_qbar);
  const int t = threadIdx.x;
  if (t < a.d) a.qbar[((int64_t)g * a.total_qblocks + qb) * a.d + t] = s_qbar[t];
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

namespace {
PlanArgs plan_args(const fp2_batch* b, const fp2_q* q, int hkv, const BatchInfo& info, const float* kbar, float tau,
                   float* scores, void* workspace) {
  const int rows = (int)(info.total_qblocks * hkv);
  const int W = plan_words(info);
  PlanArgs a;
  a.cu_seqlens_q = b->cu_seqlens_q;
  a.seqlens_k = b->seqlens_k;
  a.cu_qblocks = b->cu_qblocks;
  a.cu_kblocks = b->cu_kblocks;
  a.q = static_cast<const uint8_t*>(q->q);
  a.q_scale = q->q_scale;
  a.kbar = kbar;
  a.bits = static_cast<uint32_t*>(workspace);
  a.counts = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + (((size_t)rows * W * 4 + 255) & ~size_t(255)));
  a.scores_out = scores;
  a.qbar = nullptr;
  a.ticket = nullptr;
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
  return a;
}

// score / select (pooling Q itself, or reading the fused pass's qbar), then
// the scan and the column fill
hipError_t launch_select(const PlanArgs& a, int dtype, bool pooled, int32_t* row_ptr, int32_t* col_idx,
                         int32_t* nnz, hipStream_t stream) {
  const int rows = a.total_qblocks * a.hkv;
  const size_t lds = (size_t)a.max_kblocks * sizeof(float);
  dim3 grid((unsigned)a.total_qblocks, (unsigned)a.hkv);
  if (pooled) {
    // query blocks per workgroup: score rows of QT x max_kblocks floats in LDS (<= 64 KB)
    int QT = kMaxQT;
    while (QT > 1 && (size_t)QT * lds > (size_t)(64 << 10)) QT >>= 1;
    // enough workgroups to fill the device; each claims items until none is left
    const int nitems = ((a.total_qblocks + QT - 1) / QT) * a.hkv;
    const dim3 tgrid((unsigned)std::min(nitems, kSelectMaxWorkgroups));
    hipLaunchKernelGGL(select_tiled_kernel, tgrid, dim3(kThreads), (size_t)QT * lds, stream, a, QT);
  } else if (dtype == FP2_BF16) {
    hipLaunchKernelGGL((score_select_kernel<2, false>), grid, dim3(kThreads), lds, stream, a);
  } else {
    hipLaunchKernelGGL((score_select_kernel<1, false>), grid, dim3(kThreads), lds, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_counts_kernel, dim3(1), dim3(1024), 0, stream, a.counts, rows, row_ptr, nnz);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fill_cols_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, a.bits, a.W, row_ptr,
                     col_idx);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_plan(const fp2_batch* b, const fp2_q* q, int hkv, const BatchInfo& info,
                       const float* kbar, float tau, int32_t* row_ptr, int32_t* col_idx,
                       int32_t* nnz, float* scores, void* workspace, hipStream_t stream) {
  const PlanArgs a = plan_args(b, q, hkv, info, kbar, tau, scores, workspace);
  return launch_select(a, q->dtype, false, row_ptr, col_idx, nnz, stream);
}

hipError_t launch_stage1(const fp2_batch* b, const fp2_q* q, const fp2_kv* kv, const BatchInfo& info, float tau,
                         float* kbar, float* vbar, int32_t* row_ptr, int32_t* col_idx, int32_t* nnz, float* scores,
                         void* workspace, hipStream_t stream) {
  const int hkv = kv->num_kv_heads;
  PlanArgs a = plan_args(b, q, hkv, info, kbar, tau, scores, workspace);
  a.qbar = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan_workspace_bytes(info, hkv));
  a.ticket = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + stage1_workspace_bytes(info, hkv, q->head_dim) -
                                        kStage1TicketBytes);
  const StatsArgs sa = stats_args(b, kv, info, kbar, vbar);
  const int64_t nwg = info.total_kblocks + info.total_qblocks * hkv;
  if (nwg > 0) {
    if (kv->dtype == FP2_BF16)
      hipLaunchKernelGGL(pool_kernel<2>, dim3((unsigned)nwg), dim3(kThreads), 0, stream, sa, a);
    else
      hipLaunchKernelGGL(pool_kernel<1>, dim3((unsigned)nwg), dim3(kThreads), 0, stream, sa, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (info.total_qblocks == 0) return launch_zero_plan(row_ptr, nnz, stream);
  return launch_select(a, q->dtype, true, row_ptr, col_idx, nnz, stream);
}

}  // namespace fp2
