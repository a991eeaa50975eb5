// Stage 2 for bf16 inputs with head_dim 128: block-sparse causal GQA attention
// over the kept KV blocks plus the mean correction of every skipped block, in
// one online softmax.
//
// FlashPrefill V2 (metallab.ai paper page): Figure 3 (exact path over the
// CSR-selected blocks, correction path merged in the online softmax),
// Figure 4 (a pruned block J adds |B_J| * exp(q . kbar_J / sqrt(d)) * (vbar_J, 1)),
// Table 7 (CSR per KV head, paged KV at any page size).
//
// CDNA4 layout of the work:
//  * One workgroup = 8 waves = 256 packed query rows of one CSR row (the G
//    query heads of a KV head times B tokens); each wave owns 32 tokens of one
//    head, so every K/V tile staged in LDS feeds 256 query rows.
//  * Tiles (kept KV blocks, then mean-token tiles) stream through two LDS
//    buffers: the next tile's global loads are in flight in registers while
//    the current tile is computed, and one barrier per tile separates them.
//  * K and V tiles are stored row-major with padded rows (K 272 bytes, V 288
//    bytes per 256-byte row).  The padding makes the three access patterns
//    free of LDS bank conflicts (the staging writes, the QK^T operand reads of
//    16 rows x one 16-byte chunk, the transposing PV operand reads of
//    ds_read_tr16_b64 over 4 rows x 2 chunks) while every address stays one
//    per-lane base plus an immediate offset.
//  * S^T = K Q^T on the bf16 32x32x16 MFMA: a lane holds the keys of one query,
//    so row max / row sum are in-lane plus one lane^32 exchange.  O^T = V^T P^T
//    on the same MFMA takes P straight from the score registers (as bf16) and
//    V^T through ds_read_tr16_b64 from the row-major V tile, so V is never
//    transposed in staging.
//  * The logit scale is folded into the exponent's FMA; masks are applied only
//    on the diagonal block (causal) and on mean-token tiles (kept, block 0 and
//    non-causal mean tokens); the reference max is refreshed lazily.
#include "attn_common.h"

namespace fp2 {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;   // 512
constexpr int kWGRows = 32 * kWaves;    // packed query rows per workgroup
constexpr int kD = 128;
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left unconstrained
// (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kRowBytes = kD * 2;       // one bf16 row of K or V in global memory
constexpr int kKS = kRowBytes + 16;     // LDS row stride of the K tile (bytes)
constexpr int kVS = kRowBytes + 32;     // LDS row stride of the V tile (bytes)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ i16x4 ds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Register staging of one K tile and one V tile (BLK rows x 16 chunks each).
template <int BLK>
struct Stage {
  static constexpr int NLD = BLK * (kD / 8) / kThreads;  // chunks per thread per tile
  uint4 k[NLD], v[NLD];

  int pg[NLD];  // physical page of each staged row of the tile two ahead (-1: past the end)

  // Page-table entries of this thread's rows of exact block J (issued a full
  // tile ahead of the K/V loads that use them).
  __device__ __forceinline__ void fetch_pages(const AttnArgs& a, const int32_t* pt, int T, int J, int t) {
#pragma unroll
    for (int p = 0; p < NLD; ++p) {
      const int row = (t + kThreads * p) >> 4;
      const int pos = J * BLK + row;
      int pi, slot;
      a.pm.split(pos, pi, slot);
      pg[p] = pos < T ? pt[pi] : -1;
    }
  }

  // K/V rows of exact block J at the pages fetched by fetch_pages.
  __device__ __forceinline__ void load_exact(const AttnArgs& a, int g, int J, int t) {
#pragma unroll
    for (int p = 0; p < NLD; ++p) {
      const int ch = t + kThreads * p;
      const int row = ch >> 4, c = ch & 15;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = kv;
      if (pg[p] >= 0) {
        int pi, slot;
        a.pm.split(J * BLK + row, pi, slot);
        const int64_t off = (((int64_t)pg[p] * a.page_size + slot) * a.hkv + g) * kRowBytes + c * 16;
        kv = *reinterpret_cast<const uint4*>(a.k_pages + off);
        vv = *reinterpret_cast<const uint4*>(a.v_pages + off);
      }
      k[p] = kv;
      v[p] = vv;
    }
  }

  // mean tokens J0 + row (rows at or past jend are zero)
  __device__ __forceinline__ void load_mean(const AttnArgs& a, int64_t mrow0, int J0, int jend, int t) {
#pragma unroll
    for (int p = 0; p < NLD; ++p) {
      const int ch = t + kThreads * p;
      const int row = ch >> 4, c = ch & 15;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = kv;
      if (J0 + row < jend) {
        const int64_t off = (mrow0 + J0 + row) * kD + c * 8;
        kv = *reinterpret_cast<const uint4*>(a.kbar16 + off);
        vv = *reinterpret_cast<const uint4*>(a.vbar16 + off);
      }
      k[p] = kv;
      v[p] = vv;
    }
  }

  __device__ __forceinline__ void commit(uint8_t* Kb, uint8_t* Vb, int t) const {
#pragma unroll
    for (int p = 0; p < NLD; ++p) {
      const int ch = t + kThreads * p;
      *reinterpret_cast<uint4*>(Kb + (ch >> 4) * kKS + (ch & 15) * 16) = k[p];
      *reinterpret_cast<uint4*>(Vb + (ch >> 4) * kVS + (ch & 15) * 16) = v[p];
    }
  }
};

// bits of the 32 mean tokens [32*w, 32*w + 32) that are skipped blocks, i.e.
// in [1, diag) and not kept
__device__ __forceinline__ uint32_t skipped_word(const uint32_t* kept, int w, int diag) {
  const int j0 = 32 * w;
  if (j0 >= diag) return 0u;
  uint32_t m = ~kept[w];
  if (j0 + 32 > diag) m &= (1u << (diag - j0)) - 1u;
  if (w == 0) m &= ~1u;
  return m;
}

template <int BLK>
struct Wave {
  bf16x8 qf[kD / 16];
  f32x16 o[kD / 32];
  float m;  // reference max (log2 units), shared by lanes l and l^32
  float l;  // this lane's half of the denominator

  // mode 0: exact block; 1: diagonal block (causal mask); 2: mean-token tile
  // starting at mean token J0.  The mode is wave-uniform; one code path
  // serves all three so the register allocation is shared.
  __device__ __forceinline__ void tile(int mode, const uint8_t* Kb, const uint8_t* Vb, int lane, float scl, float bias,
                                       int tq, int J0, int diag, const uint32_t* kept) {
    const int c = lane & 31, hf = lane >> 5;
    const int i16 = lane & 15, go = lane & 16;  // tr-read lane within its 16-lane group; d offset
    // per-lane bases: K row c, chunk hf; V^T read row 4hf + i16/4, column go + 4(i16%4)
    const uint8_t* kbase = Kb + c * kKS + hf * 16;
    const uint8_t* vbase = Vb + (4 * hf + (i16 >> 2)) * kVS + (go + 4 * (i16 & 3)) * 2;
#pragma nounroll
    for (int sub = 0; sub < BLK / 64; ++sub) {
      // S^T for 64 keys: two independent accumulator chains, alternated, with the
      // K operand reads issued four MFMAs ahead
      f32x16 s[2] = {f32x16{}, f32x16{}};
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < kD / 16; ++kk)
#pragma unroll
        for (int st = 0; st < 2; ++st)
          s[st] = mfma_bf16_32x32x16(
              *reinterpret_cast<const bf16x8*>(kbase + (64 * sub + 32 * st) * kKS + 32 * kk), qf[kk], s[st]);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (mode == 1) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (64 * sub + 32 * st + 8 * (i >> 2) + 4 * hf + (i & 3) > tq) s[st][i] = -INFINITY;
      }
      if (mode == 2) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const uint32_t w = skipped_word(kept, (J0 >> 5) + 2 * sub + st, diag) >> (4 * hf);
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (!((w >> (8 * (i >> 2) + (i & 3))) & 1u)) s[st][i] = -INFINITY;
        }
      }
      float sv[32];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[i] = s[0][i];
        sv[16 + i] = s[1][i];
      }
      const float mx = max_halves(tree_max<32>(sv));
      const float mxs = mx * scl + bias;  // scl > 0; -inf stays -inf
      if (__any(mxs > m + kLazy)) {       // wave-uniform refresh of the reference max
        const float mnew = fmaxf(m, mxs);
        const float alpha = __builtin_amdgcn_exp2f(m - (mnew == -INFINITY ? 0.f : mnew));
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      }
      const float nb = bias - (m == -INFINITY ? 0.f : m);
      float pv[32];
      bf16x8 pf[2][2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][8 * r + j], scl, nb));
            pv[16 * st + 8 * r + j] = p;
            pf[st][r][j] = (__bf16)p;
          }
      l += tree_sum<32>(pv);
      // O^T += V^T P^T: four independent chains (dt), alternated, with the
      // transposing V reads (two per MFMA) issued four MFMAs ahead
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int dt = 0; dt < kD / 32; ++dt) {
            const uint8_t* vr = vbase + (64 * sub + 32 * st + 16 * r) * kVS + 64 * dt;
            const i16x4 v0 = ds_read_tr16(vr);
            const i16x4 v1 = ds_read_tr16(vr + 8 * kVS);
            const i16x4 vv[2] = {v0, v1};
            bf16x8 va;
            __builtin_memcpy(&va, vv, sizeof(va));
            o[dt] = mfma_bf16_32x32x16(va, pf[st][r], o[dt]);
          }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

template <int BLK>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_d128_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t Kb[2][BLK * kKS];
  __shared__ __attribute__((aligned(16))) uint8_t Vb[2][BLK * kVS];
  __shared__ uint32_t kept[kMaxKBlocks / 32];
  __shared__ int mtile[kMaxKBlocks / 64 + 1];
  __shared__ int s_nmean;

  // ---- tile decode (as the first kernel): 8 consecutive CSR ranks form a
  // group, the slices of one rank share blockIdx % 8 (one XCD), latest query
  // blocks first
  const int b = blockIdx.x;
  const int per_grp = 8 * a.slices;
  const int grp = b / per_grp;
  const int rem = b % per_grp;
  const int slice = rem / 8;
  const int rank = grp * 8 + (rem % 8);
  if (rank >= a.rows) return;
  const int qb = a.total_qblocks - 1 - rank / a.hkv;
  const int g = rank % a.hkv;
  const int row = g * a.total_qblocks + qb;

  const int s = find_seq(a.cu_qblocks, a.num_seqs, qb);
  const int I = qb - a.cu_qblocks[s];
  const int q0 = a.cu_seqlens_q[s];
  const int n = a.cu_seqlens_q[s + 1] - q0;
  const int T = a.seqlens_k[s];
  const int diag = (T - n) / BLK + I;
  const int G = a.hq / a.hkv;
  const int32_t* pt = a.page_table + (int64_t)s * a.max_pages;
  const int64_t mrow0 = (int64_t)g * a.total_kblocks + a.cu_kblocks[s];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int hf = lane >> 5;
  const int prow = slice * kWGRows + wave * 32;
  const bool wave_active = prow < G * BLK;
  const int h = g * G + prow / BLK;
  const int tq = prow % BLK + (lane & 31);
  const bool q_valid = wave_active && (I * BLK + tq < n);

  // uniform values: later loads indexed by them become scalar loads, which
  // do not share the vector-memory counter with the tile prefetch
  const int kbeg = ld_uniform(a.row_ptr, row);
  const int kend = ld_uniform(a.row_ptr, row + 1);
  const int nexact = kend - kbeg;

  // ---- mean-token tiles that hold at least one skipped block
  int nmean = 0;
  if (a.correction && diag > 1) {
    const int nw = (diag + 32) >> 5;
    for (int w = t; w < nw; w += kThreads) kept[w] = 0u;
    __syncthreads();
    for (int i = kbeg + t; i < kend; i += kThreads) {
      const int j = a.col_idx[i];
      atomicOr(&kept[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    if (wave == 0) {
      const int ncand = (diag + BLK - 1) / BLK;
      int base = 0;
      for (int m0 = 0; m0 < ncand; m0 += 64) {
        const int mt = m0 + lane;
        bool flag = false;
        if (mt < ncand) {
#pragma unroll
          for (int w = 0; w < BLK / 32; ++w) flag |= skipped_word(kept, mt * (BLK / 32) + w, diag) != 0u;
        }
        const uint64_t bal = __ballot(flag);
        if (flag) mtile[base + __popcll(bal & ((1ull << lane) - 1ull))] = mt * BLK;
        base += __popcll(bal);
      }
      if (lane == 0) s_nmean = base;
    }
    __syncthreads();
    nmean = s_nmean;
  }
  const int ntiles = nexact + nmean;

  Wave<BLK> ws;
  ws.m = -INFINITY;
  ws.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt) ws.o[dt] = f32x16{};
  {
    const uint8_t* qrow = a.q + ((int64_t)(q0 + I * BLK + tq) * a.hq + h) * kRowBytes;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (q_valid) v = *reinterpret_cast<const uint4*>(qrow + (16 * kk + 8 * hf) * 2);
      ws.qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
    // Complete the query loads here: otherwise the compiler's wait for them lands
    // inside the tile loop, where it would also wait for the next tile's prefetch.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }

  // Tile pipeline: at iteration i the LDS buffer i%2 holds tile i, the
  // staging registers hold tile i+1 (in flight), the page entries of tile
  // i+2 are in flight, and the block indices of tiles i..i+3 sit in uniform
  // registers.  No step of an iteration waits on a global load issued in the
  // same iteration, so global latency overlaps a full tile of compute.
  Stage<BLK> stg;
  auto block_of = [&](int idx) -> int {  // first block (KV block or mean token) of tile idx
    if (idx >= ntiles) return 0;
    if (idx < nexact) return ld_uniform(a.col_idx, kbeg + idx);
    return mtile[idx - nexact];
  };
  auto stage = [&](int idx, int j) {  // global -> staging registers
    if (idx < nexact) stg.load_exact(a, g, j, t);
    else stg.load_mean(a, mrow0, j, diag, t);
  };
  auto pages = [&](int idx, int j) {
    if (idx < nexact) stg.fetch_pages(a, pt, T, j, t);
  };

  int j0 = block_of(0), j1 = block_of(1), j2 = block_of(2), j3 = block_of(3);
  if (ntiles > 0) {
    pages(0, j0);
    stage(0, j0);
    stg.commit(Kb[0], Vb[0], t);
  }
  if (ntiles > 1) {
    pages(1, j1);
    stage(1, j1);
  }
  if (ntiles > 2) pages(2, j2);
  __syncthreads();
  const float scl = a.scale_log2;
  for (int idx = 0; idx < ntiles; ++idx) {
    const int cur = idx & 1;
    const int j4 = block_of(idx + 4);
    if (wave_active) {
      const bool exact = idx < nexact;
      const int mode = exact ? (j0 == diag ? 1 : 0) : 2;
      ws.tile(mode, Kb[cur], Vb[cur], lane, scl, exact ? 0.f : a.log2_block, tq, exact ? 0 : j0, diag, kept);
    }
    if (idx + 1 < ntiles) stg.commit(Kb[cur ^ 1], Vb[cur ^ 1], t);
    if (idx + 2 < ntiles) stage(idx + 2, j2);
    if (idx + 3 < ntiles) pages(idx + 3, j3);
    j0 = j1;
    j1 = j2;
    j2 = j3;
    j3 = j4;
    __syncthreads();
  }

  // ---- epilogue: O / l
  if (q_valid) {
    const float inv = 1.0f / sum_halves(ws.l);
    const int64_t obase = ((int64_t)(q0 + I * BLK + tq) * a.hq + h) * kD;
    if (a.out_f32) {
      float* orow = static_cast<float*>(a.out) + obase;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * q4 + 4 * hf) =
              f32x4{ws.o[dt][4 * q4 + 0] * inv, ws.o[dt][4 * q4 + 1] * inv, ws.o[dt][4 * q4 + 2] * inv,
                    ws.o[dt][4 * q4 + 3] * inv};
    } else {
      uint16_t* orow = static_cast<uint16_t*>(a.out) + obase;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          uint2 w;
          w.x = pack_bf16x2(ws.o[dt][4 * q4 + 0] * inv, ws.o[dt][4 * q4 + 1] * inv);
          w.y = pack_bf16x2(ws.o[dt][4 * q4 + 2] * inv, ws.o[dt][4 * q4 + 3] * inv);
          *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * q4 + 4 * hf) = w;
        }
    }
  }
}

}  // namespace

// Launch with a.slices computed for kWGRows rows per workgroup.
hipError_t launch_attn_bf16_d128(const AttnArgs& a_in, int block, hipStream_t stream) {
  AttnArgs a = a_in;
  const int G = a.hq / a.hkv;
  a.slices = (G * block + kWGRows - 1) / kWGRows;
  const unsigned grid = (unsigned)(((a.rows + 7) / 8) * 8 * a.slices);
  if (block == 128)
    hipLaunchKernelGGL(attn_bf16_d128_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_bf16_d128_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fp2
