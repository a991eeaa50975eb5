// Stage 2: block-sparse causal GQA attention over the kept KV blocks, with the
// mean correction of every skipped block merged into the same online softmax.
//
// FlashPrefill V2 (metallab.ai paper page): Figure 3 (exact path over the
// CSR-selected blocks; the correction path for unselected blocks merges
// inside the online softmax), Figure 4 (a pruned block J contributes
// |B_J| * exp(s_J) * (vbar_J, 1) with s_J = q . kbar_J / sqrt(d)), Table 7
// (CSR per KV head, paged KV at any page size, BF16 and FP8).
//
// CDNA4 design (not the pages' Hopper design):
//  * One workgroup = 4 waves = 128 packed query rows of one CSR row (the G
//    query heads of a KV head times B tokens are packed so every wave shares
//    the row's K/V tiles in LDS).  Each wave owns 32 query tokens of one head.
//  * Scores are computed transposed, S^T = K Q^T (bf16 32x32x16 MFMA, or the
//    OCP e4m3 32x32x64 MFMA for fp8 inputs): a lane then holds the keys of ONE
//    query, so the row max / row sum of the online softmax are in-lane plus
//    one lane^32 exchange, and rescaling the output is a per-lane scalar.
//    The output is kept transposed too, O^T = V^T P^T, computed with the fp16
//    32x32x16 MFMA whose B operand is the score accumulator itself (the
//    contraction index is permuted consistently between P and V^T).  fp16
//    (not bf16) P keeps the probability rounding at 2^-11; bf16 and e4m3 V
//    convert to fp16 exactly.
//  * K is staged row-major and V transposed (with the matching key
//    permutation) in padded LDS rows; the next block's global loads are in
//    flight while the current block is computed.
//  * Mean correction = attention over "mean tokens" (bf16 kbar, fp16 vbar
//    copies) in tiles of B, with logit bias log2(B) and masking of kept, zero
//    and non-causal blocks, through the same MFMA code path.
//  * fp8: logits carry q_scale * k_scale, and each block's v_scale is folded
//    into its probabilities before the PV product.
#include <algorithm>
#include <cstdlib>

#include "attn_common.h"

namespace fp2 {

namespace {

constexpr int kThreads = 256;

// key permutation inside each group of 16 for the V^T tile: the MFMA lane half
// h consumes keys {4h..4h+3, 8+4h..8+4h+3} of the group as one 16-byte read
__device__ __forceinline__ int vt_pos_of_quad(int quad) {
  const int sub = quad & 3;
  return 16 * (quad >> 2) + ((sub & 1) << 3) + ((sub >> 1) << 2);
}

template <int D, int BLK, bool FP8>
struct Tile {
  static constexpr int ESZ = FP8 ? 1 : 2;       // input element bytes
  static constexpr int KS = D + 8;              // bf16 K / kbar row stride (elements)
  static constexpr int KS8 = D + 16;            // e4m3 K row stride (bytes)
  static constexpr int VS = BLK + 8;            // fp16 V^T row stride (elements)
  static constexpr int CPR = D * ESZ / 16;      // 16-byte chunks per input K row
  static constexpr int RPP = kThreads / CPR;
  static constexpr int NKP = BLK / RPP;         // K rows per thread (input)
  static constexpr int CPRM = D / 8;            // 16-byte chunks per kbar (bf16) row
  static constexpr int RPPM = kThreads / CPRM;
  static constexpr int NKPM = BLK / RPPM;       // kbar rows per thread
  static constexpr int EPC = 16 / ESZ;          // V elements per 16-byte chunk (input)
  static constexpr int UNITS = (BLK / 4) * (D / EPC);
  static constexpr int NVU = (UNITS + kThreads - 1) / kThreads;
  static constexpr int UNITSM = (BLK / 4) * (D / 8);
  static constexpr int NVUM = (UNITSM + kThreads - 1) / kThreads;
  static constexpr int KK = D / 16;             // bf16 K-steps of QK^T
  static constexpr int KK8 = D / 64;            // e4m3 K-steps of QK^T
  static constexpr int DT = D / 32;             // 32-wide output tiles
  static constexpr int NREG_K = NKP > NKPM ? NKP : NKPM;
  static constexpr int NREG_V = NVU > NVUM ? NVU : NVUM;
  static constexpr int KLDS = (BLK * KS * 2 > BLK * KS8) ? BLK * KS * 2 : BLK * KS8;  // bytes
};

template <int D, int BLK, bool FP8>
struct Stager {
  using TL = Tile<D, BLK, FP8>;
  uint4 kreg[TL::NREG_K];
  uint4 vreg[TL::NREG_V][4];

  // Rows of an exact KV block J (paged input: bf16 or e4m3 bytes).
  __device__ __forceinline__ void load_block(const AttnArgs& a, const int32_t* pt, int g, int T,
                                             int J, int t) {
    const int chunk = t % TL::CPR;
    const int row0 = t / TL::CPR;
#pragma unroll
    for (int p = 0; p < TL::NKP; ++p) {
      const int k = row0 + p * TL::RPP;
      const int pos = J * BLK + k;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (pos < T) {
        int pi, slot;
        a.pm.split(pos, pi, slot);
        const int64_t off = (((int64_t)pt[pi] * a.page_size + slot) * a.hkv + g) * (D * TL::ESZ) + chunk * 16;
        v = *reinterpret_cast<const uint4*>(a.k_pages + off);
      }
      kreg[p] = v;
    }
#pragma unroll
    for (int u = 0; u < TL::NVU; ++u) {
      const int unit = t + u * kThreads;
      const int dchunk = unit % (D / TL::EPC);
      const int quad = unit / (D / TL::EPC);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = J * BLK + quad * 4 + r;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (unit < TL::UNITS && pos < T) {
          int pi, slot;
          a.pm.split(pos, pi, slot);
          const int64_t off =
              (((int64_t)pt[pi] * a.page_size + slot) * a.hkv + g) * (D * TL::ESZ) + dchunk * 16;
          v = *reinterpret_cast<const uint4*>(a.v_pages + off);
        }
        vreg[u][r] = v;
      }
    }
  }

  // Rows of a mean-token tile: mean tokens J0..J0+BLK-1 (rows >= jend are zero).
  __device__ __forceinline__ void load_means(const AttnArgs& a, int64_t mrow0, int J0, int jend, int t) {
    const int chunk = t % TL::CPRM;
    const int row0 = t / TL::CPRM;
#pragma unroll
    for (int p = 0; p < TL::NKPM; ++p) {
      const int k = row0 + p * TL::RPPM;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (J0 + k < jend)
        v = *reinterpret_cast<const uint4*>(a.kbar16 + (mrow0 + J0 + k) * D + chunk * 8);
      kreg[p] = v;
    }
#pragma unroll
    for (int u = 0; u < TL::NVUM; ++u) {
      const int unit = t + u * kThreads;
      const int dchunk = unit % (D / 8);
      const int quad = unit / (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = J0 + quad * 4 + r;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (unit < TL::UNITSM && j < jend)
          v = *reinterpret_cast<const uint4*>(a.vbar16 + (mrow0 + j) * D + dchunk * 8);
        vreg[u][r] = v;
      }
    }
  }

  // Exact block -> LDS.  K rows as they are (bf16 [BLK][KS] or e4m3 [BLK][KS8]);
  // V transposed into fp16 V^T with the key permutation (exact conversion).
  __device__ __forceinline__ void commit_block(uint8_t* Kl, uint16_t* Vt, int t) const {
    {
      const int chunk = t % TL::CPR;
      const int row0 = t / TL::CPR;
      const int rstride = FP8 ? TL::KS8 : TL::KS * 2;
#pragma unroll
      for (int p = 0; p < TL::NKP; ++p)
        *reinterpret_cast<uint4*>(Kl + (row0 + p * TL::RPP) * rstride + chunk * 16) = kreg[p];
    }
#pragma unroll
    for (int u = 0; u < TL::NVU; ++u) {
      const int unit = t + u * kThreads;
      if (unit >= TL::UNITS) break;
      const int dchunk = unit % (D / TL::EPC);
      const int quad = unit / (D / TL::EPC);
      const int kp = vt_pos_of_quad(quad);
      const uint32_t a0[4] = {vreg[u][0].x, vreg[u][0].y, vreg[u][0].z, vreg[u][0].w};
      const uint32_t a1[4] = {vreg[u][1].x, vreg[u][1].y, vreg[u][1].z, vreg[u][1].w};
      const uint32_t a2[4] = {vreg[u][2].x, vreg[u][2].y, vreg[u][2].z, vreg[u][2].w};
      const uint32_t a3[4] = {vreg[u][3].x, vreg[u][3].y, vreg[u][3].z, vreg[u][3].w};
      if constexpr (!FP8) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {  // elements 2w (low halves), 2w+1 (high halves)
          uint2 lo, hi;
          lo.x = pack_f16x2_rtz(bf16lo(a0[w]), bf16lo(a1[w]));
          lo.y = pack_f16x2_rtz(bf16lo(a2[w]), bf16lo(a3[w]));
          hi.x = pack_f16x2_rtz(bf16hi(a0[w]), bf16hi(a1[w]));
          hi.y = pack_f16x2_rtz(bf16hi(a2[w]), bf16hi(a3[w]));
          *reinterpret_cast<uint2*>(Vt + (dchunk * 8 + 2 * w) * TL::VS + kp) = lo;
          *reinterpret_cast<uint2*>(Vt + (dchunk * 8 + 2 * w + 1) * TL::VS + kp) = hi;
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {  // elements 4w..4w+3 of the 4 keys
          const f32x4 f0 = e4m3x4_to_f32(a0[w]), f1 = e4m3x4_to_f32(a1[w]);
          const f32x4 f2 = e4m3x4_to_f32(a2[w]), f3 = e4m3x4_to_f32(a3[w]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint2 v;
            v.x = pack_f16x2_rtz(f0[e], f1[e]);
            v.y = pack_f16x2_rtz(f2[e], f3[e]);
            *reinterpret_cast<uint2*>(Vt + (dchunk * 16 + 4 * w + e) * TL::VS + kp) = v;
          }
        }
      }
    }
  }

  // Mean tile -> LDS: kbar rows (bf16 [BLK][KS]) and vbar^T (already fp16).
  __device__ __forceinline__ void commit_means(uint8_t* Kl, uint16_t* Vt, int t) const {
    {
      const int chunk = t % TL::CPRM;
      const int row0 = t / TL::CPRM;
#pragma unroll
      for (int p = 0; p < TL::NKPM; ++p)
        *reinterpret_cast<uint4*>(Kl + (row0 + p * TL::RPPM) * (TL::KS * 2) + chunk * 16) = kreg[p];
    }
#pragma unroll
    for (int u = 0; u < TL::NVUM; ++u) {
      const int unit = t + u * kThreads;
      if (unit >= TL::UNITSM) break;
      const int dchunk = unit % (D / 8);
      const int quad = unit / (D / 8);
      const int kp = vt_pos_of_quad(quad);
      const uint32_t a0[4] = {vreg[u][0].x, vreg[u][0].y, vreg[u][0].z, vreg[u][0].w};
      const uint32_t a1[4] = {vreg[u][1].x, vreg[u][1].y, vreg[u][1].z, vreg[u][1].w};
      const uint32_t a2[4] = {vreg[u][2].x, vreg[u][2].y, vreg[u][2].z, vreg[u][2].w};
      const uint32_t a3[4] = {vreg[u][3].x, vreg[u][3].y, vreg[u][3].z, vreg[u][3].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint2 lo, hi;
        lo.x = __builtin_amdgcn_perm(a1[w], a0[w], 0x05040100u);
        lo.y = __builtin_amdgcn_perm(a3[w], a2[w], 0x05040100u);
        hi.x = __builtin_amdgcn_perm(a1[w], a0[w], 0x07060302u);
        hi.y = __builtin_amdgcn_perm(a3[w], a2[w], 0x07060302u);
        *reinterpret_cast<uint2*>(Vt + (dchunk * 8 + 2 * w) * TL::VS + kp) = lo;
        *reinterpret_cast<uint2*>(Vt + (dchunk * 8 + 2 * w + 1) * TL::VS + kp) = hi;
      }
    }
  }
};

// Per-wave online-softmax state and the tile compute.  A KV tile of BLK keys
// is consumed in sub-tiles of 64 keys (two 32x32 score tiles) to bound the
// live score registers.
template <int D, int BLK, bool FP8>
struct WaveState {
  using TL = Tile<D, BLK, FP8>;
  bf16x8 qf[TL::KK];     // bf16 query fragments (bf16 inputs; fp8: for the mean tiles)
  i32x8 qf8[FP8 ? TL::KK8 : 1];
  f32x16 o[TL::DT];
  float m;   // reference max (log2 domain), shared by the lane pair (l, l^32)
  float l;   // this lane's half of the running denominator

  // d-offset of the 8 bf16 query values a lane half holds at K-step kk: the
  // natural split for bf16 inputs; for fp8 inputs the split of the e4m3
  // fragments (32 contiguous d per lane half and 64-wide step), so the bf16
  // copy of an fp8 query pairs with kbar read at the same offsets.
  __device__ __forceinline__ static int koff(int kk, int hf) {
    if (FP8) return 64 * (kk >> 2) + 32 * hf + 8 * (kk & 3);
    return 16 * kk + 8 * hf;
  }

  __device__ __forceinline__ void scores_bf16(const uint8_t* Kl, int sub, int c, int hf, f32x16* s) const {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st] = f32x16{};
      const uint16_t* kr = reinterpret_cast<const uint16_t*>(Kl) + (64 * sub + 32 * st + c) * TL::KS;
#pragma unroll
      for (int kk = 0; kk < TL::KK; ++kk)
        s[st] = mfma_bf16_32x32x16(*reinterpret_cast<const bf16x8*>(kr + koff(kk, hf)), qf[kk], s[st]);
    }
  }

  __device__ __forceinline__ void scores_fp8(const uint8_t* Kl, int sub, int c, int hf, f32x16* s) const {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st] = f32x16{};
      const uint8_t* kr = Kl + (64 * sub + 32 * st + c) * TL::KS8 + 32 * hf;
#pragma unroll
      for (int kk = 0; kk < TL::KK8; ++kk) {
        const uint4 v0 = *reinterpret_cast<const uint4*>(kr + 64 * kk);
        const uint4 v1 = *reinterpret_cast<const uint4*>(kr + 64 * kk + 16);
        const i32x8 ka = {(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
        s[st] = mfma_fp8_32x32x64(ka, qf8[kk], s[st]);
      }
    }
  }

  // MODE 0: exact block (on the diagonal, keys k > qoff are masked: qoff is
  // the query's position minus the block's first key position); MODE 1:
  // mean-token tile of tokens J0.., those of skipped blocks in [1, jend)
  // count.  scl: logit scale to log2 units; pscale multiplies the
  // probabilities fed to PV (fp8 v_scale), not the denominator.
  template <int MODE>
  __device__ __forceinline__ void tile(const uint8_t* Kl, const uint16_t* Vt, int lane, float scl,
                                       float pscale, bool diagonal, int qoff, int J0, int jend,
                                       const uint32_t* kept, float bias) {
    const int c = lane & 31, hf = lane >> 5;
#pragma nounroll
    for (int sub = 0; sub < BLK / 64; ++sub) {
      f32x16 s[2];
      if (FP8 && MODE == 0) scores_fp8(Kl, sub, c, hf, s);
      else scores_bf16(Kl, sub, c, hf, s);
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int k = 64 * sub + 32 * st + 8 * (i >> 2) + 4 * hf + (i & 3);
          float x = s[st][i] * scl;
          if (MODE == 0) {
            if (diagonal && k > qoff) x = -INFINITY;
          } else {
            const int j = J0 + k;
            const bool skipped = j >= 1 && j < jend && !((kept[j >> 5] >> (j & 31)) & 1u);
            x = skipped ? x + bias : -INFINITY;
          }
          s[st][i] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, swap_halves(mx));
      if (__any(mx > m + kLazy)) {  // wave-uniform: refresh the reference max
        const float mnew = fmaxf(m, mx);
        // mnew is finite once block 0 (always kept, first in the ascending
        // list) has been seen; the guard keeps a fully masked tile NaN-free.
        const float msub = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m - msub);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < TL::DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      }
      const float msub = m == -INFINITY ? 0.f : m;
      float rs = 0.f;
      half8 pf[2][2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            const float p0 = __builtin_amdgcn_exp2f(s[st][8 * r + j] - msub);
            const float p1 = __builtin_amdgcn_exp2f(s[st][8 * r + j + 1] - msub);
            rs += p0 + p1;
            pf[st][r][j] = (_Float16)(p0 * pscale);
            pf[st][r][j + 1] = (_Float16)(p1 * pscale);
          }
        }
      }
      l += rs;
#pragma unroll
      for (int dt = 0; dt < TL::DT; ++dt) {
        const uint16_t* vr = Vt + (32 * dt + c) * TL::VS + 64 * sub + 8 * hf;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int r = 0; r < 2; ++r)
            o[dt] = mfma_f16_32x32x16(*reinterpret_cast<const half8*>(vr + 16 * (2 * st + r)),
                                      pf[st][r], o[dt]);
      }
    }
  }
};

template <int D, int BLK, bool FP8>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnArgs a) {
  using TL = Tile<D, BLK, FP8>;
  __shared__ __attribute__((aligned(16))) uint8_t Kl[TL::KLDS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * TL::VS];
  __shared__ uint32_t kept[kMaxKBlocks / 32];
  FP2_BOUNDS_GUARD(a.dbg);

  // ---- tile decode: 8 consecutive CSR ranks form a group; the slices of one
  // rank land on one XCD (blockIdx % 8); latest query blocks (most causal
  // work) are dispatched first
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
  const int P = T - n;
  const int QB = a.qblk;  // query block tokens: BLK, or 2 BLK (128-token query blocks over 64-token KV blocks)
  // the diagonal: KV blocks dlo..dhi hold the query block's own positions
  // (a single block when the query and KV blocks have one size)
  const int qpos0 = P + I * QB;  // absolute position of the block's first query
  const int dlo = qpos0 / BLK;
  const int dhi = (qpos0 + min(QB, n - I * QB) - 1) / BLK;
  const int G = a.hq / a.hkv;
  const int32_t* pt = a.page_table + (int64_t)s * a.max_pages;
  const int64_t mrow0 = (int64_t)g * a.total_kblocks + a.cu_kblocks[s];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int hf = lane >> 5;
  const int prow = slice * kRowsPerWG + wave * 32;  // first packed row of this wave
  const bool wave_active = prow < G * QB;
  const int h = g * G + prow / QB;                  // query head of this wave
  const int t0 = prow % QB;                         // first token (within the block)
  const int tq = t0 + (lane & 31);                  // this lane's query token
  const bool q_valid = wave_active && (I * QB + tq < n);

  const int kbeg = a.row_ptr[row], kend = a.row_ptr[row + 1];

  // kept-block bitmask for the correction tiles
  if (a.correction) {
    const int nw = (dhi + 32) >> 5;
    for (int w = t; w < nw; w += kThreads) kept[w] = 0u;
    __syncthreads();
    for (int i = kbeg + t; i < kend; i += kThreads) {
      const int j = a.col_idx[i];
      atomicOr(&kept[j >> 5], 1u << (j & 31));
    }
  }

  WaveState<D, BLK, FP8> ws;
  ws.m = -INFINITY;
  ws.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < TL::DT; ++dt) ws.o[dt] = f32x16{};
  float qscale = 1.f;
  {
    const uint8_t* qrow = a.q + ((int64_t)(q0 + I * QB + tq) * a.hq + h) * (D * TL::ESZ);
    if constexpr (!FP8) {
#pragma unroll
      for (int kk = 0; kk < TL::KK; ++kk) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (q_valid) v = *reinterpret_cast<const uint4*>(qrow + ws.koff(kk, hf) * 2);
        ws.qf[kk] = __builtin_bit_cast(bf16x8, v);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < TL::KK8; ++kk) {
        uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
        if (q_valid) {
          v0 = *reinterpret_cast<const uint4*>(qrow + 64 * kk + 32 * hf);
          v1 = *reinterpret_cast<const uint4*>(qrow + 64 * kk + 32 * hf + 16);
        }
        ws.qf8[kk] = i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                           (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
      }
      if (wave_active) qscale = a.q_scale[(int64_t)qb * a.hq + h];
    }
  }

  Stager<D, BLK, FP8> stg;

  // ---- exact path over the kept blocks (ascending: block 0 first)
  if (kbeg < kend) stg.load_block(a, pt, g, T, a.col_idx[kbeg], t);
  for (int i = kbeg; i < kend; ++i) {
    const int J = a.col_idx[i];
    float scl = a.scale_log2, pscale = 1.f;
    if constexpr (FP8) {
      const int64_t page = pt[J];  // page_size == BLK for e4m3
      scl *= qscale * a.k_scale[page * a.hkv + g];
      pscale = a.v_scale[page * a.hkv + g];
    }
    __syncthreads();
    stg.commit_block(Kl, Vt, t);
    __syncthreads();
    if (i + 1 < kend) stg.load_block(a, pt, g, T, a.col_idx[i + 1], t);
    // on the diagonal, keys past the query's own position are masked: its
    // offset from the block's first key
    if (wave_active)
      ws.template tile<0>(Kl, Vt, lane, scl, pscale, J >= dlo, qpos0 + tq - J * BLK, 0, dlo, kept, 0.f);
  }

  // ---- mean correction: tiles of BLK mean tokens over [1, dlo)
  if (a.correction && dlo > 1) {
    if constexpr (FP8) {
      // bf16 copy of the e4m3 query codes (exact); its scale goes into the logit scale
#pragma unroll
      for (int kk = 0; kk < TL::KK; ++kk) {
        const int w0 = 2 * (kk & 3);  // 8 codes = 2 dwords of fragment kk/4
        const i32x8 src = ws.qf8[kk >> 2];
        const f32x4 lo = e4m3x4_to_f32((uint32_t)src[w0]);
        const f32x4 hi = e4m3x4_to_f32((uint32_t)src[w0 + 1]);
        const uint4 v = make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                                   pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]));
        ws.qf[kk] = __builtin_bit_cast(bf16x8, v);
      }
    }
    const float scl_mean = a.scale_log2 * qscale;
    auto has_skipped = [&](int J0) {
      const int lo = max(1, J0), hi = min(J0 + BLK, dlo);
      int nk = 0;
      for (int j = lo; j < hi; ++j) nk += (kept[j >> 5] >> (j & 31)) & 1u;
      return hi - lo - nk > 0;
    };
    int J0 = 0;
    while (J0 < dlo && !has_skipped(J0)) J0 += BLK;
    if (J0 < dlo) stg.load_means(a, mrow0, J0, dlo, t);
    while (J0 < dlo) {
      int Jn = J0 + BLK;
      while (Jn < dlo && !has_skipped(Jn)) Jn += BLK;
      __syncthreads();
      stg.commit_means(Kl, Vt, t);
      __syncthreads();
      if (Jn < dlo) stg.load_means(a, mrow0, Jn, dlo, t);
      if (wave_active)
        ws.template tile<1>(Kl, Vt, lane, scl_mean, 1.f, false, tq, J0, dlo, kept, a.log2_block);
      J0 = Jn;
    }
  }

  // ---- epilogue: O / l -> bf16 (round to nearest even) or f32
  if (q_valid) {
    const float lt = ws.l + swap_halves(ws.l);
    const float inv = 1.0f / lt;
    const int64_t obase = ((int64_t)(q0 + I * QB + tq) * a.hq + h) * D;
    if (a.out_f32) {
      float* orow = static_cast<float*>(a.out) + obase;
#pragma unroll
      for (int dt = 0; dt < TL::DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * q4 + 4 * hf) =
              f32x4{ws.o[dt][4 * q4 + 0] * inv, ws.o[dt][4 * q4 + 1] * inv, ws.o[dt][4 * q4 + 2] * inv,
                    ws.o[dt][4 * q4 + 3] * inv};
    } else {
      uint16_t* orow = static_cast<uint16_t*>(a.out) + obase;
#pragma unroll
      for (int dt = 0; dt < TL::DT; ++dt) {
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
}

// Operand copies of the block means for the correction tiles: kbar as bf16
// (the QK^T operand type) and vbar as fp16 (the PV operand type of this
// kernel), both rounded to nearest even.
__global__ __launch_bounds__(256) void means_to_mma_kernel(const float* __restrict__ kbar,
                                                           const float* __restrict__ vbar,
                                                           uint16_t* __restrict__ k16,
                                                           uint16_t* __restrict__ v16, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4 k = reinterpret_cast<const f32x4*>(kbar)[i];
  const f32x4 v = reinterpret_cast<const f32x4*>(vbar)[i];
  reinterpret_cast<uint2*>(k16)[i] = make_uint2(pack_bf16x2(k[0], k[1]), pack_bf16x2(k[2], k[3]));
  _Float16 hv[4] = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
  uint2 bits;
  __builtin_memcpy(&bits, hv, sizeof(bits));
  reinterpret_cast<uint2*>(v16)[i] = bits;
}

template <int D, int BLK, bool FP8>
hipError_t launch_attn_t(const AttnArgs& a, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_kernel<D, BLK, FP8>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_attn_dt(int D, int BLK, const AttnArgs& a, unsigned grid, hipStream_t stream) {
  if (D == 128 && BLK == 128) return launch_attn_t<128, 128, FP8>(a, grid, stream);
  if (D == 128 && BLK == 64) return launch_attn_t<128, 64, FP8>(a, grid, stream);
  if (D == 64 && BLK == 128) return launch_attn_t<64, 128, FP8>(a, grid, stream);
  return launch_attn_t<64, 64, FP8>(a, grid, stream);
}

}  // namespace

hipError_t launch_prefill(const fp2_batch* b, const fp2_q* q, const fp2_kv* kv, const BatchInfo& info,
                          const int32_t* row_ptr, const int32_t* col_idx, const float* kbar,
                          const float* vbar, int correction, float softmax_scale, int out_f32,
                          void* out, int max_chunk_tiles, void* workspace, hipStream_t stream) {
  if (info.total_qblocks == 0) return hipSuccess;
  const int D = q->head_dim, BLK = info.kvblock, QB = info.qblock, hkv = kv->num_kv_heads;
  const bool vt = vt_path(q->dtype, D, info);
  const RunLayout L = run_layout(info, b->num_seqs, q->num_q_heads, hkv, D, q->dtype);
  uint8_t* wsb = static_cast<uint8_t*>(workspace);
  uint16_t* k16 = reinterpret_cast<uint16_t*>(wsb + L.k16);
  uint16_t* v16 = reinterpret_cast<uint16_t*>(wsb + L.v16);
  if (correction && !vt) {
    const int64_t n4 = (int64_t)hkv * info.total_kblocks * D / 4;
    hipLaunchKernelGGL(means_to_mma_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                       kbar, vbar, k16, v16, n4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  AttnArgs a;
  a.dbg = bounds_word();
  a.cu_seqlens_q = b->cu_seqlens_q;
  a.seqlens_k = b->seqlens_k;
  a.cu_qblocks = b->cu_qblocks;
  a.cu_kblocks = b->cu_kblocks;
  a.page_table = kv->page_table;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.q = static_cast<const uint8_t*>(q->q);
  a.k_pages = static_cast<const uint8_t*>(kv->k_pages);
  a.v_pages = static_cast<const uint8_t*>(kv->v_pages);
  a.q_scale = q->q_scale;
  a.k_scale = kv->k_scale;
  a.v_scale = kv->v_scale;
  a.kbar16 = k16;
  a.vbar16 = v16;
  a.vt = wsb + L.vt;
  a.vbt = wsb + L.v16;
  a.items = reinterpret_cast<int4*>(wsb + L.items);
  a.splits = reinterpret_cast<int4*>(wsb + L.splits);
  a.rank_slot = reinterpret_cast<int4*>(wsb + L.rank_slot);
  a.counters = reinterpret_cast<int32_t*>(wsb + L.counters);
  a.part = reinterpret_cast<float*>(wsb + L.part);
  a.info = reinterpret_cast<int32_t*>(wsb + L.info);
  a.skip = reinterpret_cast<uint32_t*>(wsb + L.skip);
  a.mlist = reinterpret_cast<int32_t*>(wsb + L.mlist);
  a.mcount = reinterpret_cast<int32_t*>(wsb + L.mcount);
  a.wskip = L.wskip;
  a.mtmax = L.mtmax;
  a.extra_cap = (int)L.extra_cap;
  // max_chunk_tiles > 0 caps the exact tiles of one work item below the
  // batch's own choice, < 0 turns the splitting of rows off
  if (max_chunk_tiles < 0) a.extra_cap = 0;
  a.chunk_cap = std::max(0, max_chunk_tiles);
  a.mt_cap = (int)L.mt_cap;
  a.out = out;
  a.out_f32 = out_f32;
  a.scale_log2 = softmax_scale * kLog2e;
  a.log2_block = log2f((float)BLK);
  a.num_seqs = b->num_seqs;
  a.hq = q->num_q_heads;
  a.hkv = hkv;
  a.max_pages = kv->max_pages_per_seq;
  a.page_size = kv->page_size;
  a.pm = PageMap::make(kv->page_size);
  a.total_qblocks = (int)info.total_qblocks;
  a.total_kblocks = (int)info.total_kblocks;
  a.correction = correction;
  a.qblk = QB;
  a.pair = vt && BLK == 64;
  const int G = q->num_q_heads / hkv;
  a.slices = (G * QB + kRowsPerWG - 1) / kRowsPerWG;
  a.rows = (int)(info.total_qblocks * hkv);
  const unsigned grid = (unsigned)(((a.rows + 7) / 8) * 8 * a.slices);
  if (vt) return launch_attn_d128(a, q->dtype == FP2_FP8_E4M3, kbar, vbar, (int)info.max_kblocks, stream);
  if (q->dtype == FP2_FP8_E4M3) return launch_attn_dt<true>(D, BLK, a, grid, stream);
  return launch_attn_dt<false>(D, BLK, a, grid, stream);
}

}  // namespace fp2
