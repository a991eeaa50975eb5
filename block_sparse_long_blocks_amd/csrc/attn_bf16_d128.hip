// Stage 2 for bf16 inputs with head_dim 128 and block 128: block-sparse
// causal GQA attention over the kept KV blocks plus the mean correction of
// every skipped block, in one online softmax.
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
//  * V is first transposed into V^T tiles (one 128 d x 128 key tile per KV
//    block and head, keys in the order the PV MFMA consumes them), and the
//    vbar of the mean tokens likewise; kbar is rounded to bf16 rows.
//  * Tiles stream global -> LDS by DMA (global_load_lds, 16 bytes a lane)
//    into two LDS buffers: the next tile's DMA runs while the current tile is
//    computed; one barrier per tile.  No staging registers, no LDS writes
//    from the waves.
//  * K tiles (rows = keys) and V^T tiles (rows = d) share one LDS layout:
//    256-byte rows in groups of four (one 1 KB DMA unit), groups 1088 bytes
//    apart, 16-byte chunk k of row r in slot k ^ (r & 3).  Every operand read
//    is a conflict-free ds_read_b128 at one of two per-lane bases plus an
//    immediate offset.
//  * S^T = K Q^T on the bf16 32x32x16 MFMA (a lane holds the keys of one
//    query, so row max / row sum are in-lane plus one lane^32 exchange);
//    O^T = V^T P^T on the same MFMA with P straight from the score registers.
//  * Each tile runs in 32-key steps, software-pipelined: one scheduling
//    region holds the QK^T MFMAs of step j+1, the PV MFMAs of step j-1 and
//    the softmax of step j, so matrix cores, LDS and vector ALU overlap
//    within a wave.  Masks enter as the score accumulator's initial value;
//    the reference max is refreshed lazily.
#include <type_traits>

#include "attn_common.h"

namespace fp2 {

namespace {

constexpr int kBlk = 128;
constexpr int kD = 128;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;   // 512
constexpr int kWGRows = 32 * kWaves;    // packed query rows per workgroup
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left unconstrained
// (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int kWaitVmcnt0 = 0x0F70;
// buffer resource word 3 for raw (untyped, unswizzled) 32-bit buffer loads on gfx9
constexpr int kBufferFlags = 0x00020000;
constexpr int kRowBytes = kD * 2;            // a K row (d values) or a V^T row (128 keys), bf16
constexpr int kGS = 4 * kRowBytes + 64;      // LDS stride of a 4-row group
constexpr int kTileLds = (kBlk / 4) * kGS;   // one K or V^T tile in LDS
constexpr int kTileGlobal = kBlk * kRowBytes;  // one V^T tile in global memory
// tile DMA: waves 0 .. kDmaWaves-1 each move kDmaRows rows of the K and the
// V^T tile (kDmaInstr instructions, K and V^T alternating)
constexpr int kDmaWaves = 4;
constexpr int kDmaRows = kBlk / kDmaWaves;
constexpr int kDmaHalves = kDmaRows / 16;
constexpr int kDmaInstr = kDmaRows / 2;
constexpr int kDmaSlotStep = 16 / kDmaInstr;

// Position p of a V^T row holds key key_of_pos(p): within each group of 16,
// positions 0-7 hold keys {0-3, 8-11} and positions 8-15 keys {4-7, 12-15},
// the keys that lane half 0 resp. 1 of a score accumulator holds.
__device__ __forceinline__ constexpr int key_of_pos(int p) {
  return (p & ~15) + 4 * ((p >> 3) & 1) + (p & 3) + 8 * ((p >> 2) & 1);
}

// ---------------------------------------------------------------------------
// Operand preparation
// ---------------------------------------------------------------------------
struct PrepArgs {
  const int32_t* cu_kblocks;
  const int32_t* seqlens_k;
  const int32_t* page_table;
  const uint8_t* v_pages;
  const float* kbar;
  const float* vbar;
  uint16_t* kbar16;  // bf16 [Hkv, total_kblocks, D]
  uint8_t* vt;       // V^T tiles [Hkv, total_kblocks]
  uint8_t* vbt;      // vbar^T tiles [Hkv, mt_cap]
  PageMap pm;
  int num_seqs, hkv, max_pages, page_size, total_kblocks, mt_cap;
};

// 8x8 transpose of 16-bit elements: in[e] is row e (word q = elements 2q, 2q+1);
// out[e] receives element e of every input row.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    uint32_t w[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint4 v = in[r];
      w[r] = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    }
    out[e] = make_uint4(__builtin_amdgcn_perm(w[1], w[0], sel), __builtin_amdgcn_perm(w[3], w[2], sel),
                        __builtin_amdgcn_perm(w[5], w[4], sel), __builtin_amdgcn_perm(w[7], w[6], sel));
  }
}

// One V^T tile per (KV block, head): thread t moves the 8 keys at positions
// 8(t/16) .. +7 for the 8 d values of chunk t%16.  Keys past the sequence end
// are zero.
__global__ __launch_bounds__(256) void vt_exact_kernel(PrepArgs a) {
  const int kb = blockIdx.x, g = blockIdx.y;
  const int s = find_seq(a.cu_kblocks, a.num_seqs, kb);
  const int J = kb - a.cu_kblocks[s];
  const int T = a.seqlens_k[s];
  const int32_t* pt = a.page_table + (int64_t)s * a.max_pages;
  const int t = threadIdx.x, c = t >> 4, dc = t & 15;
  uint4 in[8], out[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int pos = J * kBlk + key_of_pos(8 * c + e);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (pos < T) {
      int pi, slot;
      a.pm.split(pos, pi, slot);
      v = *reinterpret_cast<const uint4*>(a.v_pages + (((int64_t)pt[pi] * a.page_size + slot) * a.hkv + g) * kRowBytes +
                                          dc * 16);
    }
    in[e] = v;
  }
  transpose8x8(in, out);
  uint8_t* dst = a.vt + ((int64_t)g * a.total_kblocks + kb) * kTileGlobal + c * 16;
#pragma unroll
  for (int e = 0; e < 8; ++e) *reinterpret_cast<uint4*>(dst + (8 * dc + e) * kRowBytes) = out[e];
}

// Mean tokens: tile mt of sequence s holds mean tokens [128 mt, 128 mt + 128)
// of that sequence (vbar^T as bf16, zero past the sequence's blocks); the
// same workgroup rounds those tokens' kbar rows to bf16.  Tile index
// cu_kblocks[s]/128 + s + mt never collides across sequences and stays
// below mt_cap = total_kblocks/128 + num_seqs + 1.
__global__ __launch_bounds__(256) void vt_mean_kernel(PrepArgs a) {
  const int mt = blockIdx.x, s = blockIdx.y, g = blockIdx.z;
  const int kb0 = a.cu_kblocks[s];
  const int nkb = a.cu_kblocks[s + 1] - kb0;
  if (mt * kBlk >= nkb) return;
  const int t = threadIdx.x, c = t >> 4, dc = t & 15;
  const int64_t row0 = (int64_t)g * a.total_kblocks + kb0;
  uint4 in[8], out[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int jm = mt * kBlk + key_of_pos(8 * c + e);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (jm < nkb) {
      const float* src = a.vbar + (row0 + jm) * kD + dc * 8;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
      v = make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                     pack_bf16x2(hi[2], hi[3]));
    }
    in[e] = v;
  }
  transpose8x8(in, out);
  const int64_t tile = (int64_t)g * a.mt_cap + kb0 / kBlk + s + mt;
  uint8_t* dst = a.vbt + tile * kTileGlobal + c * 16;
#pragma unroll
  for (int e = 0; e < 8; ++e) *reinterpret_cast<uint4*>(dst + (8 * dc + e) * kRowBytes) = out[e];
  // kbar rows of the same mean tokens
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int id = t + 256 * u;
    const int jm = mt * kBlk + (id >> 4), ch = id & 15;
    if (jm < nkb) {
      const float* src = a.kbar + (row0 + jm) * kD + ch * 8;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
      *reinterpret_cast<uint4*>(a.kbar16 + (row0 + jm) * kD + ch * 8) =
          make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                     pack_bf16x2(hi[2], hi[3]));
    }
  }
}

// ---------------------------------------------------------------------------
// Attention
// ---------------------------------------------------------------------------

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

// bf16 pair (1, 1): the dot product with it sums two probabilities
typedef __bf16 bf16x2e __attribute__((ext_vector_type(2)));
constexpr uint32_t kOnesBf16x2 = 0x3f803f80u;
// a step whose probabilities (per lane: 16 of them) sum to this or more
// refreshes the reference max; probabilities stay below 2^64, so P (bf16),
// l and O (float32) cannot overflow
constexpr float kPmax = 18446744073709551616.0f;  // 2^64

// sched_group_barrier masks (LLVM AMDGPU IGroupLP)
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedValu = 0x002 | 0x400;  // VALU and transcendental

// Scheduling patterns for the regions of a tile: four operand reads up
// front, then each MFMA followed by the next read (while any are left) and V
// vector ALU instructions.  The counts must not exceed what the region holds,
// or the compiler drops the whole pattern (vector ALU instructions beyond the
// groups are placed freely).  Written out flat as macros: the compiler
// honours these barriers only when they sit, loop-free, in the body that
// holds the instructions.
#define FP2_SG(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)
#define FP2_MDV(V) FP2_SG(kSchedMfma, 1); FP2_SG(kSchedDsRead, 1); FP2_SG(kSchedValu, (V))
#define FP2_MV(V) FP2_SG(kSchedMfma, 1); FP2_SG(kSchedValu, (V))
#define FP2_MD FP2_SG(kSchedMfma, 1); FP2_SG(kSchedDsRead, 1)
// 8 MFMAs, 8 reads, no vector ALU
#define FP2_PATTERN_8 FP2_SG(kSchedDsRead, 4); FP2_MD; FP2_MD; FP2_MD; FP2_MD; FP2_SG(kSchedMfma, 4)
// 8 MFMAs, 8 reads, V vector ALU per MFMA
#define FP2_PATTERN_8V(V)                                                          \
  FP2_SG(kSchedDsRead, 4); FP2_MDV(V); FP2_MDV(V); FP2_MDV(V); FP2_MDV(V);         \
  FP2_MV(V); FP2_MV(V); FP2_MV(V); FP2_MV(V)
// 16 MFMAs, 16 reads, V vector ALU per MFMA
#define FP2_PATTERN_16V(V)                                                         \
  FP2_SG(kSchedDsRead, 4); FP2_MDV(V); FP2_MDV(V); FP2_MDV(V); FP2_MDV(V);         \
  FP2_MDV(V); FP2_MDV(V); FP2_MDV(V); FP2_MDV(V); FP2_MDV(V); FP2_MDV(V);          \
  FP2_MDV(V); FP2_MDV(V); FP2_MV(V); FP2_MV(V); FP2_MV(V); FP2_MV(V)

// Per-wave state and the work of one tile (32-key steps, see the header).
//
// Score accumulator element i of lane l (query l%32) is key
// 8(i/4) + 4(l/32) + i%4 of its step.  A masked score is -inf; a mean token's
// score carries log2(B)/scale extra, so that its probability carries the
// block weight B.
struct Wave {
  static constexpr int NS = kBlk / 32;  // 32-key steps per tile
  bf16x8 qf[kD / 16];
  f32x16 o[kD / 32];
  float m;    // reference max (log2 units), shared by lanes l and l^32
  float nb;   // -m (0 while m = -inf): exp2(s * scale + nb) is the probability
  float l;    // this lane's half of the denominator

  // S^T of step j accumulated onto c; K row 32j + l%32, chunk 2kk + l/32
  // (all operand reads are written before the MFMAs; the region's
  // scheduling pattern then moves them next to their MFMAs)
  __device__ __forceinline__ f32x16 qk(const uint8_t* Kt, int off0, int off1, int j, f32x16 c) const {
    bf16x8 kf[kD / 16];
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk)
      kf[kk] = *reinterpret_cast<const bf16x8*>(Kt + ((kk & 1) ? off1 : off0) + 8 * kGS * j + 64 * (kk >> 1));
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) c = mfma_bf16_32x32x16(kf[kk], qf[kk], c);
    return c;
  }

  // O^T += V^T P^T over the 32 keys of step j; V^T row 32dt + l%32, chunk
  // 4j + 2r + l/32
  __device__ __forceinline__ void pv(const uint8_t* Vt, int off0, int off1, int j, const bf16x8 (&pf)[2]) {
    bf16x8 vf[2][kD / 32];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
        vf[r][dt] = *reinterpret_cast<const bf16x8*>(Vt + (r ? off1 : off0) + 8 * kGS * dt + 64 * j);
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) o[dt] = mfma_bf16_32x32x16(vf[r][dt], pf[r], o[dt]);
  }

  // Initial score accumulator of step j on diagonal and mean-token tiles
  // (mode 1: -inf where key > query, else 0; mode 2: log2(B)/scale for a
  // skipped block's mean token, -inf for the others).
  __device__ __forceinline__ f32x16 mask(int mode, int j, int hf, int tq, float cb, const uint32_t* kept, int J0,
                                         int diag) const {
    f32x16 c;
    if (mode == 1) {
      int lim = tq - 32 * j - 4 * hf;  // element i is masked iff 8(i/4) + i%4 > lim
      asm volatile("" : "+v"(lim));    // computed here, not hoisted ahead of the branch
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = 8 * (i >> 2) + (i & 3) > lim ? -INFINITY : 0.f;
    } else {
      uint32_t w = skipped_word(kept, (J0 >> 5) + j, diag) >> (4 * hf);
      asm volatile("" : "+v"(w));
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = (w >> (8 * (i >> 2) + (i & 3))) & 1u ? cb : -INFINITY;
    }
    return c;
  }

  __device__ __forceinline__ void rescale(float alpha) {
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
  }

  // bf16 probabilities of one step against the reference max; returns the
  // sum of the rounded probabilities (two independent accumulation chains)
  __device__ __forceinline__ float probs(const f32x16& s, float scl, bf16x8 (&pf)[2]) const {
    float acc[2] = {0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[q] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * r + 2 * q], scl, nb)),
                           __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * r + 2 * q + 1], scl, nb)));
        // the denominator sums the same rounded probabilities that PV uses
        acc[q & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2e, w[q]),
                                                     __builtin_bit_cast(bf16x2e, kOnesBf16x2), acc[q & 1], false);
      }
      // computed here, not sunk into the next step's region
      asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
      pf[r] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
    return acc[0] + acc[1];
  }

  // Probabilities of one step against the current reference max, their sum
  // added to l.  The row max is not tracked on this path: the reference max
  // is set from the first step's scores (every row sees key 0 there) and
  // refreshed only when a step's probabilities reach kPmax, which keeps P,
  // l and O finite and exact while O / l does not depend on the reference.
  // Returns whether the whole wave must refresh and redo the step.
  __device__ __forceinline__ bool softmax(const f32x16& s, float scl, bf16x8 (&pf)[2]) {
    float step = probs(s, scl, pf);
    asm volatile("" : "+v"(step));
    l += step;
    return __any(!(step < kPmax));  // also catches inf
  }

  // Sets the reference max to cover this step's scores, rescales O (which
  // holds every step before this one) and l_prev (l before this step), and
  // redoes the step's probabilities.
  __device__ __forceinline__ void refresh(const f32x16& s, float scl, float l_prev, bf16x8 (&pf)[2]) {
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);  // max3 chain
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
    mx = fmaxf(mx, s[15]);
    const float mnew = fmaxf(m, max_halves(mx) * scl);  // scl > 0: -inf stays -inf
    const float alpha = __builtin_amdgcn_exp2f(m - (mnew == -INFINITY ? 0.f : mnew));
    m = mnew;
    nb = mnew == -INFINITY ? 0.f : -mnew;
    rescale(alpha);
    l = l_prev * alpha + probs(s, scl, pf);
  }

  // mode 0 exact block, 1 diagonal block, 2 mean-token tile starting at
  // mean token J0 (wave-uniform).  MASKED (modes 1, 2) sets up each step's
  // masks in a small block between the scheduling regions and starts the
  // score accumulators from them; exact blocks start from zero.
  template <bool MASKED>
  __device__ __forceinline__ void tile(int mode, bool first, const uint8_t* Kt, const uint8_t* Vt, int off0, int off1,
                                       int hf, float scl, float cb, int tq, int J0, int diag, const uint32_t* kept) {
    f32x16 cz = f32x16{};
    if constexpr (MASKED) cz = mask(mode, 0, hf, tq, cb, kept, J0, diag);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s = qk(Kt, off0, off1, 0, cz);
    FP2_PATTERN_8;
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 pp[2];  // probabilities of the previous step
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if constexpr (MASKED) {
        if (j + 1 < NS) cz = mask(mode, j + 1, hf, tq, cb, kept, J0, diag);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 sn = f32x16{};
      if (j + 1 < NS) sn = qk(Kt, off0, off1, j + 1, cz);
      if (j > 0) pv(Vt, off0, off1, j - 1, pp);
      bf16x8 pc[2];
      const float l_prev = l;
      const bool up = softmax(s, scl, pc) || (first && j == 0);
      // the softmax has about 36 vector ALU instructions
      if (j == 0 || j + 1 == NS) {
        FP2_PATTERN_8V(4);
      } else {
        FP2_PATTERN_16V(2);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (up) refresh(s, scl, l_prev, pc);  // after PV(j-1), before PV(j)
      pp[0] = pc[0];
      pp[1] = pc[1];
      s = sn;
    }
    __builtin_amdgcn_sched_barrier(0);
    pv(Vt, off0, off1, NS - 1, pp);
    FP2_PATTERN_8;
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- exact tiles on a fixed instruction schedule ----
  //
  // The 64 MFMAs of a tile run in the order QK(0) | QK(1) | QK(2),PV(0)
  // alternating | QK(3),PV(1) alternating | PV(2) | PV(3) (op n = 0..63, six
  // regions of 8, 8, 16, 16, 8, 8).  Each op is one slot closed by a
  // scheduling barrier, so the order below is the issue order: op n's LDS
  // operand is read kLA slots ahead (across regions), and the softmax of
  // step j runs in region j+1 as a stream of groups spread over the slots,
  // each value produced a group or more before it is consumed, so that no
  // vector instruction waits on the one just before it and the matrix core
  // keeps getting work.  The refresh test of step j closes region j+1,
  // before PV(j) reads P(j).
  static constexpr int kLA = 4;
  static constexpr int kGroups = 20;
  static constexpr int kDma0 = 8;  // the next tile's DMA instructions go out from op 8 on, kDmaSlotStep apart

  __device__ static constexpr bool op_qk(int n) { return n < 16 || (n < 48 && (n & 1) == 0); }
  __device__ static constexpr int op_step(int n) {
    return op_qk(n) ? (n < 8 ? 0 : n < 16 ? 1 : n < 32 ? 2 : 3) : (n < 32 ? 0 : n < 48 ? 1 : n < 56 ? 2 : 3);
  }
  // QK: d-slice kk; PV: 4 r + dt
  __device__ static constexpr int op_idx(int n) { return n < 16 ? (n & 7) : n < 48 ? ((n & 15) >> 1) : (n & 7); }

  __device__ __forceinline__ const uint8_t* op_addr(int n, const uint8_t* Kt, const uint8_t* Vt, int off0,
                                                    int off1) const {
    const int j = op_step(n), i = op_idx(n);
    if (op_qk(n)) return Kt + ((i & 1) ? off1 : off0) + 8 * kGS * j + 64 * (i >> 1);
    return Vt + ((i >> 2) ? off1 : off0) + 8 * kGS * (i & 3) + 64 * j;
  }

  // softmax stream of one step: group g computes x[g] (g < 16), e[g-2]
  // (2 <= g < 18), the bf16 pair w[(g-4)/2] (even g >= 4) and adds e[g-4]
  // to the row sum (g >= 4)
  struct Soft {
    float x[16], e[16], acc[2];
    uint32_t w[8];
  };
  // Masked tiles pass the per-lane bit mask M of the step's allowed keys
  // (bit 8(i/4) + i%4 for element i) and nbm = nb + log2(B) on mean tiles:
  // a masked element's exponent is -inf.
  template <bool MASKED>
  __device__ __forceinline__ void soft_group(int g, Soft& st, const f32x16& s, float scl, float nbm,
                                             uint32_t M) const {
    if (g < 16) {
      float x = __builtin_fmaf(s[g], scl, nbm);
      if constexpr (MASKED) {
        const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)M, 8 * (g >> 2) + (g & 3), 1);
        x = __uint_as_float((sel & __float_as_uint(x)) | (~sel & 0xff800000u));
      }
      st.x[g] = x;
      asm volatile("" : "+v"(st.x[g]));
    }
    if (g >= 2 && g < 18) {
      st.e[g - 2] = __builtin_amdgcn_exp2f(st.x[g - 2]);
      asm volatile("" : "+v"(st.e[g - 2]));
    }
    if (g >= 4 && g < 20 && (g & 1) == 0) {
      st.w[(g - 4) >> 1] = pack_bf16x2(st.e[g - 4], st.e[g - 3]);
      asm volatile("" : "+v"(st.w[(g - 4) >> 1]));
    }
    if (g >= 4 && g < 20) {
      // the row sum adds the float32 probabilities (PV takes them rounded to
      // bf16: O / l then errs by at most 2^-9 max|v| relative to exact P)
      st.acc[g & 1] += st.e[g - 4];
      asm volatile("" : "+v"(st.acc[g & 1]));
    }
  }

  // one region: ops [n0, n0 + S), with the softmax stream of s when SOFT
  template <int N0, int S, bool SOFT, bool MASKED, class Dma>
  __device__ __forceinline__ void region(bf16x8 (&fr)[8], f32x16& sn, const bf16x8 (&pp)[2], Soft& st,
                                         const f32x16& s, const uint8_t* Kt, const uint8_t* Vt, int off0, int off1,
                                         float scl, float nbm, uint32_t M, Dma& dma) {
#pragma unroll
    for (int t = 0; t < S; ++t) {
      const int n = N0 + t;
      if (op_qk(n)) {
        sn = mfma_bf16_32x32x16(fr[n & 7], qf[op_idx(n)], sn);
      } else {
        const int i = op_idx(n);
        o[i & 3] = mfma_bf16_32x32x16(fr[n & 7], pp[i >> 2], o[i & 3]);
      }
      if (n + kLA < 64) fr[(n + kLA) & 7] = *reinterpret_cast<const bf16x8*>(op_addr(n + kLA, Kt, Vt, off0, off1));
      if (n >= kDma0 && n < kDma0 + kDmaInstr * kDmaSlotStep && (n - kDma0) % kDmaSlotStep == kDmaSlotStep - 1)
        dma((n - kDma0) / kDmaSlotStep);
      if constexpr (SOFT) {
#pragma unroll
        for (int g = t * kGroups / S; g < (t + 1) * kGroups / S; ++g) soft_group<MASKED>(g, st, s, scl, nbm, M);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // closes the softmax of a step: P, l, and the refresh when the step's
  // probabilities reached kPmax (or it is the first step of the row)
  template <bool MASKED>
  __device__ __forceinline__ void soft_close(Soft& st, const f32x16& s, float scl, bool force, bf16x8 (&pc)[2],
                                             uint32_t M, float cbs) {
    pc[0] = __builtin_bit_cast(bf16x8, make_uint4(st.w[0], st.w[1], st.w[2], st.w[3]));
    pc[1] = __builtin_bit_cast(bf16x8, make_uint4(st.w[4], st.w[5], st.w[6], st.w[7]));
    const float step = st.acc[0] + st.acc[1];
    const float l_prev = l;
    l += step;
    if (__any(!(step < kPmax)) || force) {
      if constexpr (MASKED) {
        f32x16 sm;  // the scores as the stream saw them: + cbs where allowed, -inf elsewhere
#pragma unroll
        for (int i = 0; i < 16; ++i) sm[i] = (M >> (8 * (i >> 2) + (i & 3))) & 1u ? s[i] + cbs : -INFINITY;
        refresh(sm, scl, l_prev, pc);
      } else {
        refresh(s, scl, l_prev, pc);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // One tile.  MASKED: mode 1 diagonal block (key > query masked), mode 2
  // mean-token tile starting at mean token J0 (only skipped blocks' tokens
  // count, each with weight B: lb = log2 B added to the exponent, cbs = lb /
  // scl in score units).
  template <bool MASKED, class Dma>
  __device__ __forceinline__ void tile_fast(bool first, const uint8_t* Kt, const uint8_t* Vt, int off0, int off1,
                                            float scl, Dma&& dma, int mode, int tq, int hf, float lb, float cbs,
                                            int J0, int diag, const uint32_t* kept) {
    bf16x8 fr[8];
    bf16x8 pp[2] = {qf[0], qf[0]}, pc[2];
    f32x16 s = f32x16{}, sn = f32x16{};
    Soft st;
    uint32_t M[NS] = {};
    if constexpr (MASKED) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        if (mode == 0) {
          M[j] = ~0u;
        } else if (mode == 1) {
          const int lim = tq - 32 * j - 4 * hf;  // element i allowed iff 8(i/4) + i%4 <= lim
          M[j] = lim >= 31 ? ~0u : lim < 0 ? 0u : (2u << lim) - 1u;
        } else {
          M[j] = skipped_word(kept, (J0 >> 5) + j, diag) >> (4 * hf);
        }
      }
    } else {
      lb = 0.f;
      cbs = 0.f;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < kLA; ++n) fr[n] = *reinterpret_cast<const bf16x8*>(op_addr(n, Kt, Vt, off0, off1));
    __builtin_amdgcn_sched_barrier(0);
    region<0, 8, false, MASKED>(fr, sn, pp, st, s, Kt, Vt, off0, off1, scl, 0.f, 0u, dma);  // QK(0)
    s = sn;
    sn = f32x16{};
    st.acc[0] = st.acc[1] = 0.f;
    region<8, 8, true, MASKED>(fr, sn, pp, st, s, Kt, Vt, off0, off1, scl, nb + lb, M[0], dma);  // QK(1), softmax(0)
    soft_close<MASKED>(st, s, scl, first, pc, M[0], cbs);
    pp[0] = pc[0];
    pp[1] = pc[1];
    s = sn;
    sn = f32x16{};
    st.acc[0] = st.acc[1] = 0.f;
    region<16, 16, true, MASKED>(fr, sn, pp, st, s, Kt, Vt, off0, off1, scl, nb + lb, M[1], dma);  // QK(2), PV(0), softmax(1)
    soft_close<MASKED>(st, s, scl, false, pc, M[1], cbs);
    pp[0] = pc[0];
    pp[1] = pc[1];
    s = sn;
    sn = f32x16{};
    st.acc[0] = st.acc[1] = 0.f;
    region<32, 16, true, MASKED>(fr, sn, pp, st, s, Kt, Vt, off0, off1, scl, nb + lb, M[2], dma);  // QK(3), PV(1), softmax(2)
    soft_close<MASKED>(st, s, scl, false, pc, M[2], cbs);
    pp[0] = pc[0];
    pp[1] = pc[1];
    s = sn;
    st.acc[0] = st.acc[1] = 0.f;
    region<48, 8, true, MASKED>(fr, sn, pp, st, s, Kt, Vt, off0, off1, scl, nb + lb, M[3], dma);  // PV(2), softmax(3)
    soft_close<MASKED>(st, s, scl, false, pc, M[3], cbs);
    pp[0] = pc[0];
    pp[1] = pc[1];
    region<56, 8, false, MASKED>(fr, sn, pp, st, s, Kt, Vt, off0, off1, scl, 0.f, 0u, dma);  // PV(3)
  }
};

__global__ __launch_bounds__(kThreads, 1) void attn_bf16_d128_kernel(AttnArgs a) {
  // two K and two V^T buffers, as separate objects so that the compiler can
  // tell the DMA target from the buffers being read
  __shared__ __attribute__((aligned(1024))) uint8_t K0[kTileLds];
  __shared__ __attribute__((aligned(1024))) uint8_t K1[kTileLds];
  __shared__ __attribute__((aligned(1024))) uint8_t V0[kTileLds];
  __shared__ __attribute__((aligned(1024))) uint8_t V1[kTileLds];
  __shared__ uint32_t kept[kMaxKBlocks / 32];
  __shared__ int mtile[kMaxKBlocks / kBlk + 1];
  __shared__ int s_nmean;

  // ---- tile decode: 8 consecutive CSR ranks form a group, the slices of
  // one rank share blockIdx % 8 (one XCD), latest query blocks first
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
  const int diag = (T - n) / kBlk + I;
  const int G = a.hq / a.hkv;
  const int32_t* pt = a.page_table + (int64_t)s * a.max_pages;
  const int kb0 = a.cu_kblocks[s];
  const int64_t mrow0 = (int64_t)g * a.total_kblocks + kb0;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int hf = lane >> 5;
  const int prow = slice * kWGRows + wave * 32;
  const bool wave_active = prow < G * kBlk;
  const int h = g * G + prow / kBlk;
  const int tq = prow % kBlk + (lane & 31);
  const bool q_valid = wave_active && (I * kBlk + tq < n);

  // uniform values: later loads indexed by them become scalar loads, which
  // do not share the vector-memory counter with the tile DMA
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
      const int ncand = (diag + kBlk - 1) / kBlk;
      int base = 0;
      for (int m0 = 0; m0 < ncand; m0 += 64) {
        const int mt = m0 + lane;
        bool flag = false;
        if (mt < ncand) {
#pragma unroll
          for (int w = 0; w < kBlk / 32; ++w) flag |= skipped_word(kept, mt * (kBlk / 32) + w, diag) != 0u;
        }
        const uint64_t bal = __ballot(flag);
        if (flag) mtile[base + __popcll(bal & ((1ull << lane) - 1ull))] = mt * kBlk;
        base += __popcll(bal);
      }
      if (lane == 0) s_nmean = base;
    }
    __syncthreads();
    nmean = s_nmean;
  }
  const int ntiles = nexact + nmean;

  Wave ws;
  ws.m = -INFINITY;
  ws.nb = 0.f;
  ws.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt) ws.o[dt] = f32x16{};
  {
    const uint8_t* qrow = a.q + ((int64_t)(q0 + I * kBlk + tq) * a.hq + h) * kRowBytes;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (q_valid) v = *reinterpret_cast<const uint4*>(qrow + (16 * kk + 8 * hf) * 2);
      ws.qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- DMA of one tile: wave w < kDmaWaves moves rows R w .. R w + R-1
  // (R = kDmaRows; LDS row groups R w/4 ..) of the K and the V^T tile, R/4
  // instructions each; lane i of instruction p moves row R w + 4p + i/16,
  // chunk (i%16) ^ (i/16), into its 16-byte slot.  On the fast paths (each 16
  // rows lie in one page and all inside the sequence, or they are whole mean
  // tokens below the diagonal) the source of instruction p is a wave-uniform
  // base per 16 rows plus a uniform step plus a per-lane offset fixed for the
  // kernel, and exact tiles issue the instructions one by one between their
  // MFMAs; otherwise each lane looks up its own row and all go out at once.
  const bool dma_wave = wave < kDmaWaves;
  const int uoff = 16 * ((lane & 15) ^ (lane >> 4));
  const uint32_t voff = (uint32_t)((lane >> 4) * kRowBytes + uoff);  // + 1024 p: rows of 256 bytes
  const uint32_t tok = (uint32_t)a.hkv * kRowBytes;                  // K row stride in the cache
  const uint32_t koff = (uint32_t)(lane >> 4) * tok + uoff;          // + 4 p tok
  const bool pages16 = a.page_size % 16 == 0;
  // Uniform values for later tiles (block indices, page entries) come through
  // vector buffer loads: they share the vector-memory counter with the DMA,
  // so the wait at each tile barrier covers them.  Scalar loads would share
  // the LDS counter instead, and every tile's first operand-read wait would
  // then also wait for them.
  const __amdgpu_buffer_rsrc_t rcol =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.col_idx + kbeg), (short)0, nexact * 4, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rpt =
      __builtin_amdgcn_make_buffer_rsrc((void*)pt, (short)0, a.max_pages * 4, kBufferFlags);
  auto page_of = [&](int J, int hh) -> int {  // page of rows R w + 16 hh.. of block J (valid after the next barrier)
    int pi, slot;
    a.pm.split(min(J * kBlk + kDmaRows * wave + 16 * hh, T - 1), pi, slot);
    return __builtin_amdgcn_raw_buffer_load_b32(rpt, pi * 4, 0, 0);
  };
  // a value loaded before the last barrier, read as a wave-uniform scalar there
  // (pinned after the barrier so the read is not hoisted next to its load)
  auto after_barrier = [](int v) {
    asm volatile("" : "+v"(v));
    return __builtin_amdgcn_readfirstlane(v);
  };
  auto lds = [](uint8_t* p) { return (__attribute__((address_space(3))) void*)p; };
  // the fast-path sources of one tile (instruction p: kb + p * kstep + kvo, vb + 1024 p + voff)
  struct DmaPlan {
    const uint8_t* kb[kDmaHalves];
    const uint8_t* vb;
    uint32_t kstep, kvo;
    bool fast;
  };
  // Plans the DMA of tile idx (block or mean token j, page entry pg of this
  // wave's rows) into Kd / Vd; slow paths are issued here.
  auto plan = [&](int idx, int j, const int (&pg)[kDmaHalves], uint8_t* Kd, uint8_t* Vd) __attribute__((always_inline)) {
    DmaPlan pl;
    pl.fast = false;
    if (!dma_wave) return pl;
    uint8_t* kd = Kd + (kDmaRows / 4) * wave * kGS;
    uint8_t* vd = Vd + (kDmaRows / 4) * wave * kGS;
    if (idx < nexact) {
      pl.vb = a.vt + (((int64_t)g * a.total_kblocks + kb0 + j) * kBlk + kDmaRows * wave) * kRowBytes;
      const int r0 = j * kBlk + kDmaRows * wave;
      pl.fast = pages16 && r0 + kDmaRows - 1 < T;
      if (pl.fast) {
#pragma unroll
        for (int hh = 0; hh < kDmaHalves; ++hh) {
          int pi, slot;
          a.pm.split(r0 + 16 * hh, pi, slot);
          pl.kb[hh] = a.k_pages + (((int64_t)pg[hh] * a.page_size + slot) * a.hkv + g) * kRowBytes;
        }
        pl.kstep = 4 * tok;
        pl.kvo = koff;
      } else {
#pragma unroll
        for (int p = 0; p < kDmaRows / 4; ++p) {
          int pi, slot;
          a.pm.split(min(r0 + 4 * p + (lane >> 4), T - 1), pi, slot);  // rows past the end repeat the last key
          const uint8_t* ksrc = a.k_pages + (((int64_t)pt[pi] * a.page_size + slot) * a.hkv + g) * kRowBytes + uoff;
          __builtin_amdgcn_global_load_lds(ksrc, lds(kd + p * kGS), 16, 0, 0);
          __builtin_amdgcn_global_load_lds(pl.vb + voff + 1024 * p, lds(vd + p * kGS), 16, 0, 0);
        }
      }
    } else {
      pl.vb = a.vbt + (((int64_t)g * a.mt_cap + kb0 / kBlk + s + j / kBlk) * kBlk + kDmaRows * wave) * kRowBytes;
      const uint8_t* k16 = reinterpret_cast<const uint8_t*>(a.kbar16);
      const int r0 = j + kDmaRows * wave;
      pl.fast = r0 + kDmaRows - 1 < diag;
      if (pl.fast) {
#pragma unroll
        for (int hh = 0; hh < kDmaHalves; ++hh) pl.kb[hh] = k16 + (mrow0 + r0 + 16 * hh) * kRowBytes;
        pl.kstep = 1024;
        pl.kvo = voff;
      } else {
#pragma unroll
        for (int p = 0; p < kDmaRows / 4; ++p) {
          const int jm = min(r0 + 4 * p + (lane >> 4), diag - 1);  // tokens past diag repeat a real one (masked)
          __builtin_amdgcn_global_load_lds(k16 + (mrow0 + jm) * kRowBytes + uoff, lds(kd + p * kGS), 16, 0, 0);
          __builtin_amdgcn_global_load_lds(pl.vb + voff + 1024 * p, lds(vd + p * kGS), 16, 0, 0);
        }
      }
    }
    return pl;
  };
  // instruction i of a fast plan: K row group i/2 (even i) or V^T row group i/2 (odd i)
  auto issue = [&](const DmaPlan& pl, int i, uint8_t* Kd, uint8_t* Vd) __attribute__((always_inline)) {
    const int p = i >> 1;
    const int grp = (kDmaRows / 4) * wave + p;
    if ((i & 1) == 0)
      __builtin_amdgcn_global_load_lds(pl.kb[p >> 2] + (p & 3) * pl.kstep + pl.kvo, lds(Kd + grp * kGS), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(pl.vb + 1024 * p + voff, lds(Vd + grp * kGS), 16, 0, 0);
  };

  // per-lane operand offsets (see Wave::qk / Wave::pv): row l%32 of a 32-row
  // slab, chunk parity 0 / 1 of the lane's half
  const int c = lane & 31, x = c & 3;
  const int rbase = (c >> 2) * kGS + x * kRowBytes;
  const int off0 = rbase + 16 * (hf ^ x);
  const int off1 = rbase + 16 * ((2 + hf) ^ x);

  // Tile pipeline: at iteration i the LDS buffers i%2 hold tile i and the
  // DMA of tile i+1 into the other buffers is in flight; the block index of
  // tile i+2 and the page entries of tile i+1 arrived with the last barrier,
  // the loads of tile i+3's block index and tile i+2's page entries are in
  // flight.
  auto mean_of = [&](int idx) -> int { return idx < ntiles ? mtile[idx - nexact] : 0; };
  int j0 = 0, j1 = 0, j2v = 0, pgv[kDmaHalves] = {};
  if (0 < nexact) j0 = ld_uniform(a.col_idx, kbeg);
  else if (0 < ntiles) j0 = mean_of(0);
  if (1 < nexact) j1 = ld_uniform(a.col_idx, kbeg + 1);
  else if (1 < ntiles) j1 = mean_of(1);
  if (2 < nexact) j2v = __builtin_amdgcn_raw_buffer_load_b32(rcol, 2 * 4, 0, 0);
  if (ntiles > 0) {
    int pg0[kDmaHalves] = {};
    if (0 < nexact && dma_wave) {
#pragma unroll
      for (int hh = 0; hh < kDmaHalves; ++hh) pg0[hh] = __builtin_amdgcn_readfirstlane(page_of(j0, hh));
    }
    const DmaPlan pl = plan(0, j0, pg0, K0, V0);
    if (pl.fast) {
#pragma unroll
      for (int i = 0; i < kDmaInstr; ++i) issue(pl, i, K0, V0);
    }
  }
  if (1 < nexact && dma_wave) {
#pragma unroll
    for (int hh = 0; hh < kDmaHalves; ++hh) pgv[hh] = page_of(j1, hh);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  const float scl = a.scale_log2;
  const float cb = a.log2_block / scl;  // mean-token weight log2(B) in score units

  // MASKED_C: std::integral_constant<bool, ...>, the tile code path (see below)
  auto iter = [&](auto masked_c, int idx, const uint8_t* Kc, const uint8_t* Vc, uint8_t* Kn, uint8_t* Vn) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int j2 = idx + 2 < nexact ? after_barrier(j2v) : mean_of(idx + 2);
    DmaPlan pl;
    pl.fast = false;
    if (idx + 1 < ntiles) {
      int pg[kDmaHalves] = {};
      if (idx + 1 < nexact && dma_wave) {
#pragma unroll
        for (int hh = 0; hh < kDmaHalves; ++hh) pg[hh] = after_barrier(pgv[hh]);
      }
      pl = plan(idx + 1, j1, pg, Kn, Vn);
    }
    if (idx + 2 < nexact && dma_wave) {
#pragma unroll
      for (int hh = 0; hh < kDmaHalves; ++hh) pgv[hh] = page_of(j2, hh);
    }
    if (idx + 3 < nexact) j2v = __builtin_amdgcn_raw_buffer_load_b32(rcol, (idx + 3) * 4, 0, 0);
    const int mode = idx >= nexact ? 2 : (j0 == diag ? 1 : 0);
    auto dma = [&](int i) __attribute__((always_inline)) {
      if (pl.fast) issue(pl, i, Kn, Vn);
    };
    if (!wave_active) {
      if (pl.fast) {
#pragma unroll
        for (int i = 0; i < kDmaInstr; ++i) issue(pl, i, Kn, Vn);
      }
    } else if constexpr (!MASKED) {
      ws.tile_fast<false>(idx == 0, Kc, Vc, off0, off1, scl, dma, 0, tq, hf, 0.f, 0.f, 0, diag, kept);
    } else {
      const float lbm = mode == 2 ? a.log2_block : 0.f;
      ws.tile_fast<true>(idx == 0, Kc, Vc, off0, off1, scl, dma, mode, tq, hf, lbm, mode == 2 ? cb : 0.f, j0, diag,
                         kept);
    }
    j0 = j1;
    j1 = j2;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's DMA and loads for later tiles have landed
    __syncthreads();
  };
  // Two loops, each with one tile code path (one instance of the tile code
  // per loop keeps the register allocation of each loop separate): first the
  // exact tiles off the diagonal, which CSR order puts ahead of the diagonal
  // block, then everything else (diagonal, mean tiles, and any exact tile
  // that would follow them) on the masked path, whose mask lets a plain
  // exact tile through whole.
  const std::integral_constant<bool, false> plain_c;
  const std::integral_constant<bool, true> masked_c;
  int idx = 0;
  while (idx < nexact && j0 != diag) {
    iter(plain_c, idx, K0, V0, K1, V1);
    ++idx;
    if (!(idx < nexact && j0 != diag)) break;
    iter(plain_c, idx, K1, V1, K0, V0);
    ++idx;
  }
  if (idx < ntiles && (idx & 1)) {
    iter(masked_c, idx, K1, V1, K0, V0);
    ++idx;
  }
  for (; idx < ntiles; idx += 2) {
    iter(masked_c, idx, K0, V0, K1, V1);
    if (idx + 1 < ntiles) iter(masked_c, idx + 1, K1, V1, K0, V0);
  }

  // ---- epilogue: O / l
  if (q_valid) {
    const float inv = 1.0f / sum_halves(ws.l);
    const int64_t obase = ((int64_t)(q0 + I * kBlk + tq) * a.hq + h) * kD;
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

#undef FP2_PATTERN_16V
#undef FP2_PATTERN_8V
#undef FP2_PATTERN_8
#undef FP2_MD
#undef FP2_MV
#undef FP2_MDV
#undef FP2_SG

}  // namespace

hipError_t launch_attn_bf16_d128(const AttnArgs& a_in, const float* kbar, const float* vbar, int max_kblocks,
                                 hipStream_t stream) {
  AttnArgs a = a_in;
  uint16_t* kbar16 = const_cast<uint16_t*>(a.kbar16);
  uint8_t* vbt = const_cast<uint8_t*>(a.vbt);
  uint8_t* vt = const_cast<uint8_t*>(a.vt);
  PrepArgs p;
  p.cu_kblocks = a.cu_kblocks;
  p.seqlens_k = a.seqlens_k;
  p.page_table = a.page_table;
  p.v_pages = a.v_pages;
  p.kbar = kbar;
  p.vbar = vbar;
  p.kbar16 = kbar16;
  p.vt = vt;
  p.vbt = vbt;
  p.pm = a.pm;
  p.num_seqs = a.num_seqs;
  p.hkv = a.hkv;
  p.max_pages = a.max_pages;
  p.page_size = a.page_size;
  p.total_kblocks = a.total_kblocks;
  p.mt_cap = a.mt_cap;
  if (a.total_kblocks > 0) {
    hipLaunchKernelGGL(vt_exact_kernel, dim3((unsigned)a.total_kblocks, (unsigned)a.hkv), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.correction) {
      hipLaunchKernelGGL(vt_mean_kernel,
                         dim3((unsigned)((max_kblocks + kBlk - 1) / kBlk), (unsigned)a.num_seqs, (unsigned)a.hkv),
                         dim3(256), 0, stream, p);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const int G = a.hq / a.hkv;
  a.slices = (G * kBlk + kWGRows - 1) / kWGRows;
  const unsigned grid = (unsigned)(((a.rows + 7) / 8) * 8 * a.slices);
  hipLaunchKernelGGL(attn_bf16_d128_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fp2
