// Stage 2 for head_dim 128 and query blocks of 128 over KV blocks of 128 or
// of 64, bf16 or e4m3 inputs: block-sparse causal GQA attention
// over the kept KV blocks plus the mean correction of every skipped block, in
// one online softmax.
//
// FlashPrefill V2 (metallab.ai paper page): Figure 3 (exact path over the
// CSR-selected blocks, correction path merged in the online softmax),
// Figure 4 (a pruned block J adds |B_J| * exp(q . kbar_J / sqrt(d)) * (vbar_J, 1)),
// Table 7 (CSR per KV head, paged KV at any page size, 128-token query tiles
// over a CSR of 64-token KV tiles).
//
// CDNA4 layout of the work:
//  * One workgroup = 8 waves = 256 packed query rows of one CSR row (the G
//    query heads of a KV head times B tokens); each wave owns 32 tokens of one
//    head, so every K/V tile staged in LDS feeds 256 query rows.
//  * V is first transposed into V^T tiles (one 128 d x 128 key tile per KV
//    block and head, keys in the order the PV MFMA consumes them; e4m3 V
//    dequantized), and the vbar of the mean tokens likewise; kbar is rounded
//    to bf16 rows.  e4m3 K tiles stay e4m3 codes, read from the pages.
//  * Tiles stream global -> LDS by DMA (global_load_lds, 16 bytes a lane)
//    into two LDS buffers: the next tile's DMA runs while the current tile is
//    computed; one barrier per tile.  No staging registers; the waves write
//    LDS only in the epilogue (bf16 output rows).
//  * bf16 K tiles (rows = keys) and V^T tiles (rows = d) share one LDS
//    layout: 256-byte rows in groups of four (one 1 KB DMA unit), groups 1088
//    bytes apart, 16-byte chunk k of row r in slot k ^ (r & 3); e4m3 K tiles
//    are 128-byte rows, chunk c of row r in slot c ^ (r % 8).  Every operand
//    read is a conflict-free ds_read_b128 at a per-lane base plus an
//    immediate offset.
//  * S^T = K Q^T on the bf16 32x32x16 MFMA or the e4m3 32x32x64 MFMA (a lane
//    holds keys of one query, so row maxima are in-lane plus one lane^32
//    exchange); O^T = V^T P^T on the bf16 MFMA with P straight from the
//    score registers, and the row sums on the matrix core from the same P
//    (a 16x16x32 MFMA per 16-key half of a step, see Wave).
//  * Each tile runs in 32-key steps on a fixed instruction schedule: every
//    MFMA is a slot closed by a scheduling barrier, the QK^T MFMAs of step
//    j+1 and the PV MFMAs of step j-1 share a region with the softmax of
//    step j, operand reads run a few slots ahead and the softmax values are
//    consumed a group or more after they are produced.  Diagonal masks are
//    applied to the exponent; mean-token tiles take their weight and mask
//    from one more MFMA per step on the plain schedule; the reference max is
//    refreshed only when a probability would reach 2^64.  The younger wave
//    of each SIMD takes the higher issue priority for the first half of a
//    tile (the arbiter otherwise serves the older one first).
//  * 64-token KV blocks: a tile holds two kept blocks (CSR entries 2i and
//    2i+1 of the row), waves 0-1 moving the first block's K rows and 2-3 the
//    second's; V^T is kept as half tiles (128 d x 64 keys) and each lane
//    takes its 16-byte chunk from the half its key positions belong to.  A
//    row's last entry may be alone (second half masked); the diagonal mask
//    is by position and the logit scale (e4m3: the block's K scale) per
//    half.
//  * The workgroups run work items built on the device (items_kernel):
//    the first half of the KV heads, then the second, each heaviest first,
//    with the exact tiles of rows much heavier than the rest
//    cut into chunks whose float32 partials combine_kernel merges.
#include <mutex>
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
// s_waitcnt immediate for lgkmcnt(0) with vmcnt and expcnt left unconstrained
constexpr int kWaitLgkm0 = 0xC07F;
// buffer resource word 3 for raw (untyped, unswizzled) 32-bit buffer loads on gfx9
constexpr int kBufferFlags = 0x00020000;
constexpr int kRowBytes = kD * 2;            // a K row (d values) or a V^T row (128 keys), bf16
constexpr int kGS = 4 * kRowBytes + 64;      // LDS stride of a 4-row group
constexpr int kTileLds = (kBlk / 4) * kGS;   // one K or V^T tile in LDS
// bf16 output staging in the epilogue: 32 rows of 256 bytes per wave, rows
// 272 bytes apart, four waves per tile buffer
constexpr int kStageRow = kRowBytes + 16;
constexpr int kStageBytes = 32 * kStageRow;
static_assert(4 * kStageBytes <= kTileLds, "epilogue staging must fit one tile buffer");
constexpr int kTileGlobal = kBlk * kRowBytes;  // one V^T tile in global memory
// tile DMA: waves 0 .. kDmaWaves-1 each move kDmaRows rows of the K and the
// V^T tile (kDmaInstr instructions, K and V^T alternating)
constexpr int kDmaWaves = 4;
constexpr int kDmaRows = kBlk / kDmaWaves;
constexpr int kDmaHalves = kDmaRows / 16;
constexpr int kDmaInstr = kDmaRows / 2;

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
  const uint32_t* dbg;  // bounds-checking builds: the error word, else nullptr
  const int32_t* cu_kblocks;
  const int32_t* cu_seqlens_q;
  const int32_t* seqlens_k;
  const int32_t* page_table;
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const float* v_scale;  // e4m3: [num_pages, Hkv]
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
// are zero.  e4m3 V is dequantized (code times the page's scale, rounded to
// bf16).  HALF (64-token KV blocks): a half tile of 128 d rows x 64 keys per
// block (rows of 128 bytes), two blocks per workgroup.
template <bool FP8, bool HALF>
__global__ __launch_bounds__(256) void vt_exact_kernel(PrepArgs a) {
  FP2_BOUNDS_GUARD(a.dbg);
  constexpr int KB = HALF ? 64 : kBlk;  // keys of a block
  const int t = threadIdx.x;
  const int kb = HALF ? 2 * blockIdx.x + (t >> 7) : blockIdx.x, g = blockIdx.y;
  if (HALF && kb >= a.total_kblocks) return;
  const int s = find_seq(a.cu_kblocks, a.num_seqs, kb);
  const int J = kb - a.cu_kblocks[s];
  const int T = a.seqlens_k[s];
  const int32_t* pt = a.page_table + (int64_t)s * a.max_pages;
  const int c = HALF ? (t >> 4) & 7 : t >> 4, dc = t & 15;
  uint4 in[8], out[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int pos = J * KB + key_of_pos(8 * c + e);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (pos < T) {
      int pi, slot;
      a.pm.split(pos, pi, slot);
      const int64_t rowi = ((int64_t)pt[pi] * a.page_size + slot) * a.hkv + g;
      if constexpr (FP8) {
        const uint2 c8 = *reinterpret_cast<const uint2*>(a.v_pages + rowi * kD + dc * 8);
        const float sc = a.v_scale[(int64_t)pt[pi] * a.hkv + g];
        const f32x4 lo = e4m3x4_to_f32(c8.x), hi = e4m3x4_to_f32(c8.y);
        v = make_uint4(pack_bf16x2(lo[0] * sc, lo[1] * sc), pack_bf16x2(lo[2] * sc, lo[3] * sc),
                       pack_bf16x2(hi[0] * sc, hi[1] * sc), pack_bf16x2(hi[2] * sc, hi[3] * sc));
      } else {
        v = *reinterpret_cast<const uint4*>(a.v_pages + rowi * kRowBytes + dc * 16);
      }
    }
    in[e] = v;
  }
  transpose8x8(in, out);
  uint8_t* dst = a.vt + ((int64_t)g * a.total_kblocks + kb) * (KB * kRowBytes) + c * 16;
#pragma unroll
  for (int e = 0; e < 8; ++e) *reinterpret_cast<uint4*>(dst + (8 * dc + e) * (2 * KB)) = out[e];
}

// Mean tokens: tile mt of sequence s holds mean tokens [128 mt, 128 mt + 128)
// of that sequence (vbar^T as bf16, zero past the sequence's blocks); the
// same workgroup rounds those tokens' kbar rows to bf16.  Tile index
// cu_kblocks[s]/128 + s + mt never collides across sequences and stays
// below mt_cap = total_kblocks/128 + num_seqs + 1.
__global__ __launch_bounds__(256) void vt_mean_kernel(PrepArgs a) {
  FP2_BOUNDS_GUARD(a.dbg);
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


// bf16 pair (1, 1)
constexpr uint32_t kOnesBf16x2 = 0x3f803f80u;
// a step with a probability of 2^kXmax or more (an exponent, log2 units, of
// kXmax or more) refreshes the reference max; probabilities stay below 2^64,
// so P (bf16), the row sums and O (float32) cannot overflow
constexpr float kXmax = 64.0f;

// Per-wave state and the work of one tile (32-key steps, see the header).
//
// Score accumulator element i of lane l (query l%32) is key
// 8(i/4) + 4(l/32) + i%4 of its step.  A masked score is -inf; a mean token's
// score carries log2(B)/scale extra, so that its probability carries the
// block weight B.
//
// The row sums run on the matrix core beside PV, on exactly the rounded
// probabilities that PV weighs V with, so that O / l is a convex combination
// of the values whatever the rounding: a 16x16x32 MFMA takes a step half's
// B operand of PV (lane l: 8 probabilities of query l%32) as its B, whose
// column c then holds queries c and c+16 in k-groups {0, 2} and {1, 3}; an A
// of ones in row 0 at k-groups 0 and 2 and in row 1 at k-groups 1 and 3
// makes D row 0 the sum of query c and row 1 that of query c+16 (lanes 0-15,
// elements 0 and 1).
struct Wave {
  static constexpr int NS = kBlk / 32;  // 32-key steps per tile
  bf16x8 qf[kD / 16];  // bf16 query fragments (e4m3 inputs: the codes widened, for the bf16 kbar rows)
  i32x8 qf8[kD / 64];  // e4m3 query fragments (e4m3 inputs)
  f32x16 o[kD / 32];
  f32x4 lsum;    // lanes 0-15: the row sums of queries l and l+16 (see above)
  bf16x8 lones;  // the A operand of the row-sum MFMA
  float m;    // reference max (log2 units), shared by lanes l and l^32
  float nb;   // -m (0 while m = -inf): exp2(s * scale + nb) is the probability

  __device__ __forceinline__ void init_sums() {
    const int l = __lane_id();
    const bool on = (l & 15) == (l >> 4 & 1) && (l & 15) < 2;  // row 0 at k-groups 0, 2; row 1 at 1, 3
    const uint32_t w = on ? kOnesBf16x2 : 0u;
    lones = __builtin_bit_cast(bf16x8, make_uint4(w, w, w, w));
    lsum = f32x4{};
  }
  // the row sum of query l%32
  __device__ __forceinline__ float row_sum() const {
    const int l = __lane_id();
    const float a = __shfl(lsum[0], l & 15), b = __shfl(lsum[1], l & 15);
    return (l & 16) ? b : a;
  }

  __device__ __forceinline__ void rescale(float alpha) {
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    // lanes 0-15 hold the sums of queries l and l+16
    const float alpha_hi = __shfl(alpha, (__lane_id() & 15) + 16);
    lsum[0] *= alpha;
    lsum[1] *= alpha_hi;
  }

  // bf16 probabilities of one step against the reference max
  __device__ __forceinline__ void probs(const f32x16& s, float scl, bf16x8 (&pf)[2]) const {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * r + 2 * q], scl, nb)),
                           __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * r + 2 * q + 1], scl, nb)));
      // computed here, not sunk into the next step's region
      asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
      pf[r] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
  }

  // Sets the reference max to cover this step's scores, rescales O and the
  // row sums (which hold every step before this one), and redoes the step's
  // probabilities.
  __device__ __forceinline__ void refresh(const f32x16& s, float scl, bf16x8 (&pf)[2]) {
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);  // max3 chain
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
    mx = fmaxf(mx, s[15]);
    const float mnew = fmaxf(m, max_halves(mx) * scl);  // scl > 0: -inf stays -inf
    const float alpha = __builtin_amdgcn_exp2f(m - (mnew == -INFINITY ? 0.f : mnew));
    m = mnew;
    nb = mnew == -INFINITY ? 0.f : -mnew;
    rescale(alpha);
    probs(s, scl, pf);
  }

  // ---- tiles on a fixed instruction schedule ----
  //
  // A tile's MFMAs run in a fixed order of ops n: QK(0) | QK(1) | QK(2) with
  // PV(0), L(0) | QK(3) with PV(1), L(1) | PV(2), L(2) | PV(3), L(3), six
  // regions, where L(j) are the two row-sum MFMAs of step j (each after the
  // PV ops of its half of the step, on the same probabilities).  bf16 QK (QK8 false): 8 MFMAs 32x32x16
  // per step, 72 ops, regions of 8, 8, 18, 18, 10, 10 with QK and PV
  // alternating.  e4m3 QK (QK8 true): 2 MFMAs 32x32x64 per step, 48 ops,
  // regions of 2, 2, 12, 12, 10, 10 with the two QK ops at the head and the
  // middle of the PV ops of regions 2 and 3.  Each op is one slot closed by a
  // scheduling barrier, so this is the issue order: an op's LDS operand (16
  // bytes, 32 for an e4m3 QK op, none for a row-sum op) is read kLA slots
  // ahead (across regions), and the softmax of step j runs in region j+1 as
  // a stream of groups spread over the slots, each value produced a group or
  // more before it is consumed, so that no vector instruction waits on the
  // one just before it and the matrix core keeps getting work.  The refresh
  // test of step j closes region j+1, before PV(j) and L(j) read P(j).
  static constexpr int kLA = 4;
  static constexpr int kGroups = 20;
  static constexpr int kRing = 16;  // operand reads in flight (16-byte registers quads)

  enum : int { kOpQK = 0, kOpPV = 1, kOpL = 2 };
  static constexpr int kMaxOps = 72;
  // the schedule: op n's kind, step and index (QK: d-slice kk, 16 wide or 64
  // wide for e4m3; PV: 4 r + dt; L: r), its operand reads and the ring index
  // of its first read; start[r] is the first op of region r
  struct Ops {
    int n;
    int start[7];
    int kind[kMaxOps], step[kMaxOps], idx[kMaxOps], reads[kMaxOps], read0[kMaxOps];
  };
  template <bool QK8>
  static constexpr Ops make_ops() {
    Ops t{};
    int n = 0;
    auto push = [&](int kind, int j, int i) {
      t.kind[n] = kind;
      t.step[n] = j;
      t.idx[n] = i;
      t.reads[n] = kind == kOpL ? 0 : (kind == kOpQK && QK8) ? 2 : 1;
      t.read0[n] = n == 0 ? 0 : t.read0[n - 1] + t.reads[n - 1];
      ++n;
    };
    const int nqk = QK8 ? 2 : 8;
    for (int j = 0; j < 2; ++j) {  // regions 0, 1: QK(0), QK(1)
      t.start[j] = n;
      for (int i = 0; i < nqk; ++i) push(kOpQK, j, i);
    }
    for (int j = 0; j < 2; ++j) {  // regions 2, 3: QK(j+2) with PV(j) and L(j)
      t.start[2 + j] = n;
      for (int i = 0; i < 8; ++i) {
        if (QK8 ? i % 4 == 0 : true) push(kOpQK, j + 2, QK8 ? i / 4 : i);
        push(kOpPV, j, i);
        if (i % 4 == 3) push(kOpL, j, i / 4);  // after the PV ops of half i/4
      }
    }
    for (int j = 2; j < 4; ++j) {  // regions 4, 5: PV(j) and L(j)
      t.start[2 + j] = n;
      for (int i = 0; i < 8; ++i) {
        push(kOpPV, j, i);
        if (i % 4 == 3) push(kOpL, j, i / 4);
      }
    }
    t.start[6] = n;
    t.n = n;
    return t;
  }
  template <bool QK8>
  struct Sched {
    static constexpr Ops ops = make_ops<QK8>();
  };
  template <bool QK8>
  static constexpr int n_ops() { return Sched<QK8>::ops.n; }
  template <bool QK8>
  static constexpr int region_start(int r) { return Sched<QK8>::ops.start[r]; }
  template <bool QK8>
  static constexpr int op_kind(int n) { return Sched<QK8>::ops.kind[n]; }
  template <bool QK8>
  static constexpr int op_step(int n) { return Sched<QK8>::ops.step[n]; }
  template <bool QK8>
  static constexpr int op_idx(int n) { return Sched<QK8>::ops.idx[n]; }
  template <bool QK8>
  static constexpr int op_reads(int n) { return Sched<QK8>::ops.reads[n]; }
  // index of op n's first operand read
  template <bool QK8>
  static constexpr int read0(int n) { return Sched<QK8>::ops.read0[n]; }

  // LDS address of read e of op n (a QK or PV op).  bf16 K / V^T: the
  // swizzled 256-byte-row layout at the two per-lane bases off0 / off1.
  // e4m3 K: 128-byte rows, 1 KB per 8 rows, 16-byte chunk c of row r in slot
  // c ^ (r % 8); off8[2 kk + e] is lane l's slot of chunk 4 kk + 2 (l/32) + e
  // in row l%32.
  template <bool QK8>
  __device__ __forceinline__ const uint8_t* op_addr(int n, int e, const uint8_t* Kt, const uint8_t* Vt, int off0,
                                                    int off1, const int (&off8)[4]) const {
    const int j = op_step<QK8>(n), i = op_idx<QK8>(n);
    if (op_kind<QK8>(n) == kOpQK) {
      if constexpr (QK8) return Kt + off8[2 * i + e] + 4096 * j;
      return Kt + ((i & 1) ? off1 : off0) + 8 * kGS * j + 64 * (i >> 1);
    }
    return Vt + ((i >> 2) ? off1 : off0) + 8 * kGS * (i & 3) + 64 * j;
  }

  // softmax stream of one step: group g computes x[g] (g < 16), e[g-2]
  // (2 <= g < 18), the bf16 pair w[(g-4)/2] (even g >= 4) and takes x[g-2]
  // and x[g-1] into the step's largest exponent mx (even g, 2 <= g < 18)
  struct Soft {
    float x[16], e[16], mx;
    uint32_t w[8];
  };
  // Masked tiles pass the per-lane bit mask M of the step's allowed keys
  // (bit 8(i/4) + i%4 for element i): a masked element's exponent is -inf.
  template <bool MASKED>
  __device__ __forceinline__ void soft_group(int g, Soft& st, const f32x16& s, float scl, float nb,
                                             uint32_t M) const {
    if (g < 16) {
      float x = __builtin_fmaf(s[g], scl, nb);
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
    if (g >= 2 && g < 18 && (g & 1) == 0) {
      st.mx = fmaxf(fmaxf(st.mx, st.x[g - 2]), st.x[g - 1]);
      asm volatile("" : "+v"(st.mx));
    }
  }

  // one region: ops [region_start(R), region_start(R + 1)), with the softmax
  // stream of s when SOFT; the next tile's DMA instructions go out one per
  // slot in slots kDma0 .. kDma0 + 15
  template <int R, bool SOFT, bool MASKED, bool QK8, class Dma>
  __device__ __forceinline__ void region(bf16x8 (&fr)[kRing], f32x16& sn, const bf16x8 (&pp)[2], Soft& st,
                                         const f32x16& s, const uint8_t* Kt, const uint8_t* Vt, int off0, int off1,
                                         const int (&off8)[4], float scl, float nb, uint32_t M, Dma& dma) {
    constexpr int N0 = region_start<QK8>(R), S = region_start<QK8>(R + 1) - N0;
    constexpr int kDma0 = QK8 ? 4 : 8;
    // the younger wave's issue priority ends half way (see the tile loop)
    if constexpr (R == 3) __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int t = 0; t < S; ++t) {
      const int n = N0 + t;
      const int r0 = read0<QK8>(n) % kRing;
      if (op_kind<QK8>(n) == kOpQK) {
        if constexpr (QK8) {
          const uint4 lo = __builtin_bit_cast(uint4, fr[r0]), hi = __builtin_bit_cast(uint4, fr[(r0 + 1) % kRing]);
          const i32x8 ka = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          sn = mfma_fp8_32x32x64(ka, qf8[op_idx<QK8>(n)], sn);
        } else {
          sn = mfma_bf16_32x32x16(fr[r0], qf[op_idx<QK8>(n)], sn);
        }
      } else if (op_kind<QK8>(n) == kOpPV) {
        const int i = op_idx<QK8>(n);
        o[i & 3] = mfma_bf16_32x32x16(fr[r0], pp[i >> 2], o[i & 3]);
      } else {
        lsum = mfma_bf16_16x16x32(lones, pp[op_idx<QK8>(n)], lsum);
      }
      if (n + kLA < n_ops<QK8>()) {
        const int nr = n + kLA;
#pragma unroll
        for (int e = 0; e < op_reads<QK8>(nr); ++e)
          fr[(read0<QK8>(nr) + e) % kRing] =
              *reinterpret_cast<const bf16x8*>(op_addr<QK8>(nr, e, Kt, Vt, off0, off1, off8));
      }
      if (n >= kDma0 && n < kDma0 + 16) dma(n - kDma0);
      if constexpr (SOFT) {
#pragma unroll
        for (int g = t * kGroups / S; g < (t + 1) * kGroups / S; ++g) soft_group<MASKED>(g, st, s, scl, nb, M);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // closes the softmax of a step: P, and the refresh when a probability of
  // the step reached 2^kXmax (or it is the first step of the row)
  template <bool MASKED>
  __device__ __forceinline__ void soft_close(Soft& st, const f32x16& s, float scl, bool force, bf16x8 (&pc)[2],
                                             uint32_t M) {
    pc[0] = __builtin_bit_cast(bf16x8, make_uint4(st.w[0], st.w[1], st.w[2], st.w[3]));
    pc[1] = __builtin_bit_cast(bf16x8, make_uint4(st.w[4], st.w[5], st.w[6], st.w[7]));
    if (__any(!(st.mx < kXmax)) || force) {
      if constexpr (MASKED) {
        f32x16 sm;  // the scores as the stream saw them: -inf where masked
#pragma unroll
        for (int i = 0; i < 16; ++i) sm[i] = (M >> (8 * (i >> 2) + (i & 3))) & 1u ? s[i] : -INFINITY;
        refresh(sm, scl, pc);
      } else {
        refresh(s, scl, pc);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // One tile; scl is its logit scale (log2 units, input scales folded in).
  // MASKED: mode 1 diagonal block (key > query masked), mode 0 passes
  // whole.  QK8: e4m3 K tile and QK on the 32x32x64 e4m3 MFMA.
  // The operand reads of the first kLA ops, issued by the caller as early as
  // it can (see first_reads).
  template <bool QK8>
  __device__ __forceinline__ void first_reads(bf16x8 (&fr)[kRing], const uint8_t* Kt, const uint8_t* Vt, int off0,
                                              int off1, const int (&off8)[4]) const {
#pragma unroll
    for (int n = 0; n < kLA; ++n)
#pragma unroll
      for (int e = 0; e < op_reads<QK8>(n); ++e)
        fr[read0<QK8>(n) + e] = *reinterpret_cast<const bf16x8*>(op_addr<QK8>(n, e, Kt, Vt, off0, off1, off8));
  }

  // TWO: the tile's keys are two 64-token blocks: scl2 is the logit scale of
  // the second (steps NS/2 ..; e4m3 K scales differ per block); on the
  // diagonal tq is the query's position minus the first block's first key,
  // tq2 the same for the second block (very negative when the tile holds one
  // block).
  //
  // AUG (plain schedule, mean-token tile starting at mean token J0): only
  // the tokens of skipped blocks count, each with weight B, i.e. cbs =
  // log2(B) / scl more score.  Weight and mask enter the scores through one
  // more MFMA per step, at the head of the step's QK chain, instead of a bit
  // test and a select per score.  Its A holds for key l of the step (lane
  // l < 32, k = 0 and 1) cbs split into two bf16 halves when the token's
  // block is skipped, -inf and 0 when it is not; its B holds ones at k = 0
  // and 1 of every column; every other A element is finite and meets a zero
  // of B.  So the product adds cbs, or -inf, to each score of the key's row,
  // and the rest of the tile is the plain one.  nsteps: the steps that hold
  // a token below the diagonal (a row's last mean tile may end early); the
  // PV work of later steps (regions 4 and 5) is skipped.
  template <bool MASKED, bool QK8, bool TWO = false, bool AUG = false, class Dma>
  __device__ __forceinline__ void tile(bf16x8 (&fr)[kRing], bool first, const uint8_t* Kt, const uint8_t* Vt,
                                       int off0, int off1, const int (&off8)[4], float scl, float scl2, Dma&& dma,
                                       int mode, int tq, int tq2, int hf, float cbs, int J0, const uint32_t* kept,
                                       int nsteps = NS) {
    static_assert(!(MASKED && AUG), "the weight MFMA is the plain schedule's mask");
    bf16x8 pp[2] = {qf[0], qf[0]}, pc[2];
    f32x16 s = f32x16{}, sn = f32x16{};
    Soft st;
    uint32_t M[NS] = {};
    uint32_t abit = 0u, hl = 0u;  // AUG: bit j = key l%32 of step j is a skipped block's token
    auto weight = [&](int j) {
      const uint32_t ka = (abit >> j) & 1u ? hl : (hf ? 0u : 0xff80u);  // bf16 -inf at k = 0 (lanes < 32)
      const bf16x8 wa = __builtin_bit_cast(bf16x8, make_uint4(ka, 0u, 0u, 0u));
      const bf16x8 wb = __builtin_bit_cast(bf16x8, make_uint4(hf ? 0u : kOnesBf16x2, 0u, 0u, 0u));
      return mfma_bf16_32x32x16(wa, wb, f32x16{});
    };
    if constexpr (AUG) {
      const uint32_t hi = pack_bf16x2(cbs, 0.f) & 0xffffu;
      hl = pack_bf16x2(cbs, cbs - bf16lo(hi));  // cbs ~ bf16 hi + bf16 lo
      const int l = __lane_id() & 31;
#pragma unroll
      for (int j = 0; j < NS; ++j) abit |= ((kept[(J0 >> 5) + j] >> l) & 1u) << j;  // skipped-block words
      sn = weight(0);
    }
    if constexpr (MASKED) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        if (mode == 0) {
          M[j] = ~0u;
        } else {
          // element i allowed iff 8(i/4) + i%4 <= lim
          const int lim = (TWO ? (j < NS / 2 ? tq : tq2) - 32 * (j % (NS / 2)) : tq - 32 * j) - 4 * hf;
          M[j] = lim >= 31 ? ~0u : lim < 0 ? 0u : (2u << lim) - 1u;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    region<0, false, MASKED, QK8>(fr, sn, pp, st, s, Kt, Vt, off0, off1, off8, scl, 0.f, 0u, dma);  // QK(0)
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      s = sn;
      sn = f32x16{};
      if constexpr (AUG) {
        if (j + 1 < NS) sn = weight(j + 1);
      }
      st.mx = -INFINITY;
      // region j+1: QK(j+1) (j < 3), PV(j-1) (j > 0), softmax(j)
      if (j == 0) region<1, true, MASKED, QK8>(fr, sn, pp, st, s, Kt, Vt, off0, off1, off8, scl, nb, M[0], dma);
      if (j == 1) region<2, true, MASKED, QK8>(fr, sn, pp, st, s, Kt, Vt, off0, off1, off8, scl, nb, M[1], dma);
      if (j == 2) region<3, true, MASKED, QK8>(fr, sn, pp, st, s, Kt, Vt, off0, off1, off8, TWO ? scl2 : scl, nb, M[2], dma);
      if (j == 3) {
        if (AUG && nsteps <= 2) break;  // steps 2 and 3 hold no token that counts: PV(2), PV(3) and L go
        region<4, true, MASKED, QK8>(fr, sn, pp, st, s, Kt, Vt, off0, off1, off8, TWO ? scl2 : scl, nb, M[3], dma);
      }
      soft_close<MASKED>(st, s, (TWO && j >= NS / 2) ? scl2 : scl, first && j == 0, pc, M[j]);
      pp[0] = pc[0];
      pp[1] = pc[1];
    }
    if (!AUG || nsteps > 3)
      region<5, false, MASKED, QK8>(fr, sn, pp, st, s, Kt, Vt, off0, off1, off8, scl, 0.f, 0u, dma);  // PV(3)
  }
};

// One 1 KB LDS DMA instruction: lane i's 16 bytes at src land at dst + 16 i
// (dst wave-uniform).  A plain function: the builtin written straight in
// the kernel template keeps the host pass from emitting the launch stub.
__device__ __forceinline__ void dma16(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// tile code paths of the attention kernel's loops
enum : int { kPathPlain = 0, kPathMasked = 1, kPathMean = 2 };

// PAIR: 64-token KV blocks under 128-token query blocks, two blocks (two CSR
// entries) to a 128-key tile.

template <bool FP8, bool PAIR>
__global__ __launch_bounds__(kThreads, 1) void attn_d128_kernel(AttnArgs a) {
  constexpr int KB = PAIR ? 64 : kBlk;  // tokens of a KV block
  static_assert(!PAIR || (kDmaWaves / 2) * kDmaRows == 64, "a DMA wave's rows lie in one 64-token block");
  // two K and two V^T buffers, as separate objects so that the compiler can
  // tell the DMA target from the buffers being read
  __shared__ __attribute__((aligned(1024))) uint8_t K0[kTileLds];
  __shared__ __attribute__((aligned(1024))) uint8_t K1[kTileLds];
  __shared__ __attribute__((aligned(1024))) uint8_t V0[kTileLds];
  __shared__ __attribute__((aligned(1024))) uint8_t V1[kTileLds];
  __shared__ uint32_t kept[kMaxKBlocks / 32];
  __shared__ int mtile[kMaxKBlocks / kBlk + 1];
  FP2_BOUNDS_GUARD(a.dbg);

  // ---- tile decode: 8 consecutive work items form a group, the slices of
  // one item share blockIdx % 8 (one XCD); the items are in launch order,
  // by head phase, heaviest first: {CSR rank, first and end exact tile of the row, partial
  // slot or -1} (rank r: query block total_qblocks - 1 - r / Hkv, KV head
  // r % Hkv)
  const int b = blockIdx.x;
  const int per_grp = 8 * a.slices;
  const int grp = b / per_grp;
  const int rem = b % per_grp;
  const int slice = rem / 8;
  const int pos = grp * 8 + (rem % 8);
  if (pos >= a.rows + a.extra_cap) return;
  // the item's record (item_info_kernel): one load round trip for everything
  // the first two tiles need
  const int32_t* rec = a.info + (int64_t)pos * kInfoInts;
  const int rank = ld_uniform(rec, 0);
  if (rank < 0) return;
  const int tile0 = ld_uniform(rec, 1), tile1 = ld_uniform(rec, 2), pslot = ld_uniform(rec, 3);
  const int qb = ld_uniform(rec, 4);
  const int g = ld_uniform(rec, 5);
  const int row = g * a.total_qblocks + qb;
  const int s = ld_uniform(rec, 6);
  const int I = ld_uniform(rec, 7);
  const int q0 = ld_uniform(rec, 8);
  const int n = ld_uniform(rec, 9);
  const int T = ld_uniform(rec, 10);
  // the diagonal: KV blocks dlo .. diag hold the query block's own positions
  // (one block of 128 tokens; two of 64, one for a short last query block)
  const int qpos0 = T - n + I * kBlk;  // position of the block's first query
  const int diag = PAIR ? (qpos0 + min(kBlk, n - I * kBlk) - 1) / KB : (T - n) / kBlk + I;
  const int dlo = PAIR ? qpos0 / KB : diag;
  const int G = a.hq / a.hkv;
  const int32_t* pt = a.page_table + (int64_t)s * a.max_pages;
  const int kb0 = ld_uniform(rec, 11);
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
  const int rbeg = ld_uniform(rec, 12);
  const int rend = ld_uniform(rec, 13);
  // this item's exact tiles (CSR entries kbeg .. kend-1; with 64-token KV
  // blocks tile i of a row holds its entries 2i and 2i+1, the last perhaps
  // alone); the mean tiles go with the row's last item
  const int kbeg = rbeg + (PAIR ? 2 * tile0 : tile0);
  const int kend = PAIR ? min(rbeg + 2 * tile1, rend) : rbeg + tile1;
  const int nexact = PAIR ? tile1 - tile0 : kend - kbeg;
  const int ne = kend - kbeg;
  // mean-token tiles that hold at least one skipped block (the last item of
  // a row, correction on): their skipped-block words and first mean tokens
  // into LDS, read first so that their loads land before the Q and DMA ones
  const int nmean = ld_uniform(rec, 14);
  if (nmean > 0) {
    const int ncand = (dlo + kBlk - 1) / kBlk, nw = (dlo + 31) >> 5;
    const uint32_t* sk = a.skip + (int64_t)row * a.wskip;
    for (int w = (int)threadIdx.x; w < ncand * (kBlk / 32); w += kThreads) kept[w] = w < nw ? sk[w] : 0u;
    const int32_t* ml = a.mlist + (int64_t)row * a.mtmax;
    for (int k = (int)threadIdx.x; k < nmean; k += kThreads) mtile[k] = ml[k];
  }
  // PAIR: the two block indices of tile i packed as ja | jb << 16 (a lone
  // last entry goes with itself: its second half is masked)
  auto pack = [&](int ja, int jb, int i) { return ja | ((2 * i + 1 < ne ? jb : ja) << 16); };
  auto half_of = [](int J, int h) { return h ? J >> 16 : J & 0xFFFF; };
  // an exact tile on the masked path: some key past some query
  auto masked_exact = [&](int J, int i) {
    if constexpr (PAIR) return 2 * i + 1 >= ne || half_of(J, 1) >= dlo;
    return J == diag;
  };


  Wave ws;
  ws.m = -INFINITY;
  ws.nb = 0.f;
  ws.init_sums();
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt) ws.o[dt] = f32x16{};
  float qs = 1.f;  // e4m3: the query block's scale
  if constexpr (!FP8) {
    const uint8_t* qrow = a.q + ((int64_t)(q0 + I * kBlk + tq) * a.hq + h) * kRowBytes;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (q_valid) v = *reinterpret_cast<const uint4*>(qrow + (16 * kk + 8 * hf) * 2);
      ws.qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  } else {
    // e4m3 codes: 32 bytes at d = 64 kk + 32 (l/32) for the 32x32x64 MFMA, and
    // the 8 at d = 16 kk + 8 (l/32) widened to bf16 (exactly) for the bf16
    // kbar rows of mean tiles
    const uint8_t* qrow = a.q + ((int64_t)(q0 + I * kBlk + tq) * a.hq + h) * kD;
#pragma unroll
    for (int kk = 0; kk < kD / 64; ++kk) {
      uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
      if (q_valid) {
        v0 = *reinterpret_cast<const uint4*>(qrow + 64 * kk + 32 * hf);
        v1 = *reinterpret_cast<const uint4*>(qrow + 64 * kk + 32 * hf + 16);
      }
      ws.qf8[kk] = i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
    }
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) {
      uint2 v = make_uint2(0, 0);
      if (q_valid) v = *reinterpret_cast<const uint2*>(qrow + 16 * kk + 8 * hf);
      const f32x4 lo = e4m3x4_to_f32(v.x), hi = e4m3x4_to_f32(v.y);
      ws.qf[kk] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                                                        pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])));
    }
    if (wave_active) qs = a.q_scale[(int64_t)qb * a.hq + h];
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
  // e4m3 K: 128-byte rows, 8 per instruction; lane i moves row 8p + i/8,
  // chunk (i%8) ^ (i/8)
  const uint32_t tok8 = (uint32_t)a.hkv * kD;
  const uint32_t koff8 = (uint32_t)(lane >> 3) * tok8 + 16 * ((lane & 7) ^ (lane >> 3));  // + 8 p tok8
  const bool pages16 = a.page_size % 16 == 0;
  // Uniform values for later tiles (block indices, page entries) come through
  // vector buffer loads: they share the vector-memory counter with the DMA,
  // so the wait at each tile barrier covers them.  Scalar loads would share
  // the LDS counter instead, and every tile's first operand-read wait would
  // then also wait for them.
  const __amdgpu_buffer_rsrc_t rcol =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.col_idx + kbeg), (short)0, ne * 4, kBufferFlags);
  // first token row this DMA wave moves of exact tile J (PAIR: waves 0-1
  // the first block, 2-3 the second)
  auto dma_row0 = [&](int J) -> int {
    if constexpr (PAIR) return half_of(J, wave >= kDmaWaves / 2) * KB + kDmaRows * (wave % (kDmaWaves / 2));
    return J * kBlk + kDmaRows * wave;
  };
  // PAIR: lane chunk c = (l%16) ^ (l/16) of a V^T row holds keys of block
  // half c/8; a half tile of one 64-token block has 128-byte rows
  const int vhalf = ((lane & 15) ^ (lane >> 4)) >> 3;
  const uint32_t voffh = (uint32_t)((lane >> 4) * (2 * KB) + 16 * (((lane & 15) ^ (lane >> 4)) & 7));
  const __amdgpu_buffer_rsrc_t rpt =
      __builtin_amdgcn_make_buffer_rsrc((void*)pt, (short)0, a.max_pages * 4, kBufferFlags);
  auto page_of = [&](int J, int hh) -> int {  // page of rows R w + 16 hh.. of block J (valid after the next barrier)
    int pi, slot;
    a.pm.split(min(dma_row0(J) + 16 * hh, T - 1), pi, slot);
    return __builtin_amdgcn_raw_buffer_load_b32(rpt, pi * 4, 0, 0);
  };
  // a value loaded before the last barrier, read as a wave-uniform scalar there
  // (pinned after the barrier so the read is not hoisted next to its load)
  auto after_barrier = [](int v) {
    asm volatile("" : "+v"(v));
    return __builtin_amdgcn_readfirstlane(v);
  };
  // the fast-path sources of one tile: K instruction p < nk reads kb[p/4] +
  // (p%4) kstep + kvo into kd + p kds, V^T instruction p reads vb + 1024 p +
  // voff
  struct DmaPlan {
    const uint8_t* kb[kDmaHalves];
    const uint8_t* vb;
    const uint8_t* vbl;  // PAIR: this lane's V^T source of instruction 0 (+ vstep p)
    uint32_t vstep;
    uint8_t* kd;
    uint32_t kstep, kvo;
    int kds, nk;
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
    pl.kd = kd;
    pl.kds = kGS;
    pl.nk = kDmaRows / 4;
    if (idx < nexact) {
      if constexpr (PAIR) {
        pl.vbl = a.vt + ((int64_t)g * a.total_kblocks + kb0 + half_of(j, vhalf)) * (KB * kRowBytes) +
                 kDmaRows * wave * (2 * KB) + voffh;
        pl.vstep = 4 * (2 * KB);
      } else {
        pl.vb = a.vt + (((int64_t)g * a.total_kblocks + kb0 + j) * kBlk + kDmaRows * wave) * kRowBytes;
      }
      const int r0 = dma_row0(j);
      pl.fast = pages16 && r0 + kDmaRows - 1 < T;
      if (FP8) {
        // e4m3 K rows (one page per block): kDmaRows/8 instructions of 8 rows
        pl.kd = Kd + kDmaRows * wave * kD;
        pl.kds = 1024;
        pl.nk = kDmaRows / 8;
        pl.fast = r0 + kDmaRows - 1 < T;
        if (pl.fast) {
#pragma unroll
          for (int hh = 0; hh < kDmaHalves; ++hh)
            pl.kb[hh] = a.k_pages + (((int64_t)pg[0] * KB + r0 % KB) * a.hkv + g) * kD;
          pl.kstep = 8 * tok8;
          pl.kvo = koff8;
        } else {
#pragma unroll
          for (int p = 0; p < kDmaRows / 8; ++p) {
            const int r = min(r0 + 8 * p + (lane >> 3), T - 1);  // rows past the end repeat the last key
            const uint8_t* ksrc = a.k_pages + (((int64_t)pt[r / KB] * KB + r % KB) * a.hkv + g) * kD +
                                  16 * ((lane & 7) ^ (lane >> 3));
            dma16(ksrc, pl.kd + p * 1024);
          }
#pragma unroll
          for (int p = 0; p < kDmaRows / 4; ++p) {
            if constexpr (PAIR) dma16(pl.vbl + pl.vstep * p, vd + p * kGS);
            else dma16(pl.vb + voff + 1024 * p, vd + p * kGS);
          }
        }
      } else if (pl.fast) {
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
          dma16(ksrc, kd + p * kGS);
          if constexpr (PAIR) dma16(pl.vbl + pl.vstep * p, vd + p * kGS);
          else dma16(pl.vb + voff + 1024 * p, vd + p * kGS);
        }
      }
    } else {
      pl.vb = a.vbt + (((int64_t)g * a.mt_cap + kb0 / kBlk + s + j / kBlk) * kBlk + kDmaRows * wave) * kRowBytes;
      pl.vbl = pl.vb + voff;
      pl.vstep = 1024;
      const uint8_t* k16 = reinterpret_cast<const uint8_t*>(a.kbar16);
      const int r0 = j + kDmaRows * wave;
      pl.fast = r0 + kDmaRows - 1 < dlo;
      if (pl.fast) {
#pragma unroll
        for (int hh = 0; hh < kDmaHalves; ++hh) pl.kb[hh] = k16 + (mrow0 + r0 + 16 * hh) * kRowBytes;
        pl.kstep = 1024;
        pl.kvo = voff;
      } else {
#pragma unroll
        for (int p = 0; p < kDmaRows / 4; ++p) {
          const int jm = min(r0 + 4 * p + (lane >> 4), dlo - 1);  // tokens past dlo repeat a real one (masked)
          dma16(k16 + (mrow0 + jm) * kRowBytes + uoff, kd + p * kGS);
          dma16(pl.vb + voff + 1024 * p, vd + p * kGS);
        }
      }
    }
    return pl;
  };
  // instruction i of a fast plan: K row group i/2 (even i) or V^T row group i/2 (odd i)
  auto issue = [&](const DmaPlan& pl, int i, uint8_t* Vd) __attribute__((always_inline)) {
    const int p = i >> 1;
    if ((i & 1) == 0) {
      if (p < pl.nk)
        dma16(pl.kb[p >> 2] + (p & 3) * pl.kstep + pl.kvo, pl.kd + p * pl.kds);
    } else if constexpr (PAIR) {
      dma16(pl.vbl + pl.vstep * p, Vd + ((kDmaRows / 4) * wave + p) * kGS);
    } else {
      dma16(pl.vb + 1024 * p + voff, Vd + ((kDmaRows / 4) * wave + p) * kGS);
    }
  };

  // per-lane operand offsets (see Wave::qk / Wave::pv): row l%32 of a 32-row
  // slab, chunk parity 0 / 1 of the lane's half
  const int c = lane & 31, x = c & 3;
  const int rbase = (c >> 2) * kGS + x * kRowBytes;
  const int off0 = rbase + 16 * (hf ^ x);
  const int off1 = rbase + 16 * ((2 + hf) ^ x);
  // e4m3 K operand: row c, chunks 4 kk + 2 hf + e, slot = chunk ^ (c % 8)
  int off8[4];
#pragma unroll
  for (int ke = 0; ke < 4; ++ke) off8[ke] = (c >> 3) * 1024 + (c & 7) * 128 + 16 * ((4 * (ke >> 1) + 2 * hf + (ke & 1)) ^ (c & 7));

  // Tile pipeline: at iteration i the LDS buffers i%2 hold tile i and the
  // DMA of tile i+1 into the other buffers is in flight; the block index of
  // tile i+2 and the page entries of tile i+1 arrived with the last barrier,
  // the loads of tile i+3's block index and tile i+2's page entries are in
  // flight.
  // Tile 0 is an exact block (the CSR holds block 0): its DMA, the first
  // page and block-index loads go out before the mean-token setup below.
  int j0 = ld_uniform(rec, 16), j1 = ld_uniform(rec, 17), j2v = ld_uniform(rec, 18), j2vb = ld_uniform(rec, 19);
  int pgv[kDmaHalves] = {};
  // e4m3: the K scale of exact tile i (one page per block) arrives with the
  // barrier before tile i (ksv); the page entry of tile i+1 one tile earlier
  // (pgbv)
  const __amdgpu_buffer_rsrc_t rks =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.k_scale, (short)0, 0x7fffffff, kBufferFlags);
  int ksv = 0, pgbv = 0, ksvb = 0, pgbvb = 0;  // PAIR: the second block's
  if constexpr (FP8) {
    ksv = ld_uniform(rec, 20);
    ksvb = ld_uniform(rec, 21);
    pgbv = ld_uniform(rec, 22);
    pgbvb = ld_uniform(rec, 23);
  }
  if (0 < nexact) {
    int pg0[kDmaHalves] = {};
    if (dma_wave) {
#pragma unroll
      for (int hh = 0; hh < kDmaHalves; ++hh) pg0[hh] = ld_uniform(rec, 24 + 2 * wave + hh);
    }
    const DmaPlan pl = plan(0, j0, pg0, K0, V0);
    if (pl.fast) {
#pragma unroll
      for (int i = 0; i < kDmaInstr; ++i) issue(pl, i, V0);
    }
  }

  const int ntiles = nexact + nmean;
  auto mean_of = [&](int idx) -> int { return idx < ntiles ? mtile[idx - nexact] : 0; };
  if (nexact == 0 && ntiles > 0) {  // (not produced by fp2_plan_mask: every row holds block 0; j0 is mean tile 0)
    const int pg0[kDmaHalves] = {};
    const DmaPlan pl = plan(0, j0, pg0, K0, V0);
    if (pl.fast) {
#pragma unroll
      for (int i = 0; i < kDmaInstr; ++i) issue(pl, i, V0);
    }
  }
  if (1 < nexact && dma_wave) {
#pragma unroll
    for (int hh = 0; hh < kDmaHalves; ++hh) pgv[hh] = ld_uniform(rec, 32 + 2 * wave + hh);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  const float scl = a.scale_log2 * qs;  // logit scale of mean tiles (and of every bf16 tile)

  // PATH_C: std::integral_constant<int, ...>, the tile code path (see below)
  auto iter = [&](auto path_c, int idx, const uint8_t* Kc, const uint8_t* Vc, uint8_t* Kn, uint8_t* Vn)
                  __attribute__((always_inline)) {
    constexpr int PATH = decltype(path_c)::value;
    constexpr bool QK8 = FP8 && PATH != kPathMean;  // e4m3 K tile (mean tiles: bf16 kbar rows)
    // the tile's first operand reads go out before the bookkeeping below
    bf16x8 fr[Wave::kRing];
    if (wave_active) ws.first_reads<QK8>(fr, Kc, Vc, off0, off1, off8);
    __builtin_amdgcn_sched_barrier(0);
    int j2;
    if constexpr (PAIR) j2 = idx + 2 < nexact ? pack(after_barrier(j2v), after_barrier(j2vb), idx + 2) : mean_of(idx + 2);
    else j2 = idx + 2 < nexact ? after_barrier(j2v) : mean_of(idx + 2);
    float sclt = scl, sclt2 = scl;
    if constexpr (FP8) {
      if (idx < nexact) {
        sclt = scl * __uint_as_float((uint32_t)after_barrier(ksv));
        if constexpr (PAIR) sclt2 = scl * __uint_as_float((uint32_t)after_barrier(ksvb));
      }
      if (idx + 1 < nexact) {
        ksv = __builtin_amdgcn_raw_buffer_load_b32(rks, (after_barrier(pgbv) * a.hkv + g) * 4, 0, 0);
        if constexpr (PAIR)
          ksvb = __builtin_amdgcn_raw_buffer_load_b32(rks, (after_barrier(pgbvb) * a.hkv + g) * 4, 0, 0);
      }
      if (idx + 2 < nexact) {
        pgbv = __builtin_amdgcn_raw_buffer_load_b32(rpt, half_of(j2, 0) * 4, 0, 0);
        if constexpr (PAIR) pgbvb = __builtin_amdgcn_raw_buffer_load_b32(rpt, half_of(j2, 1) * 4, 0, 0);
      }
    }
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
    if (idx + 3 < nexact) {
      if constexpr (PAIR) {
        j2v = __builtin_amdgcn_raw_buffer_load_b32(rcol, 2 * (idx + 3) * 4, 0, 0);
        j2vb = __builtin_amdgcn_raw_buffer_load_b32(rcol, (2 * (idx + 3) + 1) * 4, 0, 0);
      } else {
        j2v = __builtin_amdgcn_raw_buffer_load_b32(rcol, (idx + 3) * 4, 0, 0);
      }
    }
    const int mode = idx < nexact && masked_exact(j0, idx) ? 1 : 0;  // the masked path's mask: 1 diagonal
    // The issue arbiter serves the older wave of a SIMD first (waves 0-3,
    // which also issue the DMA): the younger waves 4-7 get the higher issue
    // priority until region 3 so that the two finish a tile closer together.
    if (wave >= kDmaWaves) __builtin_amdgcn_s_setprio(1);
    auto dma = [&](int i) __attribute__((always_inline)) {
      if (pl.fast) issue(pl, i, Vn);
    };
    if (!wave_active) {
      if (pl.fast) {
#pragma unroll
        for (int i = 0; i < kDmaInstr; ++i) issue(pl, i, Vn);
      }
    } else if constexpr (PATH == kPathPlain) {
      ws.tile<false, FP8, PAIR>(fr, idx == 0, Kc, Vc, off0, off1, off8, sclt, sclt2, dma, 0, tq, 0, hf, 0.f, 0, kept);
    } else if constexpr (PATH == kPathMean) {
      // mean tiles: the plain bf16 schedule with the weight MFMA (cbs: log2 B in score units)
      ws.tile<false, false, PAIR, true>(fr, idx == 0, Kc, Vc, off0, off1, off8, sclt, sclt2, dma, 0, tq, 0, hf,
                                        a.log2_block / sclt, j0, kept, min(Wave::NS, (dlo - j0 + 31) >> 5));
    } else if constexpr (PAIR) {
      // diagonal offsets of the two blocks (a lone block: its second half masked)
      const int qd = qpos0 + tq;
      const int tqa = qd - half_of(j0, 0) * KB;
      const int tqb = 2 * idx + 1 < ne ? qd - half_of(j0, 1) * KB : -(1 << 20);
      ws.tile<true, FP8, true>(fr, idx == 0, Kc, Vc, off0, off1, off8, sclt, sclt2, dma, mode, tqa, tqb, hf, 0.f, 0,
                               kept);
    } else {
      ws.tile<true, FP8>(fr, idx == 0, Kc, Vc, off0, off1, off8, sclt, sclt, dma, mode, tq, 0, hf, 0.f, 0, kept);
    }
    __builtin_amdgcn_s_setprio(0);
    j0 = j1;
    j1 = j2;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's DMA and loads for later tiles have landed
    __syncthreads();
  };
  // Three loops, each with one tile code path (one instance of the tile code
  // per loop keeps the register allocation of each loop separate): first the
  // exact tiles off the diagonal, which the ascending CSR puts ahead of the
  // diagonal block, then the diagonal on the masked path (e4m3 inputs: both
  // on the e4m3 MFMA), then the mean tiles on the plain bf16 schedule with
  // the weight MFMA.
  const std::integral_constant<int, kPathPlain> plain_c;
  const std::integral_constant<int, kPathMasked> masked_c;
  const std::integral_constant<int, kPathMean> mean_c;
  int idx = 0;
  while (idx < nexact && !masked_exact(j0, idx)) {
    iter(plain_c, idx, K0, V0, K1, V1);
    ++idx;
    if (!(idx < nexact && !masked_exact(j0, idx))) break;
    iter(plain_c, idx, K1, V1, K0, V0);
    ++idx;
  }
  // (tile idx sits in buffers idx % 2)
  auto run = [&](auto path_c, int end) __attribute__((always_inline)) {
    if (idx < end && (idx & 1)) {
      iter(path_c, idx, K1, V1, K0, V0);
      ++idx;
    }
    while (idx < end) {
      iter(path_c, idx, K0, V0, K1, V1);
      ++idx;
      if (idx >= end) break;
      iter(path_c, idx, K1, V1, K0, V0);
      ++idx;
    }
  };
  run(masked_c, nexact);
  run(mean_c, ntiles);

  // ---- epilogue: O / l, or the chunk's partial result in register layout
  if (pslot >= 0) {
    if (wave_active) {
      float* po = a.part + ((int64_t)(pslot * a.slices + slice) * kWaves + wave) * kPartFloatsPerWave;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(po + ((dt * 4 + q4) * 64 + lane) * 4) =
              f32x4{ws.o[dt][4 * q4 + 0], ws.o[dt][4 * q4 + 1], ws.o[dt][4 * q4 + 2], ws.o[dt][4 * q4 + 3]};
      const float lsum = ws.row_sum();
      *reinterpret_cast<float2*>(po + 64 * 64 + 2 * lane) = make_float2(ws.m, lsum);
    }
  } else if (!a.out_f32) {
    // bf16: the wave's 32 x 128 output tile goes through LDS (the tile
    // buffers are free after the last barrier; 272-byte rows), so that each
    // store writes whole 256-byte rows, 16 lanes a row: a lane's own values
    // are 4-element pieces of one row, and storing them directly takes 16
    // instructions of 32 scattered pieces each, whose draining held the
    // workgroup's slot for several microseconds.
    if (wave_active) {
      const float inv = 1.0f / ws.row_sum();  // rows past the sequence end are never stored
      uint8_t* stg = (wave < 4 ? K0 : V0) + (wave & 3) * kStageBytes;
      const int r = lane & 31;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          uint2 w;
          w.x = pack_bf16x2(ws.o[dt][4 * q4 + 0] * inv, ws.o[dt][4 * q4 + 1] * inv);
          w.y = pack_bf16x2(ws.o[dt][4 * q4 + 2] * inv, ws.o[dt][4 * q4 + 3] * inv);
          *reinterpret_cast<uint2*>(stg + r * kStageRow + (32 * dt + 8 * q4 + 4 * hf) * 2) = w;
        }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rr = 4 * i + (lane >> 4);
        const uint4 v = *reinterpret_cast<const uint4*>(stg + rr * kStageRow + (lane & 15) * 16);
        const int tqr = prow % kBlk + rr;
        if (I * kBlk + tqr < n)
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + ((int64_t)(q0 + I * kBlk + tqr) * a.hq + h) * kD +
                                    (lane & 15) * 8) = v;
      }
    }
  } else if (q_valid) {
    const float inv = 1.0f / ws.row_sum();
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

// Exact tiles of CSR rank r (rank r: query block total_qblocks - 1 - r / Hkv,
// KV head r % Hkv) and, with the correction, the mean-token tiles it can have
// (an upper bound).
__device__ void rank_tiles(const AttnArgs& a, int r, int& nexact, int& nmean) {
  const int qb = a.total_qblocks - 1 - r / a.hkv;
  const int row = (r % a.hkv) * a.total_qblocks + qb;
  nexact = max(a.row_ptr[row + 1] - a.row_ptr[row], 0);
  if (a.pair) nexact = (nexact + 1) >> 1;  // 64-token KV blocks, two a tile
  nmean = a.correction ? a.mcount[row] : 0;  // (mean_prep_kernel has run)
}

// Per CSR row (correction on): the bitmask of its skipped blocks (KV blocks
// in [1, dlo) that are not kept; dlo = the row's first diagonal block) and
// the list of its mean tiles (128 consecutive mean tokens holding at least
// one skipped block, by first mean token), so that a workgroup starting the
// row reads them instead of building them.
__global__ __launch_bounds__(256) void mean_prep_kernel(AttnArgs a) {
  FP2_BOUNDS_GUARD(a.dbg);
  __shared__ uint32_t kw[kMaxKBlocks / 32];
  const int row = blockIdx.x;
  const int qb = row % a.total_qblocks;
  const int s = find_seq(a.cu_qblocks, a.num_seqs, qb);
  const int n = a.cu_seqlens_q[s + 1] - a.cu_seqlens_q[s];
  const int dlo = (a.seqlens_k[s] - n + (qb - a.cu_qblocks[s]) * kBlk) / (a.pair ? 64 : kBlk);
  const int nw = (dlo + 31) >> 5;
  const int t = threadIdx.x;
  for (int w = t; w < nw; w += 256) kw[w] = 0u;
  __syncthreads();
  const int rbeg = a.row_ptr[row], rend = a.row_ptr[row + 1];
  for (int i = rbeg + t; i < rend; i += 256) {
    const int j = a.col_idx[i];
    if (j < dlo) atomicOr(&kw[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  for (int w = t; w < nw; w += 256) {
    uint32_t m = ~kw[w];
    const int j0 = 32 * w;
    if (j0 + 32 > dlo) m &= (1u << (dlo - j0)) - 1u;
    if (w == 0) m &= ~1u;
    kw[w] = m;
    a.skip[(int64_t)row * a.wskip + w] = m;
  }
  __syncthreads();
  if (t < 64) {
    const int ncand = (dlo + kBlk - 1) / kBlk;
    int base = 0;
    for (int m0 = 0; m0 < ncand; m0 += 64) {
      const int mt = m0 + t;
      bool flag = false;
      if (mt < ncand) {
#pragma unroll
        for (int w = 0; w < kBlk / 32; ++w) flag |= (4 * mt + w < nw) && kw[4 * mt + w] != 0u;
      }
      const uint64_t bal = __ballot(flag);
      if (flag) a.mlist[(int64_t)row * a.mtmax + base + __popcll(bal & ((1ull << t) - 1ull))] = mt * kBlk;
      base += __popcll(bal);
    }
    if (t == 0) a.mcount[row] = base;
  }
}

// Tile counts of every CSR rank, one thread each, into a.rank_slot for
// items_kernel: {exact tiles, mean tiles (an upper bound), first partial slot
// (-1 until items_kernel splits the row), 0}.
__global__ __launch_bounds__(256) void rank_tiles_kernel(AttnArgs a) {
  FP2_BOUNDS_GUARD(a.dbg);
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= a.rows) return;
  int ne, nm;
  rank_tiles(a, r, ne, nm);
  a.rank_slot[r] = make_int4(ne, nm, -1, 0);
}

// Work items and their launch order.  The kept-block counts of the rows are
// very uneven under a max-based threshold (a few rows keep most of their
// causal blocks), so the exact tiles of a row with more than C of them are
// split into near-equal chunks, each its own item (the row's last chunk also
// takes its mean tiles); C is chosen so that no item holds more than a
// quarter of a CU's share of the work, and so that the extra items stay
// within extra_cap.  Items are launched in kHeadPhases phases of consecutive
// KV heads (all items of the first heads before any of the next), each phase
// heaviest first (longest processing time first: a heavy item started last
// would leave the other CUs idle).  The phases halve the K and V^T tiles the
// device reads at any time (268 MB instead of 537 at 128K tokens with 8 KV
// heads, bf16, about the size of the 256 MB last-level cache); it measured
// 1-2% faster on every workload, four phases slower.  One workgroup: a
// counting sort on (phase, tile count); items of equal key land in any order
// (no result depends on it).
constexpr int kItemsThreads = 1024;
constexpr int kItemsMaxBins = 8192;  // 32 KB of LDS; heavier items share the top bin of their phase
constexpr int kHeadPhases = 2;
constexpr int kMinChunkTiles = 16;
constexpr int kItemsPerCuShare = 4;
constexpr int kRankCache = 8;  // rank records a thread keeps in registers (8192 ranks with 1024 threads)
// The counting-sort bin of an item of w tiles of CSR rank r (KV head r %
// Hkv): nbins / kHeadPhases bins per phase, the first phase's on top.
__device__ __forceinline__ int item_bin(const AttnArgs& a, int nbins, int r, int w) {
  const int per = nbins / kHeadPhases;
  const int phase = (r % a.hkv) * kHeadPhases / a.hkv;
  return min(w, per - 1) + per * (kHeadPhases - 1 - phase);
}

__global__ __launch_bounds__(kItemsThreads) void items_kernel(AttnArgs a, int nbins) {
  FP2_BOUNDS_GUARD(a.dbg);
  extern __shared__ int hist[];  // [nbins]
  __shared__ int part[kItemsThreads];
  __shared__ int s_tot[2], s_cnt[3];
  const int t = threadIdx.x;
  for (int i = t; i < nbins; i += kItemsThreads) hist[i] = 0;
  if (t < 2) s_tot[t] = 0;
  if (t < 3) s_cnt[t] = 0;
  __syncthreads();
  // the records of this thread's ranks r = t + k kItemsThreads: the first
  // kRankCache in registers (loaded at once), the rest from memory
  int4 rc[kRankCache];
#pragma unroll
  for (int k = 0; k < kRankCache; ++k) {
    const int r = t + k * kItemsThreads;
    rc[k] = r < a.rows ? a.rank_slot[r] : make_int4(0, 0, -1, 0);
  }
  auto each_rank = [&](auto&& body) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kRankCache; ++k) {
      const int r = t + k * kItemsThreads;
      if (r < a.rows) body(r, rc[k]);
    }
    for (int r = t + kRankCache * kItemsThreads; r < a.rows; r += kItemsThreads) {
      int4 rt = a.rank_slot[r];
      body(r, rt);
      a.rank_slot[r] = rt;
    }
  };
  int ex = 0, all = 0;
  each_rank([&](int, int4& rt) {
    ex += rt.x;
    all += rt.x + rt.y;
  });
  atomicAdd(&s_tot[0], ex);
  atomicAdd(&s_tot[1], all);
  __syncthreads();
  int C = 0x7fffffff;  // tiles per chunk: no split without extra items
  if (a.extra_cap > 0) {
    const int64_t share = ((int64_t)s_tot[1] * a.slices + a.ncu - 1) / max(a.ncu, 1);
    C = (int)max<int64_t>(kMinChunkTiles, (share + kItemsPerCuShare - 1) / kItemsPerCuShare);
    if (a.chunk_cap > 0) C = min(C, a.chunk_cap);
    C = max(C, (s_tot[0] + a.extra_cap - 1) / a.extra_cap);  // sum over rows of (chunks - 1) <= extra_cap
  }
  // pass 1: histogram of the items' tile counts; partial slots of split rows
  int nitems = 0;
  each_rank([&](int r, int4& rt) {
    const int ne = rt.x, nm = rt.y;
    const int nch = ne > C ? (ne + C - 1) / C : 1;
    if (nch > 1) {
      rt.z = atomicAdd(&s_cnt[1], nch);
      a.splits[atomicAdd(&s_cnt[2], 1)] = make_int4(r, rt.z, nch, 0);
    }
    nitems += nch;
    for (int c = 0; c < nch; ++c) {
      const int w = (int)(((int64_t)(c + 1) * ne) / nch - ((int64_t)c * ne) / nch) + (c == nch - 1 ? nm : 0);
      atomicAdd(&hist[item_bin(a, nbins, r, w)], 1);
    }
  });
  atomicAdd(&s_cnt[0], nitems);
  __syncthreads();
  // exclusive scan in descending bin order: a bin starts after every item of
  // an earlier head phase or of the same phase with more tiles; thread t owns
  // bins nbins-1-k for k in its chunk
  const int chunk = (nbins + kItemsThreads - 1) / kItemsThreads;
  const int k0 = min(t * chunk, nbins), k1 = min(k0 + chunk, nbins);
  int sum = 0;
  for (int k = k0; k < k1; ++k) sum += hist[nbins - 1 - k];
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < kItemsThreads; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - sum;
  for (int k = k0; k < k1; ++k) {
    const int c = hist[nbins - 1 - k];
    hist[nbins - 1 - k] = run;
    run += c;
  }
  __syncthreads();
  // pass 2: place the items
  each_rank([&](int r, int4& rt) {
    const int ne = rt.x, nm = rt.y;
    const int nch = ne > C ? (ne + C - 1) / C : 1;
    for (int c = 0; c < nch; ++c) {
      const int c0 = (int)(((int64_t)c * ne) / nch), c1 = (int)(((int64_t)(c + 1) * ne) / nch);
      const int w = c1 - c0 + (c == nch - 1 ? nm : 0);
      a.items[atomicAdd(&hist[item_bin(a, nbins, r, w)], 1)] = make_int4(r, c0, c1, nch > 1 ? rt.z + c : -1);
    }
  });
  if (t == 0) {
    a.counters[0] = s_cnt[0];
    a.counters[1] = s_cnt[2];
  }
}

// The values the workgroups of work item pos start from, so that they read
// one record instead of walking a chain of dependent loads (item -> CSR row
// bounds -> first columns -> page entries -> DMA): int32 [kInfoInts]
//   0 rank (-1: no item), 1 first and 2 end exact tile, 3 partial slot,
//   4 query block, 5 KV head, 6 sequence, 7 query block in the sequence,
//   8 first query token, 9 new tokens, 10 keys, 11 first KV block of the
//   sequence, 12 13 CSR row bounds, 14 mean tiles of the item, 16 17 the
//   block (PAIR: block pair) of tiles 0 and 1, 18 19 the raw CSR entries of
//   tile 2, e4m3: 20 21 the K scales of tile 0's blocks, 22 23 the pages
//   of tile 1's blocks, 24-31 and 32-39 the page of each 16 rows that DMA
//   wave w (w < 4) moves of tiles 0 and 1 (entry 2 w + half).
template <bool FP8, bool PAIR>
__global__ __launch_bounds__(256) void item_info_kernel(AttnArgs a) {
  FP2_BOUNDS_GUARD(a.dbg);
  constexpr int KB = PAIR ? 64 : kBlk;
  const int pos = blockIdx.x * 256 + threadIdx.x;
  if (pos >= a.rows + a.extra_cap) return;
  int32_t* rec = a.info + (int64_t)pos * kInfoInts;
  if (pos >= a.counters[0]) {
    rec[0] = -1;
    return;
  }
  const int4 it = a.items[pos];
  const int rank = it.x, tile0 = it.y, tile1 = it.z;
  const int qb = a.total_qblocks - 1 - rank / a.hkv;
  const int g = rank % a.hkv;
  const int row = g * a.total_qblocks + qb;
  const int s = find_seq(a.cu_qblocks, a.num_seqs, qb);
  const int I = qb - a.cu_qblocks[s];
  const int q0 = a.cu_seqlens_q[s];
  const int n = a.cu_seqlens_q[s + 1] - q0;
  const int T = a.seqlens_k[s];
  const int kb0 = a.cu_kblocks[s];
  const int32_t* pt = a.page_table + (int64_t)s * a.max_pages;
  const int qpos0 = T - n + I * kBlk;
  const int diag = PAIR ? (qpos0 + min(kBlk, n - I * kBlk) - 1) / KB : (T - n) / kBlk + I;
  const int dlo = PAIR ? qpos0 / KB : diag;
  const int rbeg = a.row_ptr[row], rend = a.row_ptr[row + 1];
  const int kbeg = rbeg + (PAIR ? 2 * tile0 : tile0);
  const int kend = PAIR ? min(rbeg + 2 * tile1, rend) : rbeg + tile1;
  const int nexact = PAIR ? tile1 - tile0 : kend - kbeg;
  const int ne = kend - kbeg;
  const int nmean = (a.correction && dlo > 1 && kend == rend) ? a.mcount[row] : 0;
  const int ntiles = nexact + nmean;
  const int32_t* ml = a.mlist + (int64_t)row * a.mtmax;
  auto mean_of = [&](int idx) -> int { return idx < ntiles ? ml[idx - nexact] : 0; };
  auto pack = [&](int ja, int jb, int i) { return ja | ((2 * i + 1 < ne ? jb : ja) << 16); };
  auto half_of = [](int J, int h) { return h ? J >> 16 : J & 0xFFFF; };
  int j0 = 0, j1 = 0, j2v = 0, j2vb = 0;
  if (0 < nexact) {
    if constexpr (PAIR) j0 = pack(a.col_idx[kbeg], a.col_idx[min(kbeg + 1, kend - 1)], 0);
    else j0 = a.col_idx[kbeg];
  } else if (0 < ntiles) {
    j0 = mean_of(0);
  }
  if (1 < nexact) {
    if constexpr (PAIR) j1 = pack(a.col_idx[kbeg + 2], a.col_idx[min(kbeg + 3, kend - 1)], 1);
    else j1 = a.col_idx[kbeg + 1];
  } else if (1 < ntiles) {
    j1 = mean_of(1);
  }
  if (2 < nexact) {
    if constexpr (PAIR) {
      j2v = a.col_idx[kbeg + 4];
      j2vb = kbeg + 5 < kend ? a.col_idx[kbeg + 5] : 0;
    } else {
      j2v = a.col_idx[kbeg + 2];
    }
  }
  // the page of rows r0 + 16 hh .. of exact tile J that DMA wave w moves (as
  // the attention kernel's page_of)
  auto page = [&](int J, int w, int hh) {
    const int r0 = PAIR ? half_of(J, w >= kDmaWaves / 2) * KB + kDmaRows * (w % (kDmaWaves / 2))
                        : J * kBlk + kDmaRows * w;
    int pi, slot;
    a.pm.split(min(r0 + 16 * hh, T - 1), pi, slot);
    return pt[pi];
  };
  int v[kInfoInts] = {};
  v[0] = rank;
  v[1] = tile0;
  v[2] = tile1;
  v[3] = it.w;
  v[4] = qb;
  v[5] = g;
  v[6] = s;
  v[7] = I;
  v[8] = q0;
  v[9] = n;
  v[10] = T;
  v[11] = kb0;
  v[12] = rbeg;
  v[13] = rend;
  v[14] = nmean;
  v[16] = j0;
  v[17] = j1;
  v[18] = j2v;
  v[19] = j2vb;
  if constexpr (FP8) {
    if (0 < nexact) {
      v[20] = __float_as_int(a.k_scale[(int64_t)pt[half_of(j0, 0)] * a.hkv + g]);
      if constexpr (PAIR) v[21] = __float_as_int(a.k_scale[(int64_t)pt[half_of(j0, 1)] * a.hkv + g]);
    }
    if (1 < nexact) {
      v[22] = pt[half_of(j1, 0)];
      if constexpr (PAIR) v[23] = pt[half_of(j1, 1)];
    }
  }
  for (int w = 0; w < kDmaWaves; ++w)
    for (int hh = 0; hh < kDmaHalves; ++hh) {
      if (0 < nexact) v[24 + 2 * w + hh] = page(j0, w, hh);
      if (1 < nexact) v[32 + 2 * w + hh] = page(j1, w, hh);
    }
  for (int i = 0; i < kInfoInts; i += 4) *reinterpret_cast<int4*>(rec + i) = make_int4(v[i], v[i + 1], v[i + 2], v[i + 3]);
}

// Merges the chunks of each split row: O = sum_c 2^(m_c - M) O_c over
// sum_c 2^(m_c - M) l_c, M = max_c m_c (the chunks' reference maxima, log2
// units), then the same O / l store as the attention epilogue.  One
// workgroup per (split row, slice), the attention kernel's lane layout.
__global__ __launch_bounds__(kThreads) void combine_kernel(AttnArgs a) {
  FP2_BOUNDS_GUARD(a.dbg);
  if ((int)blockIdx.x >= ld_uniform(a.counters, 1)) return;
  const int32_t* sp = reinterpret_cast<const int32_t*>(a.splits + blockIdx.x);
  const int rank = ld_uniform(sp, 0), slot0 = ld_uniform(sp, 1), nch = ld_uniform(sp, 2);
  const int slice = blockIdx.y;
  const int qb = a.total_qblocks - 1 - rank / a.hkv;
  const int g = rank % a.hkv;
  const int s = find_seq(a.cu_qblocks, a.num_seqs, qb);
  const int I = qb - a.cu_qblocks[s];
  const int q0 = a.cu_seqlens_q[s];
  const int n = a.cu_seqlens_q[s + 1] - q0;
  const int G = a.hq / a.hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5;
  const int prow = slice * kWGRows + wave * 32;
  const int h = g * G + prow / kBlk;
  const int tq = prow % kBlk + (lane & 31);
  if (!(prow < G * kBlk) || I * kBlk + tq >= n) return;
  auto chunk_part = [&](int c) {
    return a.part + ((int64_t)((slot0 + c) * a.slices + slice) * kWaves + wave) * kPartFloatsPerWave;
  };
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, chunk_part(c)[64 * 64 + 2 * lane]);
  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int c = 0; c < nch; ++c) {
    const float* po = chunk_part(c);
    const float2 ml = *reinterpret_cast<const float2*>(po + 64 * 64 + 2 * lane);
    const float w = ml.x == -INFINITY ? 0.f : exp2f(ml.x - M);
    L = fmaf(w, ml.y, L);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(po + (j * 64 + lane) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[j][e] = fmaf(w, v[e], acc[j][e]);
    }
  }
  const float inv = 1.0f / L;
  const int64_t obase = ((int64_t)(q0 + I * kBlk + tq) * a.hq + h) * kD;
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 v = acc[dt * 4 + q4];
      const int d0 = 32 * dt + 8 * q4 + 4 * hf;
      if (a.out_f32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + obase + d0) =
            f32x4{v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv};
      } else {
        uint2 o;
        o.x = pack_bf16x2(v[0] * inv, v[1] * inv);
        o.y = pack_bf16x2(v[2] * inv, v[3] * inv);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + obase + d0) = o;
      }
    }
}

// The V^T preparation does not depend on the work-item kernels, so it runs
// on a second stream of the library's (one per device, created on first use,
// default priority) while the caller's stream builds the work items; the two
// meet before the attention kernel.  Each device's fork and join events are
// shared by all calls, so one call's record / wait pairs are enqueued under a
// host lock.
struct SidePath {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SidePath g_side[kMaxDevices];

// (g_side_mu held)
hipError_t side_path(int dev, SidePath*& out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  SidePath& sp = g_side[dev];
  if (!sp.stream) {
    SidePath n;
    hipError_t e = hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (n.join) (void)hipEventDestroy(n.join);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.stream) (void)hipStreamDestroy(n.stream);
      return e;
    }
    sp = n;
  }
  out = &sp;
  return hipSuccess;
}

// V^T tiles of every KV block and head, and the mean tokens' vbar^T tiles
// and bf16 kbar rows
hipError_t launch_prep(const PrepArgs& p, const AttnArgs& a, bool fp8, int max_kblocks, hipStream_t stream) {
  const dim3 per_block((unsigned)a.total_kblocks, (unsigned)a.hkv);
  const dim3 per_pair((unsigned)((a.total_kblocks + 1) / 2), (unsigned)a.hkv);
  if (fp8 && a.pair)
    hipLaunchKernelGGL((vt_exact_kernel<true, true>), per_pair, dim3(256), 0, stream, p);
  else if (fp8)
    hipLaunchKernelGGL((vt_exact_kernel<true, false>), per_block, dim3(256), 0, stream, p);
  else if (a.pair)
    hipLaunchKernelGGL((vt_exact_kernel<false, true>), per_pair, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((vt_exact_kernel<false, false>), per_block, dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.correction) return e;
  hipLaunchKernelGGL(vt_mean_kernel, dim3((unsigned)((max_kblocks + kBlk - 1) / kBlk), (unsigned)a.num_seqs,
                                          (unsigned)a.hkv),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

// mean-tile lists, tile counts, work items and their records
hipError_t launch_items(const AttnArgs& a, bool fp8, int max_kblocks, hipStream_t stream) {
  // bins per head phase: every tile count up to a whole causal row of exact and mean tiles
  const int nbins = kHeadPhases * min(max_kblocks + (max_kblocks + kBlk - 1) / kBlk + 1, kItemsMaxBins / kHeadPhases);
  if (a.correction) {
    hipLaunchKernelGGL(mean_prep_kernel, dim3((unsigned)a.rows), dim3(256), 0, stream, a);
    if (hipError_t e0 = hipGetLastError(); e0 != hipSuccess) return e0;
  }
  hipLaunchKernelGGL(rank_tiles_kernel, dim3((unsigned)((a.rows + 255) / 256)), dim3(256), 0, stream, a);
  if (hipError_t e0 = hipGetLastError(); e0 != hipSuccess) return e0;
  hipLaunchKernelGGL(items_kernel, dim3(1), dim3(kItemsThreads), (size_t)nbins * sizeof(int), stream, a, nbins);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int items_cap = a.rows + a.extra_cap;
  const dim3 info_grid((unsigned)((items_cap + 255) / 256));
  if (fp8 && a.pair)
    hipLaunchKernelGGL((item_info_kernel<true, true>), info_grid, dim3(256), 0, stream, a);
  else if (fp8)
    hipLaunchKernelGGL((item_info_kernel<true, false>), info_grid, dim3(256), 0, stream, a);
  else if (a.pair)
    hipLaunchKernelGGL((item_info_kernel<false, true>), info_grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((item_info_kernel<false, false>), info_grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_impl(const AttnArgs& a_in, bool fp8, const float* kbar, const float* vbar, int max_kblocks,
                       hipStream_t stream) {
  AttnArgs a = a_in;
  PrepArgs p;
  p.dbg = a.dbg;
  p.cu_kblocks = a.cu_kblocks;
  p.cu_seqlens_q = a.cu_seqlens_q;
  p.seqlens_k = a.seqlens_k;
  p.page_table = a.page_table;
  p.k_pages = a.k_pages;
  p.v_pages = a.v_pages;
  p.v_scale = a.v_scale;
  p.kbar = kbar;
  p.vbar = vbar;
  p.kbar16 = const_cast<uint16_t*>(a.kbar16);
  p.vt = const_cast<uint8_t*>(a.vt);
  p.vbt = const_cast<uint8_t*>(a.vbt);
  p.pm = a.pm;
  p.num_seqs = a.num_seqs;
  p.hkv = a.hkv;
  p.max_pages = a.max_pages;
  p.page_size = a.page_size;
  p.total_kblocks = a.total_kblocks;
  p.mt_cap = a.mt_cap;
  if (a.rows <= 0) return a.total_kblocks > 0 ? launch_prep(p, a, fp8, max_kblocks, stream) : hipSuccess;
  const int G = a.hq / a.hkv;
  a.slices = (G * kBlk + kWGRows - 1) / kWGRows;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  a.ncu = 256;
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && ncu > 0) a.ncu = ncu;
  if (a.total_kblocks > 0) {
    std::lock_guard<std::mutex> lk(g_side_mu);
    SidePath* sp = nullptr;
    e = side_path(dev, sp);
    if (e == hipSuccess) e = hipEventRecord(sp->fork, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(sp->stream, sp->fork, 0);
    if (e != hipSuccess) return e;
    // from here on the caller's stream waits for the side stream's work, also on an error
    e = launch_prep(p, a, fp8, max_kblocks, sp->stream);
    hipError_t ej = hipEventRecord(sp->join, sp->stream);
    if (e == hipSuccess && ej == hipSuccess) e = launch_items(a, fp8, max_kblocks, stream);
    if (ej == hipSuccess) ej = hipStreamWaitEvent(stream, sp->join, 0);
    if (e == hipSuccess) e = ej;
  } else {
    e = launch_items(a, fp8, max_kblocks, stream);
  }
  if (e != hipSuccess) return e;
  const int items_cap = a.rows + a.extra_cap;
  const unsigned grid = (unsigned)(((items_cap + 7) / 8) * 8 * a.slices);
  if (fp8 && a.pair)
    hipLaunchKernelGGL((attn_d128_kernel<true, true>), dim3(grid), dim3(kThreads), 0, stream, a);
  else if (fp8)
    hipLaunchKernelGGL((attn_d128_kernel<true, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  else if (a.pair)
    hipLaunchKernelGGL((attn_d128_kernel<false, true>), dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_d128_kernel<false, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.extra_cap <= 0) return e;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)a.extra_cap, (unsigned)a.slices), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_d128(const AttnArgs& a, bool fp8, const float* kbar, const float* vbar, int max_kblocks,
                            hipStream_t stream) {
  return launch_impl(a, fp8, kbar, vbar, max_kblocks, stream);
}

}  // namespace fp2
