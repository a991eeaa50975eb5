// Host-only argument checks for the C ABI.  Plain C++: no HIP call is made
// here, so every rejection happens before anything is enqueued.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>

#include "fp2_internal.h"

namespace fp2 {

namespace {
thread_local std::string g_err;

std::string S(long long v) { return std::to_string(v); }
}  // namespace

fp2_status fail(fp2_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

const char* last_error() { return g_err.c_str(); }

fp2_status check_batch(const fp2_batch* b, BatchInfo* info) {
  if (!b) return fail(FP2_ERR_INVALID, "batch is NULL");
  if (b->num_seqs < 0) return fail(FP2_ERR_INVALID, "num_seqs < 0");
  if (b->block != 64 && b->block != 128)
    return fail(FP2_ERR_UNSUPPORTED, "block must be 64 or 128, got " + S(b->block));
  if (b->num_seqs > 0) {
    if (!b->cu_seqlens_q || !b->seqlens_k || !b->cu_qblocks || !b->cu_kblocks)
      return fail(FP2_ERR_INVALID, "batch device arrays must not be NULL");
    if (!b->h_cu_seqlens_q || !b->h_seqlens_k)
      return fail(FP2_ERR_INVALID, "batch host mirrors must not be NULL");
    if (b->h_cu_seqlens_q[0] != 0) return fail(FP2_ERR_INVALID, "cu_seqlens_q[0] must be 0");
  }
  const int B = b->block;
  const int KB = b->kv_block == 0 ? B : b->kv_block;
  if (KB != B && !(B == 128 && KB == 64))
    return fail(FP2_ERR_UNSUPPORTED, "kv_block must be 0, block, or 64 with block 128; got " + S(b->kv_block));
  BatchInfo r;
  r.qblock = B;
  r.kvblock = KB;
  for (int s = 0; s < b->num_seqs; ++s) {
    const long long n = (long long)b->h_cu_seqlens_q[s + 1] - b->h_cu_seqlens_q[s];
    const long long T = b->h_seqlens_k[s];
    if (n < 0) return fail(FP2_ERR_INVALID, "cu_seqlens_q decreases at sequence " + S(s));
    if (T < n)
      return fail(FP2_ERR_INVALID, "sequence " + S(s) + ": seqlens_k (" + S(T) +
                                       ") < new queries (" + S(n) + ")");
    const long long P = T - n;
    if (T > (1LL << 21))
      return fail(FP2_ERR_UNSUPPORTED, "sequence " + S(s) + ": " + S(T) + " tokens; at most 2^21 supported");
    if (P % B != 0)
      return fail(FP2_ERR_UNSUPPORTED, "sequence " + S(s) + ": cached prefix " + S(P) +
                                           " is not a multiple of block " + S(B));
    const long long nqb = (n + B - 1) / B, nkb = (T + KB - 1) / KB;
    r.total_q += n;
    r.total_qblocks += nqb;
    r.total_kblocks += nkb;
    if (nkb > r.max_kblocks) r.max_kblocks = nkb;
    // the last diagonal KV block of query block I holds its last position:
    // (P + B(I+1) - 1)/KB = P/KB + (B/KB)(I+1) - 1 for a full block, (P +
    // n - 1)/KB for the last one; causal pairs = sum over I of that + 1
    if (nqb > 0)
      r.causal_pairs += (nqb - 1) * (P / KB) + (long long)(B / KB) * (nqb - 1) * nqb / 2 + (P + n - 1) / KB + 1;
  }
  if (r.max_kblocks > kMaxKBlocks)
    return fail(FP2_ERR_UNSUPPORTED, "a sequence has " + S(r.max_kblocks) +
                                         " KV blocks; at most " + S(kMaxKBlocks) + " supported");
  if (r.total_q > (1LL << 31) - 1 || r.total_qblocks * 64 > (1LL << 31) - 1)
    return fail(FP2_ERR_UNSUPPORTED, "batch too large for 32-bit row indices");
  *info = r;
  return FP2_OK;
}

fp2_status check_index_range(const BatchInfo& info, int num_kv_heads) {
  const long long kMax = (1LL << 31) - 1;
  if (info.total_qblocks * num_kv_heads + 1 > kMax)
    return fail(FP2_ERR_UNSUPPORTED, "total_qblocks * num_kv_heads = " + S(info.total_qblocks * num_kv_heads) +
                                         " CSR rows do not fit 32-bit row indices");
  if (info.causal_pairs * num_kv_heads > kMax)
    return fail(FP2_ERR_UNSUPPORTED, "the batch has " + S(info.causal_pairs * num_kv_heads) +
                                         " causal (query block, KV block, KV head) pairs; the CSR holds at most "
                                         "2^31 - 1 entries");
  return FP2_OK;
}

fp2_status check_q(const fp2_q* q, int num_kv_heads, const BatchInfo& info, int block) {
  if (!q) return fail(FP2_ERR_INVALID, "q is NULL");
  if (q->dtype != FP2_BF16 && q->dtype != FP2_FP8_E4M3)
    return fail(FP2_ERR_INVALID, "unknown q dtype " + S(q->dtype));
  if (q->head_dim != 64 && q->head_dim != 128)
    return fail(FP2_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got " + S(q->head_dim));
  if (num_kv_heads < 1) return fail(FP2_ERR_INVALID, "num_kv_heads < 1");
  if (q->num_q_heads < 1 || q->num_q_heads % num_kv_heads != 0)
    return fail(FP2_ERR_INVALID, "num_q_heads (" + S(q->num_q_heads) +
                                     ") must be a positive multiple of num_kv_heads (" +
                                     S(num_kv_heads) + ")");
  const int G = q->num_q_heads / num_kv_heads;
  const int esz = q->dtype == FP2_BF16 ? 2 : 1;
  if ((long long)G * q->head_dim * esz > kPoolRowBytes)
    return fail(FP2_ERR_UNSUPPORTED, "query group too wide: G*d*elem = " +
                                         S((long long)G * q->head_dim * esz) + " bytes > " +
                                         S(kPoolRowBytes));
  if ((long long)G * block > (1LL << 20))
    return fail(FP2_ERR_UNSUPPORTED, "G*block too large");
  if (info.total_q > 0 && !q->q) return fail(FP2_ERR_INVALID, "q->q is NULL");
  if (q->dtype == FP2_FP8_E4M3 && info.total_q > 0 && !q->q_scale)
    return fail(FP2_ERR_INVALID, "e4m3 queries need q_scale");
  return FP2_OK;
}

fp2_status check_kv(const fp2_kv* kv, const fp2_batch* b, const BatchInfo& info) {
  if (!kv) return fail(FP2_ERR_INVALID, "kv is NULL");
  if (kv->dtype != FP2_BF16 && kv->dtype != FP2_FP8_E4M3)
    return fail(FP2_ERR_INVALID, "unknown kv dtype " + S(kv->dtype));
  if (kv->head_dim != 64 && kv->head_dim != 128)
    return fail(FP2_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got " + S(kv->head_dim));
  if (kv->num_kv_heads < 1) return fail(FP2_ERR_INVALID, "num_kv_heads < 1");
  if ((long long)kv->num_kv_heads * kv->head_dim * 2 > (1LL << 20))
    return fail(FP2_ERR_UNSUPPORTED, "num_kv_heads too large");
  if (kv->page_size < 1) return fail(FP2_ERR_INVALID, "page_size < 1");
  if (kv->num_pages < 0 || kv->max_pages_per_seq < 0)
    return fail(FP2_ERR_INVALID, "negative page counts");
  if (kv->dtype == FP2_FP8_E4M3 && kv->page_size != info.kvblock)
    return fail(FP2_ERR_UNSUPPORTED, "e4m3 KV scales are per page: page_size (" +
                                         S(kv->page_size) + ") must equal the KV block (" +
                                         S(info.kvblock) + ")");
  long long need_pages = 0;
  for (int s = 0; s < b->num_seqs; ++s) {
    const long long np = ((long long)b->h_seqlens_k[s] + kv->page_size - 1) / kv->page_size;
    if (np > kv->max_pages_per_seq)
      return fail(FP2_ERR_INVALID, "sequence " + S(s) + " needs " + S(np) +
                                       " pages > max_pages_per_seq " + S(kv->max_pages_per_seq));
    need_pages += np;
  }
  (void)need_pages;  // pages may be shared between sequences; no lower bound on num_pages
  if (info.total_kblocks > 0) {
    if (!kv->k_pages || !kv->v_pages || !kv->page_table)
      return fail(FP2_ERR_INVALID, "k_pages, v_pages and page_table must not be NULL");
    if (kv->dtype == FP2_FP8_E4M3 && (!kv->k_scale || !kv->v_scale))
      return fail(FP2_ERR_INVALID, "e4m3 KV needs k_scale and v_scale");
    if (kv->num_pages < 1) return fail(FP2_ERR_INVALID, "num_pages < 1");
  }
  return FP2_OK;
}

size_t plan_workspace_bytes(const BatchInfo& info, int num_kv_heads) {
  const size_t rows = (size_t)info.total_qblocks * (size_t)num_kv_heads;
  if (rows == 0) return 0;
  const size_t words = (size_t)plan_words(info);
  size_t bytes = rows * words * 4;     // keep bitmask per row
  bytes = (bytes + 255) & ~size_t(255);
  bytes += rows * 4;                   // kept count per row
  return (bytes + 255) & ~size_t(255);
}

size_t stage1_workspace_bytes(const BatchInfo& info, int num_kv_heads, int head_dim) {
  const size_t plan = plan_workspace_bytes(info, num_kv_heads);
  const size_t qbar = ((size_t)info.total_qblocks * num_kv_heads * head_dim * 4 + 255) & ~size_t(255);
  return plan + qbar + kStage1TicketBytes;
}

RunLayout run_layout(const BatchInfo& info, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                     int dtype) {
  auto up = [](size_t v) { return (v + 255) & ~size_t(255); };
  RunLayout L;
  const size_t tkb = (size_t)info.total_kblocks, hkv = (size_t)num_kv_heads;
  if (tkb == 0) return L;
  const size_t rows = up(hkv * tkb * (size_t)head_dim * 2);  // one bf16/fp16 copy of kbar or vbar
  L.k16 = 0;
  L.v16 = rows;
  if (vt_path(dtype, head_dim, info)) {
    const size_t tile = (size_t)info.kvblock * (size_t)head_dim * 2;  // V^T of one KV block, bf16
    const size_t mtile = 128 * (size_t)head_dim * 2;                   // vbar^T of 128 mean tokens
    L.mt_cap = (int64_t)(tkb / 128 + (size_t)num_seqs + 1);
    L.vt = L.v16 + hkv * (size_t)L.mt_cap * mtile;
    L.total = L.vt + hkv * tkb * tile;
    // work items: one per CSR row plus the extra chunks of split rows (at
    // most one per 4 causal tiles, and kMaxExtraItems); a split row holds at
    // least two chunks, so the partial slots are at most twice the extras
    const size_t nrows = hkv * (size_t)info.total_qblocks;
    const int64_t causal_tiles = info.causal_pairs * (int64_t)num_kv_heads;
    L.extra_cap = std::min<int64_t>(kMaxExtraItems, (causal_tiles + 3) / 4);
    const size_t slices = (size_t)((std::max(num_q_heads / std::max(num_kv_heads, 1), 1) * info.qblock + 255) / 256);
    L.items = L.total;
    L.splits = L.items + up((nrows + (size_t)L.extra_cap) * 16);
    L.rank_slot = L.splits + up((size_t)L.extra_cap * 16 + 16);
    L.counters = L.rank_slot + up(nrows * 16);
    L.part = L.counters + 256;
    L.info = L.part + up(2 * (size_t)L.extra_cap * slices * 8 * (size_t)kPartFloatsPerWave * 4);
    L.wskip = (int)((info.max_kblocks + 31) / 32);
    L.mtmax = (int)((info.max_kblocks + 127) / 128);
    L.skip = L.info + up((nrows + (size_t)L.extra_cap) * kInfoInts * 4);
    L.mlist = L.skip + up(nrows * (size_t)L.wskip * 4);
    L.mcount = L.mlist + up(nrows * (size_t)L.mtmax * 4);
    L.total = L.mcount + up(nrows * 4);
  } else {
    L.total = L.v16 + rows;
  }
  return L;
}

}  // namespace fp2
