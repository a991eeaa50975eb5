// Shared by the two attention kernels: launch arguments and constants.
#pragma once

#include "fp2_device.h"
#include "fp2_internal.h"

namespace fp2 {

// The reference max of the online softmax is refreshed only when some lane's
// max grew by more than kLazy (log2 units); probabilities are otherwise taken
// against the stale max (at most 2^kLazy), which leaves O / l unchanged.
constexpr float kLazy = 8.0f;

struct AttnArgs {
  const uint32_t* dbg;  // bounds-checking builds: the error word (see fp2_device.h), else nullptr
  const int32_t* cu_seqlens_q;
  const int32_t* seqlens_k;
  const int32_t* cu_qblocks;
  const int32_t* cu_kblocks;
  const int32_t* page_table;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const uint8_t* q;
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  const uint16_t* kbar16;  // bf16 [Hkv, total_kblocks, D]
  const uint16_t* vbar16;  // fp16 [Hkv, total_kblocks, D] (register-staged kernel)
  const uint8_t* vt;       // V^T tiles of every KV block (bf16 d128 kernel)
  const uint8_t* vbt;      // vbar^T tiles of the mean tokens (bf16 d128 kernel)
  int4* items;             // d128 kernel: work items {rank, first tile, end tile, partial slot or -1},
                           // heaviest first, [rows + extra_cap]
  int4* splits;            // d128 kernel: split rows {rank, first slot, chunks, 0}, [extra_cap]
  int4* rank_slot;         // d128 kernel: per CSR rank {exact tiles, mean tiles, first partial slot, 0}
                           // (items kernel scratch)
  int32_t* counters;       // d128 kernel: [0] work items, [1] split rows
  float* part;             // d128 kernel: partial O, reference max and row sum of split-row chunks
  int32_t* info;           // d128 kernel: per work item, the values its workgroup starts from [items, kInfoInts]
  uint32_t* skip;          // d128 kernel with correction: skipped-block bitmask per CSR row [rows, wskip]
  int32_t* mlist;          // d128 kernel with correction: first mean token of each mean tile per CSR row [rows, mtmax]
  int32_t* mcount;         // d128 kernel with correction: mean tiles per CSR row [rows]
  int wskip, mtmax;
  int extra_cap, chunk_cap, ncu;
  void* out;               // bf16 or f32 [total_q, Hq, D]
  float scale_log2;        // softmax_scale * log2(e)
  float log2_block;        // log2 of the KV block size: the weight of a mean token
  PageMap pm;
  int num_seqs, hq, hkv, max_pages, page_size, total_qblocks, total_kblocks;
  int correction, slices, rows, out_f32, mt_cap;
  int qblk;                // query block tokens (register-staged kernel; the d128 kernel's is 128)
  int pair;                // d128 kernel: 64-token KV blocks, two to a 128-key tile
};


// Transposes V (and vbar, and rounds kbar) into the workspace parts that
// a.vt, a.vbt and a.kbar16 point to (e4m3: V dequantized), builds the
// work items (the exact tiles of heavy rows split into chunks, heaviest item
// first), runs the d=128 B=128 kernel and merges the chunks of split rows.
hipError_t launch_attn_d128(const AttnArgs& a, bool fp8, const float* kbar, const float* vbar, int max_kblocks,
                            hipStream_t stream);

}  // namespace fp2
