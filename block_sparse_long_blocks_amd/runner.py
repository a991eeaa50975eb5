"""Buffers and the three-call sequence of one prefill layer.

Allocates (through torch) every device buffer the C ABI needs for a batch and
runs fp2_block_stats -> fp2_plan_mask -> fp2_prefill_run on one stream.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from ._binding import (Batch, KVCache, Queries, fp2_block_stats, fp2_plan_mask, fp2_plan_max_nnz,
                       fp2_plan_workspace_bytes, fp2_prefill_run, fp2_run_workspace_bytes, fp2_stage1,
                       fp2_stage1_workspace_bytes)


class PrefillLayer:
    def __init__(self, batch: Batch, q: Queries, kv: KVCache, with_scores: bool = False,
                 out_dtype: torch.dtype = torch.bfloat16, fused_stage1: bool = False):
        self.batch, self.q, self.kv = batch, q, kv
        dev = q.q.device
        hkv, d = kv.num_kv_heads, q.q.shape[2]
        rows = batch.total_qblocks * hkv
        f32 = dict(dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.kbar = torch.empty((hkv, max(1, batch.total_kblocks), d), **f32)
        self.vbar = torch.empty_like(self.kbar)
        self.row_ptr = torch.empty(rows + 1, **i32)
        self.col_idx = torch.empty(max(1, fp2_plan_max_nnz(batch, hkv)), **i32)
        self.nnz = torch.zeros(1, **i32)
        self.plan_ws = torch.empty(max(1, fp2_plan_workspace_bytes(batch, hkv)), dtype=torch.uint8, device=dev)
        self.stage1_ws = torch.empty(max(1, fp2_stage1_workspace_bytes(batch, hkv, d)), dtype=torch.uint8, device=dev)
        # __call__: fp2_block_stats then fp2_plan_mask (the faster at 128K), or fp2_stage1
        self.fused_stage1 = fused_stage1
        self.run_ws = torch.empty(max(1, fp2_run_workspace_bytes(batch, q.q.shape[1], hkv, d, kv.dtype)), dtype=torch.uint8, device=dev)
        self.out = torch.empty((max(1, batch.total_q), q.q.shape[1], d), dtype=out_dtype, device=dev)
        self.scores = torch.empty((rows, max(1, batch.max_kblocks)), **f32) if with_scores else None
        self.max_chunk_tiles = 0  # fp2_prefill_run's chunk cap: 0 library's choice, > 0 cap, < 0 no split

    def stats(self, stream=None):
        fp2_block_stats(self.batch, self.kv, self.kbar, self.vbar, stream)

    def plan(self, tau: float, stream=None):
        fp2_plan_mask(self.batch, self.q, self.kv.num_kv_heads, self.kbar, tau, self.row_ptr, self.col_idx,
                      self.nnz, self.plan_ws, self.scores, stream)

    def stage1(self, tau: float, stream=None):
        fp2_stage1(self.batch, self.q, self.kv, tau, self.kbar, self.vbar, self.row_ptr, self.col_idx, self.nnz,
                   self.stage1_ws, self.scores, stream)

    def attend(self, correction: bool, stream=None, softmax_scale: Optional[float] = None):
        fp2_prefill_run(self.batch, self.q, self.kv, self.row_ptr, self.col_idx, self.kbar, self.vbar,
                        correction, self.out, self.run_ws, softmax_scale, stream, self.max_chunk_tiles)

    def __call__(self, tau: float, correction: bool, stream=None):
        if self.fused_stage1:
            self.stage1(tau, stream)
        else:
            self.stats(stream)
            self.plan(tau, stream)
        self.attend(correction, stream)
        return self.out

    def csr_host(self):
        rp = self.row_ptr.cpu().numpy().astype(np.int64)
        return rp, self.col_idx[:int(rp[-1])].cpu().numpy().astype(np.int64)


def from_arrays(block: int, seqlens_k, n_q, q, q_scale, k_pages, v_pages, page_table,
                k_scale=None, v_scale=None, device: str = "cuda", kv_block: int = 0):
    """Device descriptors from host arrays (numpy): bf16 data as uint16 bit patterns,
    e4m3 data as uint8 codes with float32 scales; kv_block 0 = block."""
    def dev_codes(x):
        t = torch.from_numpy(np.ascontiguousarray(x))
        if x.dtype == np.uint16:
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(device)

    def dev_f32(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)

    batch = Batch(block, [int(t) for t in seqlens_k], [int(n) for n in n_q], device, kv_block)
    queries = Queries(dev_codes(q), dev_f32(q_scale))
    kv = KVCache(dev_codes(k_pages), dev_codes(v_pages),
                 torch.from_numpy(np.ascontiguousarray(page_table, dtype=np.int32)).to(device),
                 dev_f32(k_scale), dev_f32(v_scale))
    return batch, queries, kv


def from_workload(w, device: str = "cuda"):
    """Device descriptors of a generated workload (anything with the attribute names below)."""
    return from_arrays(w.cfg.block, w.seqlens_k, w.n_q, w.q, w.q_scale, w.k_pages, w.v_pages, w.page_table,
                       w.k_scale, w.v_scale, device, getattr(w.cfg, "kv_block", 0) or 0)
