"""ctypes binding of libfp2.so, the C ABI declared in include/fp2.h.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  There is no
fallback: if the library is missing or fails to load, importing this module
raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp2.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is not built; run `python block_sparse_long_blocks_amd/build.py` from the repository root "
        "(hipcc --offload-arch=gfx950).  There is no fallback implementation.")
_lib = ctypes.CDLL(_LIB_PATH)

FP2_OK, FP2_ERR_INVALID, FP2_ERR_UNSUPPORTED, FP2_ERR_CAPACITY, FP2_ERR_HIP = range(5)
FP2_BF16, FP2_FP8_E4M3 = 0, 1
FP2_OUT_BF16, FP2_OUT_F32 = 0, 1
STATUS_NAMES = {0: "FP2_OK", 1: "FP2_ERR_INVALID", 2: "FP2_ERR_UNSUPPORTED", 3: "FP2_ERR_CAPACITY",
                4: "FP2_ERR_HIP"}

SYMBOLS = ("fp2_block_stats", "fp2_block_stats_cache_rows", "fp2_block_stats_cached", "fp2_gather_block_stats",
           "fp2_plan_workspace_bytes", "fp2_plan_max_nnz", "fp2_plan_mask", "fp2_plan_mask_noalloc",
           "fp2_stage1_workspace_bytes", "fp2_stage1", "fp2_run_workspace_bytes", "fp2_prefill_run",
           "fp2_debug_bounds_word", "fp2_last_error")

_p = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)


class CBatch(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("block", ctypes.c_int32),
                ("cu_seqlens_q", _p), ("seqlens_k", _p), ("cu_qblocks", _p), ("cu_kblocks", _p),
                ("h_cu_seqlens_q", _i32p), ("h_seqlens_k", _i32p), ("kv_block", ctypes.c_int32)]


class CQ(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("num_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q", _p), ("q_scale", _p)]


class CKV(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("k_pages", _p), ("v_pages", _p),
                ("k_scale", _p), ("v_scale", _p), ("page_table", _p)]


_lib.fp2_block_stats.argtypes = [ctypes.POINTER(CBatch), ctypes.POINTER(CKV), _p, _p, _p]
_lib.fp2_block_stats.restype = ctypes.c_int
_lib.fp2_block_stats_cache_rows.argtypes = [ctypes.POINTER(CBatch), ctypes.POINTER(CKV)]
_lib.fp2_block_stats_cache_rows.restype = ctypes.c_int64
_lib.fp2_block_stats_cached.argtypes = [ctypes.POINTER(CBatch), ctypes.POINTER(CKV), _p, _p, ctypes.c_int32, _p]
_lib.fp2_block_stats_cached.restype = ctypes.c_int
_lib.fp2_gather_block_stats.argtypes = [ctypes.POINTER(CBatch), ctypes.POINTER(CKV), _p, _p, _p, _p, _p]
_lib.fp2_gather_block_stats.restype = ctypes.c_int
_lib.fp2_plan_workspace_bytes.argtypes = [ctypes.POINTER(CBatch), ctypes.c_int32]
_lib.fp2_plan_workspace_bytes.restype = ctypes.c_size_t
_lib.fp2_plan_max_nnz.argtypes = [ctypes.POINTER(CBatch), ctypes.c_int32]
_lib.fp2_plan_max_nnz.restype = ctypes.c_int64
_lib.fp2_plan_mask.argtypes = [ctypes.POINTER(CBatch), ctypes.POINTER(CQ), ctypes.c_int32, _p,
                               ctypes.c_float, _p, _p, ctypes.c_int64, _p, _p, _p, ctypes.c_size_t, _p]
_lib.fp2_plan_mask.restype = ctypes.c_int
_lib.fp2_plan_mask_noalloc.argtypes = [ctypes.POINTER(CBatch), ctypes.POINTER(CQ), ctypes.c_int32, _p,
                                       ctypes.c_float, _p, _p, ctypes.c_int64, _p, _p, _p]
_lib.fp2_plan_mask_noalloc.restype = ctypes.c_int
_lib.fp2_stage1_workspace_bytes.argtypes = [ctypes.POINTER(CBatch), ctypes.c_int32, ctypes.c_int32]
_lib.fp2_stage1_workspace_bytes.restype = ctypes.c_size_t
_lib.fp2_stage1.argtypes = [ctypes.POINTER(CBatch), ctypes.POINTER(CQ), ctypes.POINTER(CKV), ctypes.c_float, _p, _p,
                            _p, _p, ctypes.c_int64, _p, _p, _p, ctypes.c_size_t, _p]
_lib.fp2_stage1.restype = ctypes.c_int
_lib.fp2_run_workspace_bytes.argtypes = [ctypes.POINTER(CBatch), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int]
_lib.fp2_run_workspace_bytes.restype = ctypes.c_size_t
_lib.fp2_prefill_run.argtypes = [ctypes.POINTER(CBatch), ctypes.POINTER(CQ), ctypes.POINTER(CKV), _p, _p,
                                 _p, _p, ctypes.c_int32, ctypes.c_float, ctypes.c_int, _p, ctypes.c_int32, _p,
                                 ctypes.c_size_t, _p]
_lib.fp2_prefill_run.restype = ctypes.c_int
_lib.fp2_debug_bounds_word.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
_lib.fp2_debug_bounds_word.restype = ctypes.c_int
_lib.fp2_last_error.argtypes = []
_lib.fp2_last_error.restype = ctypes.c_char_p


class Fp2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _check(status: int):
    if status != FP2_OK:
        raise Fp2Error(status, (_lib.fp2_last_error() or b"").decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


# ---------------------------------------------------------------------------
# Descriptors
# ---------------------------------------------------------------------------

@dataclass
class Batch:
    """Variable-length batch descriptors: device int32 arrays plus host mirrors.

    block: query block tokens; kv_block: KV block tokens (0: the same as block;
    64 with block 128 pairs 128-token query blocks with 64-token KV blocks).
    """
    block: int
    seqlens_k: Sequence[int]
    n_q: Sequence[int]
    device: str = "cuda"
    kv_block: int = 0

    def __post_init__(self):
        S = len(self.seqlens_k)
        kb = self.kv_block or self.block
        cu_q = [0]
        cu_qb = [0]
        cu_kb = [0]
        for T, n in zip(self.seqlens_k, self.n_q):
            cu_q.append(cu_q[-1] + int(n))
            cu_qb.append(cu_qb[-1] + _cdiv(int(n), self.block))
            cu_kb.append(cu_kb[-1] + _cdiv(int(T), kb))
        self.num_seqs = S
        self.total_q, self.total_qblocks, self.total_kblocks = cu_q[-1], cu_qb[-1], cu_kb[-1]
        self.max_kblocks = max((_cdiv(int(T), kb) for T in self.seqlens_k), default=0)
        i32 = dict(dtype=torch.int32)
        self.h_cu_seqlens_q = torch.tensor(cu_q, **i32)
        self.h_seqlens_k = torch.tensor([int(t) for t in self.seqlens_k] or [0], **i32)
        self.cu_seqlens_q = self.h_cu_seqlens_q.to(self.device)
        self.seqlens_k_dev = self.h_seqlens_k.to(self.device)
        self.cu_qblocks = torch.tensor(cu_qb, **i32).to(self.device)
        self.cu_kblocks = torch.tensor(cu_kb, **i32).to(self.device)
        self._c = CBatch(S, self.block, self.cu_seqlens_q.data_ptr(), self.seqlens_k_dev.data_ptr(),
                         self.cu_qblocks.data_ptr(), self.cu_kblocks.data_ptr(),
                         ctypes.cast(self.h_cu_seqlens_q.data_ptr(), _i32p),
                         ctypes.cast(self.h_seqlens_k.data_ptr(), _i32p), int(self.kv_block))

    @property
    def c(self) -> CBatch:
        return self._c


@dataclass
class Queries:
    """Packed queries [total_q, Hq, d] (bf16, or uint8 e4m3 codes plus q_scale)."""
    q: torch.Tensor
    q_scale: Optional[torch.Tensor] = None

    @property
    def dtype(self) -> int:
        return FP2_BF16 if self.q.dtype == torch.bfloat16 else FP2_FP8_E4M3

    @property
    def c(self) -> CQ:
        return CQ(self.dtype, self.q.shape[1], self.q.shape[2], _ptr(self.q), _ptr(self.q_scale))


@dataclass
class KVCache:
    """Paged KV cache [num_pages, page_size, Hkv, d] plus page table [S, max_pages]."""
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    page_table: torch.Tensor
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None

    @property
    def dtype(self) -> int:
        return FP2_BF16 if self.k_pages.dtype == torch.bfloat16 else FP2_FP8_E4M3

    @property
    def num_kv_heads(self) -> int:
        return self.k_pages.shape[2]

    @property
    def c(self) -> CKV:
        kp = self.k_pages
        return CKV(self.dtype, kp.shape[2], kp.shape[3], kp.shape[1], kp.shape[0],
                   self.page_table.shape[1], _ptr(kp), _ptr(self.v_pages), _ptr(self.k_scale),
                   _ptr(self.v_scale), _ptr(self.page_table))


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def fp2_block_stats(batch: Batch, kv: KVCache, kbar: torch.Tensor, vbar: torch.Tensor, stream=None):
    b, k = batch.c, kv.c
    _check(_lib.fp2_block_stats(ctypes.byref(b), ctypes.byref(k), _ptr(kbar), _ptr(vbar),
                                _stream(stream)))


def fp2_block_stats_cache_rows(batch: Batch, kv: KVCache) -> int:
    b, k = batch.c, kv.c
    return int(_lib.fp2_block_stats_cache_rows(ctypes.byref(b), ctypes.byref(k)))


def fp2_block_stats_cached(batch: Batch, kv: KVCache, kbar_cache: torch.Tensor, vbar_cache: torch.Tensor,
                           refresh_prefix: bool, stream=None):
    b, k = batch.c, kv.c
    _check(_lib.fp2_block_stats_cached(ctypes.byref(b), ctypes.byref(k), _ptr(kbar_cache), _ptr(vbar_cache),
                                       int(bool(refresh_prefix)), _stream(stream)))


def fp2_gather_block_stats(batch: Batch, kv: KVCache, kbar_cache: torch.Tensor, vbar_cache: torch.Tensor,
                           kbar: torch.Tensor, vbar: torch.Tensor, stream=None):
    b, k = batch.c, kv.c
    _check(_lib.fp2_gather_block_stats(ctypes.byref(b), ctypes.byref(k), _ptr(kbar_cache), _ptr(vbar_cache),
                                       _ptr(kbar), _ptr(vbar), _stream(stream)))


def fp2_plan_workspace_bytes(batch: Batch, num_kv_heads: int) -> int:
    b = batch.c
    return int(_lib.fp2_plan_workspace_bytes(ctypes.byref(b), num_kv_heads))


def fp2_plan_max_nnz(batch: Batch, num_kv_heads: int) -> int:
    b = batch.c
    return int(_lib.fp2_plan_max_nnz(ctypes.byref(b), num_kv_heads))


def fp2_plan_mask(batch: Batch, q: Queries, num_kv_heads: int, kbar: torch.Tensor, tau: float,
                  row_ptr: torch.Tensor, col_idx: torch.Tensor, nnz: torch.Tensor,
                  workspace: torch.Tensor, scores: Optional[torch.Tensor] = None, stream=None):
    b, qc = batch.c, q.c
    _check(_lib.fp2_plan_mask(ctypes.byref(b), ctypes.byref(qc), num_kv_heads, _ptr(kbar),
                              ctypes.c_float(tau), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                              _ptr(nnz), _ptr(scores), _ptr(workspace), workspace.numel(),
                              _stream(stream)))


def fp2_plan_mask_noalloc(batch: Batch, q: Queries, num_kv_heads: int, kbar: torch.Tensor, tau: float,
                          row_ptr: torch.Tensor, col_idx: torch.Tensor, nnz: torch.Tensor,
                          scores: Optional[torch.Tensor] = None, stream=None):
    """fp2_plan_mask with the library's own device scratch as its workspace (no allocation)."""
    b, qc = batch.c, q.c
    _check(_lib.fp2_plan_mask_noalloc(ctypes.byref(b), ctypes.byref(qc), num_kv_heads, _ptr(kbar),
                                      ctypes.c_float(tau), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                                      _ptr(nnz), _ptr(scores), _stream(stream)))


def fp2_stage1_workspace_bytes(batch: Batch, num_kv_heads: int, head_dim: int) -> int:
    b = batch.c
    return int(_lib.fp2_stage1_workspace_bytes(ctypes.byref(b), num_kv_heads, head_dim))


def fp2_stage1(batch: Batch, q: Queries, kv: KVCache, tau: float, kbar: torch.Tensor, vbar: torch.Tensor,
               row_ptr: torch.Tensor, col_idx: torch.Tensor, nnz: torch.Tensor, workspace: torch.Tensor,
               scores: Optional[torch.Tensor] = None, stream=None):
    """Block means, pooled scores, threshold and CSR in one fused pass (fp2_block_stats + fp2_plan_mask)."""
    b, qc, k = batch.c, q.c, kv.c
    _check(_lib.fp2_stage1(ctypes.byref(b), ctypes.byref(qc), ctypes.byref(k), ctypes.c_float(tau), _ptr(kbar),
                           _ptr(vbar), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _ptr(nnz), _ptr(scores),
                           _ptr(workspace), workspace.numel(), _stream(stream)))


def fp2_run_workspace_bytes(batch: Batch, num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: int) -> int:
    """dtype: FP2_BF16 or FP2_FP8_E4M3 (the KV cache's)."""
    b = batch.c
    return int(_lib.fp2_run_workspace_bytes(ctypes.byref(b), num_q_heads, num_kv_heads, head_dim, dtype))


def fp2_prefill_run(batch: Batch, q: Queries, kv: KVCache, row_ptr: torch.Tensor, col_idx: torch.Tensor,
                    kbar: torch.Tensor, vbar: torch.Tensor, mean_correction: bool, out: torch.Tensor,
                    workspace: torch.Tensor, softmax_scale: Optional[float] = None, stream=None,
                    max_chunk_tiles: int = 0):
    """max_chunk_tiles: 0 = the library's choice, > 0 caps a work item's exact tiles, < 0 never splits rows."""
    b, qc, k = batch.c, q.c, kv.c
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.q.shape[2])
    out_dtype = FP2_OUT_F32 if out.dtype == torch.float32 else FP2_OUT_BF16
    _check(_lib.fp2_prefill_run(ctypes.byref(b), ctypes.byref(qc), ctypes.byref(k), _ptr(row_ptr),
                                _ptr(col_idx), _ptr(kbar), _ptr(vbar), int(bool(mean_correction)),
                                ctypes.c_float(softmax_scale), out_dtype, _ptr(out), int(max_chunk_tiles),
                                _ptr(workspace), workspace.numel(), _stream(stream)))


def fp2_debug_bounds_word() -> int:
    """The device error word of a FP2_DEBUG_BOUNDS build (read and cleared; waits for the device).  The
    package's own libfp2.so is a release build: Fp2Error(FP2_ERR_UNSUPPORTED)."""
    w = ctypes.c_uint32(0)
    _check(_lib.fp2_debug_bounds_word(ctypes.byref(w)))
    return int(w.value)


def library_path() -> str:
    return _LIB_PATH


def exported_symbols():
    return {name: hasattr(_lib, name) for name in SYMBOLS}
