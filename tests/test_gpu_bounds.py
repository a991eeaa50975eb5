"""The FP2_DEBUG_BOUNDS build (libfp2_bounds.so): page ids and the CSR handed to
fp2_prefill_run are checked on the device ahead of the kernels that read them,
a violation sets a bit of the error word (include/fp2.h, fp2_debug_bounds_word)
and those kernels return at once.

The corrupted inputs here stay inside their buffers even if read (the bad page
id names a page the K/V tensors hold beyond the declared page count, the bad
CSR entries name blocks of the row's own sequence, the bad row pointer ends
inside the column buffer), so each test is safe whatever the checks do; the
tests check that the word reports them."""
import ctypes
import os

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BOUNDS_LIB = os.path.join(ROOT, "block_sparse_long_blocks_amd", "libfp2_bounds.so")
PAGE_BIT, CSR_ENTRY_BIT, CSR_ROW_BIT = 1, 2, 4

# d = 128, B = 128 (the d128 kernel path), page 64, three sequences with cached prefixes
CFG = synth.Config(name="bounds_varlen", seqlens=(640, 300, 1152), prefixes=(256, 0, 896), hq=8, hkv=2, d=128,
                   block=128, page_size=64, dtype="bf16", structure="band_sinks", tau=1.0, seed=21,
                   shuffle_pages=True)


def _bounds():
    import block_sparse_long_blocks_amd as lib
    assert os.path.exists(BOUNDS_LIB), "build it: python block_sparse_long_blocks_amd/build.py --debug-bounds"
    dl = ctypes.CDLL(BOUNDS_LIB)
    rel = lib._binding._lib
    for name in ("fp2_block_stats", "fp2_plan_mask", "fp2_prefill_run", "fp2_last_error",
                 "fp2_debug_bounds_word"):
        getattr(dl, name).argtypes = getattr(rel, name).argtypes
        getattr(dl, name).restype = getattr(rel, name).restype
    return lib, dl


def _word(dl):
    w = ctypes.c_uint32(0)
    st = dl.fp2_debug_bounds_word(ctypes.byref(w))
    assert st == 0, (st, dl.fp2_last_error())
    return int(w.value)


class Layer:
    """The three calls through the bounds build, on buffers of the package's PrefillLayer."""

    def __init__(self, lib, dl, w, extra_pages=0):
        import torch
        self.torch, self.lib, self.dl = torch, lib, dl
        batch, q, kv = lib.from_workload(w)
        if extra_pages:  # pages the tensors hold beyond the count the descriptor declares
            pad = lambda t: torch.cat([t, t[:extra_pages]])  # noqa: E731
            kv = lib.KVCache(pad(kv.k_pages), pad(kv.v_pages), kv.page_table.clone(), kv.k_scale, kv.v_scale)
        self.L = lib.PrefillLayer(batch, q, kv, out_dtype=torch.float32)
        # room past the plan's largest CSR, so that a row pointer past it still ends inside the buffer
        self.L.col_idx = torch.zeros(self.L.col_idx.numel() + 1024, dtype=torch.int32, device=q.q.device)
        self.num_pages = kv.k_pages.shape[0] - extra_pages
        self.stream = torch.cuda.current_stream().cuda_stream

    def ckv(self):
        c = self.L.kv.c
        c.num_pages = self.num_pages
        return c

    def stats(self):
        L, b, k = self.L, self.L.batch.c, self.ckv()
        return self.dl.fp2_block_stats(ctypes.byref(b), ctypes.byref(k), L.kbar.data_ptr(), L.vbar.data_ptr(),
                                       self.stream)

    def plan(self, tau):
        L, b, qc = self.L, self.L.batch.c, self.L.q.c
        return self.dl.fp2_plan_mask(ctypes.byref(b), ctypes.byref(qc), L.kv.num_kv_heads, L.kbar.data_ptr(),
                                     ctypes.c_float(tau), L.row_ptr.data_ptr(), L.col_idx.data_ptr(),
                                     L.col_idx.numel(), L.nnz.data_ptr(), None, L.plan_ws.data_ptr(),
                                     L.plan_ws.numel(), self.stream)

    def run(self, correction=True):
        L, b, qc, k = self.L, self.L.batch.c, self.L.q.c, self.ckv()
        return self.dl.fp2_prefill_run(ctypes.byref(b), ctypes.byref(qc), ctypes.byref(k), L.row_ptr.data_ptr(),
                                       L.col_idx.data_ptr(), L.kbar.data_ptr(), L.vbar.data_ptr(), int(correction),
                                       ctypes.c_float(1.0 / np.sqrt(CFG.d)), 1, L.out.data_ptr(), 0,
                                       L.run_ws.data_ptr(), L.run_ws.numel(), self.stream)


@pytest.mark.gpu
def test_bounds_build_clean_inputs_match_release():
    """Clean inputs: the word stays 0 and the three calls give the release library's results bit for bit."""
    lib, dl = _bounds()
    w = synth.make_custom(CFG, tau=1.0)
    t = Layer(lib, dl, w)
    assert _word(dl) == 0
    assert t.stats() == 0 and t.plan(1.0) == 0 and t.run() == 0
    t.torch.cuda.synchronize()
    assert _word(dl) == 0
    got = (t.L.kbar.clone(), t.L.row_ptr.clone(), t.L.col_idx.clone(), t.L.out.clone())
    ref = lib.PrefillLayer(t.L.batch, t.L.q, t.L.kv, out_dtype=t.torch.float32)
    ref(1.0, True)
    t.torch.cuda.synchronize()
    nnz = int(ref.nnz.item())
    assert t.torch.equal(got[0], ref.kbar) and t.torch.equal(got[1], ref.row_ptr)
    assert t.torch.equal(got[2][:nnz], ref.col_idx[:nnz])
    assert t.torch.equal(got[3][:ref.batch.total_q], ref.out[:ref.batch.total_q])


@pytest.mark.gpu
def test_bounds_build_reports_a_page_id_past_the_page_count():
    """A page id equal to the declared page count (the tensors hold that page: reading it would be safe)
    sets bit 1 in fp2_block_stats and in fp2_prefill_run; the word is cleared by reading it."""
    lib, dl = _bounds()
    w = synth.make_custom(CFG, tau=1.0)
    t = Layer(lib, dl, w, extra_pages=2)
    assert t.stats() == 0 and t.plan(1.0) == 0
    t.torch.cuda.synchronize()
    assert _word(dl) == 0
    good = t.L.kv.page_table.clone()
    t.L.kv.page_table[1, 2] = t.num_pages  # sequence 1 uses pages 0..4 (300 tokens, page 64)
    assert t.stats() == 0
    t.torch.cuda.synchronize()
    assert _word(dl) == PAGE_BIT
    assert _word(dl) == 0
    assert t.run() == 0
    t.torch.cuda.synchronize()
    assert _word(dl) == PAGE_BIT
    t.L.kv.page_table.copy_(good)
    assert t.stats() == 0 and t.run() == 0
    t.torch.cuda.synchronize()
    assert _word(dl) == 0


@pytest.mark.gpu
def test_bounds_build_reports_bad_csr_rows():
    """fp2_prefill_run's CSR: entries out of order, a row without block 0, a row running past its own
    diagonal block (to a block of the same sequence) set bit 2; row pointers out of order, or past the
    causal pair count, set bit 4.  A clean CSR afterwards leaves the word 0."""
    lib, dl = _bounds()
    w = synth.make_custom(CFG, tau=1.0)
    t = Layer(lib, dl, w)
    assert t.stats() == 0 and t.plan(1.0) == 0
    t.torch.cuda.synchronize()
    assert _word(dl) == 0
    rp0, ci0 = t.L.row_ptr.clone(), t.L.col_idx.clone()
    rp = rp0.cpu().numpy()
    # query blocks per sequence: 3, 3, 2; row 6 (KV head 0) = sequence 2's first query block, whose last
    # diagonal block is 7 of the sequence's 9 (1152 tokens, 896 cached)
    r = 6
    b, e = int(rp[r]), int(rp[r + 1])
    assert e - b >= 3 and int(ci0[b]) == 0 and int(ci0[e - 1]) == 7

    def expect(bit, edit, also=0):
        """the word is bit, or bit plus the bits in also (a neighbouring row can break as well)"""
        t.L.row_ptr.copy_(rp0)
        t.L.col_idx.copy_(ci0)
        edit()
        assert t.run() == 0
        t.torch.cuda.synchronize()
        word = _word(dl)
        assert word & ~also == bit, word

    def swap():
        a0, a1 = t.L.col_idx[b + 1].item(), t.L.col_idx[b + 2].item()
        t.L.col_idx[b + 1], t.L.col_idx[b + 2] = a1, a0
    expect(CSR_ENTRY_BIT, swap)
    expect(CSR_ENTRY_BIT, lambda: t.L.col_idx.__setitem__(b, 1))          # block 0 missing
    expect(CSR_ENTRY_BIT, lambda: t.L.col_idx.__setitem__(e - 1, 8))      # past the diagonal (block 8 exists)
    # row pointers out of order (the next row then starts inside the one before: its entries break too)
    expect(CSR_ROW_BIT, lambda: t.L.row_ptr.__setitem__(r + 1, b - 1), also=CSR_ENTRY_BIT)
    cap = int(lib.fp2_plan_max_nnz(t.L.batch, t.L.kv.num_kv_heads))
    assert t.L.col_idx.numel() > cap + 1
    expect(CSR_ROW_BIT, lambda: t.L.row_ptr.__setitem__(-1, cap + 1))  # past the causal pair count
    expect(0, lambda: None)
