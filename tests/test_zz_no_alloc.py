"""fp2_plan_mask_noalloc (the allocation-free plan call, for callers that cannot
allocate device memory) against fp2_plan_mask on the same inputs: row_ptr, the
kept columns, nnz and the float32 scores must be identical, on two calls in a
row where the second batch is smaller than the first (the library's scratch
keeps the first call's contents), at several thresholds."""
import math

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _cfg(name, seqlens, prefixes, hq, hkv, page, seed):
    return synth.Config(name=name, seqlens=tuple(seqlens), prefixes=tuple(prefixes), hq=hq, hkv=hkv, d=128,
                        block=128, page_size=page, dtype="bf16", structure="band_sinks", tau=3.0, seed=seed,
                        shuffle_pages=True)


BIG = _cfg("noalloc_big", (32768, 9000, 20480), (0, 128, 16384), 32, 8, 64, 21)
SMALL = _cfg("noalloc_small", (640, 300), (256, 0), 8, 2, 128, 22)


def _plans(L, lib, tau):
    """(row_ptr, col_idx[:nnz], nnz, scores) from fp2_plan_mask and from fp2_plan_mask_noalloc."""
    out = []
    for noalloc in (False, True):
        rp = torch.full_like(L.row_ptr, -7)
        ci = torch.full_like(L.col_idx, -7)
        nnz = torch.full_like(L.nnz, -7)
        sc = torch.full_like(L.scores, float("nan"))
        if noalloc:
            lib.fp2_plan_mask_noalloc(L.batch, L.q, L.kv.num_kv_heads, L.kbar, tau, rp, ci, nnz, sc)
        else:
            lib.fp2_plan_mask(L.batch, L.q, L.kv.num_kv_heads, L.kbar, tau, rp, ci, nnz, L.plan_ws, sc)
        torch.cuda.synchronize()
        n = int(nnz.item())
        out.append((rp.cpu(), ci[:n].cpu(), n, sc.cpu()))
    return out


def test_noalloc_plan_matches_plan_mask():
    import block_sparse_long_blocks_amd as lib
    for cfg in (BIG, SMALL):  # the second call's batch is smaller than the first's
        w = synth.make_custom(cfg)
        L = lib.PrefillLayer(*lib.from_workload(w), with_scores=True)
        L.stats()
        need = lib.fp2_plan_workspace_bytes(L.batch, w.cfg.hkv)
        print(f"\n{cfg.name}: plan workspace {need} bytes", flush=True)
        for tau in (cfg.tau, 0.5, math.inf, -1.0):
            (rp0, ci0, n0, sc0), (rp1, ci1, n1, sc1) = _plans(L, lib, tau)
            assert n0 == n1 == int(rp0[-1]) > 0
            assert torch.equal(rp0, rp1)
            assert torch.equal(ci0, ci1)
            np.testing.assert_array_equal(sc0.numpy(), sc1.numpy())
            print(f"  tau={tau}: nnz {n1}, identical", flush=True)
        del L
        torch.cuda.empty_cache()
