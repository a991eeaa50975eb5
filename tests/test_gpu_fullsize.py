"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (bf16 output, mean correction on unless stated).

Per workload: every block mean and every kept-block list is compared with the
float64 oracle (lists bit-exact except near-ties within 1e-5 of the row
threshold, which are counted); attention outputs are compared on sampled
(KV head, query block) rows that the oracle computes one by one on the GPU's
own mask: the last query block of every KV head (largest causal extent), the
first, and seeded random ones.
"""
import dataclasses
import json
import os

import numpy as np
import pytest

import oracle as O
import synth
from helpers import compare_csr, csr_well_formed, decoded_seqs, kv_block, stats_bound
from test_gpu_parity import TOL, check_out

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TAUS = json.load(open(os.path.join(ROOT, "tests", "golden", "tau.json")))


def _rows(w, seed, n_random=2):
    rng = np.random.default_rng(seed)
    rows = []
    for s in range(w.num_seqs):
        nqb = int(w.cu_qblocks[s + 1] - w.cu_qblocks[s])
        if nqb == 0:
            continue
        for g in range(w.cfg.hkv):
            picks = {nqb - 1}
            if g % 4 == 0:
                picks |= {0}
            if g % 2 == 0 and nqb > 2:
                picks |= set(rng.choice(nqb, size=min(n_random, nqb), replace=False).tolist())
            rows += [(s, g, i) for i in sorted(picks)]
    return rows


def run_full(name, corrections=(True,), out_dtype="bf16", kv_blk=0, tau=None):
    import block_sparse_long_blocks_amd as lib
    tau = TAUS[name]["tau"] if tau is None else tau
    cfg = synth.CONFIGS[name]
    if kv_blk:  # e4m3 scales are per page: pages of one KV block
        cfg = dataclasses.replace(cfg, kv_block=kv_blk, page_size=kv_blk if cfg.dtype == "fp8" else cfg.page_size)
    w = synth.make_custom(cfg, tau=tau)
    L = lib.PrefillLayer(*lib.from_workload(w), out_dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16)
    L.stats()
    L.plan(tau)
    torch.cuda.synchronize()
    rp, ci = L.csr_host()
    kb = L.kbar.cpu().numpy().astype(np.float64)
    vb = L.vbar.cpu().numpy().astype(np.float64)
    outs = {}
    for corr in corrections:
        L.attend(corr)
        torch.cuda.synchronize()
        outs[corr] = L.out[:w.total_q].float().cpu().numpy().astype(np.float64)
    del L
    torch.cuda.empty_cache()
    seqs = decoded_seqs(w)
    plan = O.plan_batch(seqs, w.cfg.block, tau, BK=kv_block(w))
    return w, seqs, plan, tau, (rp, ci, kb, vb), outs


def check_stats_and_plan(w, seqs, plan, gpu):
    rp, ci, kb, vb = gpu
    kbound, vbound = stats_bound(w, seqs)
    assert np.all(np.abs(kb[:, :w.total_kblocks] - plan["kbar"]) <= kbound)
    assert np.all(np.abs(vb[:, :w.total_kblocks] - plan["vbar"]) <= vbound)
    csr_well_formed(rp, ci, w)
    rows_bad, flips, ties, hard = compare_csr(rp, ci, plan, w)
    print(f"\n{w.cfg.name}: nnz {rp[-1]} / causal {w.causal_pairs()} "
          f"(density {rp[-1] / w.causal_pairs():.4f}); near-ties {ties}; mask flips {flips} in {rows_bad} rows")
    assert hard == 0, f"{hard} flips outside near-ties"


def check_rows(w, seqs, gpu, out, corr, rows, tol, out_dtype="bf16"):
    rp, ci = gpu[0], gpu[1]
    nqbs = [int(w.cu_qblocks[s + 1] - w.cu_qblocks[s]) for s in range(w.num_seqs)]
    nkbs = [-(-int(t) // kv_block(w)) for t in w.seqlens_k]
    keeps = O.keep_from_csr(rp, ci, w.cfg.hkv, nqbs, nkbs)
    B, G = w.cfg.block, w.cfg.hq // w.cfg.hkv
    worst = 0.0
    for s in sorted({r[0] for r in rows}):
        Q, K, V = seqs[s]
        want = [(g, i) for (ss, g, i) in rows if ss == s]
        ref, _ = O.attend(Q, K, V, keeps[s], B, corr, rows=want, BK=kv_block(w))
        q0 = int(w.cu_seqlens_q[s])
        for g, i in want:
            t0, t1 = i * B, min(i * B + B, Q.shape[0])
            got = out[q0 + t0:q0 + t1, g * G:(g + 1) * G]
            worst = max(worst, check_out(got, ref[t0:t1, g * G:(g + 1) * G], tol, out_dtype))
    return worst


@pytest.mark.parametrize("name", ["llama32k", "qwen_paged", "c128k_bf16", "c128k_fp8"])
def test_fullsize_parity(name):
    w, seqs, plan, tau, gpu, outs = run_full(name)
    check_stats_and_plan(w, seqs, plan, gpu)
    rows = _rows(w, seed=7)
    worst = check_rows(w, seqs, gpu, outs[True], True, rows, TOL[w.cfg.dtype])
    print(f"{name}: {len(rows)} sampled rows, max abs err {worst:.4f} (bf16 output)")


@pytest.mark.parametrize("name", ["c128k_bf16", "c128k_fp8"])
def test_fullsize_decoupled_tiles(name):
    """The 128K data with 128-token query blocks over 64-token KV blocks, on the attention
    kernel's pair tiles (as `bench.py --tiles` times it); tau 3.9 keeps about 5% of the
    64-token causal pairs."""
    print(f"decoupled {name}: generating and running", flush=True)
    w, seqs, plan, tau, gpu, outs = run_full(name, kv_blk=64, tau=3.9)
    check_stats_and_plan(w, seqs, plan, gpu)
    rows = _rows(w, seed=9)
    worst = check_rows(w, seqs, gpu, outs[True], True, rows, TOL[w.cfg.dtype])
    print(f"decoupled {name}: {len(rows)} sampled rows, max abs err {worst:.4f} (bf16 output)")


def test_fullsize_extreme_with_and_without_correction():
    """Extreme sparsity (~2%), fp8: parity with and without correction, and the
    approximation error of each against the oracle's dense attention."""
    w, seqs, plan, tau, gpu, outs = run_full("extreme_fp8", corrections=(True, False))
    check_stats_and_plan(w, seqs, plan, gpu)
    rows = _rows(w, seed=11, n_random=1)
    for corr in (True, False):
        worst = check_rows(w, seqs, gpu, outs[corr], corr, rows, TOL["fp8"])
        print(f"extreme_fp8 correction={corr}: max abs err vs oracle on the same mask {worst:.4f}")
    # approximation error against dense attention on the last query block of each head
    Q, K, V = seqs[0]
    B, G = w.cfg.block, w.cfg.hq // w.cfg.hkv
    nqb = int(w.cu_qblocks[1])
    t0 = (nqb - 1) * B
    dense, _ = O.dense(Q, K, V, query_rows=np.arange(t0, Q.shape[0]))
    err = {c: float(np.abs(outs[c][t0:] - dense).mean()) for c in (True, False)}
    print(f"extreme_fp8 mean abs error vs dense attention (last query block, all heads): "
          f"with correction {err[True]:.4f}, without {err[False]:.4f}")
    assert err[True] < err[False]


@pytest.mark.parametrize("kvb", [128, 64])
def test_max_kv_blocks(kvb):
    """The largest sequence the library accepts: 16,384 KV blocks (2^21 keys in blocks of 128, 2^20
    in blocks of 64 under 128-token query blocks: the kept-block bitmask, the score row of the plan
    and the mean-token list at their limits), two query blocks at the end of the cached prefix,
    4 query / 1 KV head, d 128, bf16, unstructured N(0,1) data with tau for a few percent: block
    means, kept lists and attention (with and without the correction, whose mean-token tiles then
    span all skippable blocks) against the oracle."""
    import block_sparse_long_blocks_amd as lib
    T = 16384 * kvb
    cfg = synth.Config(name="max_kv_blocks", seqlens=(T,), prefixes=(T - 256,), hq=4, hkv=1, d=128, block=128,
                       page_size=128, dtype="bf16", structure="plain", tau=0.008, seed=13,
                       kv_block=0 if kvb == 128 else kvb)
    w = synth.make_custom(cfg)
    assert w.total_kblocks == 16384
    print("\nmax_kv_blocks: inputs generated", flush=True)
    L = lib.PrefillLayer(*lib.from_workload(w), out_dtype=torch.float32)
    L.stats()
    L.plan(cfg.tau)
    torch.cuda.synchronize()
    rp, ci = L.csr_host()
    kb = L.kbar.cpu().numpy().astype(np.float64)
    vb = L.vbar.cpu().numpy().astype(np.float64)
    outs = {}
    for corr in (True, False):
        L.attend(corr)
        torch.cuda.synchronize()
        outs[corr] = L.out[:w.total_q].float().cpu().numpy().astype(np.float64)
    del L
    torch.cuda.empty_cache()
    print("max_kv_blocks: GPU calls done", flush=True)
    seqs = decoded_seqs(w)
    plan = O.plan_batch(seqs, cfg.block, cfg.tau, BK=kvb)
    print("max_kv_blocks: oracle plan done", flush=True)
    check_stats_and_plan(w, seqs, plan, (rp, ci, kb, vb))
    assert 0 < rp[-1] < w.causal_pairs()  # sparse: the correction has skipped blocks to cover
    rows = [(0, 0, 0), (0, 0, 1)]
    for corr in (True, False):
        worst = check_rows(w, seqs, (rp, ci), outs[corr], corr, rows, TOL["bf16"], out_dtype="f32")
        print(f"max_kv_blocks correction={corr}: max abs err {worst:.4f}")
