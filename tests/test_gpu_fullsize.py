"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (bf16 output, mean correction on unless stated; every run is
repeated with float32 output).

Per workload: every block mean and every kept-block list is compared with the
float64 oracle (lists bit-exact except near-ties within 1e-5 of the row
threshold, which are counted); attention outputs are compared on sampled
(KV head, query block) rows that the oracle computes one by one on the GPU's
own mask: the two CSR rows with the most kept blocks (the longest online
softmax), the last query block of every KV head (largest causal extent), the
first, and seeded random ones.  A 128-token chunk after a 130,944-token
cached prefix checks every row with the heavy rows split into chunks and
merged (the default) and unsplit.

Each test adds its counts and worst errors to a table written at the end of
the module to gpurun_out/parity_fullsize.md (nnz, near-ties, mask flips, rows
checked, max-abs error for bf16 and f32 outputs).
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
REPORT = []


@pytest.fixture(scope="module", autouse=True)
def _write_report():
    yield
    if not REPORT:
        return
    out = os.path.join(ROOT, "gpurun_out")
    os.makedirs(out, exist_ok=True)
    cols = ["case", "correction", "nnz", "causal", "density", "near_ties", "mask_flips", "rows_flipped",
            "rows_checked", "max_err_bf16", "max_err_f32", "tol"]
    with open(os.path.join(out, "parity_fullsize.md"), "w") as f:
        f.write("| " + " | ".join(cols) + " |\n|" + "---|" * len(cols) + "\n")
        for r in REPORT:
            f.write("| " + " | ".join(str(r.get(c, "")) for c in cols) + " |\n")
    with open(os.path.join(out, "parity_fullsize.json"), "w") as f:
        json.dump(REPORT, f, indent=1)


def _heaviest(w, rp, k=2):
    """(sequence, KV head, query block) of the k CSR rows with the most kept blocks."""
    counts = np.diff(rp)
    out = []
    for r in np.argsort(-counts, kind="stable")[:k]:
        g, qb = divmod(int(r), w.total_qblocks)
        s = int(np.searchsorted(w.cu_qblocks, qb, side="right")) - 1
        out.append((s, g, qb - int(w.cu_qblocks[s])))
    return out


def _rows(w, seed, rp, n_random=2):
    rng = np.random.default_rng(seed)
    rows = set(_heaviest(w, rp))
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
            rows |= {(s, g, i) for i in picks}
    return sorted(rows)


def run_layer(w, tau, corrections=(True,), chunk_caps=(0,)):
    """The three calls on the GPU: CSR, block means, and the outputs of
    fp2_prefill_run for each correction and chunk cap, in bf16 and in f32."""
    import block_sparse_long_blocks_amd as lib
    L = lib.PrefillLayer(*lib.from_workload(w))
    L.stats()
    L.plan(tau)
    torch.cuda.synchronize()
    rp, ci = L.csr_host()
    kb = L.kbar.cpu().numpy().astype(np.float64)
    vb = L.vbar.cpu().numpy().astype(np.float64)
    # the fused stage-1 pass gives the same means and CSR, bit for bit
    L.kbar.fill_(float("nan"))
    L.vbar.fill_(float("nan"))
    L.col_idx.fill_(-1)
    L.stage1(tau)
    torch.cuda.synchronize()
    rp2, ci2 = L.csr_host()
    assert np.array_equal(rp, rp2) and np.array_equal(ci, ci2)
    assert np.array_equal(L.kbar.cpu().numpy().astype(np.float64), kb)
    assert np.array_equal(L.vbar.cpu().numpy().astype(np.float64), vb)
    outs = {}
    bf16_out = L.out
    f32_out = torch.empty(L.out.shape, dtype=torch.float32, device=L.out.device)
    for corr in corrections:
        for cap in chunk_caps:
            L.max_chunk_tiles = cap
            for od, buf in (("bf16", bf16_out), ("f32", f32_out)):
                L.out = buf
                L.attend(corr)
                torch.cuda.synchronize()
                outs[(corr, cap, od)] = buf[:w.total_q].float().cpu().numpy().astype(np.float64)
    del L, bf16_out, f32_out
    torch.cuda.empty_cache()
    return (rp, ci, kb, vb), outs


def run_full(name, corrections=(True,), kv_blk=0, tau=None):
    tau = TAUS[name]["tau"] if tau is None else tau
    cfg = synth.CONFIGS[name]
    if kv_blk:  # e4m3 scales are per page: pages of one KV block
        cfg = dataclasses.replace(cfg, kv_block=kv_blk, page_size=kv_blk if cfg.dtype == "fp8" else cfg.page_size)
    w = synth.make_custom(cfg, tau=tau)
    gpu, outs = run_layer(w, tau, corrections)
    seqs = decoded_seqs(w)
    plan = O.plan_batch(seqs, w.cfg.block, tau, BK=kv_block(w))
    return w, seqs, plan, tau, gpu, outs


def check_stats_and_plan(w, seqs, plan, gpu):
    """Block means and kept lists; returns the counts the report lists."""
    rp, ci, kb, vb = gpu
    kbound, vbound = stats_bound(w, seqs)
    assert np.all(np.abs(kb[:, :w.total_kblocks] - plan["kbar"]) <= kbound)
    assert np.all(np.abs(vb[:, :w.total_kblocks] - plan["vbar"]) <= vbound)
    csr_well_formed(rp, ci, w)
    rows_bad, flips, ties, hard = compare_csr(rp, ci, plan, w)
    print(f"\n{w.cfg.name}: nnz {rp[-1]} / causal {w.causal_pairs()} "
          f"(density {rp[-1] / w.causal_pairs():.4f}); near-ties {ties}; mask flips {flips} in {rows_bad} rows")
    assert hard == 0, f"{hard} flips outside near-ties"
    return dict(nnz=int(rp[-1]), causal=int(w.causal_pairs()), density=round(float(rp[-1] / w.causal_pairs()), 5),
                near_ties=int(ties), mask_flips=int(flips), rows_flipped=int(rows_bad))


def check_rows(w, seqs, gpu, outs, corr, rows, tol):
    """outs: {out dtype: output}; the oracle's rows once, every output against them.
    Returns {out dtype: max abs error}."""
    rp, ci = gpu[0], gpu[1]
    nqbs = [int(w.cu_qblocks[s + 1] - w.cu_qblocks[s]) for s in range(w.num_seqs)]
    nkbs = [-(-int(t) // kv_block(w)) for t in w.seqlens_k]
    keeps = O.keep_from_csr(rp, ci, w.cfg.hkv, nqbs, nkbs)
    B, G = w.cfg.block, w.cfg.hq // w.cfg.hkv
    worst = {od: 0.0 for od in outs}
    for s in sorted({r[0] for r in rows}):
        Q, K, V = seqs[s]
        want = [(g, i) for (ss, g, i) in rows if ss == s]
        ref, _ = O.attend(Q, K, V, keeps[s], B, corr, rows=want, BK=kv_block(w))
        q0 = int(w.cu_seqlens_q[s])
        for g, i in want:
            t0, t1 = i * B, min(i * B + B, Q.shape[0])
            for od, out in outs.items():
                got = out[q0 + t0:q0 + t1, g * G:(g + 1) * G]
                worst[od] = max(worst[od], check_out(got, ref[t0:t1, g * G:(g + 1) * G], tol, od))
    return worst


def _report(case, corr, counts, rows, worst, tol):
    REPORT.append(dict(case=case, correction=corr, **counts, rows_checked=len(rows),
                       max_err_bf16=round(worst["bf16"], 5), max_err_f32=round(worst["f32"], 5), tol=tol))
    print(f"{case} correction={corr}: {len(rows)} rows checked, max abs err bf16 {worst['bf16']:.4f} "
          f"f32 {worst['f32']:.4f}")


def _dtype_outs(outs, corr, cap=0):
    return {od: outs[(corr, cap, od)] for od in ("bf16", "f32")}


@pytest.mark.parametrize("name", ["llama32k", "qwen_paged", "c128k_bf16", "c128k_fp8"])
def test_fullsize_parity(name):
    w, seqs, plan, tau, gpu, outs = run_full(name)
    counts = check_stats_and_plan(w, seqs, plan, gpu)
    rows = _rows(w, 7, gpu[0])
    tol = TOL[w.cfg.dtype]
    _report(name, True, counts, rows, check_rows(w, seqs, gpu, _dtype_outs(outs, True), True, rows, tol), tol)


@pytest.mark.parametrize("name", ["c128k_bf16", "c128k_fp8"])
def test_fullsize_decoupled_tiles(name):
    """The 128K data with 128-token query blocks over 64-token KV blocks, on the attention
    kernel's pair tiles (as `bench.py --tiles` times it); tau 3.9 keeps about 5% of the
    64-token causal pairs."""
    print(f"decoupled {name}: generating and running", flush=True)
    w, seqs, plan, tau, gpu, outs = run_full(name, kv_blk=64, tau=3.9)
    counts = check_stats_and_plan(w, seqs, plan, gpu)
    rows = _rows(w, 9, gpu[0])
    tol = TOL[w.cfg.dtype]
    _report(f"{name} (128 x 64 tiles)", True, counts, rows,
            check_rows(w, seqs, gpu, _dtype_outs(outs, True), True, rows, tol), tol)


def test_fullsize_extreme_with_and_without_correction():
    """Extreme sparsity (~2%), fp8: parity with and without correction, and the
    approximation error of each against the oracle's dense attention."""
    w, seqs, plan, tau, gpu, outs = run_full("extreme_fp8", corrections=(True, False))
    counts = check_stats_and_plan(w, seqs, plan, gpu)
    rows = _rows(w, 11, gpu[0], n_random=1)
    for corr in (True, False):
        _report("extreme_fp8", corr, counts, rows,
                check_rows(w, seqs, gpu, _dtype_outs(outs, corr), corr, rows, TOL["fp8"]), TOL["fp8"])
    # approximation error against dense attention on the last query block of each head
    Q, K, V = seqs[0]
    B = w.cfg.block
    nqb = int(w.cu_qblocks[1])
    t0 = (nqb - 1) * B
    dense, _ = O.dense(Q, K, V, query_rows=np.arange(t0, Q.shape[0]))
    err = {c: float(np.abs(outs[(c, 0, "f32")][t0:] - dense).mean()) for c in (True, False)}
    print(f"extreme_fp8 mean abs error vs dense attention (last query block, all heads): "
          f"with correction {err[True]:.4f}, without {err[False]:.4f}")
    assert err[True] < err[False]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_fullsize_chunk_after_prefix_split_rows(dtype):
    """One 128-token query chunk after a 130,944-token cached prefix (8 CSR rows of up to 1024
    blocks, 32 query / 8 KV heads, band + sinks data, tau 4.5: rows keep from 4 to about 700
    blocks, the rest corrected).  With the library's chunk size the heavy rows run as several
    work items merged by the combine kernel; with splitting off each row is one item.  Every
    row of both runs, with and without correction, against the oracle; the two runs must
    differ in their last bits (the split path really ran)."""
    cfg = synth.Config(name=f"chunk_after_128k_{dtype}", seqlens=(131072,), prefixes=(131072 - 128,), hq=32, hkv=8,
                       d=128, block=128, page_size=128, dtype=dtype, structure="band_sinks", tau=4.5, seed=7)
    w = synth.make_custom(cfg)
    print(f"\nchunk_after_128k_{dtype}: inputs generated", flush=True)
    gpu, outs = run_layer(w, cfg.tau, corrections=(True, False), chunk_caps=(0, -1))
    seqs = decoded_seqs(w)
    plan = O.plan_batch(seqs, cfg.block, cfg.tau)
    counts = check_stats_and_plan(w, seqs, plan, gpu)
    tiles = np.diff(gpu[0])
    assert tiles.max() > 64 and tiles.min() < 64  # heavy rows beside light ones
    rows = [(0, g, 0) for g in range(cfg.hkv)]
    tol = TOL[w.cfg.dtype]
    for corr in (True, False):
        for cap, label in ((0, "split"), (-1, "unsplit")):
            worst = check_rows(w, seqs, gpu, _dtype_outs(outs, corr, cap), corr, rows, tol)
            _report(f"chunk after 128K prefix {dtype} ({label})", corr, counts, rows, worst, tol)
        assert not np.array_equal(outs[(corr, 0, "f32")], outs[(corr, -1, "f32")])


@pytest.mark.parametrize("kvb", [128, 64])
def test_max_kv_blocks(kvb):
    """The largest sequence the library accepts: 16,384 KV blocks (2^21 keys in blocks of 128, 2^20
    in blocks of 64 under 128-token query blocks: the kept-block bitmask, the score row of the plan
    and the mean-token list at their limits), two query blocks at the end of the cached prefix,
    4 query / 1 KV head, d 128, bf16, unstructured N(0,1) data with tau for a few percent: block
    means, kept lists and attention (with and without the correction, whose mean-token tiles then
    span all skippable blocks) against the oracle."""
    T = 16384 * kvb
    cfg = synth.Config(name="max_kv_blocks", seqlens=(T,), prefixes=(T - 256,), hq=4, hkv=1, d=128, block=128,
                       page_size=128, dtype="bf16", structure="plain", tau=0.008, seed=13,
                       kv_block=0 if kvb == 128 else kvb)
    w = synth.make_custom(cfg)
    assert w.total_kblocks == 16384
    print("\nmax_kv_blocks: inputs generated", flush=True)
    gpu, outs = run_layer(w, cfg.tau, corrections=(True, False))
    print("max_kv_blocks: GPU calls done", flush=True)
    seqs = decoded_seqs(w)
    plan = O.plan_batch(seqs, cfg.block, cfg.tau, BK=kvb)
    print("max_kv_blocks: oracle plan done", flush=True)
    counts = check_stats_and_plan(w, seqs, plan, gpu)
    assert 0 < gpu[0][-1] < w.causal_pairs()  # sparse: the correction has skipped blocks to cover
    rows = [(0, 0, 0), (0, 0, 1)]
    for corr in (True, False):
        _report(f"max KV blocks ({kvb}-token)", corr, counts, rows,
                check_rows(w, seqs, gpu, _dtype_outs(outs, corr), corr, rows, TOL["bf16"]), TOL["bf16"])
