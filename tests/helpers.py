"""Glue shared by the GPU tests: decoded oracle inputs of a generated workload,
and comparisons in the terms the parity bar is stated in."""
import numpy as np

import oracle as O


def decoded_seqs(w):
    cfg = w.cfg
    return [O.decode_sequence(cfg.dtype, cfg.block, w.q_seq(s), w.q_scale_seq(s), w.k_seq[s],
                              w.k_scale_seq[s], w.v_seq[s], w.v_scale_seq[s], kv_block=cfg.kv_block or None)
            for s in range(w.num_seqs)]


def kv_block(w):
    """KV block tokens of a workload (its query block unless set apart)."""
    return w.cfg.kv_block or w.cfg.block


def stats_bound(w, seqs):
    """Per-element bound on |float32 block mean - exact mean|: a float32 sum of n
    terms errs by at most (n-1)*2^-24*sum|x| (any order), the scale product and
    the division add 2^-24 each, relative."""
    B = kv_block(w)
    ks, vs = [], []
    for (_, K, V) in seqs:
        T = K.shape[0]
        for j in range(-(-T // B)):
            blk = slice(j * B, min(j * B + B, T))
            n = blk.stop - blk.start
            ks.append(((n + 2) * 2.0 ** -24) * np.abs(K[blk]).mean(axis=0))
            vs.append(((n + 2) * 2.0 ** -24) * np.abs(V[blk]).mean(axis=0))
    kb = np.stack(ks).transpose(1, 0, 2)
    vb = np.stack(vs).transpose(1, 0, 2)
    return kb + 1e-30, vb + 1e-30


def compare_csr(gpu_rp, gpu_ci, plan, w):
    """Row-by-row comparison of the GPU CSR with the oracle's plan.

    A mismatch is allowed only where the oracle flags a near-tie (score within
    1e-5 of its row threshold).  Returns (rows_mismatched, entries_flipped,
    near_ties_total, flips_not_near_tie)."""
    Hkv = w.cfg.hkv
    nqbs = plan["nqb"]
    total_qb = sum(nqbs)
    rp, ci = plan["row_ptr"], plan["col_idx"]
    assert gpu_rp.shape == rp.shape
    rows_bad = flips = hard = 0
    ties = sum(int(t.sum()) for t in plan["near_tie"])
    base = 0
    for si, nqb in enumerate(nqbs):
        tie = plan["near_tie"][si]
        for g in range(Hkv):
            for i in range(nqb):
                r = g * total_qb + base + i
                a = set(gpu_ci[gpu_rp[r]:gpu_rp[r + 1]].tolist())
                b = set(ci[rp[r]:rp[r + 1]].tolist())
                if a != b:
                    rows_bad += 1
                    for j in a ^ b:
                        flips += 1
                        if not tie[g, i, j]:
                            hard += 1
        base += nqb
    return rows_bad, flips, ties, hard


def csr_well_formed(rp, ci, w):
    B = w.cfg.block
    Hkv = w.cfg.hkv
    KB = kv_block(w)
    total_qb = w.total_qblocks
    assert rp[0] == 0 and np.all(np.diff(rp) > 0)
    for g in range(Hkv):
        for s in range(w.num_seqs):
            P = int(w.seqlens_k[s] - w.n_q[s])
            for i in range(int(w.cu_qblocks[s + 1] - w.cu_qblocks[s])):
                r = g * total_qb + int(w.cu_qblocks[s]) + i
                row = ci[rp[r]:rp[r + 1]]
                lo, hi = O.diag_range(P, int(w.n_q[s]), i, B, KB)
                assert row[0] == 0 and row[-1] == hi and np.all(np.diff(row) > 0), (g, s, i)
                assert set(range(lo, hi + 1)) <= set(row.tolist()), (g, s, i)
