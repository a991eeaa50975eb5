"""Write tests/golden/tau.json: the threshold tau of each workload whose tau is
given as a target density (about 5% at 128K, about 2% for the extreme case).

Calls only the generator (synth) and the float64 oracle.  Density is the
fraction of causal (query block, KV block, KV head) triples that are kept,
forced blocks included.  tau is the smallest float32 value (by bisection on
the oracle's float32 scores) whose density reaches the target.

Usage: python tests/golden/calibrate_tau.py [config ...]
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tau.json")


def scores_of(w):
    cfg = w.cfg
    B, G = cfg.block, cfg.hq // cfg.hkv
    res = []
    for s in range(w.num_seqs):
        Q, K, _ = O.decode_sequence(cfg.dtype, B, w.q_seq(s), w.q_scale_seq(s), w.k_seq[s],
                                    w.k_scale_seq[s], w.v_seq[s], w.v_scale_seq[s])
        P = int(w.seqlens_k[s] - w.n_q[s])
        kbar = O.block_means(K, B)
        qbar = O.pooled_query_means(Q, B, G)
        del Q, K
        res.append((O.block_scores(qbar, kbar, P, B, cfg.d), P))
    return res


def density(scores, B, tau):
    kept = causal = 0
    for s, P in scores:
        keep, _, _ = O.select_blocks(s, P, B, tau)
        kept += int(keep.sum())
        causal += int(np.isfinite(s).sum())
    return kept / causal


def main(names):
    table = json.load(open(OUT)) if os.path.exists(OUT) else {}
    for name in names:
        cfg = synth.CONFIGS[name]
        w = synth.make(name, tau=0.0)
        sc = scores_of(w)
        del w
        if cfg.target_density is None:
            table[name] = {"tau": cfg.tau, "density": density(sc, cfg.block, cfg.tau),
                           "target_density": None}
        else:
            lo, hi = np.float32(0.0), np.float32(64.0)
            for _ in range(60):
                mid = np.float32(0.5 * (lo + hi))
                if mid == lo or mid == hi:
                    break
                if density(sc, cfg.block, float(mid)) >= cfg.target_density:
                    hi = mid
                else:
                    lo = mid
            table[name] = {"tau": float(hi), "density": density(sc, cfg.block, float(hi)),
                           "target_density": cfg.target_density}
        print(name, table[name], flush=True)
        json.dump(table, open(OUT, "w"), indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["tiny", "llama32k", "qwen_paged", "c128k_bf16", "c128k_fp8",
                          "extreme_fp8"])
