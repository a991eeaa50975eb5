"""GPU parity on seeded random small batches: block and head sizes, KV block, dtype, page size (shuffled
or not), GQA group, sequence count, lengths and cached prefixes, score structure and threshold are drawn
from the values the library accepts (a cached prefix is a whole number of query blocks), so that
combinations the named cases do not spell out also meet the bar: kept-block lists equal to the oracle's
except at near-ties, and the attention output within 1e-2 (bf16) / 4e-2 (e4m3) of the float64 oracle run
on the GPU's own mask, with and without the mean correction."""
import math

import numpy as np
import pytest

import oracle as O
import synth
from helpers import compare_csr, csr_well_formed, decoded_seqs, kv_block
from test_gpu_parity import TOL, check_out, layer

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# (head size, query block, KV block or 0 for the query block's): every kernel layout; the first 16
# cases take each with both dtypes, the rest draw them
LAYOUTS = [(128, 128, 0), (128, 128, 64), (128, 64, 0), (64, 128, 0), (64, 64, 0), (64, 128, 64), (128, 128, 0),
           (128, 128, 64)]
N_CASES = 24


def random_config(i):
    r = np.random.default_rng(7100 + i)
    if i < 2 * len(LAYOUTS):
        d, B, kvb = LAYOUTS[i % len(LAYOUTS)]
        dtype = ("bf16", "fp8")[i // len(LAYOUTS)]
    else:
        d, B, kvb = LAYOUTS[int(r.integers(len(LAYOUTS)))]
        dtype = str(r.choice(["bf16", "fp8"]))
    KB = kvb or B
    page = KB if dtype == "fp8" else int(r.choice([8, 16, 24, 32, 64, 128, 256]))
    hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 8]))
    seqlens, prefixes = [], []
    for _ in range(int(r.integers(1, 4))):
        T = int(r.integers(1, 1500))
        P = B * int(r.integers(0, (T - 1) // B + 1)) if r.random() < 0.5 else 0  # a whole number of query blocks
        seqlens.append(T)
        prefixes.append(P)
    structure = str(r.choice(["band_sinks", "hot", "slash", "plain"]))
    tau = float(r.choice([0.0, 0.5, 1.0, 3.0]))
    cfg = synth.Config(name=f"random{i}", seqlens=tuple(seqlens), prefixes=tuple(prefixes), hq=hkv * G, hkv=hkv,
                       d=d, block=B, page_size=page, dtype=dtype, structure=structure, tau=1.0, seed=300 + i,
                       shuffle_pages=bool(r.random() < 0.7), kv_block=kvb)
    return cfg, tau


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_batch_parity(i):
    cfg, tau = random_config(i)
    w = synth.make_custom(cfg, tau=1.0)
    seqs = decoded_seqs(w)
    print(f"case {i}: {cfg}, tau {tau}", flush=True)
    L = layer(w)
    nqbs = [int(w.cu_qblocks[s + 1] - w.cu_qblocks[s]) for s in range(w.num_seqs)]
    nkbs = [-(-int(t) // kv_block(w)) for t in w.seqlens_k]
    plan = O.plan_batch(seqs, w.cfg.block, tau, BK=kv_block(w))
    for corr in (True, False):
        out = L(tau, corr)
        torch.cuda.synchronize()
        rp, ci = L.csr_host()
        csr_well_formed(rp, ci, w)
        _, flips, ties, hard = compare_csr(rp, ci, plan, w)
        assert hard == 0, f"{hard} mask flips outside near-ties ({flips} flips, {ties} ties)"
        keeps = O.keep_from_csr(rp, ci, w.cfg.hkv, nqbs, nkbs)
        ref = O.run_batch(seqs, w.cfg.block, tau, corr, keeps=keeps, BK=kv_block(w))["out"]
        got = out[:w.total_q].float().cpu().numpy().astype(np.float64)
        check_out(got, ref, TOL[w.cfg.dtype], "bf16")
        assert math.isfinite(float(np.abs(got).max()))
