"""GPU parity of the three C-ABI calls against the float64 oracle (small and
ragged shapes that the oracle finishes in seconds but that span several tiles).

Bar: block means within a rigorous float32 summation bound; kept-block lists
identical except where the oracle flags a near-tie (score within 1e-5 of the
row threshold); attention output within 1e-2 (bf16) / 4e-2 (fp8) max-abs of
the oracle run on the GPU's own mask.
"""
import math

import numpy as np
import pytest

import oracle as O
import synth
from helpers import compare_csr, csr_well_formed, decoded_seqs, kv_block, stats_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = {"bf16": 1e-2, "fp8": 4e-2}


def bf16_half_ulp(x):
    """Half a bfloat16 ulp at |x|: the rounding every bf16 output carries."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 0.5 * 2.0 ** (np.floor(np.log2(a)) - 7)


def check_out(got, ref, tol, out_dtype, extra=0.0):
    """fp32 output: max-abs <= tol (+ extra).  bf16 output: <= tol plus the
    output's own half-ulp rounding (which alone exceeds 1e-2 once |O| >= 4)."""
    err = np.abs(got - ref)
    bound = (tol if out_dtype == "f32" else tol + bf16_half_ulp(ref)) + extra
    bad = err > bound
    assert np.all(np.isfinite(got))
    assert not bad.any(), (f"{int(bad.sum())} outputs over the bound; max err {err.max():.5f}, "
                           f"worst |O| {np.abs(ref[np.unravel_index(np.argmax(err - bound), err.shape)]):.3f}")
    return float(err.max())


def _cfg(name, seqlens, prefixes, hq, hkv, d, B, page, dtype="bf16", structure="band_sinks",
         shuffle=True, seed=11, kv_block=0):
    return synth.Config(name=name, seqlens=tuple(seqlens), prefixes=tuple(prefixes), hq=hq, hkv=hkv, d=d,
                        block=B, page_size=page, dtype=dtype, structure=structure, tau=1.0, seed=seed,
                        shuffle_pages=shuffle, kv_block=kv_block)


SMALL = {
    "tiny": synth.CONFIGS["tiny"],
    "varlen_p64": _cfg("varlen_p64", (640, 300, 1152), (256, 0, 896), 8, 2, 128, 128, 64),
    "d64_b128_p16": _cfg("d64_b128_p16", (512, 384), (128, 256), 8, 4, 64, 128, 16),
    "d128_b64_g8": _cfg("d128_b64_g8", (768,), (192,), 16, 2, 128, 64, 32),
    "single_token": _cfg("single_token", (257, 1), (256, 0), 4, 2, 128, 128, 128, structure="plain"),
    "fp8_varlen": _cfg("fp8_varlen", (1024, 512), (0, 256), 8, 2, 128, 128, 128, dtype="fp8", shuffle=True),
    # bf16 d=128 B=128 with pages that split a 16-row DMA group (per-lane page lookups), one query
    # head per KV head (half of each workgroup idle) and eight (four slices per query block)
    "d128_p24_g1": _cfg("d128_p24_g1", (900, 260), (128, 0), 2, 2, 128, 128, 24),
    "d128_p8_g8": _cfg("d128_p8_g8", (700,), (384,), 16, 2, 128, 128, 8),
    # chunked prefill: one query block after a 6016-token cached prefix (4 CSR rows of up to 48
    # blocks, so the default work-item builder splits them), bf16 and e4m3
    "chunk_after_prefix": _cfg("chunk_after_prefix", (6144,), (6016,), 8, 4, 128, 128, 128),
    "chunk_after_prefix_fp8": _cfg("chunk_after_prefix_fp8", (6144,), (6016,), 8, 4, 128, 128, 128,
                                   dtype="fp8"),
    # pages that hold two blocks each (B = 64, page 128)
    "d128_b64_p128": _cfg("d128_b64_p128", (700, 300), (256, 0), 8, 2, 128, 64, 128),
    # 128-token query blocks over 64-token KV blocks: ragged last query blocks whose diagonal is one
    # KV block (44 and 60 tokens), prefixes, shuffled pages smaller than, equal to and larger than
    # the KV block, e4m3 (page = KV block), d = 64 and eight query heads per KV head
    "dec_varlen": _cfg("dec_varlen", (640, 300, 1152), (256, 0, 896), 8, 2, 128, 128, 32, kv_block=64),
    "dec_fp8": _cfg("dec_fp8", (1024, 512), (0, 256), 8, 2, 128, 128, 64, dtype="fp8", kv_block=64),
    "dec_d64_p128": _cfg("dec_d64_p128", (512, 384), (128, 256), 8, 4, 64, 128, 128, kv_block=64),
    "dec_g8": _cfg("dec_g8", (700,), (384,), 16, 2, 128, 128, 64, kv_block=64),
    # the same on the DMA kernel's pair tiles (d = 128): one query block after a long prefix (rows
    # split into chunks; e4m3: masked pair tiles that hold prefix blocks), and pages of 24 tokens
    # (per-lane DMA sources) with G = 1
    "dec_chunk": _cfg("dec_chunk", (6144,), (6016,), 8, 4, 128, 128, 128, kv_block=64),
    "dec_p24_g1": _cfg("dec_p24_g1", (900, 260), (128, 0), 2, 2, 128, 128, 24, kv_block=64),
    "dec_chunk_fp8": _cfg("dec_chunk_fp8", (6144,), (6016,), 8, 4, 128, 128, 64, dtype="fp8", kv_block=64),
}
TAUS = {"tiny": (0.0, 0.005, 0.01, 0.02, 2.0), "varlen_p64": (0.0, 0.5, 3.0),
        "d64_b128_p16": (0.3, 3.0), "d128_b64_g8": (0.2, 2.0), "single_token": (0.0, 1.0),
        "fp8_varlen": (0.0, 0.5, 3.0), "d128_p24_g1": (0.0, 1.0), "d128_p8_g8": (0.0, 1.0),
        "chunk_after_prefix": (0.5, 1e9), "chunk_after_prefix_fp8": (0.5, 1e9), "d128_b64_p128": (0.0, 1.0),
        "dec_varlen": (0.0, 0.5, 3.0), "dec_fp8": (0.0, 0.5, 3.0), "dec_d64_p128": (0.3, 3.0), "dec_g8": (0.0, 1.0),
        "dec_chunk": (0.5, 1e9), "dec_p24_g1": (0.0, 1.0), "dec_chunk_fp8": (0.5, 1e9)}

_cache = {}


def workload(name, pad_fill="zero"):
    key = (name, pad_fill)
    if key not in _cache:
        w = synth.make_custom(SMALL[name], tau=1.0, pad_fill=pad_fill)
        _cache[key] = (w, decoded_seqs(w))
    return _cache[key]


def layer(w, with_scores=False, out_dtype="bf16"):
    import block_sparse_long_blocks_amd as lib
    return lib.PrefillLayer(*lib.from_workload(w), with_scores=with_scores,
                            out_dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16)


@pytest.mark.parametrize("name", list(SMALL))
def test_block_stats_parity(name):
    w, seqs = workload(name)
    L = layer(w)
    L.stats()
    torch.cuda.synchronize()
    plan = O.plan_batch(seqs, w.cfg.block, 1.0, BK=kv_block(w))
    kb_bound, vb_bound = stats_bound(w, seqs)
    kb = L.kbar.cpu().numpy().astype(np.float64)
    vb = L.vbar.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(kb - plan["kbar"]) <= kb_bound)
    assert np.all(np.abs(vb - plan["vbar"]) <= vb_bound)


@pytest.mark.parametrize("name", list(SMALL))
def test_plan_parity(name):
    w, seqs = workload(name)
    L = layer(w, with_scores=True)
    L.stats()
    for tau in TAUS[name] + (math.inf, -1.0):
        L.plan(tau)
        torch.cuda.synchronize()
        rp, ci = L.csr_host()
        plan = O.plan_batch(seqs, w.cfg.block, tau, BK=kv_block(w))
        csr_well_formed(rp, ci, w)
        rows_bad, flips, ties, hard = compare_csr(rp, ci, plan, w)
        assert hard == 0, f"tau={tau}: {hard} mask flips outside near-ties ({flips} flips, {ties} ties)"
        assert int(L.nnz.item()) == rp[-1]
        # float32 scores agree with the oracle's float32 scores to ~ulp level
        sc = L.scores.cpu().numpy()
        off = 0
        for s, S in enumerate(plan["s"]):
            nqb = S.shape[1]
            for g in range(w.cfg.hkv):
                gs = sc[g * w.total_qblocks + off: g * w.total_qblocks + off + nqb, :S.shape[2]]
                fin = np.isfinite(S[g])
                assert np.array_equal(np.isfinite(gs), fin)
                assert np.max(np.abs(gs[fin] - S[g][fin]), initial=0.0) <= 2e-6
            off += nqb
        if tau == math.inf:
            assert rp[-1] == w.causal_pairs()
        if tau == -1.0:  # only the forced blocks: block 0 and the diagonal run
            assert rp[-1] == sum(len({0} | set(range(lo, hi + 1)))
                                 for s in range(w.num_seqs)
                                 for i in range(int(w.cu_qblocks[s + 1] - w.cu_qblocks[s]))
                                 for lo, hi in [O.diag_range(int(w.seqlens_k[s] - w.n_q[s]), int(w.n_q[s]), i,
                                                             w.cfg.block, kv_block(w))]) * w.cfg.hkv


@pytest.mark.parametrize("name", list(SMALL))
def test_stage1_fused_matches_separate_calls(name):
    """fp2_stage1 (one pass over K, V and Q, then the selection) gives fp2_block_stats' block means and
    fp2_plan_mask's CSR, nnz and float32 scores bit for bit, at every threshold (so the oracle parity
    of the separate calls carries over)."""
    w, _ = workload(name)
    L = layer(w, with_scores=True)
    for tau in TAUS[name] + (math.inf, -1.0):
        L.stats()
        L.plan(tau)
        torch.cuda.synchronize()
        ref = [x.clone() for x in (L.kbar, L.vbar, L.row_ptr, L.nnz, L.scores)]
        n = int(L.nnz.item())
        ref_ci = L.col_idx[:n].clone()
        for x in (L.kbar, L.vbar, L.scores):
            x.fill_(float("nan"))
        L.row_ptr.fill_(-5)
        L.col_idx.fill_(-5)
        L.nnz.fill_(-5)
        L.stage1(tau)
        torch.cuda.synchronize()
        got = (L.kbar, L.vbar, L.row_ptr, L.nnz, L.scores)
        for a, b in zip(got[:2], ref[:2]):
            assert torch.equal(a[:, :w.total_kblocks], b[:, :w.total_kblocks])
        assert torch.equal(got[2], ref[2]) and torch.equal(got[3], ref[3])
        assert torch.equal(L.col_idx[:n], ref_ci)
        assert torch.equal(torch.nan_to_num(got[4], nan=7.0), torch.nan_to_num(ref[4], nan=7.0))


def _attention_case(name, tau, corr, pad_fill="zero", out_dtype="bf16", max_chunk_tiles=0):
    w, seqs = workload(name, pad_fill)
    L = layer(w, out_dtype=out_dtype)
    L.max_chunk_tiles = max_chunk_tiles
    out = L(tau, corr)
    torch.cuda.synchronize()
    rp, ci = L.csr_host()
    nqbs = [int(w.cu_qblocks[s + 1] - w.cu_qblocks[s]) for s in range(w.num_seqs)]
    nkbs = [-(-int(t) // kv_block(w)) for t in w.seqlens_k]
    keeps = O.keep_from_csr(rp, ci, w.cfg.hkv, nqbs, nkbs)
    ref = O.run_batch(seqs, w.cfg.block, tau, corr, keeps=keeps, BK=kv_block(w))["out"]
    got = out[:w.total_q].float().cpu().numpy().astype(np.float64)
    return got, ref, w, L


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("corr", [True, False])
@pytest.mark.parametrize("name", list(SMALL))
def test_attention_parity(name, corr, out_dtype):
    for tau in TAUS[name]:
        got, ref, w, _ = _attention_case(name, tau, corr, out_dtype=out_dtype)
        check_out(got, ref, TOL[w.cfg.dtype], out_dtype)


@pytest.mark.parametrize("name", ["varlen_p64", "fp8_varlen", "chunk_after_prefix", "d128_b64_p128", "d64_b128_p16",
                                  "dec_varlen", "dec_d64_p128"])
def test_cached_block_stats(name):
    """The block means kept in a cache beside the KV pages: with refresh_prefix the gathered
    kbar / vbar equal fp2_block_stats bit for bit; without it, the rows of blocks holding new
    tokens are computed again (planted NaNs vanish) and the rows of cached-prefix blocks are left
    as they were (a planted sentinel comes back from the gather)."""
    import block_sparse_long_blocks_amd as lib
    w, _ = workload(name)
    L = layer(w)
    L.stats()
    rows = lib.fp2_block_stats_cache_rows(L.batch, L.kv)
    B, ps = kv_block(w), w.cfg.page_size
    bpp = max(1, ps // B)
    assert rows == w.k_pages.shape[0] * bpp
    kc = torch.full((rows, w.cfg.hkv, w.cfg.d), float("nan"), device="cuda")
    vc = kc.clone()
    lib.fp2_block_stats_cached(L.batch, L.kv, kc, vc, True)
    kb, vb = torch.empty_like(L.kbar), torch.empty_like(L.vbar)
    lib.fp2_gather_block_stats(L.batch, L.kv, kc, vc, kb, vb)
    torch.cuda.synchronize()
    assert torch.equal(kb, L.kbar) and torch.equal(vb, L.vbar)
    prefix, new = [], []
    for s in range(w.num_seqs):
        T, n = int(w.seqlens_k[s]), int(w.n_q[s])
        for J in range(-(-T // B)):
            row = int(w.page_table[s, J * B // ps]) * bpp + J % bpp
            (prefix if J < (T - n) // B else new).append((int(w.cu_kblocks[s]) + J, row))
    assert prefix and new
    kc[[r for _, r in new]] = float("nan")
    vc[[r for _, r in new]] = float("nan")
    kc[[r for _, r in prefix]] = 7.0
    vc[[r for _, r in prefix]] = -3.0
    lib.fp2_block_stats_cached(L.batch, L.kv, kc, vc, False)
    lib.fp2_gather_block_stats(L.batch, L.kv, kc, vc, kb, vb)
    torch.cuda.synchronize()
    nk = [k for k, _ in new]
    pk = [k for k, _ in prefix]
    assert torch.equal(kb[:, nk], L.kbar[:, nk]) and torch.equal(vb[:, nk], L.vbar[:, nk])
    assert bool((kb[:, pk] == 7.0).all()) and bool((vb[:, pk] == -3.0).all())


@pytest.mark.parametrize("corr", [True, False])
@pytest.mark.parametrize("name", ["varlen_p64", "fp8_varlen", "dec_varlen", "dec_fp8"])
def test_split_rows_match_oracle(name, corr):
    """Rows whose exact tiles are cut into chunks (fp2_prefill_run's
    max_chunk_tiles caps the chunk; the batch bounds it below by its tiles over its extra-item budget,
    4 tiles here) run as separate work items whose float32 partials (O, the
    reference max, the row sum) a combine kernel merges: the result stays
    within the bar of the oracle, and differs in its last bits from the
    unsplit run (so the split path really ran)."""
    for tau in (math.inf, 0.5):
        whole, ref, w, L = _attention_case(name, tau, corr, out_dtype="f32")
        rp, _ = L.csr_host()
        extra_cap = min(256, -(-w.causal_pairs() // 4))
        # exact tiles per row: one per kept block, or one per two with 64-token KV blocks
        tiles = np.diff(rp) if kv_block(w) == w.cfg.block else -(-np.diff(rp) // 2)
        chunk = max(2, -(-int(tiles.sum()) // extra_cap))
        if tau != math.inf and int(tiles.max()) <= chunk:
            continue  # no row long enough to split at this threshold
        assert int(tiles.max()) > chunk  # some row is split
        split, ref2, _, _ = _attention_case(name, tau, corr, out_dtype="f32", max_chunk_tiles=2)
        assert np.array_equal(ref, ref2)
        check_out(split, ref, TOL[w.cfg.dtype], "f32")
        check_out(whole, ref, TOL[w.cfg.dtype], "f32")
        assert not np.array_equal(split, whole)


@pytest.mark.parametrize("name", ["tiny", "varlen_p64", "d128_b64_g8", "dec_varlen", "dec_fp8"])
def test_dense_mode_is_causal_attention(name):
    got, _, w, _ = _attention_case(name, math.inf, True, out_dtype="f32")
    _, seqs = workload(name)
    ref = np.concatenate([O.dense(Q, K, V)[0] for Q, K, V in seqs], axis=0)
    check_out(got, ref, TOL[w.cfg.dtype], "f32")


@pytest.mark.parametrize("name", ["varlen_p64", "d64_b128_p16", "fp8_varlen", "dec_varlen", "dec_p24_g1"])
def test_pad_slots_are_never_read(name):
    """Unused slots of each last page hold NaN; results must equal the zero-padded run."""
    got_z, _, w, Lz = _attention_case(name, 0.5, True, "zero")
    got_n, _, _, Ln = _attention_case(name, 0.5, True, "nan")
    assert np.all(np.isfinite(got_n))
    np.testing.assert_array_equal(got_z, got_n)
    np.testing.assert_array_equal(Lz.kbar.cpu().numpy(), Ln.kbar.cpu().numpy())


def test_repeat_runs_bit_identical():
    w, _ = workload("varlen_p64")
    L = layer(w)
    a = L(0.5, True).clone()
    rp_a, ci_a = L.csr_host()
    b = L(0.5, True).clone()
    rp_b, ci_b = L.csr_host()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    np.testing.assert_array_equal(rp_a, rp_b)
    np.testing.assert_array_equal(ci_a, ci_b)


def test_concurrent_calls_on_two_streams():
    """fp2_prefill_run runs its V^T preparation on a second stream of the library's, forked from and
    joined to the caller's stream by events that all calls on a device share (under a host lock): two
    host threads driving two layers on two streams at once get, every time, what each layer gives alone."""
    import threading
    layers = [layer(workload(n)[0]) for n in ("varlen_p64", "fp8_varlen")]
    ref = [L(0.5, True).clone() for L in layers]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in layers]
    outs = [[] for _ in layers]
    errors = []

    def drive(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(16):
                    outs[i].append(layers[i](0.5, True).clone())
            streams[i].synchronize()
        except Exception as e:  # reported below, in the test's own thread
            errors.append(e)

    threads = [threading.Thread(target=drive, args=(i,)) for i in range(len(layers))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(len(layers)):
        assert len(outs[i]) == 16
        for o in outs[i]:
            assert torch.equal(o, ref[i])


def test_page_shuffle_and_varlen_metamorphic():
    """Shuffled pages == identity pages (bit-identical); a varlen batch == each sequence alone."""
    cfg = SMALL["varlen_p64"]
    import dataclasses
    w_shuf = synth.make_custom(cfg, tau=0.5)
    w_id = synth.make_custom(dataclasses.replace(cfg, shuffle_pages=False), tau=0.5)
    o_shuf = layer(w_shuf)(0.5, True).clone()
    o_id = layer(w_id)(0.5, True).clone()
    torch.cuda.synchronize()
    assert torch.equal(o_shuf, o_id)
    off = 0
    for s in range(w_id.num_seqs):
        one_cfg = dataclasses.replace(cfg, seqlens=(cfg.seqlens[s],), prefixes=(cfg.prefixes[s],),
                                      shuffle_pages=False)
        w1 = synth.make_custom(one_cfg, tau=0.5, seq_seeds=(cfg.seed + 1000 * s,))
        o1 = layer(w1)(0.5, True).clone()
        torch.cuda.synchronize()
        n = int(w1.n_q[0])
        assert torch.equal(o1[:n], o_id[off:off + n])
        off += n


def test_empty_batch_and_empty_sequence():
    import block_sparse_long_blocks_amd as lib
    # a batch whose middle sequence has no new queries (prefix only)
    cfg = _cfg("with_empty", (384, 256, 200), (128, 256, 0), 4, 2, 128, 128, 64)
    w = synth.make_custom(cfg, tau=0.5)
    seqs = decoded_seqs(w)
    L = layer(w)
    out = L(0.5, True)
    torch.cuda.synchronize()
    rp, ci = L.csr_host()
    nqbs = [int(w.cu_qblocks[s + 1] - w.cu_qblocks[s]) for s in range(w.num_seqs)]
    nkbs = [-(-int(t) // 128) for t in w.seqlens_k]
    keeps = O.keep_from_csr(rp, ci, 2, nqbs, nkbs)
    ref = O.run_batch(seqs, 128, 0.5, True, keeps=keeps)["out"]
    check_out(out[:w.total_q].float().cpu().numpy().astype(np.float64), ref, 1e-2, "bf16")
    # an empty batch: every call is a no-op that succeeds
    b = lib.Batch(128, [], [], device="cuda")
    q = lib.Queries(torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda"))
    kv = lib.KVCache(torch.zeros((1, 128, 2, 128), dtype=torch.bfloat16, device="cuda"),
                     torch.zeros((1, 128, 2, 128), dtype=torch.bfloat16, device="cuda"),
                     torch.zeros((1, 1), dtype=torch.int32, device="cuda"))
    Le = lib.PrefillLayer(b, q, kv)
    Le(1.0, True)
    torch.cuda.synchronize()
    assert int(Le.nnz.item()) == 0 and int(Le.row_ptr[0].item()) == 0


@pytest.mark.parametrize("kvb", [128, 64])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_reference_max_refresh_in_every_tile_kind(dtype, kvb):
    """Scores that climb by far more than 64 log2 units along the keys (about 2 per
    key), and one 128-token span (keys 256-383) lying far above every other, under a
    hand-made mask (block 0, the block at query block I//2's start and the diagonal
    run per query block I): the running reference max must be raised after the first
    step inside exact tiles, diagonal tiles and mean-token tiles (the high span
    skipped, its mean tokens on top), and the result must still match the oracle on
    the same mask.  One or two keys carry each row here, so a row sum that did not
    add exactly the bf16-rounded probabilities PV weighs V with would show whole
    (up to 2^-9 max|v|); the bar is the plain 1e-2 (4e-2 for e4m3), and the
    measured worst error is printed.  e4m3: one scale per KV block and head (query block and
    head for Q).  kvb = 64: 64-token KV blocks under 128-token query blocks, two to a
    tile, each half with its own K scale; rows of three or four entries give full and
    lone-entry pair tiles."""
    import block_sparse_long_blocks_amd as lib
    rng = np.random.default_rng(5)
    B, d, hq, hkv, T = 128, 128, 8, 2, 1024
    r = B // kvb
    pos = np.arange(T, dtype=np.float64)
    q = 1.0 + 0.25 * rng.standard_normal((T, hq, d))
    k = (0.125 * pos)[:, None, None] + 0.25 * rng.standard_normal((T, hkv, d))
    k[2 * B:3 * B] += 200.0
    v = rng.standard_normal((T, hkv, d))
    nq, nb = T // B, T // kvb
    page_table = np.arange(nb, dtype=np.int32)[None, :]
    if dtype == "bf16":
        qc, kc, vc = (synth.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))
        qs = ks = vs = None
    else:
        qc, qs = synth.quantize_blocks_e4m3(q.astype(np.float32), B)
        (kc, ks), (vc, vs) = (synth.quantize_blocks_e4m3(x.astype(np.float32), kvb) for x in (k, v))
    batch, queries, kv = lib.from_arrays(B, [T], [T], qc, qs, kc.reshape(nb, kvb, hkv, d),
                                         vc.reshape(nb, kvb, hkv, d), page_table, k_scale=ks, v_scale=vs,
                                         kv_block=0 if kvb == B else kvb)
    keep = np.zeros((hkv, nq, nb), dtype=bool)
    for i in range(nq):
        keep[:, i, [0, r * (i // 2)] + list(range(r * i, r * i + r))] = True
    rp = [0]
    ci = []
    for g in range(hkv):
        for i in range(nq):
            cols = np.nonzero(keep[g, i])[0]
            ci.extend(cols.tolist())
            rp.append(len(ci))
    dec = O.decode_sequence(dtype, B, qc, qs, kc, ks, vc, vs, kv_block=kvb)
    for corr in (True, False):
        L = lib.PrefillLayer(batch, queries, kv, out_dtype=torch.float32)
        L.stats()
        L.row_ptr.copy_(torch.tensor(rp, dtype=torch.int32))
        L.col_idx[:len(ci)].copy_(torch.tensor(ci, dtype=torch.int32))
        L.attend(corr)
        torch.cuda.synchronize()
        got = L.out[:T].cpu().numpy().astype(np.float64)
        ref = O.run_batch([tuple(dec)], B, 0.0, corr, keeps=[keep], BK=kvb)["out"]
        worst = check_out(got, ref, TOL[dtype], "f32")
        print(f"\nrefresh stress {dtype} kvb={kvb} correction={corr}: max abs err {worst:.4f} (bar {TOL[dtype]})")
