"""Pins for the float64 oracle: it is checked against things other than itself.

- pure-Python brute force on tiny inputs (every step re-derived per query);
- tau = +inf reduces to textbook causal softmax attention (torch float64 SDPA);
- mean correction is exact when the keys of every block are identical;
- constant V gives constant output; output is linear in V;
- Jensen: lse(sparse) <= lse(corrected) <= lse(dense);
- threshold special cases (tau < 0, tau = 0, nesting in tau) and CSR shape;
- varlen batch == per-sequence runs; prefix+chunk rows == tail of a full run;
- exact block means on small integers (fractions).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

torch = pytest.importorskip("torch")


def _rand_seq(rng, T, n, Hq, Hkv, d, scale=1.0):
    Q = rng.standard_normal((n, Hq, d)) * scale
    K = rng.standard_normal((T, Hkv, d)) * scale
    V = rng.standard_normal((T, Hkv, d))
    return Q, K, V


# ---------------------------------------------------------------------------
# brute force: every step per query in plain Python
# ---------------------------------------------------------------------------

def brute_force(Q, K, V, B, tau, correction, BK=None):
    """B: query block size; BK: KV block size (B unless given)."""
    BK = B if BK is None else BK
    n, Hq, d = Q.shape
    T, Hkv, _ = K.shape
    G = Hq // Hkv
    P = T - n
    c = 1.0 / math.sqrt(d)
    nkb = -(-T // BK)
    nqb = -(-n // B)

    def mean_rows(rows):
        return [sum(r[e] for r in rows) / len(rows) for e in range(d)]

    kbar = [[mean_rows([K[t, g] for t in range(j * BK, min(j * BK + BK, T))]) for g in range(Hkv)]
            for j in range(nkb)]
    vbar = [[mean_rows([V[t, g] for t in range(j * BK, min(j * BK + BK, T))]) for g in range(Hkv)]
            for j in range(nkb)]
    qbar = [[mean_rows([Q[t, h] for t in range(i * B, min(i * B + B, n))
                        for h in range(g * G, g * G + G)]) for g in range(Hkv)]
            for i in range(nqb)]
    out = np.zeros((n, Hq, d))
    keep_all = {}
    for g in range(Hkv):
        for i in range(nqb):
            # the query block's own positions; its diagonal = the KV blocks
            # that hold one of them; causal blocks = those with a visible key
            own = set(range(P + i * B, P + min(i * B + B, n)))
            diag = [j for j in range(nkb) if own & set(range(j * BK, min(j * BK + BK, T)))]
            causal = [j for j in range(nkb) if j * BK <= max(own)]
            s = []
            for j in causal:
                dot = sum(float(np.float32(qbar[i][g][e])) * float(np.float32(kbar[j][g][e]))
                          for e in range(d))
                s.append(np.float32(dot * c))
            thr = np.float32(max(s) - np.float32(tau))
            keep = [j for j in causal if s[j] >= thr or j == 0 or j in diag]
            keep_all[(g, i)] = keep
            for t in range(i * B, min(i * B + B, n)):
                p = P + t
                for h in range(g * G, g * G + G):
                    terms = []
                    for j in keep:
                        for u in range(j * BK, min(j * BK + BK, T)):
                            if u <= p:
                                lg = sum(Q[t, h, e] * K[u, g, e] for e in range(d)) * c
                                terms.append((lg, 1.0, V[u, g]))
                    if correction:
                        for j in range(1, min(diag)):
                            if j not in keep:
                                lg = sum(Q[t, h, e] * kbar[j][g][e] for e in range(d)) * c
                                terms.append((lg, float(BK), vbar[j][g]))
                    m = max(lg for lg, _, _ in terms)
                    den = sum(w * math.exp(lg - m) for lg, w, _ in terms)
                    for e in range(d):
                        out[t, h, e] = sum(w * math.exp(lg - m) * v[e] for lg, w, v in terms) / den
    return out, keep_all


@pytest.mark.parametrize("T,n,Hq,Hkv,d,B,tau,corr,seed", [
    (96, 96, 2, 1, 8, 16, 0.3, True, 1),
    (128, 64, 4, 1, 8, 32, 0.2, True, 2),     # prefix of 64
    (112, 48, 4, 2, 16, 16, 0.25, True, 3),   # prefix 64, ragged last blocks
    (80, 80, 4, 4, 8, 16, 0.4, False, 4),     # G = 1
    (100, 68, 2, 1, 8, 16, 0.1, True, 5),     # prefix 32, T not a multiple of B
])
def test_oracle_matches_brute_force(T, n, Hq, Hkv, d, B, tau, corr, seed):
    rng = np.random.default_rng(seed)
    Q, K, V = _rand_seq(rng, T, n, Hq, Hkv, d)
    # block-level offsets spread the pooled scores so the threshold drops blocks
    for j in range(-(-T // B)):
        K[j * B:(j + 1) * B] += rng.standard_normal((1, Hkv, d)) * 0.7
    for i in range(-(-n // B)):
        Q[i * B:(i + 1) * B] += rng.standard_normal((1, Hq, d)) * 0.7
    res = O.run_batch([(Q, K, V)], B, tau, corr)
    ref, keep_ref = brute_force(Q, K, V, B, tau, corr)
    keep = res["keep"][0]
    nskipped = 0
    for (g, i), js in keep_ref.items():
        assert list(np.nonzero(keep[g, i])[0]) == js, (g, i)
        nskipped += (T - n) // B + i + 1 - len(js)
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)
    if tau < 1.0 and T >= 96:
        assert nskipped > 0, "case should exercise skipped blocks"


@pytest.mark.parametrize("T,n,Hq,Hkv,d,B,BK,tau,corr,seed", [
    (128, 128, 2, 1, 8, 32, 16, 0.3, True, 11),
    (160, 96, 4, 2, 8, 32, 16, 0.2, True, 12),    # prefix 64, ragged: last query block 1 KV block
    (150, 86, 4, 1, 8, 32, 16, 0.25, True, 13),   # prefix 64, T and n ragged inside a KV block
    (176, 112, 2, 2, 8, 64, 16, 0.3, False, 14),  # four KV blocks per query block
])
def test_oracle_matches_brute_force_decoupled(T, n, Hq, Hkv, d, B, BK, tau, corr, seed):
    """Query blocks of B tokens scored against KV blocks of BK < B tokens."""
    rng = np.random.default_rng(seed)
    Q, K, V = _rand_seq(rng, T, n, Hq, Hkv, d)
    for j in range(-(-T // BK)):
        K[j * BK:(j + 1) * BK] += rng.standard_normal((1, Hkv, d)) * 0.7
    for i in range(-(-n // B)):
        Q[i * B:(i + 1) * B] += rng.standard_normal((1, Hq, d)) * 0.7
    res = O.run_batch([(Q, K, V)], B, tau, corr, BK=BK)
    ref, keep_ref = brute_force(Q, K, V, B, tau, corr, BK=BK)
    keep = res["keep"][0]
    nskipped = 0
    for (g, i), js in keep_ref.items():
        assert list(np.nonzero(keep[g, i])[0]) == js, (g, i)
        nskipped += O.diag_range(T - n, n, i, B, BK)[1] + 1 - len(js)
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)
    assert nskipped > 0, "case should exercise skipped blocks"


def test_decoupled_scores_average_to_coupled():
    """Linearity of the means: a full 2BK-token KV block's mean is the average
    of its two BK halves, so its score is the average of theirs."""
    rng = np.random.default_rng(21)
    T, n, Hq, Hkv, d, B = 256, 256, 4, 2, 16, 32
    Q, K, V = _rand_seq(rng, T, n, Hq, Hkv, d)
    G = Hq // Hkv
    qbar = O.pooled_query_means(Q, B, G)
    s32 = O.block_scores(qbar, O.block_means(K, B), 0, B, d)
    s16 = O.block_scores(qbar, O.block_means(K, B // 2), 0, B, d, n, B // 2)
    for i in range(n // B):
        for J in range(i + 1):
            np.testing.assert_allclose(s32[:, i, J], 0.5 * (s16[:, i, 2 * J] + s16[:, i, 2 * J + 1]),
                                       rtol=0, atol=1e-5)
        assert np.all(np.isinf(s16[:, i, 2 * i + 2:]))


@pytest.mark.parametrize("corr", [False, True])
def test_tau_inf_is_dense_attention_decoupled(corr):
    rng = np.random.default_rng(31)
    T, n = 200, 136
    Q, K, V = _rand_seq(rng, T, n, 4, 2, 8)
    res = O.run_batch([(Q, K, V)], 32, float("inf"), corr, BK=16)
    np.testing.assert_allclose(res["out"], _torch_sdpa(Q, K, V), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# tau = +inf reduces to dense causal attention (torch float64 SDPA)
# ---------------------------------------------------------------------------

def _torch_sdpa(Q, K, V):
    n, Hq, d = Q.shape
    T, Hkv, _ = K.shape
    G = Hq // Hkv
    P = T - n
    q = torch.from_numpy(Q).permute(1, 0, 2)                     # [Hq, n, d]
    k = torch.from_numpy(K).repeat_interleave(G, dim=1).permute(1, 0, 2)
    v = torch.from_numpy(V).repeat_interleave(G, dim=1).permute(1, 0, 2)
    mask = torch.arange(T)[None, :] <= (P + torch.arange(n))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("T,n,Hq,Hkv,d,B", [(256, 256, 4, 2, 16, 32), (320, 128, 4, 1, 16, 64),
                                          (200, 72, 8, 2, 8, 32)])
@pytest.mark.parametrize("corr", [False, True])
def test_tau_inf_is_dense_attention(T, n, Hq, Hkv, d, B, corr):
    rng = np.random.default_rng(T + n)
    Q, K, V = _rand_seq(rng, T, n, Hq, Hkv, d)
    res = O.run_batch([(Q, K, V)], B, float("inf"), corr)
    assert all(k.sum() == sum((T - n) // B + i + 1 for i in range(k.shape[1])) * k.shape[0]
               for k in res["keep"])
    ref = _torch_sdpa(Q, K, V)
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)
    dense, _ = O.dense(Q, K, V)
    np.testing.assert_allclose(dense, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# mean correction: exact with identical keys per block; Jensen bounds
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("P", [0, 64])
def test_correction_exact_for_identical_block_keys(P):
    rng = np.random.default_rng(7 + P)
    B, Hq, Hkv, d, n = 16, 4, 2, 16, 192
    T = P + n
    Q, K, V = _rand_seq(rng, T, n, Hq, Hkv, d)
    nkb = -(-T // B)
    for j in range(nkb):
        K[j * B:(j + 1) * B] = rng.standard_normal((1, Hkv, d))
    for tau in (0.0, 0.05, 0.5):
        res = O.run_batch([(Q, K, V)], B, tau, True)
        causal = sum(P // B + i + 1 for i in range(-(-n // B))) * Hkv
        skipped = causal - sum(int(k.sum()) for k in res["keep"])
        dense, _ = O.dense(Q, K, V)
        np.testing.assert_allclose(res["out"], dense, rtol=0, atol=1e-12)
        if tau == 0.0:
            assert skipped > 0


def test_jensen_and_constant_v_and_linearity():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, d, T, n = 16, 4, 2, 16, 256, 192
    Q, K, V = _rand_seq(rng, T, n, Hq, Hkv, d)
    plan = O.plan_batch([(Q, K, V)], B, 0.1)
    keep = plan["keep"][0]
    _, lse_s = O.attend(Q, K, V, keep, B, correction=False)
    Oc, lse_c = O.attend(Q, K, V, keep, B, correction=True)
    _, lse_d = O.dense(Q, K, V)
    assert np.all(lse_s <= lse_c + 1e-12)
    assert np.all(lse_c <= lse_d + 1e-12)
    assert np.any(lse_c > lse_s + 1e-6)
    # constant V -> constant output, with and without correction
    Vc = np.full_like(V, 0.625)
    for corr in (False, True):
        Oo, _ = O.attend(Q, K, Vc, keep, B, correction=corr)
        np.testing.assert_allclose(Oo, 0.625, rtol=0, atol=1e-13)
    # linear in V for a fixed mask
    V2 = rng.standard_normal(V.shape)
    a, b = 0.7, -1.3
    O1, _ = O.attend(Q, K, V, keep, B, True)
    O2, _ = O.attend(Q, K, V2, keep, B, True)
    O12, _ = O.attend(Q, K, a * V + b * V2, keep, B, True)
    np.testing.assert_allclose(O12, a * O1 + b * O2, rtol=0, atol=1e-12)


def test_correction_has_no_effect_at_tau_inf():
    rng = np.random.default_rng(12)
    Q, K, V = _rand_seq(rng, 160, 160, 4, 1, 8)
    a = O.run_batch([(Q, K, V)], 32, float("inf"), True)["out"]
    b = O.run_batch([(Q, K, V)], 32, float("inf"), False)["out"]
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------------------
# threshold special cases and CSR shape
# ---------------------------------------------------------------------------

def test_threshold_special_cases_and_nesting():
    rng = np.random.default_rng(13)
    B, T, n = 16, 320, 256
    Q, K, V = _rand_seq(rng, T, n, 4, 2, 16)
    P = T - n
    forced_only = O.plan_batch([(Q, K, V)], B, -1.0)["keep"][0]
    for g in range(2):
        for i in range(n // B):
            diag = P // B + i
            assert set(np.nonzero(forced_only[g, i])[0]) == {0, diag}
    p0 = O.plan_batch([(Q, K, V)], B, 0.0)
    s, keep0 = p0["s"][0], p0["keep"][0]
    for g in range(2):
        for i in range(n // B):
            diag = P // B + i
            row = s[g, i, :diag + 1]
            assert len(set(row.tolist())) == row.size  # distinct scores
            assert set(np.nonzero(keep0[g, i])[0]) == {0, diag, int(np.argmax(row))}
    prev = None
    for tau in (0.0, 0.01, 0.05, 0.2, 1.0, float("inf")):
        k = O.plan_batch([(Q, K, V)], B, tau)["keep"][0]
        if prev is not None:
            assert np.all(k >= prev)
        prev = k


def test_csr_is_well_formed_varlen():
    rng = np.random.default_rng(14)
    B = 16
    seqs = [_rand_seq(rng, 96, 64, 4, 2, 8), _rand_seq(rng, 48, 48, 4, 2, 8),
            _rand_seq(rng, 130, 66, 4, 2, 8)]
    plan = O.plan_batch(seqs, B, 0.05)
    rp, ci = plan["row_ptr"], plan["col_idx"]
    nqbs = plan["nqb"]
    total_qb = sum(nqbs)
    assert rp[0] == 0 and rp[-1] == ci.size and rp.size == 2 * total_qb + 1
    base = 0
    for (Q, K, V), nqb in zip(seqs, nqbs):
        P = K.shape[0] - Q.shape[0]
        for g in range(2):
            for i in range(nqb):
                r = g * total_qb + base + i
                row = ci[rp[r]:rp[r + 1]]
                diag = P // B + i
                assert np.all(np.diff(row) > 0) and row[0] == 0 and row[-1] == diag
        base += nqb


# ---------------------------------------------------------------------------
# metamorphic: varlen batch == per sequence; prefix+chunk == tail of full run
# ---------------------------------------------------------------------------

def test_varlen_batch_equals_per_sequence_runs():
    rng = np.random.default_rng(15)
    B = 16
    seqs = [_rand_seq(rng, 96, 64, 4, 2, 8), _rand_seq(rng, 80, 80, 4, 2, 8),
            _rand_seq(rng, 130, 66, 4, 2, 8)]
    res = O.run_batch(seqs, B, 0.05, True)
    off = 0
    for Q, K, V in seqs:
        one = O.run_batch([(Q, K, V)], B, 0.05, True)["out"]
        np.testing.assert_array_equal(res["out"][off:off + Q.shape[0]], one)
        off += Q.shape[0]


@pytest.mark.parametrize("P", [32, 96])
def test_prefix_chunk_equals_tail_of_full_run(P):
    rng = np.random.default_rng(16)
    B, T = 32, 224
    Qf, K, V = _rand_seq(rng, T, T, 4, 2, 16)
    full = O.run_batch([(Qf, K, V)], B, 0.1, True)
    part = O.run_batch([(Qf[P:], K, V)], B, 0.1, True)
    np.testing.assert_allclose(part["out"], full["out"][P:], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# exact means on small integers
# ---------------------------------------------------------------------------

def test_block_and_pooled_means_exact():
    rng = np.random.default_rng(17)
    T, Hkv, G, d, B = 45, 2, 3, 5, 8
    K = rng.integers(-50, 50, size=(T, Hkv, d)).astype(np.float64)
    Q = rng.integers(-50, 50, size=(T, Hkv * G, d)).astype(np.float64)
    kb = O.block_means(K, B)
    qb = O.pooled_query_means(Q, B, G)
    for j in range(-(-T // B)):
        toks = range(j * B, min(j * B + B, T))
        for g in range(Hkv):
            for e in range(d):
                ref = Fraction(sum(int(K[t, g, e]) for t in toks), len(toks))
                assert abs(Fraction(kb[j, g, e]) - ref) <= Fraction(1, 2 ** 40)
                refq = Fraction(sum(int(Q[t, h, e]) for t in toks for h in range(g * G, g * G + G)),
                                len(toks) * G)
                assert abs(Fraction(qb[j, g, e]) - refq) <= Fraction(1, 2 ** 40)
