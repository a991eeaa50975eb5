"""The oracle's pins have teeth: plausible mistakes planted in a copy of the
oracle (on the CPU) must each be caught by at least one pin."""
import math
import types

import numpy as np
import pytest

import oracle.fp2_oracle as ref_mod
from test_oracle import brute_force, _rand_seq, _torch_sdpa
from test_oracle_decode import _codes, _expect, _scales


def _mutant(old: str, new: str):
    import inspect
    src = inspect.getsource(ref_mod)
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def pin_brute(mod):
    rng = np.random.default_rng(5)
    T, n, Hq, Hkv, d, B = 100, 68, 2, 1, 8, 16
    Q, K, V = _rand_seq(rng, T, n, Hq, Hkv, d)
    for j in range(-(-T // B)):
        K[j * B:(j + 1) * B] += rng.standard_normal((1, Hkv, d)) * 0.7
    res = mod.run_batch([(Q, K, V)], B, 0.1, True)
    ref, keep_ref = brute_force(Q, K, V, B, 0.1, True)
    for (g, i), js in keep_ref.items():
        assert list(np.nonzero(res["keep"][0][g, i])[0]) == js
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)


def pin_dense(mod):
    rng = np.random.default_rng(3)
    Q, K, V = _rand_seq(rng, 200, 72, 8, 2, 8)
    res = mod.run_batch([(Q, K, V)], 32, float("inf"), True)
    np.testing.assert_allclose(res["out"], _torch_sdpa(Q, K, V), rtol=0, atol=1e-12)


def pin_identical_keys(mod):
    rng = np.random.default_rng(8)
    B, n, P = 16, 192, 64
    T = P + n
    Q, K, V = _rand_seq(rng, T, n, 4, 2, 16)
    for j in range(-(-T // B)):
        K[j * B:(j + 1) * B] = rng.standard_normal((1, 2, 16))
    res = mod.run_batch([(Q, K, V)], B, 0.0, True)
    np.testing.assert_allclose(res["out"], mod.dense(Q, K, V)[0], rtol=0, atol=1e-12)


def pin_tau_zero(mod):
    rng = np.random.default_rng(13)
    B, T, n = 16, 320, 256
    Q, K, V = _rand_seq(rng, T, n, 4, 2, 16)
    p0 = mod.plan_batch([(Q, K, V)], B, 0.0)
    for g in range(2):
        for i in range(n // B):
            diag = (T - n) // B + i
            row = p0["s"][0][g, i, :diag + 1]
            assert set(np.nonzero(p0["keep"][0][g, i])[0]) == {0, diag, int(np.argmax(row))}


def pin_prefix(mod):
    rng = np.random.default_rng(16)
    Qf, K, V = _rand_seq(rng, 224, 224, 4, 2, 16)
    full = mod.run_batch([(Qf, K, V)], 32, 0.1, True)
    part = mod.run_batch([(Qf[96:], K, V)], 32, 0.1, True)
    np.testing.assert_allclose(part["out"], full["out"][96:], rtol=0, atol=1e-12)


def pin_brute_decoupled(mod):
    rng = np.random.default_rng(12)
    T, n, Hq, Hkv, d, B, BK = 160, 96, 4, 2, 8, 32, 16
    Q, K, V = _rand_seq(rng, T, n, Hq, Hkv, d)
    for j in range(-(-T // BK)):
        K[j * BK:(j + 1) * BK] += rng.standard_normal((1, Hkv, d)) * 0.7
    res = mod.run_batch([(Q, K, V)], B, 0.2, True, BK=BK)
    ref, keep_ref = brute_force(Q, K, V, B, 0.2, True, BK=BK)
    for (g, i), js in keep_ref.items():
        assert list(np.nonzero(res["keep"][0][g, i])[0]) == js
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)


def pin_threshold_decoupled(mod):
    rng = np.random.default_rng(17)
    T, n, Hq, Hkv, d, B, BK = 192, 128, 4, 2, 8, 32, 16
    Q, K, V = _rand_seq(rng, T, n, Hq, Hkv, d)
    # tau = 0 on random scores: block 0, the diagonal run and the row's argmax
    res = mod.run_batch([(Q, K, V)], B, 0.0, True, BK=BK)
    ref, keep_ref = brute_force(Q, K, V, B, 0.0, True, BK=BK)
    for (g, i), js in keep_ref.items():
        assert list(np.nonzero(res["keep"][0][g, i])[0]) == js
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)
    # scores rising with J (a direction shared by Q and, growing, by the KV
    # blocks): the row max sits on the last diagonal block and tau spans
    # about one block's step
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    Q2 = Q + 2.0 * u
    K2 = K.copy()
    for j in range(-(-T // BK)):
        K2[j * BK:(j + 1) * BK] += 0.5 * j * u
    res = mod.run_batch([(Q2, K2, V)], B, 0.5, True, BK=BK)
    ref, keep_ref = brute_force(Q2, K2, V, B, 0.5, True, BK=BK)
    for (g, i), js in keep_ref.items():
        assert list(np.nonzero(res["keep"][0][g, i])[0]) == js


def pin_decode_e4m3(mod):
    # 128-token query blocks over 64-token KV blocks after a cached prefix
    rng = np.random.default_rng(23)
    block, kv_block, P, n, Hq, Hkv, d = 128, 64, 128, 200, 4, 2, 4
    T = P + n
    q, k, v = _codes(rng, (n, Hq, d)), _codes(rng, (T, Hkv, d)), _codes(rng, (T, Hkv, d))
    qs = _scales(-(-n // block), Hq, 0.0)
    ks = _scales(-(-T // kv_block), Hkv, 100.0)
    vs = _scales(-(-T // kv_block), Hkv, 1000.0)
    Q, K, V = mod.decode_sequence("fp8", block, q, qs, k, ks, v, vs, kv_block=kv_block)
    np.testing.assert_array_equal(Q, _expect(q, qs, block))
    np.testing.assert_array_equal(K, _expect(k, ks, kv_block))
    np.testing.assert_array_equal(V, _expect(v, vs, kv_block))


def pin_keep_from_csr(mod):
    # two sequences (2 and 1 query blocks, 3 and 2 KV blocks), two KV heads
    rows = [[0], [0, 2], [0, 1], [0, 1], [1, 2], [1]]
    row_ptr = np.cumsum([0] + [len(r) for r in rows])
    col_idx = np.array([j for r in rows for j in r])
    keeps = mod.keep_from_csr(row_ptr, col_idx, 2, [2, 1], [3, 2])
    got = [sorted(np.nonzero(keeps[s][g, i])[0].tolist())
           for g in range(2) for s, nqb in enumerate([2, 1]) for i in range(nqb)]
    assert got == rows


PINS = [pin_brute, pin_dense, pin_identical_keys, pin_tau_zero, pin_prefix, pin_brute_decoupled,
        pin_threshold_decoupled, pin_decode_e4m3, pin_keep_from_csr]

MUTATIONS = [
    ("surrogate weight 1 instead of B", "* c + logB", "* c"),
    ("causal mask off by one", "keys[None, :] <= qpos[:, None]", "keys[None, :] < qpos[:, None] + 1 - 1"),
    ("kept blocks also corrected", "for j in range(1, dlo) if not keep[g, i, j]", "for j in range(1, dlo) if True"),
    ("strict threshold", "keep = s >= thr[:, :, None]", "keep = s > thr[:, :, None]"),
    ("score scale dropped", "full = (q32[:, g, :] @ k32[:, g, :].T) * c", "full = (q32[:, g, :] @ k32[:, g, :].T)"),
    ("diag ignores prefix in attend", "dlo, dhi = diag_range(P, n, i, B, BK)\n        kept",
     "dlo, dhi = diag_range(0, n, i, B, BK)\n        kept"),
    ("pooled over tokens only", "out[i] = blk.mean(axis=(0, 2))", "out[i] = blk[:, :, 0].mean(axis=0)"),
    ("value mean taken from keys", "kbar, vbar = block_means(K, BK or B), block_means(V, BK or B)\n        O, lse",
     "kbar, vbar = block_means(K, BK or B), block_means(K, BK or B)\n        O, lse"),
    ("diagonal run ignores the prefix", "first = P + i * B", "first = i * B"),
    ("diagonal taken as one KV block", "return first // BK, last // BK", "return last // BK, last // BK"),
    ("surrogate weight of the query block", "logB = math.log(BK)", "logB = math.log(B)"),
    ("scores stop at the first diagonal block", "s[g, i, :hi + 1] = full[i, :hi + 1]",
     "s[g, i, :hi] = full[i, :hi]"),
    ("exp base 2", "w = np.exp(L - m)", "w = np.exp2(L - m)"),
    ("threshold above the row max", "thr = (rowmax - t32)", "thr = (rowmax + t32)"),
    ("K/V scales indexed by the query block", "kb = kv_block or block", "kb = block"),
    ("scales taken per token", "tok_block = np.arange(T) // block",
     "tok_block = np.minimum(np.arange(T), scales.shape[0] - 1)"),
    ("CSR row base off by one sequence", "r = g * total_qb + base + i\n                keep[g, i",
     "r = g * total_qb + i\n                keep[g, i"),
    ("CSR rows read head-minor", "r = g * total_qb + base + i\n                keep[g, i",
     "r = (base + i) * Hkv + g\n                keep[g, i"),
]


def test_reference_passes_every_pin():
    for pin in PINS:
        pin(ref_mod)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new):
    mod = _mutant(old, new)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught: {name}"
