"""Pins for the oracle's input decoders and its CSR reader, against values
written out by hand rather than against the oracle itself.

- decode_sequence / dequant_blocks: e4m3 codes whose values the OCP FP8
  definition fixes (listed literally below), one scale per (block, head) set
  to distinct numbers; every token position must come out as value x the
  scale of its own block and head.  Queries are blocked by their index among
  the new tokens, keys and values by absolute position in KV blocks of
  kv_block tokens (Table 7's 128-token query tiles over 64-token KV tiles).
- keep_from_csr: a CSR written by hand for a two-sequence batch with two KV
  heads must give back the masks written by hand; a CSR from plan_batch must
  give back plan_batch's masks.
"""
import numpy as np
import pytest

import oracle as O

# OCP FP8 E4M3 (bias 7, 3 mantissa bits): code -> value, from the definition
E4M3_BY_HAND = {
    0x38: 1.0,          # 0.0111.000
    0x40: 2.0,          # 0.1000.000
    0x30: 0.5,          # 0.0110.000
    0x3C: 1.5,          # 0.0111.100
    0xB8: -1.0,         # 1.0111.000
    0xC4: -3.0,         # 1.1000.100
    0x7E: 448.0,        # 0.1111.110, the largest finite value
    0x01: 2.0 ** -9,    # smallest subnormal
    0x00: 0.0,
}
CODES = np.array(sorted(E4M3_BY_HAND), dtype=np.uint8)


def _codes(rng, shape):
    return CODES[rng.integers(0, CODES.size, size=shape)]


def _expect(codes, scales, blk):
    """value(code) x scales[t // blk, h], one element at a time."""
    T, H, d = codes.shape
    out = np.empty((T, H, d))
    for t in range(T):
        for h in range(H):
            for e in range(d):
                out[t, h, e] = E4M3_BY_HAND[int(codes[t, h, e])] * float(scales[t // blk, h])
    return out


def _scales(nb, H, base):
    # distinct per block and head, not powers of two: a scale taken from the
    # wrong block or head changes the value
    return np.array([[base + 10.0 * b + 1.0 + h + 0.25 for h in range(H)] for b in range(nb)],
                    dtype=np.float32)


@pytest.mark.parametrize("blk,T", [(128, 300), (64, 130), (128, 128)])
def test_dequant_blocks_each_token_takes_its_blocks_scale(blk, T):
    rng = np.random.default_rng(31 + T)
    H, d = 3, 4
    codes = _codes(rng, (T, H, d))
    sc = _scales(-(-T // blk), H, 0.0)
    np.testing.assert_array_equal(O.dequant_blocks(codes, sc, blk), _expect(codes, sc, blk))


@pytest.mark.parametrize("block,kv_block,P,n", [
    (128, None, 0, 300),     # one sequence, no prefix, ragged last block
    (128, None, 256, 130),   # cached prefix of two blocks, a 2-token last query block
    (128, 64, 0, 300),       # 128-token query blocks over 64-token KV blocks
    (128, 64, 128, 200),     # the same with a cached prefix
    (64, None, 64, 100),
])
def test_decode_sequence_e4m3_scales_per_block_and_head(block, kv_block, P, n):
    rng = np.random.default_rng(7 + P + n)
    Hq, Hkv, d = 4, 2, 4
    T = P + n
    kb = kv_block or block
    q = _codes(rng, (n, Hq, d))
    k = _codes(rng, (T, Hkv, d))
    v = _codes(rng, (T, Hkv, d))
    qs = _scales(-(-n // block), Hq, 0.0)        # [query blocks, Hq]: by new-token index
    ks = _scales(-(-T // kb), Hkv, 100.0)        # [KV blocks, Hkv]: by absolute position
    vs = _scales(-(-T // kb), Hkv, 1000.0)
    Q, K, V = O.decode_sequence("fp8", block, q, qs, k, ks, v, vs, kv_block=kv_block)
    np.testing.assert_array_equal(Q, _expect(q, qs, block))
    np.testing.assert_array_equal(K, _expect(k, ks, kb))
    np.testing.assert_array_equal(V, _expect(v, vs, kb))
    # spot check written out in full: the last key of KV block 1, head 1
    t = 2 * kb - 1
    assert K[t, 1, 0] == E4M3_BY_HAND[int(k[t, 1, 0])] * (100.0 + 10.0 * 1 + 1.0 + 1 + 0.25)


def test_decode_sequence_bf16_is_the_bit_pattern():
    # bfloat16 is the top half of a binary32: 0x3F80 = 1.0, 0xC040 = -3.0,
    # 0x3F81 = 1 + 2^-7, 0x0001 = 2^-133 (subnormal)
    bits = np.array([0x3F80, 0xC040, 0x3F81, 0x0001, 0x0000, 0x8000], dtype=np.uint16).reshape(6, 1, 1)
    Q, K, V = O.decode_sequence("bf16", 64, bits, None, bits, None, bits, None)
    want = np.array([1.0, -3.0, 1.0 + 2.0 ** -7, 2.0 ** -133, 0.0, -0.0]).reshape(6, 1, 1)
    for X in (Q, K, V):
        np.testing.assert_array_equal(X, want)
    assert np.signbit(K[5, 0, 0])


def test_keep_from_csr_hand_written():
    # batch of two sequences: 2 and 1 query blocks, 3 and 2 KV blocks, 2 KV
    # heads; rows r = g * total_qblocks + global query block, total 3
    Hkv, nqbs, nkbs = 2, [2, 1], [3, 2]
    rows = [
        [0],        # g0, seq0 block0
        [0, 2],     # g0, seq0 block1
        [0, 1],     # g0, seq1 block0
        [0, 1],     # g1, seq0 block0
        [1, 2],     # g1, seq0 block1
        [1],        # g1, seq1 block0
    ]
    row_ptr = np.cumsum([0] + [len(r) for r in rows])
    col_idx = np.array([j for r in rows for j in r])
    keeps = O.keep_from_csr(row_ptr, col_idx, Hkv, nqbs, nkbs)
    want0 = np.zeros((2, 2, 3), bool)
    want0[0, 0, [0]] = True
    want0[0, 1, [0, 2]] = True
    want0[1, 0, [0, 1]] = True
    want0[1, 1, [1, 2]] = True
    want1 = np.zeros((2, 1, 2), bool)
    want1[0, 0, [0, 1]] = True
    want1[1, 0, [1]] = True
    assert len(keeps) == 2
    np.testing.assert_array_equal(keeps[0], want0)
    np.testing.assert_array_equal(keeps[1], want1)


@pytest.mark.parametrize("BK", [None, 16])
def test_keep_from_csr_round_trip_varlen_with_prefixes(BK):
    rng = np.random.default_rng(44)
    B, Hq, Hkv, d = 32, 4, 2, 8
    seqs = []
    for P, n in [(64, 80), (0, 100), (96, 33)]:
        T = P + n
        seqs.append((rng.standard_normal((n, Hq, d)), rng.standard_normal((T, Hkv, d)),
                     rng.standard_normal((T, Hkv, d))))
    plan = O.plan_batch(seqs, B, 0.3, BK)
    nkbs = [-(-K.shape[0] // (BK or B)) for _, K, _ in seqs]
    keeps = O.keep_from_csr(plan["row_ptr"], plan["col_idx"], Hkv, plan["nqb"], nkbs)
    assert sum(k.sum() for k in keeps) == plan["row_ptr"][-1] > 0
    for got, want in zip(keeps, plan["keep"]):
        np.testing.assert_array_equal(got, want)
