"""Plain float64 reference of the FlashPrefill V2 prefill path (CPU, numpy).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP kernels.

Source: "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context LLM
Serving" (metallab.ai page), Figure 3 (Stage 1: PackGQA query packing,
block-mean pooling, a CSR index of selected blocks; Stage 2: exact attention
over the selected blocks merged in one online softmax with the mean
correction of the unselected ones), Figure 4 (each pruned block J enters
numerator and denominator as |B_J| * exp(s_J) * (vbar_J, 1)), Table 7 (CSR
per KV head), and the abstract's "instantaneous pattern discovery and
max-based dynamic thresholding".  The pages state the method in words; the
exact definition followed here is:

  1. kbar_J, vbar_J: mean of K and V over the tokens of KV block J.
  2. qbar_I: mean of Q over the tokens of query block I and the G query
     heads that share one KV head (PackGQA packing, then pooling).
  3. s_IJ = (qbar_I . kbar_J) / sqrt(d) for every causal J <= diag(I).
  4. keep J iff s_IJ >= max_J s_IJ - tau; block 0 and the diagonal block are
     always kept.  The decision is taken in float32 (the scores are defined
     as float32 values), everything else in float64.
  5. exact softmax attention over the kept blocks' tokens (causal), plus for
     every skipped J in [1, diag) a surrogate term
     B * exp(q . kbar_J / sqrt(d) - m) * (vbar_J, 1), merged into the same
     softmax normaliser.

Query blocks hold B tokens and KV blocks BK tokens (BK = B unless given; BK
must divide B).  Table 7 pairs 128-token query tiles with 64-token KV tiles.
With BK < B the diagonal of query block I is the run of KV blocks that hold
one of its own positions, [diag_lo(I), diag_hi(I)]: all of them are forced,
scores and keys reach up to diag_hi, the surrogate covers skipped J in
[1, diag_lo) and its weight is the KV block size BK.  With BK = B the run is
the single block diag(I) = P/B + I.

Every input is the exact value the GPU sees: bfloat16 bits widened, or
OCP E4M3 codes times their float32 block scale.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "decode_bf16", "decode_e4m3", "E4M3_VALUES", "dequant_blocks", "decode_sequence",
    "block_means", "pooled_query_means", "diag_range", "block_scores", "select_blocks",
    "attend", "dense", "plan_batch", "run_batch", "NEAR_TIE",
]

NEAR_TIE = 1e-5  # scores this close to their row threshold may fall either way


# ---------------------------------------------------------------------------
# Storage formats
# ---------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64.  bfloat16 is the top half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    """Value of one OCP FP8 E4M3 code: sign, 4-bit exponent (bias 7), 3-bit mantissa.

    Exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there are
    no infinities.
    """
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_VALUES = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def dequant_blocks(codes: np.ndarray, scales: np.ndarray, block: int) -> np.ndarray:
    """E4M3 codes[T, H, d] times one scale per (block of tokens, head) -> float64."""
    x = decode_e4m3(codes)
    T = x.shape[0]
    tok_block = np.arange(T) // block
    return x * scales.astype(np.float64)[tok_block][:, :, None]


def decode_sequence(dtype: str, block: int, q, q_scale, k, k_scale, v, v_scale,
                    kv_block: Optional[int] = None):
    """Storage codes of one sequence -> float64 (Q[n,Hq,d], K[T,Hkv,d], V[T,Hkv,d]).

    e4m3: one query scale per (query block, head), one K / V scale per (KV
    block, head); kv_block = block unless given.
    """
    if dtype == "bf16":
        return decode_bf16(q), decode_bf16(k), decode_bf16(v)
    if dtype == "fp8":
        kb = kv_block or block
        return (dequant_blocks(q, q_scale, block), dequant_blocks(k, k_scale, kb),
                dequant_blocks(v, v_scale, kb))
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Stage 1: block statistics, pooled scores, max-based threshold
# ---------------------------------------------------------------------------

def block_means(X: np.ndarray, B: int) -> np.ndarray:
    """Mean over the valid tokens of each block of B: X[T, H, d] -> [ceil(T/B), H, d]."""
    T = X.shape[0]
    nb = -(-T // B)
    out = np.empty((nb,) + X.shape[1:], dtype=np.float64)
    for j in range(nb):
        out[j] = X[j * B:min((j + 1) * B, T)].mean(axis=0)
    return out


def pooled_query_means(Q: np.ndarray, B: int, G: int) -> np.ndarray:
    """qbar[I, g] = mean of Q over the tokens of query block I and heads g*G..g*G+G-1.

    Q[n, Hq, d] holds the n new tokens; block I covers new-token indices
    [I*B, min((I+1)*B, n)).  Returns [ceil(n/B), Hq/G, d].
    """
    n, Hq, d = Q.shape
    Hkv = Hq // G
    nb = -(-n // B)
    out = np.empty((nb, Hkv, d), dtype=np.float64)
    for i in range(nb):
        blk = Q[i * B:min((i + 1) * B, n)].reshape(-1, Hkv, G, d)
        out[i] = blk.mean(axis=(0, 2))
    return out


def diag_range(P: int, n: int, i: int, B: int, BK: Optional[int] = None) -> Tuple[int, int]:
    """First and last KV block (BK tokens) holding a position of query block i (B tokens).

    Query block i covers the absolute positions P + i*B .. P + min((i+1)*B, n) - 1.
    """
    BK = B if BK is None else BK
    first = P + i * B
    last = P + min((i + 1) * B, n) - 1
    return first // BK, last // BK


def block_scores(qbar: np.ndarray, kbar: np.ndarray, P: int, B: int, d: int,
                 n: Optional[int] = None, BK: Optional[int] = None) -> np.ndarray:
    """float32 scores s[g, I, J] = (qbar_I . kbar_J) / sqrt(d) for J <= diag_hi(I); -inf above.

    The pooled means are held as float32 (the precision the scores are
    defined in); the dot product of those float32 values is formed in
    float64 and rounded once to float32.  n (new tokens) is needed when
    BK < B; with BK = B, diag(I) = P/B + I.
    """
    nqb, Hkv, _ = qbar.shape
    nkb = kbar.shape[0]
    if n is None:
        if BK is not None and BK != B:
            raise ValueError("n is needed when the KV block differs from the query block")
        n = nqb * B
    q32 = qbar.astype(np.float32).astype(np.float64)
    k32 = kbar.astype(np.float32).astype(np.float64)
    c = 1.0 / math.sqrt(d)
    s = np.full((Hkv, nqb, nkb), -np.inf, dtype=np.float32)
    for g in range(Hkv):
        full = (q32[:, g, :] @ k32[:, g, :].T) * c  # [nqb, nkb]
        for i in range(nqb):
            _, hi = diag_range(P, n, i, B, BK)
            s[g, i, :hi + 1] = full[i, :hi + 1].astype(np.float32)
    return s


def select_blocks(s: np.ndarray, P: int, B: int, tau: float, n: Optional[int] = None,
                  BK: Optional[int] = None):
    """Max-based dynamic threshold with forced blocks.

    thr[g, I] = float32(max_J s[g, I, J] - tau); keep J iff s >= thr, or
    J == 0, or J is on the diagonal of I (diag_range).  Returns (keep[g, I, J]
    bool, thr[g, I] float32, rowmax[g, I] float32).
    """
    Hkv, nqb, nkb = s.shape
    if n is None:
        if BK is not None and BK != B:
            raise ValueError("n is needed when the KV block differs from the query block")
        n = nqb * B
    t32 = np.float32(tau)
    rowmax = s.max(axis=2)
    with np.errstate(invalid="ignore", over="ignore"):
        thr = (rowmax - t32).astype(np.float32)
    keep = s >= thr[:, :, None]
    for i in range(nqb):
        lo, hi = diag_range(P, n, i, B, BK)
        keep[:, i, hi + 1:] = False
        keep[:, i, 0] = True
        keep[:, i, lo:hi + 1] = True
    return keep, thr, rowmax


# ---------------------------------------------------------------------------
# Stage 2: exact attention over kept blocks plus mean correction
# ---------------------------------------------------------------------------

def attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, keep: np.ndarray, B: int,
           correction: bool, kbar: Optional[np.ndarray] = None,
           vbar: Optional[np.ndarray] = None,
           rows: Optional[Sequence[Tuple[int, int]]] = None, BK: Optional[int] = None):
    """Block-sparse causal GQA attention with optional mean correction, one sequence.

    Q[n, Hq, d]; K, V[T, Hkv, d]; the n queries sit at absolute positions
    P..T-1 with P = T - n (a cached prefix of P tokens).  keep[g, I, J]
    selects KV blocks (BK tokens, BK = B unless given) per (KV head, query
    block of B tokens).  A query at position p sees a key at position u of a
    kept block iff u <= p.  With correction, every J in [1, diag_lo(I)) that
    is not kept adds the surrogate logit q . kbar_J / sqrt(d) with weight BK
    and value vbar_J.

    rows: optional list of (g, I) to compute; other outputs stay NaN.
    Returns (O[n, Hq, d], lse[n, Hq]) with lse = log of the softmax
    normaliser (sum of exp(logit) times weight) in absolute terms.
    """
    n, Hq, d = Q.shape
    T, Hkv, _ = K.shape
    G = Hq // Hkv
    P = T - n
    BK = B if BK is None else BK
    c = 1.0 / math.sqrt(d)
    if correction and (kbar is None or vbar is None):
        kbar, vbar = block_means(K, BK), block_means(V, BK)
    nqb = -(-n // B)
    O = np.full((n, Hq, d), np.nan, dtype=np.float64)
    lse = np.full((n, Hq), np.nan, dtype=np.float64)
    if rows is None:
        rows = [(g, i) for g in range(Hkv) for i in range(nqb)]
    logB = math.log(BK)
    for g, i in rows:
        t0, t1 = i * B, min((i + 1) * B, n)
        dlo, dhi = diag_range(P, n, i, B, BK)
        kept = np.nonzero(keep[g, i, :dhi + 1])[0]
        keys = np.concatenate([np.arange(j * BK, min((j + 1) * BK, T)) for j in kept])
        qpos = P + np.arange(t0, t1)                       # absolute query positions
        Qb = Q[t0:t1, g * G:(g + 1) * G, :]               # [nt, G, d]
        logit = (Qb @ K[keys, g, :].T) * c                # [nt, G, nk]
        visible = keys[None, :] <= qpos[:, None]          # [nt, nk]
        logit = np.where(visible[:, None, :], logit, -np.inf)
        parts_l = [logit]
        parts_v = [V[keys, g, :]]
        if correction:
            skipped = np.array([j for j in range(1, dlo) if not keep[g, i, j]], dtype=np.int64)
            if skipped.size:
                lbar = (Qb @ kbar[skipped, g, :].T) * c + logB
                parts_l.append(lbar)
                parts_v.append(vbar[skipped, g, :])
        L = np.concatenate(parts_l, axis=2)               # [nt, G, nk_total]
        Vv = np.concatenate(parts_v, axis=0)              # [nk_total, d]
        m = L.max(axis=2, keepdims=True)
        w = np.exp(L - m)
        den = w.sum(axis=2)
        O[t0:t1, g * G:(g + 1) * G, :] = (w @ Vv) / den[..., None]
        lse[t0:t1, g * G:(g + 1) * G] = m[..., 0] + np.log(den)
    return O, lse


def dense(Q: np.ndarray, K: np.ndarray, V: np.ndarray,
          query_rows: Optional[Sequence[int]] = None):
    """Textbook causal softmax attention with a cached prefix (bottom-right aligned).

    Q[n, Hq, d], K, V[T, Hkv, d]; query t (new-token index) sits at absolute
    position T - n + t and sees keys 0..T-n+t.  query_rows restricts the
    computation to some new-token indices.  Returns (O[len, Hq, d], lse[len, Hq]).
    """
    n, Hq, d = Q.shape
    T, Hkv, _ = K.shape
    G = Hq // Hkv
    P = T - n
    idx = np.arange(n) if query_rows is None else np.asarray(query_rows)
    O = np.empty((idx.size, Hq, d))
    lse = np.empty((idx.size, Hq))
    for h in range(Hq):
        g = h // G
        S = (Q[idx, h, :] @ K[:, g, :].T) / math.sqrt(d)   # [len, T]
        S = np.where(np.arange(T)[None, :] <= (P + idx)[:, None], S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        w = np.exp(S - m)
        den = w.sum(axis=1)
        O[:, h, :] = (w @ V[:, g, :]) / den[:, None]
        lse[:, h] = m[:, 0] + np.log(den)
    return O, lse


# ---------------------------------------------------------------------------
# Batch level: CSR plan and outputs in the library's layouts
# ---------------------------------------------------------------------------

def plan_batch(seqs: List[Tuple[np.ndarray, np.ndarray, np.ndarray]], B: int, tau: float,
               BK: Optional[int] = None) -> Dict:
    """Stage 1 over a variable-length batch (query blocks of B tokens, KV blocks of BK = B unless given).

    seqs: per sequence (Q[n,Hq,d], K[T,Hkv,d], V[T,Hkv,d]) in float64.
    Returns a dict with
      kbar, vbar : [Hkv, total_kblocks, d] float64 (block means)
      row_ptr    : int64 [Hkv*total_qblocks + 1]; row r = g*total_qblocks + global q-block
      col_idx    : int64 [nnz], KV-block indices within the sequence, ascending per row
      keep, s, thr, rowmax : per-sequence lists ([Hkv, nqb, nkb] / [Hkv, nqb])
      near_tie   : per-sequence bool [Hkv, nqb, nkb], |s - thr| <= NEAR_TIE
    """
    Hkv = seqs[0][1].shape[1]
    d = seqs[0][0].shape[2]
    G = seqs[0][0].shape[1] // Hkv
    kb_list, vb_list, keeps, ss, thrs, maxes, ties = [], [], [], [], [], [], []
    nqbs = []
    for Q, K, V in seqs:
        n, T = Q.shape[0], K.shape[0]
        P = T - n
        kbar, vbar = block_means(K, BK or B), block_means(V, BK or B)
        qbar = pooled_query_means(Q, B, G)
        s = block_scores(qbar, kbar, P, B, d, n, BK)
        keep, thr, rowmax = select_blocks(s, P, B, tau, n, BK)
        with np.errstate(invalid="ignore"):
            tie = np.abs(s.astype(np.float64) - thr.astype(np.float64)[:, :, None]) <= NEAR_TIE
        kb_list.append(kbar)
        vb_list.append(vbar)
        keeps.append(keep)
        ss.append(s)
        thrs.append(thr)
        maxes.append(rowmax)
        ties.append(tie)
        nqbs.append(qbar.shape[0])
    total_qb = int(sum(nqbs))
    counts = np.zeros(Hkv * total_qb, dtype=np.int64)
    cols = [[None] * total_qb for _ in range(Hkv)]
    base = 0
    for si, keep in enumerate(keeps):
        for g in range(Hkv):
            for i in range(nqbs[si]):
                js = np.nonzero(keep[g, i])[0]
                cols[g][base + i] = js
                counts[g * total_qb + base + i] = js.size
        base += nqbs[si]
    row_ptr = np.zeros(Hkv * total_qb + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.concatenate([cols[g][q] for g in range(Hkv) for q in range(total_qb)]) \
        if total_qb else np.zeros(0, dtype=np.int64)
    kbar_all = np.concatenate(kb_list, axis=0).transpose(1, 0, 2) if kb_list else None
    vbar_all = np.concatenate(vb_list, axis=0).transpose(1, 0, 2) if vb_list else None
    return dict(kbar=kbar_all, vbar=vbar_all, row_ptr=row_ptr, col_idx=col_idx.astype(np.int64),
                keep=keeps, s=ss, thr=thrs, rowmax=maxes, near_tie=ties, nqb=nqbs)


def keep_from_csr(row_ptr: np.ndarray, col_idx: np.ndarray, Hkv: int, nqbs: Sequence[int],
                  nkbs: Sequence[int]) -> List[np.ndarray]:
    """Per-sequence keep[g, I, J] masks from a CSR plan (e.g. the GPU's)."""
    total_qb = int(sum(nqbs))
    out = []
    base = 0
    for nqb, nkb in zip(nqbs, nkbs):
        keep = np.zeros((Hkv, nqb, nkb), dtype=bool)
        for g in range(Hkv):
            for i in range(nqb):
                r = g * total_qb + base + i
                keep[g, i, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
        out.append(keep)
        base += nqb
    return out


__all__.append("keep_from_csr")


def run_batch(seqs: List[Tuple[np.ndarray, np.ndarray, np.ndarray]], B: int, tau: float,
              correction: bool, keeps: Optional[List[np.ndarray]] = None,
              BK: Optional[int] = None) -> Dict:
    """Whole path over a batch: plan (unless keeps is given) then attention.

    Returns the plan dict plus out: [total_q, Hq, d] float64 and lse [total_q, Hq].
    """
    plan = plan_batch(seqs, B, tau, BK)
    if keeps is None:
        keeps = plan["keep"]
    outs, lses = [], []
    for (Q, K, V), keep in zip(seqs, keeps):
        kbar, vbar = block_means(K, BK or B), block_means(V, BK or B)
        O, lse = attend(Q, K, V, keep, B, correction, kbar, vbar, BK=BK)
        outs.append(O)
        lses.append(lse)
    plan["out"] = np.concatenate(outs, axis=0)
    plan["lse"] = np.concatenate(lses, axis=0)
    return plan
