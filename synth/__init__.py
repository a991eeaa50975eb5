"""Seeded synthetic inputs for block-sparse causal GQA prefill attention.

This module is shared by the float64 oracle's tests and by the GPU path's
tests and benchmark.  It holds input generation only: random draws, the
planted attention structure of each workload, casts to the storage formats
(bfloat16, OCP FP8 E4M3 with one scale per 128x128 block), paging of the KV
cache and the variable-length batch descriptors.  No step of the attention
method itself (block statistics, scoring, thresholding, attention,
correction) is computed here.

Workload shapes follow the five synthetic configurations of the build
contract (tiny, a Llama-3.1-8B-shaped 32K layer, a 128K layer in bf16 and
fp8, a Qwen3-30B-A3B-shaped paged continuous batch, and an extreme-sparsity
fp8 layer).  The needle-in-a-haystack inputs that the FlashPrefill V2 pages
measure on (Table 1, Table 3) are stood in for by planted structure: hot
keys, a local band, sink columns and fixed-offset slashes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Config", "Workload", "CONFIGS", "make", "make_custom",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "f32_to_e4m3", "quantize_blocks_e4m3",
    "E4M3_MAX",
]

E4M3_MAX = 448.0  # largest finite OCP E4M3 magnitude (S.1111.110)


# ---------------------------------------------------------------------------
# Storage-format casts (written from the bfloat16 and OCP FP8 definitions)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    bfloat16 keeps the top 16 bits of an IEEE binary32.  Rounding adds
    0x7FFF plus the lowest kept bit before truncation.  Inputs here are
    finite; NaN handling is not needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_e4m3(y: np.ndarray) -> np.ndarray:
    """float32 -> OCP FP8 E4M3 codes (uint8), round to nearest even, saturating.

    E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
    infinities, S.1111.111 is NaN, so the largest finite value is
    1.75 * 2^8 = 448.  Normal numbers start at 2^-6; subnormals are
    m * 2^-9 for m = 1..7.  Magnitudes above 448 saturate to 448.
    """
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    flat_y = y.reshape(-1)
    flat_o = out.reshape(-1)
    chunk = 1 << 24
    for s in range(0, flat_y.size, chunk):
        a = np.abs(flat_y[s:s + chunk])
        sign = (flat_y[s:s + chunk].view(np.uint32) >> np.uint32(31)).astype(np.uint8)
        bits = a.view(np.uint32)
        # normal range: round the 23-bit mantissa to 3 bits (RNE) in the bit pattern
        lsb = (bits >> np.uint32(20)) & np.uint32(1)
        rb = (bits + np.uint32(0x7FFFF) + lsb) & np.uint32(0xFFF00000)
        e = (rb >> np.uint32(23)).astype(np.int32) - 127 + 7
        m = ((rb >> np.uint32(20)) & np.uint32(7)).astype(np.int32)
        code_n = (e << 3) | m
        # subnormal range: multiples of 2^-9, RNE via rint; 8 * 2^-9 is the min normal (code 8)
        code_s = np.rint(a.astype(np.float64) * 512.0).astype(np.int32)
        code = np.where(a >= np.float32(2.0 ** -6), code_n, code_s)
        code = np.minimum(code, 0x7E)  # saturate at 448, never emit the NaN code
        flat_o[s:s + chunk] = (code.astype(np.uint8) | (sign << np.uint8(7)))
    return out


def quantize_blocks_e4m3(x: np.ndarray, block: int) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise x[T, H, d] to E4M3 with one float32 scale per (block of tokens, head).

    scale = amax / 448 over the block's tokens and the head's d channels
    (amax == 0 gives scale 1); code = E4M3(x / scale).  A partial last block
    is scaled over its valid tokens.  Returns (codes[T, H, d] uint8,
    scales[ceil(T/block), H] float32).
    """
    T, H, d = x.shape
    nb = (T + block - 1) // block
    codes = np.empty((T, H, d), dtype=np.uint8)
    scales = np.empty((nb, H), dtype=np.float32)
    for b in range(nb):
        blk = np.asarray(x[b * block:(b + 1) * block], dtype=np.float32)
        amax = np.abs(blk).max(axis=(0, 2)).astype(np.float32)  # [H]
        sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        scales[b] = sc
        codes[b * block:(b + 1) * block] = f32_to_e4m3(blk / sc[None, :, None])
    return codes, scales


# ---------------------------------------------------------------------------
# Configurations
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    name: str
    seqlens: Tuple[int, ...]      # total key length T of each sequence (prefix + new)
    prefixes: Tuple[int, ...]     # cached prefix length P of each sequence
    hq: int
    hkv: int
    d: int
    block: int                    # B: query block size (and KV block size unless kv_block is set)
    page_size: int
    dtype: str                    # "bf16" or "fp8"
    structure: str                # "hot", "band_sinks", "slash" or "plain"
    tau: Optional[float]          # None: calibrated to a target density (see target_density)
    seed: int
    shuffle_pages: bool = False
    target_density: Optional[float] = None
    seq_seeds: Optional[Tuple[int, ...]] = None   # one seed per request (varlen batch)
    shuffle_seed: int = 4999
    description: str = ""
    kv_block: int = 0             # KV block size; 0: the same as block


_QWEN_T = (4096, 8192, 16384, 16384, 32768, 32768, 65536, 8192)

CONFIGS = {
    "tiny": Config(
        name="tiny", seqlens=(1024,), prefixes=(0,), hq=4, hkv=1, d=64, block=64, page_size=64,
        dtype="bf16", structure="hot", tau=2.0, seed=1,
        description="1 seq, L=1024, 4q/1kv, d=64, B=64, N(0,1) fp32 rounded to bf16, 8 hot keys +3"),
    "llama32k": Config(
        name="llama32k", seqlens=(32768,), prefixes=(0,), hq=32, hkv=8, d=128, block=128,
        page_size=128, dtype="bf16", structure="band_sinks", tau=3.0, seed=2,
        description="Llama-3.1-8B-shaped layer, L=32768, 32q/8kv, d=128, B=128, bf16, band+16 sinks"),
    "c128k_bf16": Config(
        name="c128k_bf16", seqlens=(131072,), prefixes=(0,), hq=32, hkv=8, d=128, block=128,
        page_size=128, dtype="bf16", structure="band_sinks", tau=None, target_density=0.05, seed=3,
        description="L=131072, 32q/8kv, d=128, B=128, bf16, band+16 sinks, tau for ~5% density"),
    "c128k_fp8": Config(
        name="c128k_fp8", seqlens=(131072,), prefixes=(0,), hq=32, hkv=8, d=128, block=128,
        page_size=128, dtype="fp8", structure="band_sinks", tau=None, target_density=0.05, seed=3,
        description="L=131072, 32q/8kv, d=128, B=128, fp8-e4m3 (scale per 128x128), band+sinks, ~5%"),
    "qwen_paged": Config(
        name="qwen_paged", seqlens=_QWEN_T, prefixes=tuple(t // 2 for t in _QWEN_T), hq=32, hkv=4,
        d=128, block=128, page_size=64, dtype="bf16", structure="band_sinks", tau=3.0, seed=4,
        shuffle_pages=True, seq_seeds=tuple(4000 + r for r in range(len(_QWEN_T))),
        description="Qwen3-30B-A3B-shaped, 8 requests {4K..64K}, 50% cached prefix, 32q/4kv, "
                    "d=128, B=128, bf16, page 64, shuffled page table"),
    "extreme_fp8": Config(
        name="extreme_fp8", seqlens=(131072,), prefixes=(0,), hq=32, hkv=8, d=128, block=128,
        page_size=128, dtype="fp8", structure="slash", tau=None, target_density=0.02, seed=5,
        description="L=131072, 32q/8kv, d=128, fp8-e4m3, Gaussian + slashes at {0,64,4096}, ~2%"),
}


# ---------------------------------------------------------------------------
# Planted structure (one sequence at a time)
# ---------------------------------------------------------------------------

def _unit(rng: np.random.Generator, d: int) -> np.ndarray:
    u = rng.standard_normal(d)
    return (u / np.linalg.norm(u)).astype(np.float32)


def _plant_hot(rng, Q, K, V):
    """8 hot key positions boosted by +3 along one shared random direction."""
    T = K.shape[0]
    pos = rng.choice(T, size=min(8, T), replace=False)
    u = _unit(rng, K.shape[2])
    K[pos] += 3.0 * u[None, None, :]


def _plant_band_sinks(rng, Q, K, V, G):
    """Local band (keys within 512 positions correlated ~0.5) and 16 sink columns at +4.

    Band: per KV head, c_t = (1/sqrt(512)) * sum of 512 iid N(0, I) vectors
    xi_{t-511..t}; the group's queries and the head's keys become
    sqrt(1/2) * x + sqrt(1/2) * c_t, so channels of q_t and k_s correlate by
    0.5 * max(0, 1 - |t - s| / 512).
    Sinks: position 0 plus 15 distinct uniform positions in [1, T).  Per KV
    head a unit direction u is removed from every query and key of the group,
    each query's u-component is set to 1 and each sink key's to 4*sqrt(d), so
    the sink logit carries +4 after the 1/sqrt(d) scale.
    """
    T, Hkv, d = K.shape
    W = 512
    h = np.float32(math.sqrt(0.5))
    for g in range(Hkv):
        xi = rng.standard_normal((T + W - 1, d), dtype=np.float32)
        cs = np.zeros((T + W, d), dtype=np.float64)
        np.cumsum(xi, axis=0, dtype=np.float64, out=cs[1:])
        c = ((cs[W:] - cs[:T]) / math.sqrt(W)).astype(np.float32)  # [T, d]
        del cs, xi
        qs = slice(g * G, (g + 1) * G)
        Q[:, qs, :] *= h
        Q[:, qs, :] += h * c[:, None, :]
        K[:, g, :] *= h
        K[:, g, :] += h * c
        del c
    n_extra = min(15, T - 1)
    cols = np.concatenate([[0], np.sort(rng.choice(np.arange(1, T), size=n_extra, replace=False))]) \
        if T > 1 else np.array([0])
    for g in range(Hkv):
        u = _unit(rng, d)
        qs = slice(g * G, (g + 1) * G)
        Qg = Q[:, qs, :]
        Qg -= (Qg @ u)[..., None] * u
        Qg += u
        Q[:, qs, :] = Qg
        Kg = K[:, g, :]
        Kg -= (Kg @ u)[:, None] * u[None, :]
        Kg[cols] += np.float32(4.0 * math.sqrt(d)) * u[None, :]
        K[:, g, :] = Kg


def _plant_slash(rng, Q, K, V, G, offsets=(0, 64, 4096)):
    """Fixed-offset diagonals: q_t . k_{t-o} / sqrt(d) has mean +4 for o in offsets."""
    T, Hkv, d = K.shape
    a = np.float32(4.0 / math.sqrt(d))
    for g in range(Hkv):
        z = rng.standard_normal((T, d), dtype=np.float32)
        Q[:, g * G:(g + 1) * G, :] += z[:, None, :]
        for o in offsets:
            if o < T:
                K[:T - o, g, :] += a * z[o:]
        del z


def _gen_sequence(cfg: Config, T: int, seed: int):
    """Logical float32 Q[T,Hq,d], K[T,Hkv,d], V[T,Hkv,d] for one sequence.

    Draw order: Q, K, V as N(0,1) float32 in C order, then the structure draws.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    G = cfg.hq // cfg.hkv
    Q = rng.standard_normal((T, cfg.hq, cfg.d), dtype=np.float32)
    K = rng.standard_normal((T, cfg.hkv, cfg.d), dtype=np.float32)
    V = rng.standard_normal((T, cfg.hkv, cfg.d), dtype=np.float32)
    if cfg.structure == "hot":
        _plant_hot(rng, Q, K, V)
    elif cfg.structure == "band_sinks":
        _plant_band_sinks(rng, Q, K, V, G)
    elif cfg.structure == "slash":
        _plant_slash(rng, Q, K, V, G)
    elif cfg.structure != "plain":
        raise ValueError(f"unknown structure {cfg.structure!r}")
    return Q, K, V


# ---------------------------------------------------------------------------
# Workload: storage-format tensors, paging and batch descriptors
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    cfg: Config
    tau: float
    seqlens_k: np.ndarray          # int32 [S]
    n_q: np.ndarray                # int32 [S] new query tokens
    cu_seqlens_q: np.ndarray       # int32 [S+1]
    cu_qblocks: np.ndarray         # int32 [S+1]
    cu_kblocks: np.ndarray         # int32 [S+1]
    q: np.ndarray                  # [total_q, Hq, d] uint16 (bf16 bits) or uint8 (e4m3)
    q_scale: Optional[np.ndarray]  # fp8: float32 [total_qblocks, Hq]
    k_pages: np.ndarray            # [num_pages, page_size, Hkv, d]
    v_pages: np.ndarray
    k_scale: Optional[np.ndarray]  # fp8: float32 [num_pages, Hkv]
    v_scale: Optional[np.ndarray]
    page_table: np.ndarray         # int32 [S, max_pages]
    # logical (unpaged) per-sequence storage codes and scales, for the oracle
    k_seq: List[np.ndarray] = field(default_factory=list)
    v_seq: List[np.ndarray] = field(default_factory=list)
    k_scale_seq: List[Optional[np.ndarray]] = field(default_factory=list)
    v_scale_seq: List[Optional[np.ndarray]] = field(default_factory=list)

    @property
    def num_seqs(self) -> int:
        return int(self.seqlens_k.shape[0])

    @property
    def prefixes(self) -> np.ndarray:
        return (self.seqlens_k - self.n_q).astype(np.int32)

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def total_qblocks(self) -> int:
        return int(self.cu_qblocks[-1])

    @property
    def total_kblocks(self) -> int:
        return int(self.cu_kblocks[-1])

    def q_seq(self, s: int) -> np.ndarray:
        return self.q[self.cu_seqlens_q[s]:self.cu_seqlens_q[s + 1]]

    def q_scale_seq(self, s: int) -> Optional[np.ndarray]:
        if self.q_scale is None:
            return None
        return self.q_scale[self.cu_qblocks[s]:self.cu_qblocks[s + 1]]

    def causal_pairs(self) -> int:
        """Number of (q-block, k-block <= last diagonal k-block, KV head) triples."""
        B = self.cfg.block
        KB = self.cfg.kv_block or B
        tot = 0
        for s in range(self.num_seqs):
            n = int(self.n_q[s])
            P = int(self.seqlens_k[s]) - n
            for i in range(-(-n // B)):
                tot += (P + min((i + 1) * B, n) - 1) // KB + 1
        return tot * self.cfg.hkv


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def make_custom(cfg: Config, tau: Optional[float] = None, pad_fill: str = "zero",
                seq_seeds: Optional[Sequence[int]] = None) -> Workload:
    """Build a Workload for an arbitrary Config.

    pad_fill: what the unused token slots of each sequence's last page hold
    ("zero", or "nan" to check that no kernel ever reads them).
    """
    S = len(cfg.seqlens)
    assert len(cfg.prefixes) == S
    if seq_seeds is None:
        seq_seeds = cfg.seq_seeds if cfg.seq_seeds is not None else \
            tuple(cfg.seed + 1000 * r for r in range(S))
    B, ps = cfg.block, cfg.page_size
    KB = cfg.kv_block or B
    seqlens = np.array(cfg.seqlens, dtype=np.int32)
    n_q = np.array([T - P for T, P in zip(cfg.seqlens, cfg.prefixes)], dtype=np.int32)
    cu_q = np.zeros(S + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(n_q)
    cu_qb = np.zeros(S + 1, dtype=np.int32)
    cu_qb[1:] = np.cumsum([_cdiv(int(n), B) for n in n_q])
    cu_kb = np.zeros(S + 1, dtype=np.int32)
    cu_kb[1:] = np.cumsum([_cdiv(int(t), KB) for t in seqlens])
    total_q = int(cu_q[-1])

    fp8 = cfg.dtype == "fp8"
    if fp8 and ps != KB:
        raise ValueError("fp8 KV scales are per page and need page_size == the KV block")
    code_t = np.uint8 if fp8 else np.uint16
    q = np.empty((total_q, cfg.hq, cfg.d), dtype=code_t)
    q_scale = np.empty((int(cu_qb[-1]), cfg.hq), dtype=np.float32) if fp8 else None

    k_seq, v_seq, ks_seq, vs_seq = [], [], [], []
    for s in range(S):
        T, P = int(seqlens[s]), int(cfg.prefixes[s])
        Qf, Kf, Vf = _gen_sequence(cfg, T, int(seq_seeds[s]))
        Qn = Qf[P:]
        del Qf
        if fp8:
            qc, qs = quantize_blocks_e4m3(Qn, B)
            q[cu_q[s]:cu_q[s + 1]] = qc
            q_scale[cu_qb[s]:cu_qb[s + 1]] = qs
            kc, kss = quantize_blocks_e4m3(Kf, KB)
            vc, vss = quantize_blocks_e4m3(Vf, KB)
        else:
            q[cu_q[s]:cu_q[s + 1]] = f32_to_bf16_bits(Qn)
            kc, kss = f32_to_bf16_bits(Kf), None
            vc, vss = f32_to_bf16_bits(Vf), None
        del Qn, Kf, Vf
        k_seq.append(kc)
        v_seq.append(vc)
        ks_seq.append(kss)
        vs_seq.append(vss)

    # paging
    npages = [_cdiv(int(t), ps) for t in seqlens]
    num_pages = int(sum(npages))
    max_pages = max(npages) if npages else 0
    logical_page = np.arange(num_pages, dtype=np.int64)
    if cfg.shuffle_pages:
        perm = np.random.Generator(np.random.PCG64(cfg.shuffle_seed)).permutation(num_pages)
    else:
        perm = logical_page
    page_table = np.zeros((S, max(1, max_pages)), dtype=np.int32)
    fill = {"zero": 0, "nan": (0x7F if fp8 else 0x7FC0)}[pad_fill]
    k_pages = np.empty((num_pages, ps, cfg.hkv, cfg.d), dtype=code_t)
    v_pages = np.empty_like(k_pages)
    k_scale = np.ones((num_pages, cfg.hkv), dtype=np.float32) if fp8 else None
    v_scale = np.ones((num_pages, cfg.hkv), dtype=np.float32) if fp8 else None
    base = 0
    for s in range(S):
        T = int(seqlens[s])
        for j in range(npages[s]):
            phys = int(perm[base + j])
            page_table[s, j] = phys
            lo, hi = j * ps, min((j + 1) * ps, T)
            k_pages[phys, :hi - lo] = k_seq[s][lo:hi]
            v_pages[phys, :hi - lo] = v_seq[s][lo:hi]
            if hi - lo < ps:
                k_pages[phys, hi - lo:] = fill
                v_pages[phys, hi - lo:] = fill
            if fp8:
                k_scale[phys] = ks_seq[s][j]
                v_scale[phys] = vs_seq[s][j]
        base += npages[s]

    if tau is None:
        tau = cfg.tau
    if tau is None:
        raise ValueError(f"config {cfg.name} needs a calibrated tau (pass tau=...)")
    return Workload(cfg=cfg, tau=float(tau), seqlens_k=seqlens, n_q=n_q, cu_seqlens_q=cu_q,
                    cu_qblocks=cu_qb, cu_kblocks=cu_kb, q=q, q_scale=q_scale,
                    k_pages=k_pages, v_pages=v_pages, k_scale=k_scale, v_scale=v_scale,
                    page_table=page_table, k_seq=k_seq, v_seq=v_seq,
                    k_scale_seq=ks_seq, v_scale_seq=vs_seq)


def make(name: str, tau: Optional[float] = None, pad_fill: str = "zero") -> Workload:
    """Build one of the named workloads in CONFIGS."""
    return make_custom(CONFIGS[name], tau=tau, pad_fill=pad_fill)
