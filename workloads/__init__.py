"""Seeded synthetic inputs for attention decode and causal prefill.

This module holds no attention arithmetic. It fixes the five workload shapes,
draws N(0, 1) float32 values from counter-keyed NumPy PCG64 streams, and rounds
them to bfloat16 (default) or IEEE fp16 bit patterns (round to nearest, ties to
even). Both the CPU oracle and the GPU path read the same uint16 bit patterns
produced here.

Recipe (deterministic, independent of thread count):
  * every tensor is cut into chunks of CHUNK elements in C order; chunk ``i``
    of tensor ``tid`` (sub-stream ``sub``, the batch row for KV-cache rows)
    under seed ``seed`` is drawn by
    ``default_rng(SeedSequence([seed, tid, sub, i])).standard_normal(n, float32)``;
  * decode inputs: KV lengths first (stream ``TID_LEN``), then q, then for each
    batch row b the K rows [0, L_b) and the V rows [0, L_b); cache rows at and
    beyond L_b are filled with ``pad`` (NaN by default, so that a kernel that
    reads past a sequence end poisons its output);
  * prefill inputs: q, k, v in that order.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22
TID_Q, TID_K, TID_V, TID_LEN, TID_DO = 1, 2, 3, 4, 5
BF16_NAN = np.uint16(0x7FC0)
BF16_ZERO = np.uint16(0)
F16_NAN = np.uint16(0x7E00)
NAN_BITS = {"bf16": BF16_NAN, "f16": F16_NAN}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (nearest, ties to even); return uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def normal_bits(seed: int, tid: int, n: int, sub: int = 0, dtype: str = "bf16") -> np.ndarray:
    """n bit patterns (bf16, or fp16 with dtype="f16") of N(0,1) draws from stream (seed, tid, sub)."""
    to_bits = {"bf16": f32_to_bf16_bits, "f16": f32_to_f16_bits}[dtype]
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(i: int) -> None:
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        g = np.random.default_rng(np.random.SeedSequence([seed, tid, sub, i]))
        out[lo:hi] = to_bits(g.standard_normal(hi - lo, dtype=np.float32))

    if nchunks <= 1:
        for i in range(nchunks):
            work(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def normal_bf16(seed: int, tid: int, n: int, sub: int = 0) -> np.ndarray:
    """n bf16 bit patterns of N(0,1) draws from stream (seed, tid, sub)."""
    return normal_bits(seed, tid, n, sub, "bf16")


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    d: int
    seqlen_q: int
    max_seqlen_k: int
    len_lo: int  # KV lengths are uniform integers in [len_lo, len_hi]
    len_hi: int
    seed: int
    note: str = ""

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    d: int
    seqlen: int
    causal: bool
    seed: int
    note: str = ""


# The five workloads, with seeds 1000 + index (index 0..4).
DECODE_CONFIGS = {
    "gqa-decode-small": DecodeConfig("gqa-decode-small", 1, 8, 1, 64, 1, 512, 512, 512, 1000,
                       "single-token GQA decode, 8 q heads on 1 kv head, d=64, L=512"),
    "gqa-decode": DecodeConfig("gqa-decode", 32, 64, 8, 128, 1, 8192, 1024, 8192, 1001,
                       "GQA decode, B=32, 64/8 heads, d=128, L ~ U{1024..8192}"),
    "multi-token-decode": DecodeConfig("multi-token-decode", 16, 32, 8, 64, 4, 4096, 4096, 4096, 1002,
                       "multi-token decode, B=16, 32/8 heads, d=64, 4 causal new tokens, L=4096"),
    "long-context-decode": DecodeConfig("long-context-decode", 4, 32, 8, 128, 1, 131072, 131072, 131072, 1003,
                       "long-context decode, B=4, 32/8 heads, d=128, L=131072"),
}
PREFILL_CONFIGS = {
    "causal-prefill": PrefillConfig("causal-prefill", 2, 32, 32, 128, 8192, True, 1004,
                        "causal prefill, B=2, 32 heads MHA, d=128, S=8192"),
}


@dataclass
class DecodeInputs:
    q: np.ndarray  # uint16 [B, sq, Hq, d]
    k: np.ndarray  # uint16 [B, S_max, Hkv, d]
    v: np.ndarray  # uint16 [B, S_max, Hkv, d]
    seqlens: np.ndarray  # int32 [B]
    meta: dict = field(default_factory=dict)
    dtype: str = "bf16"  # element type of q, k, v: "bf16" or "f16"


@dataclass
class PrefillInputs:
    q: np.ndarray  # uint16 [B, S, Hq, d]
    k: np.ndarray  # uint16 [B, S, Hkv, d]
    v: np.ndarray  # uint16 [B, S, Hkv, d]
    meta: dict = field(default_factory=dict)
    dtype: str = "bf16"


def draw_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    if lo == hi:
        return np.full(batch, lo, dtype=np.int32)
    g = np.random.default_rng(np.random.SeedSequence([seed, TID_LEN, 0, 0]))
    return g.integers(lo, hi + 1, size=batch).astype(np.int32)


def make_decode(batch, n_q_heads, n_kv_heads, d, seqlen_q, max_seqlen_k, seqlens,
                seed, pad=None, dtype="bf16") -> DecodeInputs:
    """Decode inputs of an arbitrary shape with given per-sequence lengths.

    pad: bit pattern of the cache rows past each sequence end (default: NaN of
    the element type)."""
    if pad is None:
        pad = NAN_BITS[dtype]
    seqlens = np.asarray(seqlens, dtype=np.int32).reshape(batch)
    q = normal_bits(seed, TID_Q, batch * seqlen_q * n_q_heads * d, dtype=dtype).reshape(
        batch, seqlen_q, n_q_heads, d)
    k = np.full((batch, max_seqlen_k, n_kv_heads, d), pad, dtype=np.uint16)
    v = np.full((batch, max_seqlen_k, n_kv_heads, d), pad, dtype=np.uint16)
    row = n_kv_heads * d
    for b in range(batch):
        L = int(min(max(seqlens[b], 0), max_seqlen_k))
        if L == 0:
            continue
        k[b, :L] = normal_bits(seed, TID_K, L * row, sub=b, dtype=dtype).reshape(L, n_kv_heads, d)
        v[b, :L] = normal_bits(seed, TID_V, L * row, sub=b, dtype=dtype).reshape(L, n_kv_heads, d)
    return DecodeInputs(q, k, v, seqlens, dict(seed=seed), dtype)


def decode_inputs(cfg: DecodeConfig | str, pad=None) -> DecodeInputs:
    if isinstance(cfg, str):
        cfg = DECODE_CONFIGS[cfg]
    lens = draw_lengths(cfg.seed, cfg.batch, cfg.len_lo, cfg.len_hi)
    out = make_decode(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.d, cfg.seqlen_q,
                      cfg.max_seqlen_k, lens, cfg.seed, pad)
    out.meta["config"] = cfg.name
    return out


def make_prefill(batch, n_q_heads, n_kv_heads, d, seqlen_q, seqlen_k, seed,
                 dtype="bf16") -> PrefillInputs:
    q = normal_bits(seed, TID_Q, batch * seqlen_q * n_q_heads * d, dtype=dtype).reshape(
        batch, seqlen_q, n_q_heads, d)
    k = normal_bits(seed, TID_K, batch * seqlen_k * n_kv_heads * d, dtype=dtype).reshape(
        batch, seqlen_k, n_kv_heads, d)
    v = normal_bits(seed, TID_V, batch * seqlen_k * n_kv_heads * d, dtype=dtype).reshape(
        batch, seqlen_k, n_kv_heads, d)
    return PrefillInputs(q, k, v, dict(seed=seed), dtype)


@dataclass
class VarlenInputs:
    q: np.ndarray        # uint16 [total_q, Hq, d], sequences packed back to back
    k: np.ndarray        # uint16 [total_k, Hkv, d]
    v: np.ndarray        # uint16 [total_k, Hkv, d]
    cu_q: np.ndarray     # int32 [B + 1], cu_q[b] = first query row of sequence b
    cu_k: np.ndarray     # int32 [B + 1]
    meta: dict = field(default_factory=dict)
    dtype: str = "bf16"


def make_varlen(lens_q, lens_k, n_q_heads, n_kv_heads, d, seed, dtype="bf16") -> VarlenInputs:
    """Packed variable-length batch: sequence b has lens_q[b] queries and lens_k[b] keys."""
    lq = np.asarray(lens_q, dtype=np.int64)
    lk = np.asarray(lens_k, dtype=np.int64)
    if lq.shape != lk.shape or (lq < 0).any() or (lk < 0).any():
        raise ValueError("lens_q and lens_k must be non-negative and of equal length")
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = normal_bits(seed, TID_Q, tq * n_q_heads * d, dtype=dtype).reshape(tq, n_q_heads, d)
    k = normal_bits(seed, TID_K, tk * n_kv_heads * d, dtype=dtype).reshape(tk, n_kv_heads, d)
    v = normal_bits(seed, TID_V, tk * n_kv_heads * d, dtype=dtype).reshape(tk, n_kv_heads, d)
    return VarlenInputs(q, k, v, cu_q, cu_k, dict(seed=seed), dtype)


def varlen_prefill_inputs(seed: int = 1006, batch: int = 16, lo: int = 256, hi: int = 4096,
                          n_heads: int = 32, d: int = 128) -> VarlenInputs:
    """Variable-length causal prefill: `batch` sequences with query = key lengths
    uniform in [lo, hi] (stream TID_LEN), MHA, packed."""
    lens = draw_lengths(seed, batch, lo, hi)
    out = make_varlen(lens, lens, n_heads, n_heads, d, seed)
    out.meta["config"] = f"varlen-prefill b={batch} h={n_heads} d={d} len~U[{lo},{hi}] (seed {seed})"
    return out


def make_grad_out(q: np.ndarray, seed: int, dtype: str = "bf16") -> np.ndarray:
    """Output gradient dO shaped like q: N(0,1) draws of stream (seed, TID_DO)."""
    return normal_bits(seed, TID_DO, q.size, dtype=dtype).reshape(q.shape)


def prefill_inputs(cfg: PrefillConfig | str) -> PrefillInputs:
    if isinstance(cfg, str):
        cfg = PREFILL_CONFIGS[cfg]
    out = make_prefill(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.d, cfg.seqlen,
                       cfg.seqlen, cfg.seed)
    out.meta["config"] = cfg.name
    return out
