"""Plain fp64 attention: the definition written out, no tiling, no online softmax.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed ([FA4-decode] §Recap on the FA4 forward pass):
    S = Q K^T / sqrt(d),  P = softmax(S) row-wise,  O = P V.
Tiled online-softmax kernels reach exactly this result up to rounding order
(same section), so the oracle is the definition itself, in fp64, from the same
bf16 or fp16 bytes (both convert to fp64 exactly).

Readings where the pages leave a step open (each is listed in the design notes):
  * GQA head map: query head h reads KV head h // G with G = Hq / Hkv, i.e. the
    G heads that share a KV head are contiguous ([FA4-edges] §Edge 2 · GQA packs
    the GQA_RATIO query heads of one KV head into one tile).
  * Causal alignment: bottom-right. With L keys of which the last sq belong to
    the sq new queries, query t sees keys j <= L - sq + t. For prefill with
    Sq == Sk this is the usual lower triangle ([FA4-edges] §Edge 1 · causal
    masking: a query must not attend to keys in its future).
  * LSE is the natural log of sum_j exp(s_j) (the convention the backward pass
    consumes as P = exp(S - L), [FA4-bwd] §Recap on the FA4 backward pass).
  * An empty visible set gives O = 0 and LSE = -inf ([GQA-SM100] §Removing the
    max reset: an entirely empty sequence produces zero output).
"""
from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact bf16 -> fp64: the bf16 pattern is the top half of a float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact IEEE binary16 -> fp64 (NumPy's half-precision type as the decoder)."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def to_f64(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Decode 16-bit element patterns of the given type ("bf16" or "f16") to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    raise ValueError(f"unknown element type {dtype!r}")


def _visible(L: int, sq: int, t: int, causal: bool) -> int:
    """Number of visible keys (a prefix [0, n)) for query t of sq, L keys."""
    if not causal:
        return max(L, 0)
    return max(0, min(L, L - sq + t + 1))


def _attend(qrows: np.ndarray, kk: np.ndarray, vv: np.ndarray, nvis: np.ndarray, d: int):
    """qrows [R, d], kk/vv [L, d], nvis [R] -> O [R, d], LSE [R] (fp64).

    Row r attends to keys [0, nvis[r]). Scores are formed in full, masked to
    -inf beyond the visible prefix, then softmax-normalised per row.
    """
    R, L = qrows.shape[0], kk.shape[0]
    O = np.zeros((R, d), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    if L == 0 or R == 0:
        return O, lse
    s = (qrows @ kk.T) / math.sqrt(d)  # [R, L]
    cols = np.arange(L)[None, :]
    s = np.where(cols < nvis[:, None], s, -np.inf)
    live = nvis > 0
    if not np.any(live):
        return O, lse
    s = s[live]
    m = np.max(s, axis=1, keepdims=True)
    p = np.exp(s - m)
    ell = np.sum(p, axis=1, keepdims=True)
    O[live] = (p @ vv) / ell
    lse[live] = (m + np.log(ell))[:, 0]
    return O, lse


def attention(q, k, v, seqlens=None, causal=True, row_block=512, dtype="bf16"):
    """Reference attention for decode and prefill.

    q: uint16 bf16 bits [B, sq, Hq, d]; k, v: uint16 [B, S, Hkv, d].
    seqlens: int[B] (decode: keys [0, L_b) of the cache are valid, L_b clamped
    to [0, S]); None means every row has S keys (prefill).
    causal: bottom-right causal mask among the sq queries.
    Returns (O fp64 [B, sq, Hq, d], LSE fp64 [B, Hq, sq]).
    Work is cut per (batch, KV head) and into blocks of query rows only to bound
    memory; each row is still computed from the full definition.
    """
    B, sq, Hq, d = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    G = Hq // Hkv
    O = np.zeros((B, sq, Hq, d), dtype=np.float64)
    LSE = np.full((B, Hq, sq), -np.inf, dtype=np.float64)
    for b in range(B):
        L = S if seqlens is None else int(min(max(int(seqlens[b]), 0), S))
        for g in range(Hkv):
            kk = to_f64(k[b, :L, g], dtype)
            vv = to_f64(v[b, :L, g], dtype)
            for t0 in range(0, sq, max(1, row_block // G)):
                t1 = min(sq, t0 + max(1, row_block // G))
                # rows ordered (t, head-in-group)
                qr = to_f64(q[b, t0:t1, g * G:(g + 1) * G], dtype).reshape(-1, d)
                nv = np.array([_visible(L, sq, t, causal) for t in range(t0, t1)
                               for _ in range(G)], dtype=np.int64)
                Lmax = int(nv.max()) if nv.size else 0
                o, lse = _attend(qr, kk[:Lmax], vv[:Lmax], nv, d)
                O[b, t0:t1, g * G:(g + 1) * G] = o.reshape(t1 - t0, G, d)
                LSE[b, g * G:(g + 1) * G, t0:t1] = lse.reshape(t1 - t0, G).T
    return O, LSE


def attention_rows(q, k, v, rows, seqlens=None, causal=True, dtype="bf16"):
    """Reference O and LSE for selected (b, t, h) rows only (for large shapes).

    rows: iterable of (b, t, h). Returns (O [n, d], LSE [n]) in the given order.
    """
    B, sq, Hq, d = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    rows = list(rows)
    O = np.zeros((len(rows), d), dtype=np.float64)
    LSE = np.full(len(rows), -np.inf, dtype=np.float64)
    for i, (b, t, h) in enumerate(rows):
        L = S if seqlens is None else int(min(max(int(seqlens[b]), 0), S))
        n = _visible(L, sq, t, causal)
        g = h // G
        qr = to_f64(q[b, t, h], dtype).reshape(1, d)
        o, lse = _attend(qr, to_f64(k[b, :n, g], dtype), to_f64(v[b, :n, g], dtype),
                         np.array([n]), d)
        O[i], LSE[i] = o[0], lse[0]
    return O, LSE


def probabilities(q, k, b, t, h, seqlens=None, causal=True, dtype="bf16"):
    """The softmax row P[b, h, t, :] over all S cache positions (zeros where masked)."""
    B, sq, Hq, d = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    L = S if seqlens is None else int(min(max(int(seqlens[b]), 0), S))
    n = _visible(L, sq, t, causal)
    out = np.zeros(S, dtype=np.float64)
    if n == 0:
        return out
    s = to_f64(k[b, :n, h // G], dtype) @ to_f64(q[b, t, h], dtype) / math.sqrt(d)
    e = np.exp(s - s.max())
    out[:n] = e / e.sum()
    return out


def decode_row_counts(L: int, sq: int, causal: bool = True):
    """Visible key counts of the sq query rows (exposed for tests)."""
    return [_visible(L, sq, t, causal) for t in range(sq)]


# --- split-KV partials and their merge ---------------------------------------
#
# [GQA-SM100] §Combining the KV splits: each split s of the key range returns an
# unnormalised output, its maximum and its denominator (m_s, l_s, O~_s); the
# maxima use base-2 score scaling. The merge brings all partials to a common
# scale before normalising. The formula itself did not survive on the page; it
# is reconstructed from the combine path shown in §Removing the max reset:
#     M  = max_s m_s                       (empty splits have m_s = -inf, skipped)
#     w_s = 2^(m_s - M)
#     l  = sum_s w_s l_s,   O = (sum_s w_s O~_s) / l
# and an entirely empty row gives O = 0.

_LOG2E = 1.0 / math.log(2.0)


def split_partials(qrow: np.ndarray, kk: np.ndarray, vv: np.ndarray, bounds):
    """Per-split base-2 partials of one query row (fp64 vectors, not bf16 bits).

    bounds: list of (lo, hi) key ranges. Returns lists m, l, Ot (m in base 2:
    m_s = max_j s_j * log2(e), l_s = sum_j 2^(s_j log2 e - m_s),
    Ot_s = sum_j 2^(s_j log2 e - m_s) v_j).
    """
    d = qrow.shape[0]
    ms, ls, Os = [], [], []
    for lo, hi in bounds:
        if hi <= lo:
            ms.append(-np.inf)
            ls.append(0.0)
            Os.append(np.zeros(d))
            continue
        s2 = (kk[lo:hi] @ qrow) / math.sqrt(d) * _LOG2E
        m = float(np.max(s2))
        w = np.exp2(s2 - m)
        ms.append(m)
        ls.append(float(np.sum(w)))
        Os.append(w @ vv[lo:hi])
    return ms, ls, Os


def combine_partials(ms, ls, Os):
    """Merge base-2 split partials; returns (O, LSE natural log)."""
    d = Os[0].shape[0] if Os else 0
    live = [i for i, m in enumerate(ms) if m > -np.inf]
    if not live:
        return np.zeros(d), -np.inf
    M = max(ms[i] for i in live)
    ell = 0.0
    acc = np.zeros(d)
    for i in live:  # fixed split order
        w = 2.0 ** (ms[i] - M)
        ell += w * ls[i]
        acc += w * Os[i]
    return acc / ell, math.log(2.0) * (M + math.log2(ell))


def attention_varlen(q, k, v, cu_q, cu_k, causal=True, dtype="bf16"):
    """Reference attention over a packed variable-length batch.

    q: uint16 [total_q, Hq, d]; k, v: uint16 [total_k, Hkv, d]; cu_q, cu_k:
    int[B + 1] row offsets of each sequence. Each sequence is an independent
    prefill (bottom-right causal within it when causal). Returns
    (O fp64 [total_q, Hq, d], LSE fp64 [Hq, total_q]).
    """
    tq, Hq, d = q.shape
    O = np.zeros((tq, Hq, d), dtype=np.float64)
    LSE = np.full((Hq, tq), -np.inf, dtype=np.float64)
    for b in range(len(cu_q) - 1):
        s0, s1 = int(cu_q[b]), int(cu_q[b + 1])
        t0, t1 = int(cu_k[b]), int(cu_k[b + 1])
        if s1 <= s0:
            continue
        o, lse = attention(q[None, s0:s1], k[None, t0:t1], v[None, t0:t1], None, causal, dtype=dtype)
        O[s0:s1] = o[0]
        LSE[:, s0:s1] = lse[0]
    return O, LSE
