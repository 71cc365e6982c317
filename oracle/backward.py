"""Plain fp64 attention backward: the gradient formulas written out, no tiling.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition ([FA4-bwd] §Recap on the FA4 backward pass), with the forward's
scale s = 1/sqrt(d) written explicitly (the recap leaves it folded into S):
    S  = s Q K^T,        P  = exp(S - L)   (L: natural-log LSE of the row),
    dP = dO V^T,         dS = P o (dP - D),
    dV = P^T dO,         dK = s dS^T Q,     dQ = s dS K.

Readings where the pages leave a step open (each is listed in the design notes):
  * D is used but not defined on the page. It is the row sum of P o dP, which
    equals the row sum of dO o O because O = P V; the oracle forms it as
    rowsum(P o dP) from its own exact P.
  * Masked (query, key) pairs have P = 0 and contribute nothing; a query row
    that sees no key has P = 0 everywhere, so dQ = 0 there.
  * GQA: the dK and dV of a KV head are the sums over the G query heads that
    read it (the forward's head map, query head h reads KV head h // G).
  * Causal masking is bottom-right aligned, as in the forward: query i of Sq
    sees keys j <= i + Sk - Sq.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import to_f64


def _mask(Sq: int, Sk: int, causal: bool, i0: int = 0, i1: int | None = None) -> np.ndarray:
    """Boolean visibility of keys [0, Sk) for query rows [i0, i1)."""
    i1 = Sq if i1 is None else i1
    rows = np.arange(i0, i1)[:, None]
    cols = np.arange(Sk)[None, :]
    if not causal:
        return np.ones((i1 - i0, Sk), dtype=bool)
    return cols <= rows + (Sk - Sq)


def _probs(qq: np.ndarray, kk: np.ndarray, vis: np.ndarray, scale: float) -> np.ndarray:
    """Exact softmax rows P (zeros where masked or where a row sees nothing)."""
    s = np.where(vis, (qq @ kk.T) * scale, -np.inf)
    live = vis.any(axis=1)
    p = np.zeros_like(s)
    if np.any(live):
        sl = s[live]
        e = np.exp(sl - sl.max(axis=1, keepdims=True))
        p[live] = e / e.sum(axis=1, keepdims=True)
    return p


def backward_f64(q, k, v, do, causal=True, row_block=512):
    """Gradients of attention from fp64 arrays.

    q, do: [B, Sq, Hq, d]; k, v: [B, Sk, Hkv, d] (float64).
    Returns (dq [B, Sq, Hq, d], dk [B, Sk, Hkv, d], dv [B, Sk, Hkv, d],
    D [B, Hq, Sq]). Query rows are processed in blocks only to bound memory;
    dK and dV sum the blocks' contributions.
    """
    B, Sq, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros((B, Sq, Hq, d))
    dk = np.zeros((B, Sk, Hkv, d))
    dv = np.zeros((B, Sk, Hkv, d))
    D = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            kk, vv = k[b, :, g], v[b, :, g]
            for i0 in range(0, Sq, row_block):
                i1 = min(Sq, i0 + row_block)
                qq, dd = q[b, i0:i1, h], do[b, i0:i1, h]
                p = _probs(qq, kk, _mask(Sq, Sk, causal, i0, i1), scale)
                dp = dd @ vv.T
                Di = np.sum(p * dp, axis=1)
                ds = p * (dp - Di[:, None])
                dv[b, :, g] += p.T @ dd
                dk[b, :, g] += scale * (ds.T @ qq)
                dq[b, i0:i1, h] = scale * (ds @ kk)
                D[b, h, i0:i1] = Di
    return dq, dk, dv, D


def attention_backward(q, k, v, do, causal=True, dtype="bf16", row_block=512):
    """attention gradients from 16-bit element patterns (bf16 or fp16).

    q, do: uint16 [B, Sq, Hq, d]; k, v: uint16 [B, Sk, Hkv, d]. The inputs
    convert to fp64 exactly; all arithmetic is fp64 and nothing is rounded.
    """
    return backward_f64(to_f64(q, dtype), to_f64(k, dtype), to_f64(v, dtype), to_f64(do, dtype),
                        causal, row_block)


def backward_kv_head(q, k, v, do, b, g, causal=True, dtype="bf16", row_block=512):
    """dK and dV of one (batch b, KV head g), and dQ and D of its G query heads.

    For large shapes, where only a few heads can be checked. Returns
    (dq [Sq, G, d], dk [Sk, d], dv [Sk, d], D [G, Sq]).
    """
    Hq, Hkv = q.shape[2], k.shape[2]
    G = Hq // Hkv
    sl = slice(g * G, (g + 1) * G)
    dq, dk, dv, D = backward_f64(to_f64(q[b:b + 1, :, sl], dtype), to_f64(k[b:b + 1, :, g:g + 1], dtype),
                                 to_f64(v[b:b + 1, :, g:g + 1], dtype), to_f64(do[b:b + 1, :, sl], dtype),
                                 causal, row_block)
    return dq[0], dk[0, :, 0], dv[0, :, 0], D[0]


def backward_error_scales(q, k, v, do, causal=True, dtype="bf16", row_block=512):
    """Sums of absolute values of the terms of each gradient element.

    A product rounded to a precision with unit roundoff u (relative error at
    most u per term) errs by at most u times the sum of its terms' absolute
    values. Returns (eq [B, Sq, Hq, d], ek [B, Sk, Hkv, d], ev [B, Sk, Hkv, d]):
        ev = P^T |dO|,   ek = s A^T |Q|,   eq = s A |K|,
    with A = |dS| + 2 P o delta and delta_i = sum_d |dO_i| (P |V|)_i, the scale
    by which an error of O (itself bounded by u (P |V|)) moves D = rowsum(dO o O).
    """
    qf, kf, vf, dof = (to_f64(t, dtype) for t in (q, k, v, do))
    B, Sq, Hq, d = qf.shape
    Sk, Hkv = kf.shape[1], kf.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    eq = np.zeros((B, Sq, Hq, d))
    ek = np.zeros((B, Sk, Hkv, d))
    ev = np.zeros((B, Sk, Hkv, d))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            kk, vv = kf[b, :, g], vf[b, :, g]
            for i0 in range(0, Sq, row_block):
                i1 = min(Sq, i0 + row_block)
                qq, dd = qf[b, i0:i1, h], dof[b, i0:i1, h]
                p = _probs(qq, kk, _mask(Sq, Sk, causal, i0, i1), scale)
                dp = dd @ vv.T
                ds = p * (dp - np.sum(p * dp, axis=1)[:, None])
                delta = np.sum(np.abs(dd) * (p @ np.abs(vv)), axis=1)
                a = np.abs(ds) + 2.0 * p * delta[:, None]
                ev[b, :, g] += p.T @ np.abs(dd)
                ek[b, :, g] += scale * (a.T @ np.abs(qq))
                eq[b, i0:i1, h] = scale * (a @ np.abs(kk))
    return eq, ek, ev


def _varlen_apply(fn, q, k, v, do, cu_q, cu_k, causal, dtype):
    """Run a per-batch backward function on each sequence of a packed batch; pack the results."""
    tq, Hq, d = q.shape
    tk, Hkv = k.shape[0], k.shape[1]
    out_q, out_k, out_v = np.zeros((tq, Hq, d)), np.zeros((tk, Hkv, d)), np.zeros((tk, Hkv, d))
    for b in range(len(cu_q) - 1):
        s0, s1, t0, t1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if s1 <= s0 or t1 <= t0:
            continue
        r = fn(q[None, s0:s1], k[None, t0:t1], v[None, t0:t1], do[None, s0:s1], causal, dtype=dtype)
        out_q[s0:s1], out_k[t0:t1], out_v[t0:t1] = r[0][0], r[1][0], r[2][0]
    return out_q, out_k, out_v


def attention_backward_varlen(q, k, v, do, cu_q, cu_k, causal=True, dtype="bf16"):
    """dq [total_q, Hq, d], dk and dv [total_k, Hkv, d] of a packed variable-length batch
    (uint16 element patterns in, fp64 out): each sequence is an independent problem."""
    return _varlen_apply(attention_backward, q, k, v, do, cu_q, cu_k, causal, dtype)


def backward_error_scales_varlen(q, k, v, do, cu_q, cu_k, causal=True, dtype="bf16"):
    """backward_error_scales of each sequence of a packed batch, packed."""
    return _varlen_apply(backward_error_scales, q, k, v, do, cu_q, cu_k, causal, dtype)
