"""Scalar brute-force attention in pure Python (tiny shapes only).

TEST INFRASTRUCTURE ONLY (see the package docstring). Written independently of
``attention.py``: own bf16 decoding (struct), own masking loop, math.fsum, and
the log-sum-exp taken as log(sum exp(s - max)) + max per row.
Definition: [FA4-decode] §Recap on the FA4 forward pass; GQA head map and
bottom-right causal reading as stated in ``attention.py``.
"""
from __future__ import annotations

import math
import struct


def _bf16(x: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(x) & 0xFFFF) << 16))[0]


def _f16(x: int) -> float:
    return struct.unpack("<e", struct.pack("<H", int(x) & 0xFFFF))[0]


def brute_attention(q, k, v, seqlens=None, causal=True, dtype="bf16"):
    """Nested-list result: O[b][t][h][e], LSE[b][h][t] (floats)."""
    dec = {"bf16": _bf16, "f16": _f16}[dtype]
    B, sq, Hq, d = (int(x) for x in q.shape)
    S, Hkv = int(k.shape[1]), int(k.shape[2])
    G = Hq // Hkv
    O = [[[[0.0] * d for _ in range(Hq)] for _ in range(sq)] for _ in range(B)]
    LSE = [[[float("-inf")] * sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        L = S if seqlens is None else min(max(int(seqlens[b]), 0), S)
        for h in range(Hq):
            g = h // G
            for t in range(sq):
                js = [j for j in range(L) if (not causal) or j <= L - sq + t]
                if not js:
                    continue
                qv = [dec(q[b, t, h, e]) for e in range(d)]
                sc = []
                for j in js:
                    dot = math.fsum(qv[e] * dec(k[b, j, g, e]) for e in range(d))
                    sc.append(dot / math.sqrt(d))
                mx = max(sc)
                ws = [math.exp(s - mx) for s in sc]
                den = math.fsum(ws)
                for e in range(d):
                    O[b][t][h][e] = math.fsum(w * dec(v[b, j, g, e]) for w, j in zip(ws, js)) / den
                LSE[b][h][t] = mx + math.log(den)
    return O, LSE
