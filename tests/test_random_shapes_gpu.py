"""Seeded random shapes through every entry point, each against the fp64 oracle.

The hand-picked cases elsewhere aim at specific edges; these sweep the
parameter space (head sizes, group sizes, new-token counts, ragged and empty
lengths, piece counts, element types, causal or not) with a fixed seed, so a
failure names its case and reproduces.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests import _gpu as G
from tests._libload import ensure_built

pytestmark = pytest.mark.gpu
U = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


@pytest.fixture(scope="module")
def aa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    ensure_built()
    import attention_attn_decode_amd as mod
    return mod


def _decode_cases(n, seed=901):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128, 256]))
        cap = 16 if d == 256 else 32
        sq = int(rng.choice([1, 1, 2, 4]))
        G_ = int(rng.choice([g for g in (1, 2, 4, 8, 16, 32) if g * sq <= cap]))
        Hkv = int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 9))
        lens = [int(x) for x in rng.integers(0, 2500, B)]
        if rng.random() < 0.3:
            lens[int(rng.integers(0, B))] = 0
        lens = [max(L, sq) if L else 0 for L in lens]
        ns = int(rng.choice([0, 0, 1, 2, 7, 64, 300]))
        dtype = "f16" if rng.random() < 0.25 else "bf16"
        out.append((i, B, G_ * Hkv, Hkv, d, sq, lens, ns, dtype))
    return out


@pytest.mark.parametrize("case", _decode_cases(64), ids=lambda c: f"dec{c[0]}")
def test_random_decode(aa, case):
    i, B, Hq, Hkv, d, sq, lens, ns, dtype = case
    torch = G.torch()
    S = max(max(lens), 1) + 5
    x = wl.make_decode(B, Hq, Hkv, d, sq, S, lens, seed=911 + i, pad=wl.BF16_NAN, dtype=dtype)
    q, k, v = G.dev_bf16(x.q, x.dtype), G.dev_bf16(x.k, x.dtype), G.dev_bf16(x.v, x.dtype)
    o = G.nan_like_bf16((B, sq, Hq, d), x.dtype)
    lse = G.nan_f32((B, Hq, sq))
    nbytes = aa.attn_decode_workspace_size(B, Hq, Hkv, sq, d, S, ns)
    ws = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    aa.attn_decode(q, k, v, G.dev_i32(x.seqlens), o, lse, workspace=ws, num_splits=ns)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, x.seqlens, True, dtype=x.dtype)
    G.assert_parity(G.host_f64(o), G.host_f64(lse), O_ref, L_ref, f"decode case {case}")


def _prefill_cases(n, seed=921, dims=(64, 128)):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice(dims))
        Hkv = int(rng.choice([1, 2, 4]))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 3))
        Sq = int(rng.integers(1, 700))
        Sk = int(rng.choice([Sq, int(rng.integers(1, 900))]))
        causal = bool(rng.random() < 0.7)
        dtype = "f16" if rng.random() < 0.25 else "bf16"
        out.append((i, B, Sq, Sk, Hq, Hkv, d, causal, dtype))
    return out


@pytest.mark.parametrize("case", _prefill_cases(32) + [(32 + c[0],) + c[1:] for c in _prefill_cases(12, seed=927, dims=(256,))],
                         ids=lambda c: f"fwd{c[0]}")
def test_random_prefill(aa, case):
    i, B, Sq, Sk, Hq, Hkv, d, causal, dtype = case
    torch = G.torch()
    x = wl.make_prefill(B, Hq, Hkv, d, Sq, Sk, seed=931 + i, dtype=dtype)
    q, k, v = G.dev_bf16(x.q, x.dtype), G.dev_bf16(x.k, x.dtype), G.dev_bf16(x.v, x.dtype)
    o = G.nan_like_bf16((B, Sq, Hq, d), x.dtype)
    lse = G.nan_f32((B, Hq, Sq))
    aa.attn_fwd(q, k, v, o, lse, causal=causal)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, None, causal, dtype=x.dtype)
    G.assert_parity(G.host_f64(o), G.host_f64(lse), O_ref, L_ref, f"prefill case {case}")


def _grad_parity(got, ref, scale, u, tag):
    assert not np.isnan(got).any(), f"{tag}: NaN"
    bound = 2.0 * u * (scale + np.abs(ref)) + 1e-6 * np.abs(ref).max()
    worst = float((np.abs(got - ref) / bound).max())
    assert worst <= 1.0, f"{tag}: max err/bound = {worst:.3f}"


@pytest.mark.parametrize("case", _prefill_cases(24, seed=941), ids=lambda c: f"bwd{c[0]}")
def test_random_backward(aa, case):
    """Forward and backward on the same random shape (gradient bound as in the backward tests)."""
    i, B, Sq, Sk, Hq, Hkv, d, causal, dtype = case
    torch = G.torch()
    x = wl.make_prefill(B, Hq, Hkv, d, Sq, Sk, seed=951 + i, dtype=dtype)
    do_bits = wl.make_grad_out(x.q, 961 + i, dtype=dtype)
    q, k, v = G.dev_bf16(x.q, x.dtype), G.dev_bf16(x.k, x.dtype), G.dev_bf16(x.v, x.dtype)
    do = G.dev_bf16(do_bits, x.dtype)
    o = G.nan_like_bf16(q.shape, x.dtype)
    lse = G.nan_f32((B, Hq, Sq))
    aa.attn_fwd(q, k, v, o, lse, causal=causal)
    dq, dk, dv = (G.nan_like_bf16(t.shape, x.dtype) for t in (q, k, v))
    ws = torch.full((aa.attn_bwd_workspace_size(B, Hq, Sq) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    aa.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv, _ = oracle.attention_backward(x.q, x.k, x.v, do_bits, causal, dtype=x.dtype)
    eq, ek, ev = oracle.backward_error_scales(x.q, x.k, x.v, do_bits, causal, dtype=x.dtype)
    u = U[x.dtype]
    _grad_parity(G.host_f64(dq), rq, eq, u, f"backward case {case} dq")
    _grad_parity(G.host_f64(dk), rk, ek, u, f"backward case {case} dk")
    _grad_parity(G.host_f64(dv), rv, ev, u, f"backward case {case} dv")


def _varlen_cases(n, seed=971):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        nseq = int(rng.integers(1, 6))
        lq = [int(x) for x in rng.integers(0, 500, nseq)]
        lk = [int(x) if rng.random() < 0.5 else lq[j] for j, x in enumerate(rng.integers(0, 600, nseq))]
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2]))
        out.append((i, lq, lk, Hkv * int(rng.choice([1, 2, 4])), Hkv, d, bool(rng.random() < 0.7)))
    return out


@pytest.mark.parametrize("case", _varlen_cases(24), ids=lambda c: f"var{c[0]}")
def test_random_varlen_prefill(aa, case):
    i, lq, lk, Hq, Hkv, d, causal = case
    torch = G.torch()
    if sum(lq) == 0 or sum(lk) == 0:
        pytest.skip("no rows to pack")
    x = wl.make_varlen(lq, lk, Hq, Hkv, d, seed=981 + i)
    q, k, v = G.dev_bf16(x.q, x.dtype), G.dev_bf16(x.k, x.dtype), G.dev_bf16(x.v, x.dtype)
    o = G.nan_like_bf16(q.shape, x.dtype)
    lse = G.nan_f32((Hq, q.shape[0]))
    aa.attn_fwd_varlen(q, k, v, G.dev_i32(x.cu_q), G.dev_i32(x.cu_k), o, max(max(lq), 1), lse=lse, causal=causal)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, causal)
    G.assert_parity(G.host_f64(o), G.host_f64(lse), O_ref, L_ref, f"varlen case {case}")
