"""Pins of the backward oracle against facts that do not come from its own formulas.

- central finite differences of the oracle's forward definition (the gradient of
  the scalar loss sum(O * dO) is what the backward pass returns);
- torch's CPU autograd in fp64 through a plain masked-softmax attention (a
  library routine differentiating the definition, not our formulas);
- invariants of softmax attention: every row of dS sums to zero, so the dK rows
  of a head sum to zero; dV rows sum to the dO rows of the queries that see a key;
- special cases: one key (softmax constant: dQ = dK = 0, dV = sum of dO);
- GQA equals MHA with repeated K/V heads whose gradients are summed back;
- the two forms of D (rowsum of P o dP and rowsum of dO o O) agree.
CPU only.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from oracle.attention import _attend


def _forward_f64(q, k, v, causal):
    """O [B, Sq, Hq, d] from fp64 arrays through the oracle's forward core."""
    B, Sq, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    O = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            nv = np.array([min(Sk, i + Sk - Sq + 1) if causal else Sk for i in range(Sq)])
            nv = np.maximum(nv, 0)
            O[b, :, h], _ = _attend(q[b, :, h], k[b, :, h // G], v[b, :, h // G], nv, d)
    return O


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 5, 7, 2, 1, 4), (2, 6, 6, 4, 2, 8), (1, 7, 4, 2, 2, 4)])
def test_backward_matches_finite_differences(shape, causal):
    B, Sq, Sk, Hq, Hkv, d = shape
    q, k, v = _rand((B, Sq, Hq, d), 1), _rand((B, Sk, Hkv, d), 2), _rand((B, Sk, Hkv, d), 3)
    do = _rand((B, Sq, Hq, d), 4)
    dq, dk, dv, _ = oracle.backward_f64(q, k, v, do, causal)
    loss = lambda q_, k_, v_: float(np.sum(_forward_f64(q_, k_, v_, causal) * do))
    eps = 1e-6
    rng = np.random.default_rng(5)
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_torch_autograd_fp64(causal):
    torch = pytest.importorskip("torch")
    B, Sq, Sk, Hq, Hkv, d = 2, 37, 53, 4, 2, 16
    G = Hq // Hkv
    q, k, v = _rand((B, Sq, Hq, d), 11), _rand((B, Sk, Hkv, d), 12), _rand((B, Sk, Hkv, d), 13)
    do = _rand((B, Sq, Hq, d), 14)
    dq, dk, dv, _ = oracle.backward_f64(q, k, v, do, causal)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    kr = tk.repeat_interleave(G, dim=2)  # [B, Sk, Hq, d]
    vr = tv.repeat_interleave(G, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", tq, kr) / math.sqrt(d)
    if causal:  # bottom-right alignment, built explicitly
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Sk)[None, :]
        s = s.masked_fill(~(j <= i + (Sk - Sq)), float("-inf"))
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), vr)
    o.backward(torch.tensor(do, dtype=torch.float64))
    assert np.allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_invariants(causal):
    """sum_j dK_j = 0 (rows of dS sum to zero); sum_j dV_j = sum of dO over rows seeing a key."""
    B, Sq, Sk, Hq, Hkv, d = 1, 40, 30, 4, 2, 8
    G = Hq // Hkv
    q, k, v = _rand((B, Sq, Hq, d), 21), _rand((B, Sk, Hkv, d), 22), _rand((B, Sk, Hkv, d), 23)
    do = _rand((B, Sq, Hq, d), 24)
    dq, dk, dv, D = oracle.backward_f64(q, k, v, do, causal)
    assert np.abs(dk.sum(axis=1)).max() < 1e-12
    live = np.array([(min(Sk, i + Sk - Sq + 1) if causal else Sk) > 0 for i in range(Sq)])
    for g in range(Hkv):
        want = do[0][live][:, g * G:(g + 1) * G].sum(axis=(0, 1))
        assert np.allclose(dv[0, :, g].sum(axis=0), want, atol=1e-12)
    # rows that see nothing (causal with Sq > Sk) have zero dQ and zero D
    if causal:
        assert np.all(dq[0][~live] == 0) and np.all(D[0][:, ~live] == 0)


def test_backward_single_key():
    """One key: the softmax is constant 1, so dQ = dK = 0 and dV = sum of dO."""
    q, k, v, do = _rand((1, 6, 2, 8), 31), _rand((1, 1, 2, 8), 32), _rand((1, 1, 2, 8), 33), _rand((1, 6, 2, 8), 34)
    dq, dk, dv, D = oracle.backward_f64(q, k, v, do, causal=False)
    assert np.all(dq == 0) and np.abs(dk).max() < 1e-15
    assert np.allclose(dv[0, 0], do[0].sum(axis=0), atol=1e-14)
    # D = rowsum(dO o O) with O = v_0
    assert np.allclose(D[0], np.einsum("ihd,hd->hi", do[0], v[0, 0]), atol=1e-13)


def test_backward_gqa_equals_mha_with_summed_heads():
    B, Sq, Sk, Hq, Hkv, d = 1, 20, 25, 6, 2, 8
    G = Hq // Hkv
    q, k, v, do = _rand((B, Sq, Hq, d), 41), _rand((B, Sk, Hkv, d), 42), _rand((B, Sk, Hkv, d), 43), _rand((B, Sq, Hq, d), 44)
    dq, dk, dv, _ = oracle.backward_f64(q, k, v, do, True)
    dq2, dk2, dv2, _ = oracle.backward_f64(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), do, True)
    assert np.allclose(dq, dq2, atol=1e-13)
    assert np.allclose(dk, dk2.reshape(B, Sk, Hkv, G, d).sum(axis=3), atol=1e-13)
    assert np.allclose(dv, dv2.reshape(B, Sk, Hkv, G, d).sum(axis=3), atol=1e-13)


def test_backward_D_forms_agree():
    """D from rowsum(P o dP) equals rowsum(dO o O) with O from the oracle forward."""
    B, Sq, Sk, Hq, Hkv, d = 1, 30, 30, 2, 1, 16
    q, k, v, do = _rand((B, Sq, Hq, d), 51), _rand((B, Sk, Hkv, d), 52), _rand((B, Sk, Hkv, d), 53), _rand((B, Sq, Hq, d), 54)
    _, _, _, D = oracle.backward_f64(q, k, v, do, True)
    O = _forward_f64(q, k, v, True)
    assert np.allclose(D, np.einsum("bihd,bihd->bhi", do, O), atol=1e-12)


def test_backward_bits_wrappers_agree():
    """attention_backward decodes bf16 / fp16 bits exactly; backward_kv_head slices one KV head."""
    x = wl.make_prefill(1, 4, 2, 16, 24, 24, seed=61)
    do = wl.make_grad_out(x.q, 62)
    dq, dk, dv, D = oracle.attention_backward(x.q, x.k, x.v, do, True)
    ref = oracle.backward_f64(*(oracle.bf16_bits_to_f64(t) for t in (x.q, x.k, x.v, do)), True)
    for a, r in zip((dq, dk, dv, D), ref):
        assert np.array_equal(a, r)
    hq, hk, hv, hD = oracle.backward_kv_head(x.q, x.k, x.v, do, 0, 1, True)
    assert np.allclose(hq, dq[0, :, 2:4]) and np.allclose(hk, dk[0, :, 1]) and np.allclose(hv, dv[0, :, 1])
    assert np.allclose(hD, D[0, 2:4])
    xf = wl.make_prefill(1, 2, 2, 8, 9, 9, seed=63, dtype="f16")
    dof = wl.make_grad_out(xf.q, 64, "f16")
    got = oracle.attention_backward(xf.q, xf.k, xf.v, dof, False, dtype="f16")
    ref = oracle.backward_f64(*(oracle.f16_bits_to_f64(t) for t in (xf.q, xf.k, xf.v, dof)), False)
    for a, r in zip(got, ref):
        assert np.array_equal(a, r)


def test_backward_error_scales_bound_the_gradients():
    """|dX| <= the sum of its terms' absolute values (triangle inequality), for every element."""
    x = wl.make_prefill(2, 4, 2, 16, 33, 41, seed=71)
    do = wl.make_grad_out(x.q, 72)
    for causal in (True, False):
        dq, dk, dv, _ = oracle.attention_backward(x.q, x.k, x.v, do, causal)
        eq, ek, ev = oracle.backward_error_scales(x.q, x.k, x.v, do, causal)
        assert np.all(np.abs(dv) <= ev + 1e-12)
        assert np.all(np.abs(dk) <= ek + 1e-12)
        assert np.all(np.abs(dq) <= eq + 1e-12)
        # and they are not vacuous: within a modest factor of the gradients' own size
        assert ev.max() < 50 * np.abs(dv).max() and ek.max() < 200 * np.abs(dk).max()


def test_backward_varlen_equal_lengths_match_batched():
    """A packed batch of equal-length sequences has the batched [B, S, H, d] gradients."""
    B, S, Hq, Hkv, d = 3, 21, 4, 2, 8
    x = wl.make_varlen([S] * B, [S] * B, Hq, Hkv, d, seed=81)
    do = wl.make_grad_out(x.q, 82)
    got = oracle.attention_backward_varlen(x.q, x.k, x.v, do, x.cu_q, x.cu_k, True)
    ref = oracle.attention_backward(x.q.reshape(B, S, Hq, d), x.k.reshape(B, S, Hkv, d), x.v.reshape(B, S, Hkv, d),
                                    do.reshape(B, S, Hq, d), True)
    for a, r, n in zip(got, ref[:3], (Hq, Hkv, Hkv)):
        assert np.array_equal(a, r.reshape(B * S, n, d))
    es = oracle.backward_error_scales_varlen(x.q, x.k, x.v, do, x.cu_q, x.cu_k, True)
    er = oracle.backward_error_scales(x.q.reshape(B, S, Hq, d), x.k.reshape(B, S, Hkv, d), x.v.reshape(B, S, Hkv, d),
                                      do.reshape(B, S, Hq, d), True)
    for a, r, n in zip(es, er, (Hq, Hkv, Hkv)):
        assert np.array_equal(a, r.reshape(B * S, n, d))
