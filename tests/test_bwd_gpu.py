"""Parity of the HIP backward pass (attn_bwd) with the fp64 oracle.

The backward's inputs are what a training step hands it: q, k, v, dO, and the
O and LSE the HIP forward produced for them. The oracle differentiates the
exact attention of the same q, k, v, dO bit patterns.

Tolerance, derived from the arithmetic (element by element): the kernels
round P and dS to the element type before their products, take D from the
rounded forward output O, and round dQ, dK, dV once at the end. With unit
roundoff u (2^-8 for bf16, 2^-11 for fp16), each of these rounds a term by at
most u relative, so
    |dX - dX_ref| <= u (E_X + |dX_ref|),
where E_X is the sum of the absolute values of dX's terms (the oracle's
backward_error_scales, which also covers D's dependence on the forward's own
rounding of O). The test allows twice that, for the fp32 accumulations and the
fp32 LSE, plus 1e-6 of the tensor's largest element.
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


def run_bwd(aa, x, do_bits, causal=True, poison=True):
    """HIP forward then HIP backward on the same inputs; returns fp64 host copies of dq, dk, dv."""
    torch = G.torch()
    B, Sq, Hq, d = x.q.shape
    q, k, v = G.dev_bf16(x.q, x.dtype), G.dev_bf16(x.k, x.dtype), G.dev_bf16(x.v, x.dtype)
    do = G.dev_bf16(do_bits, x.dtype)
    o = G.nan_like_bf16(q.shape, x.dtype)
    lse = G.nan_f32((B, Hq, Sq))
    aa.attn_fwd(q, k, v, o, lse, causal=causal)
    dq, dk, dv = G.nan_like_bf16(q.shape, x.dtype), G.nan_like_bf16(k.shape, x.dtype), G.nan_like_bf16(k.shape, x.dtype)
    nbytes = aa.attn_bwd_workspace_size(B, Hq, Sq)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    if poison:
        ws.fill_(float("nan"))  # the workspace needs no initialisation
    aa.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal)
    torch.cuda.synchronize()
    return G.host_f64(dq), G.host_f64(dk), G.host_f64(dv)


def assert_grad_parity(got, ref, scale, u, tag):
    assert not np.isnan(got).any(), f"{tag}: NaN"
    err = np.abs(got - ref)
    bound = 2.0 * u * (scale + np.abs(ref)) + 1e-6 * np.abs(ref).max()
    worst = float((err / bound).max())
    assert worst <= 1.0, f"{tag}: max err/bound = {worst:.3f} (max err {err.max():.3e}, max |ref| {np.abs(ref).max():.3e})"
    return worst


def check(aa, x, do, causal, tag):
    dq, dk, dv = run_bwd(aa, x, do, causal)
    rq, rk, rv, _ = oracle.attention_backward(x.q, x.k, x.v, do, causal, dtype=x.dtype)
    eq, ek, ev = oracle.backward_error_scales(x.q, x.k, x.v, do, causal, dtype=x.dtype)
    u = U[x.dtype]
    return (assert_grad_parity(dq, rq, eq, u, f"{tag} dq"), assert_grad_parity(dk, rk, ek, u, f"{tag} dk"),
            assert_grad_parity(dv, rv, ev, u, f"{tag} dv"))


SHAPES = [
    # B, Sq, Sk, Hq, Hkv, d, causal
    (1, 200, 200, 4, 4, 128, True),
    (2, 130, 130, 4, 2, 64, True),
    (1, 128, 300, 2, 1, 128, True),     # bottom-right, Sk > Sq
    (1, 300, 128, 2, 2, 128, True),     # Sq > Sk: early rows see no key
    (1, 257, 257, 2, 2, 128, False),
    (2, 64, 1000, 4, 4, 64, False),
    (1, 1, 1, 1, 1, 128, True),
    (1, 513, 513, 3, 1, 128, True),     # G = 3
    (1, 700, 700, 8, 2, 64, True),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_bwd_small_shapes(aa, shape):
    B, Sq, Sk, Hq, Hkv, d, causal = shape
    x = wl.make_prefill(B, Hq, Hkv, d, Sq, Sk, seed=301 + Sq + Sk + d)
    do = wl.make_grad_out(x.q, 302 + Sq)
    w = check(aa, x, do, causal, f"bwd {shape}")
    print(f"[bwd parity] {shape}: err/bound dq {w[0]:.3f} dk {w[1]:.3f} dv {w[2]:.3f}", flush=True)


@pytest.mark.parametrize("shape", [(1, 200, 200, 4, 4, 128, True), (2, 130, 130, 4, 2, 64, True),
                                   (1, 300, 128, 2, 2, 128, True), (2, 64, 1000, 4, 4, 64, False)])
def test_bwd_f16_small_shapes(aa, shape):
    B, Sq, Sk, Hq, Hkv, d, causal = shape
    x = wl.make_prefill(B, Hq, Hkv, d, Sq, Sk, seed=401 + Sq + Sk + d, dtype="f16")
    do = wl.make_grad_out(x.q, 402 + Sq, "f16")
    check(aa, x, do, causal, f"bwd f16 {shape}")


def test_bwd_deterministic(aa):
    x = wl.make_prefill(1, 4, 2, 128, 700, 700, seed=501)
    do = wl.make_grad_out(x.q, 502)
    a = run_bwd(aa, x, do)
    b = run_bwd(aa, x, do, poison=False)
    for u_, v_ in zip(a, b):
        assert np.array_equal(u_, v_)


def test_bwd_gqa_equals_mha_with_summed_heads(aa):
    """GQA dK/dV equal the MHA gradients of K/V heads repeated G times, summed back over the group."""
    B, Sq, Sk, Hq, Hkv, d = 1, 300, 300, 4, 2, 128
    x = wl.make_prefill(B, Hq, Hkv, d, Sq, Sk, seed=511)
    do = wl.make_grad_out(x.q, 512)
    dq, dk, dv = run_bwd(aa, x, do)
    x.k = np.ascontiguousarray(np.repeat(x.k, Hq // Hkv, axis=2))
    x.v = np.ascontiguousarray(np.repeat(x.v, Hq // Hkv, axis=2))
    dq2, dk2, dv2 = run_bwd(aa, x, do)
    assert np.array_equal(dq, dq2)
    # The GQA kernel sums the group in fp32 before one rounding; the MHA
    # gradients are rounded per head, then summed here: agreement to rounding.
    G_ = Hq // Hkv
    for a_, b_ in ((dk, dk2), (dv, dv2)):
        s = b_.reshape(B, Sk, Hkv, G_, d).sum(axis=3)
        assert np.abs(a_ - s).max() <= 2 * 2.0 ** -8 * (np.abs(b_).reshape(B, Sk, Hkv, G_, d).sum(axis=3).max() + 1e-3)


def test_bwd_causal_prefill_workload_sampled(aa):
    """Full-size causal prefill backward (B=2, 32 heads, S=8192, d=128): one head against the
    oracle element by element, and a property of every head (sum_j dV_j = sum_i dO_i)."""
    x = wl.prefill_inputs("causal-prefill")
    do = wl.make_grad_out(x.q, 1005)
    B, S, H, d = x.q.shape
    print(f"[bwd parity] causal prefill shape {x.q.shape}", flush=True)
    dq, dk, dv = run_bwd(aa, x, do)
    b, h = 1, 5
    rq, rk, rv, _ = oracle.backward_kv_head(x.q, x.k, x.v, do, b, h, True)
    sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
    eq, ek, ev = oracle.backward_error_scales(x.q[sl], x.k[sl], x.v[sl], do[sl], True)
    u = U["bf16"]
    w = (assert_grad_parity(dq[b, :, h], rq[:, 0], eq[0, :, 0], u, "causal prefill dq"),
         assert_grad_parity(dk[b, :, h], rk, ek[0, :, 0], u, "causal prefill dk"),
         assert_grad_parity(dv[b, :, h], rv, ev[0, :, 0], u, "causal prefill dv"))
    print(f"[bwd parity] causal prefill head (1, 5): err/bound dq {w[0]:.3f} dk {w[1]:.3f} dv {w[2]:.3f}", flush=True)
    # Every row sees a key (causal, Sq == Sk), so the dV rows of a head sum to its dO rows:
    # sum_j dV_j = sum_i dO_i exactly, and to u (sum_i |dO_i| + sum_j |dV_j|) after roundings.
    dof = oracle.bf16_bits_to_f64(do)
    lhs, rhs = dv.sum(axis=1), dof.sum(axis=1)
    tol = 2 * u * (np.abs(dof).sum(axis=1) + np.abs(dv).sum(axis=1))
    assert np.all(np.abs(lhs - rhs) <= tol)


@pytest.mark.parametrize("b", [0, 1])
def test_bwd_causal_prefill_workload_every_head(aa, b):
    """Full-size causal prefill backward (B=2, 32 heads, S=8192, d=128): dQ, dK and dV of
    every head of batch row b against the oracle element by element, within the
    rounding bound, heads in parallel (the two rows together cover all 64 pairs)."""
    x = wl.prefill_inputs("causal-prefill")
    do = wl.make_grad_out(x.q, 1005)
    B, S, H, d = x.q.shape
    print(f"[bwd parity] causal prefill every head, shape {x.q.shape}", flush=True)
    dq, dk, dv = run_bwd(aa, x, do)
    u = U["bf16"]

    def head(h):
        rq, rk, rv, _ = oracle.backward_kv_head(x.q, x.k, x.v, do, b, h, True)
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        eq, ek, ev = oracle.backward_error_scales(x.q[sl], x.k[sl], x.v[sl], do[sl], True)
        return max(assert_grad_parity(dq[b, :, h], rq[:, 0], eq[0, :, 0], u, f"({b}, {h}) dq"),
                   assert_grad_parity(dk[b, :, h], rk, ek[0, :, 0], u, f"({b}, {h}) dk"),
                   assert_grad_parity(dv[b, :, h], rv, ev[0, :, 0], u, f"({b}, {h}) dv"))

    worst = G.parallel_map(head, list(range(H)))
    print(f"[bwd parity] causal prefill batch row {b}, every head: worst err/bound {max(worst):.3f}", flush=True)


# --- packed variable-length batches -------------------------------------------

def run_bwd_varlen(aa, x, do_bits, causal=True):
    torch = G.torch()
    tq, Hq, d = x.q.shape
    q, k, v = G.dev_bf16(x.q, x.dtype), G.dev_bf16(x.k, x.dtype), G.dev_bf16(x.v, x.dtype)
    do = G.dev_bf16(do_bits, x.dtype)
    cq, ck = G.dev_i32(x.cu_q), G.dev_i32(x.cu_k)
    mq, mk = int(np.diff(x.cu_q).max()), int(np.diff(x.cu_k).max())
    o = G.nan_like_bf16(q.shape, x.dtype)
    lse = G.nan_f32((Hq, tq))
    aa.attn_fwd_varlen(q, k, v, cq, ck, o, mq, lse=lse, causal=causal)
    dq, dk, dv = G.nan_like_bf16(q.shape, x.dtype), G.nan_like_bf16(k.shape, x.dtype), G.nan_like_bf16(k.shape, x.dtype)
    ws = torch.full((aa.attn_bwd_varlen_workspace_size(Hq, tq) // 4,), float("nan"), dtype=torch.float32,
                    device="cuda")
    aa.attn_bwd_varlen(q, k, v, o, lse, do, dq, dk, dv, cq, ck, mq, mk, ws, causal=causal)
    torch.cuda.synchronize()
    return G.host_f64(dq), G.host_f64(dk), G.host_f64(dv)


VARLEN_CASES = [
    # lens_q, lens_k, Hq, Hkv, d, causal
    ([200, 1, 513, 64, 300], [200, 1, 513, 64, 128], 4, 2, 128, True),
    ([100, 257, 30], [900, 257, 31], 2, 2, 64, True),
    ([77, 300, 5, 256], [77, 300, 5, 256], 4, 4, 64, False),
    ([129, 40, 3], [129, 50, 7], 3, 1, 128, False),
    ([129, 0, 40, 70], [129, 50, 0, 70], 2, 2, 128, True),   # a sequence without queries, one without keys
]


@pytest.mark.parametrize("case", VARLEN_CASES)
def test_bwd_varlen_against_oracle(aa, case):
    lq, lk, Hq, Hkv, d, causal = case
    x = wl.make_varlen(lq, lk, Hq, Hkv, d, seed=801 + sum(lq))
    do = wl.make_grad_out(x.q, 802 + sum(lk))
    dq, dk, dv = run_bwd_varlen(aa, x, do, causal)
    rq, rk, rv = oracle.attention_backward_varlen(x.q, x.k, x.v, do, x.cu_q, x.cu_k, causal)
    eq, ek, ev = oracle.backward_error_scales_varlen(x.q, x.k, x.v, do, x.cu_q, x.cu_k, causal)
    u = U["bf16"]
    assert_grad_parity(dq, rq, eq, u, f"varlen {case} dq")
    assert_grad_parity(dk, rk, ek, u, f"varlen {case} dk")
    assert_grad_parity(dv, rv, ev, u, f"varlen {case} dv")


def test_bwd_varlen_equal_lengths_bitwise_equal_dense(aa):
    B, S, Hq, Hkv, d = 3, 333, 4, 2, 128
    x = wl.make_varlen([S] * B, [S] * B, Hq, Hkv, d, seed=811)
    do = wl.make_grad_out(x.q, 812)
    got = run_bwd_varlen(aa, x, do, True)
    xd = wl.make_prefill(B, Hq, Hkv, d, S, S, seed=811)  # same streams and sizes: the same bits
    assert np.array_equal(xd.q.reshape(x.q.shape), x.q) and np.array_equal(xd.k.reshape(x.k.shape), x.k)
    ref = run_bwd(aa, xd, do.reshape(B, S, Hq, d), True)
    for a, r in zip(got, ref):
        assert np.array_equal(a, r.reshape(a.shape))


def test_hip_graph_replay_forward_and_backward(aa):
    """attn_fwd + attn_bwd (and their packed forms) captured once, replayed with new dO and a
    reused workspace, eager work and synchronisation between replays; every replay equals
    the eager calls bit for bit."""
    torch = G.torch()
    B, S, Hq, Hkv, d = 2, 300, 4, 2, 128
    x = wl.make_prefill(B, Hq, Hkv, d, S, S, seed=901)
    q, k, v = G.dev_bf16(x.q), G.dev_bf16(x.k), G.dev_bf16(x.v)
    do = G.dev_bf16(wl.make_grad_out(x.q, 902))
    o, lse = G.nan_like_bf16(q.shape), G.nan_f32((B, Hq, S))
    dq, dk, dv = G.nan_like_bf16(q.shape), G.nan_like_bf16(k.shape), G.nan_like_bf16(k.shape)
    ws = torch.full((aa.attn_bwd_workspace_size(B, Hq, S) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    xv = wl.make_varlen([S, 77], [S, 90], Hq, Hkv, d, seed=903)
    qv, kv_, vv = G.dev_bf16(xv.q), G.dev_bf16(xv.k), G.dev_bf16(xv.v)
    cq, ck = G.dev_i32(xv.cu_q), G.dev_i32(xv.cu_k)
    ov, lv = G.nan_like_bf16(qv.shape), G.nan_f32((Hq, qv.shape[0]))

    def calls(stream):
        aa.attn_fwd(q, k, v, o, lse, causal=True, stream=stream)
        aa.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, causal=True, stream=stream)
        aa.attn_fwd_varlen(qv, kv_, vv, cq, ck, ov, S, lse=lv, causal=True, stream=stream)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls(s)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls(s)
    for rep in range(3):
        do.copy_(G.dev_bf16(wl.make_grad_out(x.q, 910 + rep)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [G.host_f64(t) for t in (o, lse, dq, dk, dv, ov, lv)]
        for t in (o, dq, dk, dv, ov):
            t.fill_(float("nan"))
        calls(torch.cuda.current_stream())
        torch.cuda.synchronize()
        want = [G.host_f64(t) for t in (o, lse, dq, dk, dv, ov, lv)]
        for i, (a_, b_) in enumerate(zip(got, want)):
            assert np.array_equal(a_, b_), f"replay {rep}, output {i}"
