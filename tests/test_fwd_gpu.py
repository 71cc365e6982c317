"""Parity of the HIP prefill kernel (attn_fwd) with the fp64 oracle."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as wl
from tests import _gpu as G
from tests._libload import ensure_built

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def aa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    ensure_built()
    import attention_attn_decode_amd as mod
    return mod


def run_fwd(aa, x, causal=True):
    B, Sq, Hq, d = x.q.shape
    q, k, v = G.dev_bf16(x.q, x.dtype), G.dev_bf16(x.k, x.dtype), G.dev_bf16(x.v, x.dtype)
    o = G.nan_like_bf16((B, Sq, Hq, d), x.dtype)
    lse = G.nan_f32((B, Hq, Sq))
    aa.attn_fwd(q, k, v, o, lse, causal=causal)
    G.torch().cuda.synchronize()
    return G.host_f64(o), G.host_f64(lse)


@pytest.mark.parametrize("shape", [
    # B, Sq, Sk, Hq, Hkv, d, causal
    (1, 200, 200, 4, 4, 128, True),
    (2, 130, 130, 4, 2, 64, True),
    (1, 128, 300, 2, 1, 128, True),     # bottom-right, Sk > Sq
    (1, 300, 128, 2, 2, 128, True),     # Sq > Sk: early rows see no key
    (1, 257, 257, 2, 2, 128, False),
    (2, 64, 1000, 4, 4, 64, False),
    (1, 1, 1, 1, 1, 128, True),
    (1, 513, 513, 3, 1, 128, True),
    (1, 40, 40, 2, 2, 128, True),       # one partial key block
    (1, 70, 1, 2, 1, 128, True),        # a single key: only the last row sees it
    (1, 1, 700, 2, 2, 128, True),       # one query row over a ragged key range
    (2, 333, 191, 4, 2, 128, False),    # ragged both ways, GQA, non-causal
    (1, 300, 300, 2, 2, 256, True),     # head size 256: 32-key blocks
    (2, 200, 333, 4, 1, 256, True),     # d = 256, GQA, bottom-right, ragged
    (1, 333, 120, 2, 2, 256, False),    # d = 256, Sq > Sk, non-causal
    (1, 1, 33, 1, 1, 256, True),
])
def test_fwd_small_shapes(aa, shape):
    B, Sq, Sk, Hq, Hkv, d, causal = shape
    x = wl.make_prefill(B, Hq, Hkv, d, Sq, Sk, seed=81 + Sq + Sk + d)
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, None, causal)
    o, lse = run_fwd(aa, x, causal)
    G.assert_parity(o, lse, O_ref, L_ref, f"fwd {shape}")


def test_fwd_page_correctness_config(aa):
    """The FA4 lesson's correctness shape (GQA 32/8, S=1024, D=128) at its 1e-2 tolerance and at our bar."""
    g = json.load(open(os.path.join(GOLD, "fa4_correctness_config.json")))
    x = wl.make_prefill(g["batch"], g["n_q_heads"], g["n_kv_heads"], g["head_dim"], g["seqlen"],
                        g["seqlen"], seed=83)
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, None, True)
    o, lse = run_fwd(aa, x, True)
    assert np.allclose(o, O_ref, rtol=g["rtol"], atol=g["atol"])
    G.assert_parity(o, lse, O_ref, L_ref, "fa4 correctness config")


def test_fwd_causal_prefill_workload_sampled(aa):
    """Full-size causal prefill (B=2, 32 heads, S=8192, d=128), oracle on sampled rows."""
    x = wl.prefill_inputs("causal-prefill")
    B, S, H, d = x.q.shape
    print(f"[fwd parity] causal prefill shape {x.q.shape}", flush=True)
    o, lse = run_fwd(aa, x, True)
    rng = np.random.default_rng(5)
    rows = set()
    for t in [0, 1, 2, 31, 32, 63, 64, 127, 128, 129, 4095, 4096, 8063, 8064, 8190, 8191]:
        rows.add((int(rng.integers(B)), t, int(rng.integers(H))))
    for _ in range(150):
        rows.add((int(rng.integers(B)), int(rng.integers(S)), int(rng.integers(H))))
    rows = sorted(rows)
    O_ref, L_ref = oracle.attention_rows(x.q, x.k, x.v, rows, None, True)
    og = np.stack([o[b, t, h] for b, t, h in rows])
    lg = np.array([lse[b, h, t] for b, t, h in rows])
    err, scale = G.assert_parity(og, lg, O_ref, L_ref, "causal prefill sampled")
    print(f"[fwd parity] causal prefill sampled {len(rows)} rows: max|dO| = {err:.3e}", flush=True)
    # property at any size: O rows are convex combinations of V rows -> |O| <= max|V| per column
    assert np.abs(o).max() <= np.abs(oracle.bf16_bits_to_f64(x.v)).max() + 1e-2


def test_fwd_causal_prefill_workload_every_row(aa):
    """Full-size causal prefill (B=2, 32 heads, S=8192, d=128): every one of the
    524,288 (batch, query, head) rows of O and LSE against the oracle at the
    parity bar, one (batch, head) per oracle call, heads in parallel."""
    x = wl.prefill_inputs("causal-prefill")
    B, S, H, d = x.q.shape
    print(f"[fwd parity] causal prefill every row, shape {x.q.shape}", flush=True)
    o, lse = run_fwd(aa, x, True)

    def head(bh):
        b, h = bh
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        O_ref, L_ref = oracle.attention(x.q[sl], x.k[sl], x.v[sl], None, True)
        return G.assert_parity(o[sl], lse[b:b + 1, h:h + 1], O_ref, L_ref, f"causal prefill (b={b}, h={h})")[0]

    errs = G.parallel_map(head, [(b, h) for b in range(B) for h in range(H)])
    print(f"[fwd parity] causal prefill every row: {B * S * H} rows, max|dO| = {max(errs):.3e}", flush=True)


def test_fwd_tile_rounds_ragged_gqa_every_row(aa):
    """The 868-tile ragged GQA prefill of the sampled test below (Sq = 15653 < Sk = 15700,
    14 query heads on 2 KV heads): every row against the oracle, heads in parallel."""
    B, Sq, Sk, Hq, Hkv, d = 1, 15653, 15700, 14, 2, 128
    x = wl.make_prefill(B, Hq, Hkv, d, Sq, Sk, seed=97)
    print(f"[fwd parity] rounds every row, q {x.q.shape} k {x.k.shape}", flush=True)
    o, lse = run_fwd(aa, x, True)
    Gq = Hq // Hkv

    def head(h):
        g = h // Gq
        O_ref, L_ref = oracle.attention(x.q[:, :, h:h + 1], x.k[:, :, g:g + 1], x.v[:, :, g:g + 1], None, True)
        return G.assert_parity(o[:, :, h:h + 1], lse[:, h:h + 1], O_ref, L_ref, f"rounds head {h}")[0]

    errs = G.parallel_map(head, list(range(Hq)))
    print(f"[fwd parity] rounds every row: {Sq * Hq} rows, max|dO| = {max(errs):.3e}", flush=True)


def test_fwd_tile_rounds_ragged_gqa_sampled(aa):
    """868 query tiles (62 of 256 rows x 14 heads): three full rounds of resident
    work-groups and a partial reversed fourth, ragged Sq = 15653 < Sk = 15700
    (bottom-right causal), 7 query heads per KV head; oracle on sampled rows,
    among them each round's first and last tiles and the ragged ends."""
    B, Sq, Sk, Hq, Hkv, d = 1, 15653, 15700, 14, 2, 128
    x = wl.make_prefill(B, Hq, Hkv, d, Sq, Sk, seed=97)
    print(f"[fwd parity] rounds shape q {x.q.shape} k {x.k.shape}", flush=True)
    o, lse = run_fwd(aa, x, True)
    rng = np.random.default_rng(9)
    rows = set()
    for t in [0, 1, 63, 64, 255, 256, 5119, 5120, 15359, 15360, 15615, 15616, 15651, 15652]:
        for h in (0, 6, 7, 13):
            rows.add((0, t, h))
    for _ in range(60):
        rows.add((0, int(rng.integers(Sq)), int(rng.integers(Hq))))
    rows = sorted(rows)
    O_ref, L_ref = oracle.attention_rows(x.q, x.k, x.v, rows, None, True)
    og = np.stack([o[b, t, h] for b, t, h in rows])
    lg = np.array([lse[b, h, t] for b, t, h in rows])
    err, _ = G.assert_parity(og, lg, O_ref, L_ref, "rounds sampled")
    print(f"[fwd parity] rounds sampled {len(rows)} rows: max|dO| = {err:.3e}", flush=True)
    assert not np.isnan(o).any() and not np.isnan(lse).any()


def test_fwd_deterministic(aa):
    x = wl.make_prefill(1, 4, 4, 128, 700, 700, seed=85)
    a = run_fwd(aa, x)
    b = run_fwd(aa, x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fwd_gqa_equals_mha_with_repeated_kv_heads(aa):
    """Prefill GQA equals MHA over K/V heads repeated G times (head h reads KV head h // G)."""
    B, Sq, Sk, Hq, Hkv, d = 1, 300, 300, 4, 2, 128
    x = wl.make_prefill(B, Hq, Hkv, d, Sq, Sk, seed=99)
    o_gqa, l_gqa = run_fwd(aa, x, True)
    x.k = np.ascontiguousarray(np.repeat(x.k, Hq // Hkv, axis=2))
    x.v = np.ascontiguousarray(np.repeat(x.v, Hq // Hkv, axis=2))
    o_mha, l_mha = run_fwd(aa, x, True)
    # The same kernel computes both with identical per-column arithmetic.
    assert np.array_equal(o_gqa, o_mha) and np.array_equal(l_gqa, l_mha)


@pytest.mark.parametrize("shape", [
    # B, Sq, Sk, Hq, Hkv, d, causal
    (1, 200, 200, 4, 4, 128, True),
    (2, 130, 130, 4, 2, 64, True),
    (1, 128, 300, 2, 1, 128, True),
    (1, 300, 128, 2, 2, 128, True),
    (1, 257, 257, 2, 2, 128, False),
    (2, 64, 1000, 4, 4, 64, False),
    (1, 300, 300, 2, 1, 256, True),
])
def test_fwd_f16_small_shapes(aa, shape):
    """IEEE fp16 inputs and outputs (attn_fwd_f16) against the oracle reading the same fp16 bits."""
    B, Sq, Sk, Hq, Hkv, d, causal = shape
    x = wl.make_prefill(B, Hq, Hkv, d, Sq, Sk, seed=181 + Sq + Sk + d, dtype="f16")
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, None, causal, dtype="f16")
    o, lse = run_fwd(aa, x, causal)
    G.assert_parity(o, lse, O_ref, L_ref, f"fwd f16 {shape}")


def test_fwd_page_correctness_config_in_its_dtype(aa):
    """The FA4 lesson's correctness test as stated: fp16 in, GQA 32/8, S=1024, D=128, rtol = atol = 1e-2."""
    g = json.load(open(os.path.join(GOLD, "fa4_correctness_config.json")))
    x = wl.make_prefill(g["batch"], g["n_q_heads"], g["n_kv_heads"], g["head_dim"], g["seqlen"],
                        g["seqlen"], seed=183, dtype="f16")
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, None, True, dtype="f16")
    o, lse = run_fwd(aa, x, True)
    assert np.allclose(o, O_ref, rtol=g["rtol"], atol=g["atol"])
    G.assert_parity(o, lse, O_ref, L_ref, "fa4 correctness config, fp16")


def test_prefill_graph_replay_without_memset(aa):
    """Captured prefill calls (the persistent d = 128 grid, whose launch reads
    the CU count, and the packed path at d = 64 and d = 128), replayed with new
    queries; each replay must equal an eager call on the same inputs and match
    the oracle."""
    torch = G.torch()
    B, S, Hq, Hkv, d = 1, 700, 4, 2, 128
    x = wl.make_prefill(B, Hq, Hkv, d, S, S, seed=151)
    q, k, v = G.dev_bf16(x.q), G.dev_bf16(x.k), G.dev_bf16(x.v)
    o = G.nan_like_bf16((B, S, Hq, d))
    lse = G.nan_f32((B, Hq, S))
    xv = wl.make_varlen([300, 0, 257], [300, 40, 400], 2, 1, 64, seed=153)
    qv, kv, vv = G.dev_bf16(xv.q), G.dev_bf16(xv.k), G.dev_bf16(xv.v)
    cq, ck = G.dev_i32(xv.cu_q), G.dev_i32(xv.cu_k)
    ov = G.nan_like_bf16(qv.shape)
    lv = G.nan_f32((qv.shape[1], qv.shape[0]))
    xw = wl.make_varlen([260, 513], [260, 600], 4, 2, 128, seed=157)
    qw, kw, vw = G.dev_bf16(xw.q), G.dev_bf16(xw.k), G.dev_bf16(xw.v)
    cqw, ckw = G.dev_i32(xw.cu_q), G.dev_i32(xw.cu_k)
    ow = G.nan_like_bf16(qw.shape)
    lw = G.nan_f32((qw.shape[1], qw.shape[0]))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def calls(stream):
        aa.attn_fwd(q, k, v, o, lse, causal=True, stream=stream)
        aa.attn_fwd_varlen(qv, kv, vv, cq, ck, ov, 300, lse=lv, causal=True, stream=stream)
        aa.attn_fwd_varlen(qw, kw, vw, cqw, ckw, ow, 513, lse=lw, causal=True, stream=stream)

    with torch.cuda.stream(s):
        calls(s)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls(s)
    for rep in range(3):
        xq = wl.make_prefill(B, Hq, Hkv, d, S, S, seed=160 + rep)
        q.copy_(G.dev_bf16(xq.q))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        og, lg, ovg, lvg = G.host_f64(o), G.host_f64(lse), G.host_f64(ov), G.host_f64(lv)
        owg, lwg = G.host_f64(ow), G.host_f64(lw)
        o2, l2 = G.nan_like_bf16((B, S, Hq, d)), G.nan_f32((B, Hq, S))
        aa.attn_fwd(q, k, v, o2, l2, causal=True)
        ov2, lv2 = G.nan_like_bf16(qv.shape), G.nan_f32((qv.shape[1], qv.shape[0]))
        aa.attn_fwd_varlen(qv, kv, vv, cq, ck, ov2, 300, lse=lv2, causal=True)
        ow2, lw2 = G.nan_like_bf16(qw.shape), G.nan_f32((qw.shape[1], qw.shape[0]))
        aa.attn_fwd_varlen(qw, kw, vw, cqw, ckw, ow2, 513, lse=lw2, causal=True)
        torch.cuda.synchronize()
        assert np.array_equal(og, G.host_f64(o2)) and np.array_equal(lg, G.host_f64(l2)), f"dense replay {rep}"
        assert np.array_equal(ovg, G.host_f64(ov2)) and np.array_equal(lvg, G.host_f64(lv2)), f"packed replay {rep}"
        assert np.array_equal(owg, G.host_f64(ow2)) and np.array_equal(lwg, G.host_f64(lw2)), f"packed d=128 {rep}"
        O_ref, L_ref = oracle.attention(xq.q, x.k, x.v, None, True)
        G.assert_parity(og, lg, O_ref, L_ref, f"prefill graph replay {rep}")
