"""Parity of the HIP decode path (split kernel + combine) with the fp64 oracle.

All calls go through the C ABI (libattn.so) via the ctypes binding.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests import _gpu as G
from tests._libload import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def aa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    ensure_built()
    import attention_attn_decode_amd as mod
    return mod


def piece_spans(lens, P, max_len, min_piece=64, sub=32):
    """Pieces each sequence spans under the balanced split (the plan the header
    documents): sub-blocks of all sequences end to end, cut into P_eff equal
    pieces. Used only to check that a test reaches the merge paths it names."""
    n = [-(-min(max(L, 0), max_len) // sub) for L in lens]
    T = sum(n)
    if T == 0:
        return [0] * len(lens)
    mu = max(1, min_piece // sub)
    p_eff = max(1, min(P, -(-T // mu)))
    piece = lambda xx: ((xx + 1) * p_eff - 1) // T
    out, st = [], 0
    for nb in n:
        out.append(piece(st + nb - 1) - piece(st) + 1 if nb else 0)
        st += nb
    return out


def run_decode(aa, x, num_splits=0, workspace="auto", poison=True):
    torch = G.torch()
    B, sq, Hq, d = x.q.shape
    S, Hkv = x.k.shape[1], x.k.shape[2]
    q, k, v = G.dev_bf16(x.q, x.dtype), G.dev_bf16(x.k, x.dtype), G.dev_bf16(x.v, x.dtype)
    sl = G.dev_i32(x.seqlens)
    o = G.nan_like_bf16((B, sq, Hq, d), x.dtype) if poison else torch.empty((B, sq, Hq, d), dtype=q.dtype, device="cuda")
    lse = G.nan_f32((B, Hq, sq)) if poison else torch.empty((B, Hq, sq), dtype=torch.float32, device="cuda")
    ws = None
    if workspace == "auto":
        nbytes = aa.attn_decode_workspace_size(B, Hq, Hkv, sq, d, S, num_splits)
        ws = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    aa.attn_decode(q, k, v, sl, o, lse, workspace=ws, num_splits=num_splits)
    torch.cuda.synchronize()
    return G.host_f64(o), G.host_f64(lse)


def check(aa, x, tag, **kw):
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, x.seqlens, True, dtype=x.dtype)
    o, lse = run_decode(aa, x, **kw)
    return G.assert_parity(o, lse, O_ref, L_ref, tag)


@pytest.mark.parametrize("cfg", ["gqa-decode-small", "multi-token-decode", "gqa-decode", "long-context-decode"])
def test_decode_workload_parity(aa, cfg):
    """Full-size workloads (cache rows past each sequence end are NaN)."""
    x = wl.decode_inputs(cfg)
    print(f"[decode parity] {cfg} shape q{x.q.shape} k{x.k.shape}", flush=True)
    err, scale = check(aa, x, cfg)
    print(f"[decode parity] {cfg}: max|dO| = {err:.3e} (max|O| {scale:.3e})", flush=True)


@pytest.mark.parametrize("num_splits", [1, 2, 3, 5, 16, 45, 64, 4096])
def test_piece_count_invariance(aa, num_splits):
    """Any number of pieces per KV head gives the oracle's result (pieces cross
    sequence boundaries, sequences span several pieces, short ones fit in one)."""
    x = wl.make_decode(5, 16, 4, 64, 2, 2000, [2000, 777, 129, 0, 1500], seed=51)
    check(aa, x, f"pieces={num_splits}", num_splits=num_splits)


def test_no_workspace_single_split(aa):
    x = wl.make_decode(2, 32, 8, 128, 1, 3000, [3000, 1234], seed=53)
    check(aa, x, "no-workspace", workspace=None)


def test_bitwise_determinism(aa):
    x = wl.make_decode(4, 64, 8, 128, 1, 5000, [5000, 4097, 100, 2048], seed=55)
    a = run_decode(aa, x)
    b = run_decode(aa, x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("d", [64, 128, 256])
def test_needles_at_block_and_split_boundaries(aa, d):
    """Key j* = 8 q (score gap >> 40) must dominate: O = v[j*] for that head."""
    L, chunk_splits = 700, 33  # 13 x 700 keys in 33 pieces: piece boundaries fall inside sequences
    needles = [0, 1, 31, 32, 63, 127, 128, 255, 256, 257, 511, 512, 699]
    B = len(needles)
    x = wl.make_decode(B, 8, 1, d, 1, 768, [L] * B, seed=57 + d)
    qf = oracle.bf16_bits_to_f64(x.q[:, 0, 0])  # head 0 of each batch row
    for b, j in enumerate(needles):
        x.k[b, j, 0] = wl.f32_to_bf16_bits((8.0 * qf[b]).astype(np.float32))
    o, lse = run_decode(aa, x, num_splits=chunk_splits)
    for b, j in enumerate(needles):
        want = oracle.bf16_bits_to_f64(x.v[b, j, 0])
        assert np.abs(o[b, 0, 0] - want).max() <= 2.0 ** -7 * max(1.0, np.abs(want).max()), f"needle {j}"
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    G.assert_parity(o, lse, O_ref, L_ref, "needles")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("pattern", ["ramp", "steps", "descending"])
def test_rising_running_max(aa, d, pattern):
    """Scores that climb along the sequence (a ramp, or jumps of 3-12 in base 2
    every 96 keys) move each column's running max many times, by more and by
    less than the rescale threshold, inside pieces, across piece boundaries and
    in the grouped kernel; a descending ramp never moves it after the first
    sub-block. Keys j get k = c_j * q + noise, so s_j grows with c_j."""
    L, B = 1500, 3
    x = wl.make_decode(B, 4, 4, d, 1, 1536, [L, L - 37, L - 700], seed=71 + d)
    rng = np.random.default_rng(7 + d)
    j = np.arange(L, dtype=np.float64)
    if pattern == "ramp":
        c = 3.0 * j / L
    elif pattern == "steps":
        c = np.cumsum(np.where(j % 96 == 95, rng.uniform(3.0, 12.0, L), 0.0)) / np.sqrt(d) / np.log2(np.e)
    else:
        c = 3.0 * (1.0 - j / L)
    for b in range(B):
        for h in range(4):
            qf = oracle.bf16_bits_to_f64(x.q[b, 0, h])
            noise = rng.normal(0.0, 0.3, (L, d))
            x.k[b, :L, h] = wl.f32_to_bf16_bits((c[:, None] * qf[None, :] + noise).astype(np.float32))
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    for ns, ws in ((0, "auto"), (1, "auto"), (7, "auto"), (0, None)):
        o, lse = run_decode(aa, x, num_splits=ns, workspace=ws)
        G.assert_parity(o, lse, O_ref, L_ref, f"{pattern} d={d} splits={ns} ws={'none' if ws is None else 'yes'}")


def test_future_needle_is_masked_for_earlier_tokens(aa):
    """sq = 4: key L-1 is visible only to the last new token (bottom-right)."""
    L, sq = 1000, 4
    x = wl.make_decode(1, 4, 1, 64, sq, 1024, [L], seed=59)
    for t in range(sq):
        qf = oracle.bf16_bits_to_f64(x.q[0, t, 0])
        x.k[0, L - 1, 0] = wl.f32_to_bf16_bits((8.0 * qf).astype(np.float32)) if t == 0 else x.k[0, L - 1, 0]
    o, lse = run_decode(aa, x)
    vneedle = oracle.bf16_bits_to_f64(x.v[0, L - 1, 0])
    assert np.abs(o[0, 0, 0] - vneedle).max() > 0.1  # token 0 must not see key L-1
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    G.assert_parity(o, lse, O_ref, L_ref, "future-needle")


@pytest.mark.parametrize("sq", [1, 4])
def test_empty_short_and_ragged_sequences(aa, sq):
    lens = [0, 1, 2, 3, 5, 31, 32, 33, 127, 128, 129, 300]
    x = wl.make_decode(len(lens), 8, 2, 64, sq, 300, lens, seed=61 + sq)
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    for ns in (0, 1, 3):
        o, lse = run_decode(aa, x, num_splits=ns)
        G.assert_parity(o, lse, O_ref, L_ref, f"ragged sq={sq} splits={ns}")
        empty = np.isneginf(L_ref)
        assert np.all(o[np.transpose(empty, (0, 2, 1))] == 0.0)


def test_seqlens_are_clamped_to_capacity(aa):
    x = wl.make_decode(2, 8, 1, 128, 1, 256, [256, 100], seed=63)
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    x.seqlens = np.array([10_000, 100], dtype=np.int32)
    o, lse = run_decode(aa, x)
    G.assert_parity(o, lse, O_ref, L_ref, "clamp")


@pytest.mark.parametrize("shape", [(16, 1, 1), (8, 2, 4), (4, 4, 4), (1, 1, 1), (2, 1, 8), (32, 2, 1)])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_group_shapes(aa, shape, d):
    """Packed query columns from 1 up to one full 16-column group, G*sq = 16 included."""
    Hq, Hkv, sq = shape
    x = wl.make_decode(2, Hq, Hkv, d, sq, 600, [600, 333], seed=67 + Hq + sq + d)
    check(aa, x, f"Hq={Hq} Hkv={Hkv} sq={sq} d={d}")


def test_hip_graph_replay_without_memset(aa):
    """Captured decode + combine, replayed with new queries and a reused workspace."""
    torch = G.torch()
    x = wl.make_decode(4, 32, 8, 128, 1, 4096, [4096, 3000, 17, 2049], seed=71)
    B, sq, Hq, d = x.q.shape
    q, k, v = G.dev_bf16(x.q), G.dev_bf16(x.k), G.dev_bf16(x.v)
    sl = G.dev_i32(x.seqlens)
    o = G.nan_like_bf16((B, sq, Hq, d))
    lse = G.nan_f32((B, Hq, sq))
    nbytes = aa.attn_decode_workspace_size(B, Hq, 8, sq, d, x.k.shape[1])
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        aa.attn_decode(q, k, v, sl, o, lse, workspace=ws, stream=s)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        aa.attn_decode(q, k, v, sl, o, lse, workspace=ws, stream=s)
    for rep in range(3):
        xq = wl.make_decode(B, Hq, 8, d, sq, 4096, x.seqlens, seed=100 + rep)
        q.copy_(G.dev_bf16(xq.q))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        og, lg = G.host_f64(o), G.host_f64(lse)
        # eager call on fresh outputs for the same inputs
        o2 = G.nan_like_bf16((B, sq, Hq, d))
        l2 = G.nan_f32((B, Hq, sq))
        aa.attn_decode(q, k, v, sl, o2, l2, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(og, G.host_f64(o2)) and np.array_equal(lg, G.host_f64(l2)), f"replay {rep}"
        O_ref, L_ref = oracle.attention(xq.q, x.k, x.v, x.seqlens, True)
        G.assert_parity(og, lg, O_ref, L_ref, f"graph replay {rep}")


def test_errors_are_reported_without_launch(aa):
    torch = G.torch()
    x = wl.make_decode(1, 8, 1, 64, 1, 4096, [4096], seed=73)
    q, k, v = G.dev_bf16(x.q), G.dev_bf16(x.k), G.dev_bf16(x.v)
    sl = G.dev_i32(x.seqlens)
    o = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(aa.AttnError) as e:
        aa.attn_decode(q, k, v, sl, o, None, workspace=small, num_splits=4)
    assert e.value.status == aa.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert float(o.abs().max()) == 0.0  # nothing was written


@pytest.mark.parametrize("shape", [
    # B, Hq, Hkv, d, sq, lengths
    (2, 4, 2, 64, 1, [70, 33]),
    (1, 2, 1, 64, 3, [65]),
    (2, 3, 3, 128, 2, [1, 40]),
])
def test_tiny_shapes_against_brute_force(aa, shape):
    """Tiny shapes against the pure-Python scalar oracle (math.fsum, own bf16 decode)."""
    from oracle.brute import brute_attention
    B, Hq, Hkv, d, sq, lens = shape
    x = wl.make_decode(B, Hq, Hkv, d, sq, max(lens), lens, seed=91 + d + sq)
    Ob, Lb = brute_attention(x.q, x.k, x.v, x.seqlens, True)
    O_ref, L_ref = np.array(Ob, dtype=np.float64), np.array(Lb, dtype=np.float64)
    for ns in (0, 1, 3):
        o, lse = run_decode(aa, x, num_splits=ns)
        G.assert_parity(o, lse, O_ref, L_ref, f"brute {shape} pieces={ns}")


def test_gqa_equals_mha_with_repeated_kv_heads(aa):
    """GQA output equals MHA over K/V heads repeated G times (head h reads KV head h // G)."""
    B, Hq, Hkv, d, sq, S = 3, 8, 2, 128, 2, 700
    x = wl.make_decode(B, Hq, Hkv, d, sq, S, [700, 257, 64], seed=97)
    o_gqa, l_gqa = run_decode(aa, x)
    G_ = Hq // Hkv
    x.k = np.ascontiguousarray(np.repeat(x.k, G_, axis=2))
    x.v = np.ascontiguousarray(np.repeat(x.v, G_, axis=2))
    o_mha, l_mha = run_decode(aa, x)
    # Different column packing changes only the fp32 summation order.
    assert np.abs(o_gqa - o_mha).max() <= 8e-3
    assert np.abs(l_gqa - l_mha).max() <= 1e-4 * max(1.0, np.abs(l_mha).max())
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    G.assert_parity(o_mha, l_mha, O_ref, L_ref, "mha-repeated")


@pytest.mark.parametrize("shape", [
    # B, Hq, Hkv, d, sq, S, lengths
    (1, 8, 1, 64, 1, 512, [512]),
    (4, 32, 8, 128, 1, 3000, [3000, 1, 0, 1777]),
    (3, 16, 8, 64, 4, 2048, [2048, 900, 5]),
    (2, 16, 2, 128, 2, 1500, [1500, 64]),
])
@pytest.mark.parametrize("num_splits", [0, 1, 5])
def test_f16_decode_parity(aa, shape, num_splits):
    """IEEE fp16 decode (attn_decode_f16) against the oracle reading the same fp16 bits; NaN-poisoned cache tail."""
    B, Hq, Hkv, d, sq, S, lens = shape
    x = wl.make_decode(B, Hq, Hkv, d, sq, S, lens, seed=301 + d + sq, dtype="f16")
    check(aa, x, f"f16 {shape} pieces={num_splits}", num_splits=num_splits)


# --- more than 16 packed query rows: two column groups sharing the K/V reads ---

WIDE = [
    # Hq, Hkv, sq, d, lengths
    (32, 1, 1, 128, [4096, 3000, 17, 2049]),      # MQA-style group of 32
    (64, 2, 1, 64, [1500, 1, 777]),               # G = 32 at d = 64
    (8, 1, 4, 64, [4096, 513, 4, 3]),             # 8 heads x 4 new tokens (causal among them)
    (16, 2, 2, 128, [2048, 1000]),                # G = 8, sq = 2: 16 rows, the one-group boundary
    (20, 4, 4, 128, [1200, 64, 0, 333]),          # G = 5, sq = 4: 20 rows, a partly used second group
    (16, 1, 2, 128, [700, 64, 65]),               # G = 16, sq = 2: exactly 32 rows
]


@pytest.mark.parametrize("shape", WIDE)
def test_wide_groups_against_oracle(aa, shape):
    Hq, Hkv, sq, d, lens = shape
    x = wl.make_decode(len(lens), Hq, Hkv, d, sq, max(lens) + 5, lens, seed=601 + Hq + sq, pad=wl.BF16_NAN)
    check(aa, x, f"wide {shape}")


@pytest.mark.parametrize("num_splits", [1, 3, 64])
def test_wide_group_piece_invariance(aa, num_splits):
    x = wl.make_decode(3, 32, 1, 128, 1, 5000, [5000, 4096, 1], seed=611, pad=wl.BF16_NAN)
    ref = run_decode(aa, x, num_splits=0)
    got = run_decode(aa, x, num_splits=num_splits)
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    G.assert_parity(got[0], got[1], O_ref, L_ref, f"wide splits={num_splits}")
    # piece count changes only the merge order: results agree to rounding
    assert np.abs(got[0] - ref[0]).max() <= 2e-2


def test_wide_group_f16(aa):
    x = wl.make_decode(2, 32, 1, 128, 1, 3000, [3000, 1234], seed=621, dtype="f16")
    check(aa, x, "wide f16")


# Sequences spread over many pieces: K partials per sequence, including K = 127
# and odd counts that leave one piece over in the combine's piece groups.
MERGE = [
    # Hq, Hkv, sq, d, lengths, num_splits, the spans K that must occur
    (16, 2, 2, 128, [576], 9, {9}),
    (16, 2, 2, 128, [512], 8, {8}),
    (8, 1, 1, 64, [1024], 16, {16}),
    (8, 1, 1, 64, [1088], 17, {17}),
    (32, 1, 1, 128, [8192, 40, 33], 128, {127, 2, 1}),
    (16, 4, 1, 128, [3000, 64, 4000, 0, 1], 40, {17, 23, 1}),
    # one sequence over every piece of the automatic plan (the batch-1 shapes:
    # each sequence's merge is split over its output slices)
    (16, 1, 1, 128, [20000], 0, {313}),
    (16, 2, 1, 64, [9000, 0], 0, {141, 0}),
]


@pytest.mark.parametrize("case", MERGE)
def test_many_piece_merges_against_oracle(aa, case):
    Hq, Hkv, sq, d, lens, ns, spans = case
    S = max(lens) + 3
    K = piece_spans(lens, aa.attn_decode_plan(len(lens), Hq, Hkv, d, sq, S, ns)[0], S)
    assert spans <= set(K), (K, spans)
    x = wl.make_decode(len(lens), Hq, Hkv, d, sq, S, lens, seed=631 + sum(lens) % 97, pad=wl.BF16_NAN)
    check(aa, x, f"merge K={K}", num_splits=ns)


def test_largest_batch_against_oracle(aa):
    """batch = ATTN_MAX_BATCH (every length staged on chip), ragged lengths 0..64."""
    rng = np.random.default_rng(651)
    lens = rng.integers(0, 65, aa.ATTN_MAX_BATCH).astype(np.int32)
    x = wl.make_decode(len(lens), 8, 1, 64, 1, 64, lens, seed=651, pad=wl.BF16_NAN)
    check(aa, x, "largest batch")


def test_million_key_sequence_against_oracle(aa):
    """One sequence of 2^20 + 3 keys over every piece of the automatic plan."""
    L = (1 << 20) + 3
    x = wl.make_decode(1, 8, 1, 64, 1, L, [L], seed=653)
    check(aa, x, "million keys")


# Head size 256 (one column group, single register slot per wave).
D256 = [
    # Hq, Hkv, sq, lengths, num_splits
    (16, 1, 1, [5000, 1, 0, 777, 33], 0),
    (8, 2, 2, [4096, 513, 64, 65], 0),
    (4, 4, 4, [300, 4, 3, 2000], 3),
    (16, 2, 1, [20000], 0),             # one sequence over every piece (slice combine)
    (8, 1, 1, [1200, 900], 1),          # one piece per KV head: no partials
    (8, 8, 1, [3000, 2999], 4096),
]


@pytest.mark.parametrize("case", D256)
def test_head_size_256_against_oracle(aa, case):
    Hq, Hkv, sq, lens, ns = case
    x = wl.make_decode(len(lens), Hq, Hkv, 256, sq, max(lens) + 7, lens, seed=661 + Hq + sq, pad=wl.BF16_NAN)
    check(aa, x, f"d=256 {case}", num_splits=ns)


def test_head_size_256_f16(aa):
    x = wl.make_decode(3, 16, 2, 256, 1, 3000, [3000, 1234, 5], seed=671, dtype="f16")
    check(aa, x, "d=256 f16")


# Shapes the launcher serves with one work-group per (sequence, KV head): whole caches of at most
# 256 KB of K/V, or 128-512 sequence-head pairs of at most 512 KB each (at capacity). Lengths include
# empty sequences and sequences shorter than the four 32-key sub-blocks the work-group's waves share.
GROUPED = [
    # B, Hq, Hkv, d, sq, max_len, lengths (None = random in [0, max_len]), seed
    (32, 64, 8, 128, 1, 512, None, 611),
    (16, 32, 8, 64, 4, 1024, None, 612),
    (16, 32, 8, 64, 8, 512, None, 613),           # 32 packed rows: two column groups
    (32, 16, 16, 256, 1, 128, None, 614),         # d = 256, 512 pairs
    (2, 8, 1, 64, 1, 300, [300, 0], 615),         # tiny call, one empty sequence
    (1, 8, 1, 64, 1, 512, [97], 616),             # one short sequence: waves 0-3 get 0-1 sub-blocks
    (128, 8, 1, 128, 2, 512, None, 617),          # 128 pairs, 2 causal new tokens
]


@pytest.mark.parametrize("case", GROUPED, ids=lambda c: f"B{c[0]}h{c[1]}:{c[2]}d{c[3]}sq{c[4]}L{c[5]}")
def test_grouped_shapes_against_oracle(aa, case):
    B, Hq, Hkv, d, sq, S, lens, seed = case
    if lens is None:
        rng = np.random.default_rng(seed)
        lens = rng.integers(0, S + 1, size=B)
        lens[: min(B, 4)] = [0, 1, 33, S][: min(B, 4)]
    x = wl.make_decode(B, Hq, Hkv, d, sq, S, lens, seed=seed)
    check(aa, x, f"grouped {case[:6]}")


@pytest.mark.parametrize("hkv,sq", [(1, 2), (2, 4)])
def test_batch1_long_cache_short_pieces(aa, hkv, sq):
    """Batch-1 GQA decode over 131072 keys, 16 query heads, d = 128, several new tokens: the automatic plan
    spreads the cache over 1024 workers of 4-8 sub-blocks each, and the combine merges 512-1024 partials per
    KV head."""
    x = wl.make_decode(1, 16, hkv, 128, sq, 131072, [131072], seed=9400 + hkv + sq)
    assert aa.attn_decode_plan(1, 16, hkv, 128, sq, 131072)[0] == 1024 // hkv
    check(aa, x, f"batch-1 L=131072 16:{hkv} sq={sq}")
