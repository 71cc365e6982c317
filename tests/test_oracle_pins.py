"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test targets a mistake a plausible oracle bug would make (dropped scale,
wrong head map, wrong causal alignment, wrong LSE base, transposed operand,
wrong split merge). CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bits(x):
    return wl.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def f64(b):
    return oracle.bf16_bits_to_f64(b)


# --- bf16 decoding is exact ----------------------------------------------------

def test_bf16_roundtrip_exact():
    vals = np.array([0.0, 1.0, -2.5, 0.15625, 3.0e38, -1.0e-38, 65504.0], dtype=np.float32)
    b = bits(vals)
    back = f64(b)
    # every bf16 value is a float32 whose low 16 bits are zero
    assert np.all((back.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    # RNE: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even mantissa (1.0)
    assert f64(bits([1.0 + 2.0 ** -8]))[0] == 1.0
    assert f64(bits([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert np.array_equal(back[:5], np.array([0.0, 1.0, -2.5, 0.15625, back[4]]))


# --- brute force on tiny shapes (independent pure-Python implementation) -----

@pytest.mark.parametrize("B,sq,Hq,Hkv,d,S,lens,causal", [
    (2, 1, 4, 2, 4, 9, [9, 5], True),
    (1, 3, 2, 1, 8, 11, [11], True),
    (2, 4, 4, 1, 4, 13, [13, 6], True),
    (1, 2, 2, 2, 4, 7, [0], True),        # empty sequence
    (1, 4, 2, 1, 4, 6, [2], True),        # fewer keys than queries: early rows empty
    (2, 3, 6, 3, 4, 10, None, False),     # prefill-like, no mask
    (1, 5, 2, 1, 4, 5, None, True),       # square causal prefill
])
def test_oracle_matches_brute_force(B, sq, Hq, Hkv, d, S, lens, causal):
    x = wl.make_prefill(B, Hq, Hkv, d, sq, S, seed=7 + B * 31 + S)
    seq = None if lens is None else np.asarray(lens)
    O, L = oracle.attention(x.q, x.k, x.v, seq, causal)
    Ob, Lb = oracle.brute_attention(x.q, x.k, x.v, seq, causal)
    assert np.allclose(O, np.asarray(Ob), rtol=0, atol=1e-12)
    Lb = np.asarray(Lb)
    assert np.array_equal(np.isinf(L), np.isinf(Lb))
    fin = np.isfinite(Lb)
    assert np.allclose(L[fin], Lb[fin], rtol=0, atol=1e-12)


def test_oracle_brute_force_d64_decode():
    x = wl.make_decode(1, 4, 1, 64, 2, 70, [70], seed=3)
    O, L = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    Ob, Lb = oracle.brute_attention(x.q, x.k, x.v, x.seqlens, True)
    assert np.allclose(O, np.asarray(Ob), atol=1e-12)
    assert np.allclose(L, np.asarray(Lb), atol=1e-12)


# --- closed forms ----------------------------------------------------------------

def test_single_key_closed_form():
    """L = 1: softmax of one score is 1, so O = v0 exactly and LSE = s0.

    q = 2 e_0 and k0 = 4 e_0 with d = 64 give s0 = 8 / sqrt(64) = 1 exactly;
    a dropped 1/sqrt(d) would give 8.
    """
    d = 64
    q = np.zeros((1, 1, 1, d), np.float32); q[..., 0] = 2.0
    k = np.zeros((1, 1, 1, d), np.float32); k[..., 0] = 4.0
    v = np.random.default_rng(0).standard_normal((1, 1, 1, d)).astype(np.float32)
    O, L = oracle.attention(bits(q), bits(k), bits(v), np.array([1]), True)
    assert np.array_equal(O[0, 0, 0], f64(bits(v))[0, 0, 0])
    assert L[0, 0, 0] == 1.0


def test_identical_values_give_that_value():
    """Every V row equal to v: O = v whatever the scores (rows of P sum to 1)."""
    x = wl.make_decode(2, 8, 2, 64, 1, 300, [300, 17], seed=11, pad=wl.BF16_ZERO)
    vrow = bits(np.linspace(-3, 3, 64))
    x.v[:] = vrow
    O, _ = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    assert np.allclose(O, f64(vrow)[None, None, None, :], rtol=0, atol=1e-14)


def test_zero_query_is_uniform_mean_and_log_length():
    """q = 0: all scores 0, P uniform, O = mean of visible V rows, LSE = ln L (natural log)."""
    L = 37
    x = wl.make_decode(1, 2, 1, 64, 1, 64, [L], seed=5, pad=wl.BF16_ZERO)
    x.q[:] = 0
    O, LSE = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    mean = f64(x.v[0, :L, 0]).mean(axis=0)
    assert np.allclose(O[0, 0, 0], mean, atol=1e-14)
    assert np.allclose(LSE[0, :, 0], math.log(L), atol=1e-14)


@pytest.mark.parametrize("jstar", [0, 1, 63, 64, 199])
def test_one_hot_limit(jstar):
    """A key aligned with q and a score gap >> 40 selects its value row."""
    d, L = 64, 200
    x = wl.make_decode(1, 1, 1, d, 1, L, [L], seed=9)
    qf = f64(x.q[0, 0, 0])
    x.k[0, jstar, 0] = bits(8.0 * qf)
    O, LSE = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    assert np.allclose(O[0, 0, 0], f64(x.v[0, jstar, 0]), atol=1e-12)
    s_star = float(f64(x.k[0, jstar, 0]) @ qf) / math.sqrt(d)
    assert s_star > 40
    assert abs(LSE[0, 0, 0] - s_star) < 1e-12


def test_probability_rows_sum_to_one_and_respect_mask():
    x = wl.make_decode(2, 4, 2, 64, 3, 90, [90, 40], seed=21)
    for b in range(2):
        for t in range(3):
            for h in range(4):
                p = oracle.probabilities(x.q, x.k, b, t, h, x.seqlens, True)
                assert abs(p.sum() - 1.0) < 1e-14
                L = int(x.seqlens[b])
                assert np.all(p[L - 3 + t + 1:] == 0.0)
                assert np.all(p[:L - 3 + t + 1] > 0.0)


# --- structure -------------------------------------------------------------------

def test_gqa_equals_mha_with_repeated_kv_heads():
    x = wl.make_decode(2, 8, 2, 64, 2, 50, [50, 23], seed=13)
    O, L = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    k4 = np.repeat(x.k, 4, axis=2)  # repeat_interleave along the head axis
    v4 = np.repeat(x.v, 4, axis=2)
    Om, Lm = oracle.attention(x.q, k4, v4, x.seqlens, True)
    assert np.array_equal(O, Om) and np.array_equal(L, Lm)


def test_gqa_head_map_matches_page_packing():
    """Query head h reads KV head h // G, the page's 32/8 packing (ratio 4).

    Each KV head g carries a constant V row equal to g, so O of query head h
    reveals which KV head it read.
    """
    gold = json.load(open(os.path.join(GOLD, "gqa_packing.json")))
    Hq, Hkv = gold["num_qo_heads"], gold["num_kv_heads"]
    G = Hq // Hkv
    assert G == gold["gqa_ratio"] and gold["blk_m"] // G == gold["seq_q_per_tile"]
    for row, seq_pos, q_head in gold["sample_rows"]:
        assert (row // G, row % G) == (seq_pos, q_head)
    x = wl.make_decode(1, Hq, Hkv, 64, 1, 16, [16], seed=17)
    for g in range(Hkv):
        x.v[0, :, g, :] = bits(np.full(64, float(g)))
    O, _ = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    for h in range(Hq):
        assert np.allclose(O[0, 0, h], h // G, atol=1e-12)


def test_causal_rows_equal_shorter_single_token_decode():
    """Bottom-right causal: multi-token row t equals decode of that query with L' = L - sq + t + 1."""
    sq, L = 4, 77
    x = wl.make_decode(1, 4, 2, 64, sq, 80, [L], seed=23)
    O, LSE = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    for t in range(sq):
        Lp = L - sq + t + 1
        o1, l1 = oracle.attention(x.q[:, t:t + 1], x.k, x.v, np.array([Lp]), True)
        assert np.allclose(O[:, t], o1[:, 0], atol=1e-14)
        assert np.allclose(LSE[:, :, t], l1[:, :, 0], atol=1e-14)
    assert oracle.decode_row_counts(L, sq) == [74, 75, 76, 77]


def test_prefill_square_causal_is_lower_triangle():
    x = wl.make_prefill(1, 2, 2, 8, 6, 6, seed=29)
    for t in range(6):
        p = oracle.probabilities(x.q, x.k, 0, t, 1, None, True)
        assert np.all(p[t + 1:] == 0) and np.all(p[:t + 1] > 0)


# --- split-KV combine -----------------------------------------------------------

def test_combine_rules_golden():
    gold = json.load(open(os.path.join(GOLD, "combine_rules.json")))
    conv = lambda a: [float(z) for z in a]
    for c in gold["cases"]:
        O, lse = oracle.combine_partials(conv(c["m"]), conv(c["l"]), [np.array(o, float) for o in c["o"]])
        assert np.allclose(O, c["expect_o"], atol=1e-15)
        M = float(c["expect_M"])
        if M == -np.inf:
            assert lse == -np.inf
        else:
            assert abs(lse - math.log(2) * (M + math.log2(c["expect_l_common"]))) < 1e-14


@pytest.mark.parametrize("chunk", [1, 7, 64, 100, 1000])
def test_split_and_combine_equals_unsplit(chunk):
    d, L = 64, 250
    x = wl.make_decode(1, 1, 1, d, 1, L, [L], seed=31)
    q, kk, vv = f64(x.q[0, 0, 0]), f64(x.k[0, :, 0]), f64(x.v[0, :, 0])
    bounds = [(lo, min(lo + chunk, L)) for lo in range(0, L, chunk)] + [(L, L)]  # one empty split
    ms, ls, Os = oracle.split_partials(q, kk, vv, bounds)
    Oc, lsec = oracle.combine_partials(ms, ls, Os)
    O, LSE = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    assert np.allclose(Oc, O[0, 0, 0], atol=1e-13)
    assert abs(lsec - LSE[0, 0, 0]) < 1e-12
    # the natural-log LSE of the whole is the logsumexp of the split LSEs
    split_lse = [math.log(2) * (m + math.log2(l)) for m, l in zip(ms, ls) if m > -np.inf]
    mx = max(split_lse)
    assert abs(mx + math.log(sum(math.exp(s - mx) for s in split_lse)) - LSE[0, 0, 0]) < 1e-12


# --- library special case ---------------------------------------------------------

def _sdpa_f64(q, k, v, causal_bottom_right):
    torch = pytest.importorskip("torch")
    Q = torch.from_numpy(f64(q)).permute(0, 2, 1, 3)
    K = torch.from_numpy(f64(k)).permute(0, 2, 1, 3)
    V = torch.from_numpy(f64(v)).permute(0, 2, 1, 3)
    sq, sk = Q.shape[2], K.shape[2]
    mask = None
    if causal_bottom_right:
        i = torch.arange(sq)[:, None]
        j = torch.arange(sk)[None, :]
        mask = j <= i + (sk - sq)  # explicit bottom-right mask
    O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, enable_gqa=True)
    return O.permute(0, 2, 1, 3).numpy()


def test_against_torch_sdpa_on_page_correctness_config():
    """The page validates FA4 against SDPA with GQA at B=1, S=1024, 32/8 heads, D=128."""
    g = json.load(open(os.path.join(GOLD, "fa4_correctness_config.json")))
    x = wl.make_prefill(g["batch"], g["n_q_heads"], g["n_kv_heads"], g["head_dim"],
                        g["seqlen"], g["seqlen"], seed=41)
    O, _ = oracle.attention(x.q, x.k, x.v, None, True)
    ref = _sdpa_f64(x.q, x.k, x.v, True)
    assert np.abs(O - ref).max() < 1e-12


def test_against_torch_sdpa_bottom_right_decode():
    x = wl.make_prefill(2, 8, 2, 64, 4, 33, seed=43)
    O, _ = oracle.attention(x.q, x.k, x.v, None, True)
    ref = _sdpa_f64(x.q, x.k, x.v, True)
    assert np.abs(O - ref).max() < 1e-13


def test_attention_rows_matches_full():
    x = wl.make_decode(3, 8, 2, 64, 2, 120, [120, 60, 1], seed=47)
    O, LSE = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    rows = [(0, 1, 7), (1, 0, 3), (2, 0, 0), (2, 1, 5), (1, 1, 4)]
    Or, Lr = oracle.attention_rows(x.q, x.k, x.v, rows, x.seqlens, True)
    for i, (b, t, h) in enumerate(rows):
        assert np.allclose(Or[i], O[b, t, h], atol=1e-14)
        assert (Lr[i] == LSE[b, h, t]) or abs(Lr[i] - LSE[b, h, t]) < 1e-14


# --- fp16 (IEEE binary16) inputs ------------------------------------------------

def _binary16_by_formula(p):
    """Value of a binary16 pattern from its fields: (-1)^s * 2^(e-15) * (1 + m/1024),
    subnormals 2^-14 * m/1024 (written out here, not taken from any library)."""
    s, e, m = (p >> 15) & 1, (p >> 10) & 0x1F, p & 0x3FF
    sign = -1.0 if s else 1.0
    if e == 0:
        return sign * 2.0 ** -14 * (m / 1024.0)
    assert e != 31
    return sign * 2.0 ** (e - 15) * (1.0 + m / 1024.0)


@pytest.mark.parametrize("pattern", [0x3C00, 0xC000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0x3555, 0xB266, 0x0000, 0x8000])
def test_f16_decoders_match_the_binary16_definition(pattern):
    from oracle.brute import _f16
    want = _binary16_by_formula(pattern)
    assert oracle.f16_bits_to_f64(np.array([pattern], dtype=np.uint16))[0] == want
    assert _f16(pattern) == want
    assert oracle.to_f64(np.array([pattern], dtype=np.uint16), "f16")[0] == want


def test_f16_generator_rounds_to_nearest_even():
    def f(x):
        return int(wl.f32_to_f16_bits(np.array([x], dtype=np.float32))[0])
    assert f(1.0 + 2.0 ** -11) == 0x3C00        # tie -> even (1.0)
    assert f(1.0 + 3 * 2.0 ** -11) == 0x3C02    # tie -> even (1 + 2^-9)
    assert f(1.0 + 2.0 ** -11 + 2.0 ** -20) == 0x3C01  # above the tie
    assert f(65504.0) == 0x7BFF


def test_f16_brute_force_matches_vectorised_oracle():
    x = wl.make_decode(2, 4, 2, 16, 3, 40, [40, 7], seed=23, pad=wl.BF16_ZERO, dtype="f16")
    O, L = oracle.attention(x.q, x.k, x.v, x.seqlens, True, dtype="f16")
    Ob, Lb = oracle.brute_attention(x.q, x.k, x.v, x.seqlens, True, dtype="f16")
    assert np.abs(O - np.array(Ob)).max() <= 1e-12
    assert np.abs(L - np.array(Lb)).max() <= 1e-12
    # the same bits read as bf16 give a different result: the type is honoured
    Ox, _ = oracle.attention(x.q, x.k, x.v, x.seqlens, True, dtype="bf16")
    assert np.abs(O - Ox).max() > 1e-3


def test_f16_one_hot_limit():
    """A key equal to a large multiple of q dominates: O is that key's value row (fp16 exact)."""
    x = wl.make_decode(1, 1, 1, 16, 1, 9, [9], seed=29, pad=wl.BF16_ZERO, dtype="f16")
    qv = oracle.f16_bits_to_f64(x.q[0, 0, 0])
    x.k[0, 4, 0] = wl.f32_to_f16_bits((8.0 * qv).astype(np.float32))
    O, L = oracle.attention(x.q, x.k, x.v, x.seqlens, True, dtype="f16")
    assert np.abs(O[0, 0, 0] - oracle.f16_bits_to_f64(x.v[0, 4, 0])).max() <= 1e-6


# --- variable-length batches ---------------------------------------------------

def test_varlen_equal_lengths_match_the_batched_oracle():
    """A packed batch of equal-length sequences is the batched [B, S, H, d] problem."""
    B, S, Hq, Hkv, d = 3, 37, 4, 2, 16
    x = wl.make_varlen([S] * B, [S] * B, Hq, Hkv, d, seed=91)
    for causal in (True, False):
        O, L = oracle.attention_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, causal)
        Ob, Lb = oracle.attention(x.q.reshape(B, S, Hq, d), x.k.reshape(B, S, Hkv, d), x.v.reshape(B, S, Hkv, d),
                                  None, causal)
        assert np.array_equal(O, Ob.reshape(B * S, Hq, d))
        assert np.array_equal(L, Lb.transpose(1, 0, 2).reshape(Hq, B * S))


def test_varlen_sequences_are_independent_and_edges_hold():
    """Each sequence sees only its own keys (a needle in another sequence is invisible);
    an empty key range gives O = 0 and LSE = -inf; Sq > Sk puts the causal diagonal bottom-right."""
    lq, lk = [5, 0, 7, 3], [5, 4, 3, 0]
    x = wl.make_varlen(lq, lk, 2, 1, 8, seed=92)
    O, L = oracle.attention_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, True)
    # sequence 3 has no keys
    s0, s1 = x.cu_q[3], x.cu_q[4]
    assert np.all(O[s0:s1] == 0) and np.all(np.isneginf(L[:, s0:s1]))
    # sequence 2: 7 queries over 3 keys, bottom-right: query t sees keys j <= t - 4
    s0 = x.cu_q[2]
    assert np.all(np.isneginf(L[:, s0:s0 + 4])) and np.isfinite(L[:, s0 + 4:s0 + 7]).all()
    # row 4 of sequence 2 sees exactly key 0 of that sequence: O = v_0
    assert np.array_equal(O[s0 + 4, 0], f64(x.v[x.cu_k[2], 0]))
    # changing sequence 0's keys leaves sequence 2 unchanged
    k2 = x.k.copy()
    k2[x.cu_k[0]:x.cu_k[1]] = bits(np.full((5, 1, 8), 3.0))
    O2, _ = oracle.attention_varlen(x.q, k2, x.v, x.cu_q, x.cu_k, True)
    assert np.array_equal(O2[x.cu_q[2]:], O[x.cu_q[2]:])
