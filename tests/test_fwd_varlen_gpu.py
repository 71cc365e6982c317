"""Parity of the packed variable-length prefill (attn_fwd_varlen) with the fp64 oracle."""
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


def run_varlen(aa, x, causal=True, max_q=None):
    torch = G.torch()
    tq, Hq, d = x.q.shape
    q, k, v = G.dev_bf16(x.q, x.dtype), G.dev_bf16(x.k, x.dtype), G.dev_bf16(x.v, x.dtype)
    cq, ck = G.dev_i32(x.cu_q), G.dev_i32(x.cu_k)
    o = G.nan_like_bf16(q.shape, x.dtype)
    lse = G.nan_f32((Hq, tq))
    mq = int(np.diff(x.cu_q).max()) if max_q is None else max_q
    aa.attn_fwd_varlen(q, k, v, cq, ck, o, mq, lse=lse, causal=causal)
    torch.cuda.synchronize()
    return G.host_f64(o), G.host_f64(lse)


CASES = [
    # lens_q, lens_k, Hq, Hkv, d, causal
    ([200, 1, 513, 64, 300], [200, 1, 513, 64, 128], 4, 2, 128, True),    # ragged, Sq > Sk in the last
    ([100, 257, 30], [900, 257, 31], 2, 2, 128, True),                     # Sk > Sq: bottom-right
    ([77, 300, 5, 256], [77, 300, 5, 256], 4, 4, 64, False),
    ([129, 0, 40], [129, 50, 0], 3, 1, 128, True),                         # an empty query range, an empty key range
    ([1000], [1000], 2, 1, 64, True),
    ([150, 0, 300, 33], [150, 40, 300, 90], 4, 2, 256, True),            # d = 256, an empty query range
]


@pytest.mark.parametrize("case", CASES)
def test_varlen_against_oracle(aa, case):
    lq, lk, Hq, Hkv, d, causal = case
    x = wl.make_varlen(lq, lk, Hq, Hkv, d, seed=701 + sum(lq))
    O_ref, L_ref = oracle.attention_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, causal)
    o, lse = run_varlen(aa, x, causal)
    G.assert_parity(o, lse, O_ref, L_ref, f"varlen {case}")


def test_varlen_equal_lengths_bitwise_equal_dense(aa):
    """Equal lengths: the packed call computes exactly what the dense attn_fwd does."""
    torch = G.torch()
    B, S, Hq, Hkv, d = 3, 333, 4, 2, 128
    x = wl.make_varlen([S] * B, [S] * B, Hq, Hkv, d, seed=711)
    o, lse = run_varlen(aa, x, True)
    qd = G.dev_bf16(x.q.reshape(B, S, Hq, d))
    kd, vd = G.dev_bf16(x.k.reshape(B, S, Hkv, d)), G.dev_bf16(x.v.reshape(B, S, Hkv, d))
    od = G.nan_like_bf16(qd.shape)
    ld = G.nan_f32((B, Hq, S))
    aa.attn_fwd(qd, kd, vd, od, ld, causal=True)
    torch.cuda.synchronize()
    assert np.array_equal(o, G.host_f64(od).reshape(B * S, Hq, d))
    assert np.array_equal(lse, G.host_f64(ld).transpose(1, 0, 2).reshape(Hq, B * S))


@pytest.mark.parametrize("causal", [True, False])
def test_dense_tile_rounds_bitwise_equal_packed(aa, causal):
    """356 query tiles of 256 rows (B=2, S=22784, 2 heads) are more than one
    round of resident work-groups, and the second (reversed) round is partial:
    the dense d = 128 call, which walks the tile list in rounds, must write
    every row exactly as the packed call, which dispatches one work-group per
    tile, does (outputs start as NaN, so a skipped tile shows)."""
    torch = G.torch()
    B, S, Hq, Hkv, d = 2, 89 * 256, 2, 1, 128
    x = wl.make_varlen([S] * B, [S] * B, Hq, Hkv, d, seed=741)
    o, lse = run_varlen(aa, x, causal)
    qd = G.dev_bf16(x.q.reshape(B, S, Hq, d))
    kd, vd = G.dev_bf16(x.k.reshape(B, S, Hkv, d)), G.dev_bf16(x.v.reshape(B, S, Hkv, d))
    od = G.nan_like_bf16(qd.shape)
    ld = G.nan_f32((B, Hq, S))
    aa.attn_fwd(qd, kd, vd, od, ld, causal=causal)
    torch.cuda.synchronize()
    assert not np.isnan(o).any()
    assert np.array_equal(o, G.host_f64(od).reshape(B * S, Hq, d))
    assert np.array_equal(lse, G.host_f64(ld).transpose(1, 0, 2).reshape(Hq, B * S))


def test_varlen_larger_max_seqlen_changes_nothing(aa):
    x = wl.make_varlen([300, 20], [300, 20], 2, 2, 64, seed=721)
    a = run_varlen(aa, x, True)
    b = run_varlen(aa, x, True, max_q=1500)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_varlen_f16(aa):
    lq, lk = [200, 1, 513, 64], [200, 1, 600, 30]
    x = wl.make_varlen(lq, lk, 4, 2, 128, seed=731, dtype="f16")
    O_ref, L_ref = oracle.attention_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, True, dtype="f16")
    o, lse = run_varlen(aa, x, True)
    G.assert_parity(o, lse, O_ref, L_ref, "varlen f16")


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_many_sequences_both_grids(aa, causal):
    """At d = 128 a packed batch of up to 4096 sequences runs on the persistent grid (the sequences' tile counts
    sit in LDS) and a larger one on one work-group per tile. 4097 short sequences, empty query and key ranges
    among them, go against the oracle; their first 4096 alone must give the same rows bit for bit, since both
    grids run the same tile code."""
    rng = np.random.default_rng(4097)
    n = 4097
    lq = rng.integers(0, 40, n)
    lk = lq + rng.integers(0, 9, n)
    lq[::97] = 0
    lk[5::131] = 0
    Hq, Hkv, d = 2, 1, 128
    x = wl.make_varlen(lq, lk, Hq, Hkv, d, seed=4097 + causal)
    O_ref, L_ref = oracle.attention_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, causal)
    o, lse = run_varlen(aa, x, causal)
    G.assert_parity(o, lse, O_ref, L_ref, f"varlen 4097 sequences causal={causal}")
    tq, tk = int(x.cu_q[n - 1]), int(x.cu_k[n - 1])
    head = wl.VarlenInputs(x.q[:tq], x.k[:tk], x.v[:tk], x.cu_q[:n], x.cu_k[:n], x.meta, x.dtype)
    o2, lse2 = run_varlen(aa, head, causal)
    assert np.array_equal(o2, o[:tq]), "4096-sequence call differs from the 4097-sequence call"
    assert np.array_equal(lse2, lse[:, :tq]), "4096-sequence LSE differs from the 4097-sequence call"
