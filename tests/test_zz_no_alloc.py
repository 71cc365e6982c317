"""attn_decode_noalloc (the decode entry point that allocates nothing and works in
the library's fixed per-device scratch) against attn_decode_ex with a caller
workspace: two calls in a row on one device, the second with a smaller input,
so the second runs over what the first left in the shared scratch."""
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


def both(aa, x, num_splits):
    """Outputs of attn_decode_ex (caller workspace) and attn_decode_noalloc on the same inputs."""
    torch = G.torch()
    B, sq, Hq, d = x.q.shape
    S, Hkv = x.k.shape[1], x.k.shape[2]
    q, k, v = G.dev_bf16(x.q), G.dev_bf16(x.k), G.dev_bf16(x.v)
    sl = G.dev_i32(x.seqlens)
    nbytes = aa.attn_decode_workspace_size(B, Hq, Hkv, sq, d, S, num_splits)
    assert 0 < nbytes <= aa.ATTN_NOALLOC_SCRATCH_BYTES
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    o1, l1 = G.nan_like_bf16((B, sq, Hq, d)), G.nan_f32((B, Hq, sq))
    aa.attn_decode(q, k, v, sl, o1, l1, workspace=ws, num_splits=num_splits)
    o2, l2 = G.nan_like_bf16((B, sq, Hq, d)), G.nan_f32((B, Hq, sq))
    aa.attn_decode_noalloc(q, k, v, sl, o2, l2, num_splits=num_splits)
    torch.cuda.synchronize()
    return (G.host_f64(o1), G.host_f64(l1)), (G.host_f64(o2), G.host_f64(l2))


def test_noalloc_matches_workspace_call_twice_second_smaller(aa):
    cases = [
        # first: 8 ragged sequences, 64/8 heads, d = 128, automatic plan (sequences span several pieces)
        (wl.make_decode(8, 64, 8, 128, 1, 6000, [6000, 3001, 4500, 1, 5999, 2048, 3333, 4097], seed=301), 0),
        # second, smaller: 3 sequences (one empty), 16/4 heads, d = 64, 4 causal new tokens, 7 pieces per KV head
        (wl.make_decode(3, 16, 4, 64, 4, 900, [900, 17, 0], seed=302), 7),
    ]
    for i, (x, ns) in enumerate(cases):
        print(f"[noalloc] call {i}: q {x.q.shape} k {x.k.shape} pieces {ns}", flush=True)
        (o1, l1), (o2, l2) = both(aa, x, ns)
        # the same kernels and plan: the outputs agree bit for bit, and both meet the oracle bar
        assert np.array_equal(o1, o2, equal_nan=False), f"call {i}: O differs from the workspace call"
        assert np.array_equal(l1, l2), f"call {i}: LSE differs from the workspace call"
        O_ref, L_ref = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
        G.assert_parity(o2, l2, O_ref, L_ref, f"noalloc call {i}")


def test_noalloc_rejects_plans_beyond_the_scratch(aa):
    torch = G.torch()
    B, Hq, Hkv, d, S = 2048, 16, 8, 128, 64
    assert aa.attn_decode_workspace_size(B, Hq, Hkv, 1, d, S, 0) > aa.ATTN_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, 1, Hq, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, S, Hkv, d), dtype=torch.bfloat16, device="cuda")
    sl = torch.full((B,), S, dtype=torch.int32, device="cuda")
    o = torch.full_like(q, 7.0)
    with pytest.raises(aa.AttnError) as e:
        aa.attn_decode_noalloc(q, kv, kv, sl, o)
    assert e.value.status == aa.ATTN_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()), "nothing may be enqueued for a rejected call"
