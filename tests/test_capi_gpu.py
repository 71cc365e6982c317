"""The library through its C header alone: tests/capi/attn_capi_check, a plain C program (built by
build(); no Python and no framework in its process, only the HIP runtime), runs one decode and one
causal prefill from seeded inputs written here, and its outputs must match the fp64 oracle at the
parity bar of the other GPU tests."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads as wl
from attention_attn_decode_amd import build as _build
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _bf16_bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _run_c(tmp_path, header, arrays, o_shape, lse_shape):
    if not os.path.exists(_build.CAPI_BIN):
        pytest.fail("the C caller is not built: run build()")
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        np.asarray(header, dtype="<i4").tofile(f)
        for a in arrays:
            np.ascontiguousarray(a).tofile(f)
    r = subprocess.run([_build.CAPI_BIN, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"C caller failed ({r.returncode}): {r.stderr[-2000:]}"
    raw = np.fromfile(out, dtype=np.uint8)
    no, nl = int(np.prod(o_shape)), int(np.prod(lse_shape))
    assert raw.size == 2 * no + 4 * nl
    o = raw[:2 * no].view(np.uint16).reshape(o_shape)
    lse = raw[2 * no:].view(np.float32).reshape(lse_shape)
    return _bf16_bits_to_f64(o), lse.astype(np.float64)


def test_decode_from_c(tmp_path):
    """GQA decode, 4 query heads per KV head, 2 new tokens, ragged lengths (one of a single key); the
    cache rows past each length hold NaN."""
    x = wl.make_decode(3, 16, 4, 128, 2, 700, [700, 1, 333], seed=1201)
    B, sq, Hq, d = x.q.shape
    S, Hkv = x.k.shape[1], x.k.shape[2]
    o, lse = _run_c(tmp_path, [1, B, sq, Hq, Hkv, d, S, 0],
                    [x.q, x.k, x.v, x.seqlens.astype("<i4")], (B, sq, Hq, d), (B, Hq, sq))
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, x.seqlens, True)
    G.assert_parity(o, lse, O_ref, L_ref, "decode from C")


def test_causal_prefill_from_c(tmp_path):
    """Causal GQA prefill with more keys than queries (bottom-right alignment) and a ragged tile."""
    x = wl.make_prefill(2, 8, 2, 64, 300, 420, seed=1203)
    B, Sq, Hq, d = x.q.shape
    Sk, Hkv = x.k.shape[1], x.k.shape[2]
    o, lse = _run_c(tmp_path, [2, B, Sq, Sk, Hq, Hkv, d, 1], [x.q, x.k, x.v], (B, Sq, Hq, d), (B, Hq, Sq))
    O_ref, L_ref = oracle.attention(x.q, x.k, x.v, None, True)
    G.assert_parity(o, lse, O_ref, L_ref, "causal prefill from C")
