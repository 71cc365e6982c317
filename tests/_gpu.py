"""GPU-test helpers: move generator bit patterns to the device and check parity.

The parity bar: max |O - O_ref| <= 2e-2 on bf16 O and a relative LSE error
<= 1e-3 (relative to max(1, |LSE_ref|)), against the fp64 oracle on the same
bf16 inputs. A second bar pins the O error to the output scale: at long key
ranges |O| is small (about sqrt(e / L)) and 2e-2 alone would pass an all-zero
output, so max |O - O_ref| must also stay within 1% of max |O_ref|
(bf16 rounding of P and of O contributes at most about 2 * 2^-9 relative).
"""
import numpy as np

O_ATOL = 2e-2
O_REL_SCALE = 1e-2
LSE_RTOL = 1e-3


def torch():
    import torch as _t
    return _t


def _tdtype(dtype):
    t = torch()
    return {"bf16": t.bfloat16, "f16": t.float16}[dtype]


def dev_bf16(bits: np.ndarray, dtype: str = "bf16"):
    """Device tensor of the generator's 16-bit patterns, as bf16 (default) or fp16."""
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(_tdtype(dtype)).cuda()


def dev_i32(x):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).cuda()


def host_f64(t):
    return t.detach().double().cpu().numpy()


def nan_like_bf16(shape, dtype: str = "bf16"):
    t = torch()
    return t.full(shape, float("nan"), dtype=_tdtype(dtype), device="cuda")


def nan_f32(shape):
    t = torch()
    return t.full(shape, float("nan"), dtype=t.float32, device="cuda")


def assert_parity(o, lse, O_ref, LSE_ref, tag=""):
    """o, lse: fp64 numpy copies of the GPU outputs; *_ref from the oracle."""
    assert not np.isnan(o).any(), f"{tag}: NaN in O"
    err = float(np.abs(o - O_ref).max())
    scale = float(np.abs(O_ref).max())
    assert err <= O_ATOL, f"{tag}: max|dO| = {err:.3e} > {O_ATOL}"
    assert err <= O_REL_SCALE * scale + 1e-6, f"{tag}: max|dO| = {err:.3e} vs scale {scale:.3e}"
    if lse is not None:
        assert not np.isnan(lse).any(), f"{tag}: NaN in LSE"
        empty = np.isneginf(LSE_ref)
        assert np.array_equal(np.isneginf(lse), empty), f"{tag}: -inf LSE pattern differs"
        fin = ~empty
        if fin.any():
            rel = np.abs(lse[fin] - LSE_ref[fin]) / np.maximum(1.0, np.abs(LSE_ref[fin]))
            assert rel.max() <= LSE_RTOL, f"{tag}: LSE rel err {rel.max():.3e}"
    return err, scale


def host_threads() -> int:
    """Worker threads for oracle checks: the host cores this process may use (at most 16)."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def parallel_map(fn, items):
    """fn over items on host_threads() threads, BLAS held to one thread each (NumPy
    releases the interpreter lock inside BLAS calls and large array loops, so the
    oracle's per-head work runs in parallel). Returns the results in item order;
    the first exception raised by any call is re-raised."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1), ThreadPoolExecutor(host_threads()) as ex:
        return list(ex.map(fn, items))
