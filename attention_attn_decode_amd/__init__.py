"""Python binding of libattn.so, the gfx950 attention library (decode, prefill, backward).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/attn.h. The functions here take
torch tensors (device memory allocated by the caller), check dtypes, shapes and
contiguity, and pass raw pointers and sizes. Nothing is allocated here, and
there is no fallback: if libattn.so is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

ATTN_OK = 0
ATTN_ERR_INVALID = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_MISALIGNED = -3
ATTN_ERR_WORKSPACE = -4
ATTN_ERR_LAUNCH = -5
ATTN_ERR_DEVICE = -6
ATTN_ERR_TOO_LARGE = -7
ATTN_NOALLOC_SCRATCH_BYTES = 32 << 20
ATTN_MAX_PIECES = 4096
ATTN_MIN_PIECE = 64
ATTN_MAX_BATCH = 8192

# Every symbol include/attn.h declares.
EXPORTS = ("attn_decode_plan", "attn_decode_workspace_size", "attn_decode", "attn_decode_ex",
           "attn_decode_f16", "attn_fwd", "attn_fwd_f16", "attn_fwd_varlen", "attn_fwd_varlen_f16",
           "attn_bwd_workspace_size", "attn_bwd", "attn_bwd_varlen_workspace_size", "attn_bwd_varlen",
           "attn_bwd_varlen_f16",
           "attn_bwd_f16", "attn_decode_noalloc", "attn_status_string", "attn_version")
# Every symbol include/attn_probe.h declares (measurement kernels, not the attention path).
PROBE_EXPORTS = ("attn_probe_stream_read", "attn_probe_mfma_bf16")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libattn.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libattn.so not built at {LIB_PATH}; run attention_attn_decode_amd.build.build()")
    # torch carries its own copy of the HIP runtime under the same soname, but asks for it by a name that
    # an already-loaded /opt/rocm runtime does not match. Loaded before torch, this library would pull in
    # the system runtime and torch would then load its own beside it: two runtimes that share no devices,
    # memory or streams, so every launch on torch's tensors fails. With torch loaded first, this library
    # binds to torch's runtime.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.attn_decode_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32,
                                   ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.attn_decode_plan.restype = i32
    L.attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.attn_decode_workspace_size.restype = sz
    dec = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    L.attn_decode.argtypes = dec
    L.attn_decode.restype = i32
    for name in ("attn_decode_ex", "attn_decode_f16"):
        getattr(L, name).argtypes = dec + [i32]
        getattr(L, name).restype = i32
    L.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, i32]
    L.attn_decode_noalloc.restype = i32
    for name in ("attn_fwd", "attn_fwd_f16"):
        getattr(L, name).argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
        getattr(L, name).restype = i32
    for name in ("attn_fwd_varlen", "attn_fwd_varlen_f16"):
        getattr(L, name).argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp]
        getattr(L, name).restype = i32
    L.attn_bwd_workspace_size.argtypes = [i32, i32, i32]
    L.attn_bwd_workspace_size.restype = sz
    for name in ("attn_bwd", "attn_bwd_f16"):
        getattr(L, name).argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, sz,
                                     vp]
        getattr(L, name).restype = i32
    L.attn_bwd_varlen_workspace_size.argtypes = [i32, i32]
    L.attn_bwd_varlen_workspace_size.restype = sz
    for name in ("attn_bwd_varlen", "attn_bwd_varlen_f16"):
        getattr(L, name).argtypes = [vp] * 11 + [i32] * 9 + [vp, sz, vp]
        getattr(L, name).restype = i32
    L.attn_probe_stream_read.argtypes = [vp, sz, vp, i32, vp]
    L.attn_probe_stream_read.restype = i32
    L.attn_probe_mfma_bf16.argtypes = [vp, i32, i32, vp, vp]
    L.attn_probe_mfma_bf16.restype = i32
    L.attn_status_string.argtypes = [i32]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_version.argtypes = []
    L.attn_version.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def version() -> str:
    return lib().attn_version().decode()


def attn_decode_plan(batch, n_q_heads, n_kv_heads, d, seqlen_q, max_seqlen_k, num_splits=0):
    """(pieces per KV head, minimum piece length) of the decode plan (host-only)."""
    ns, ch = ctypes.c_int(0), ctypes.c_int(0)
    st = lib().attn_decode_plan(batch, n_q_heads, n_kv_heads, d, seqlen_q, max_seqlen_k,
                                num_splits, ctypes.byref(ns), ctypes.byref(ch))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_plan")
    return ns.value, ch.value


def attn_decode_workspace_size(batch, n_q_heads, n_kv_heads, seqlen_q, d, max_seqlen_k,
                               num_splits=0) -> int:
    return int(lib().attn_decode_workspace_size(batch, n_q_heads, n_kv_heads, seqlen_q, d,
                                                max_seqlen_k, num_splits))


def _stream_ptr(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be device memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def _elem(q):
    """Entry-point suffix for the element type of q (bf16 or fp16)."""
    import torch
    if q.dtype == torch.bfloat16:
        return torch.bfloat16, False
    if q.dtype == torch.float16:
        return torch.float16, True
    raise TypeError(f"q must be bfloat16 or float16, got {q.dtype}")


def attn_decode(q, k_cache, v_cache, seqlens_k, o, lse=None, workspace=None, num_splits=0,
                stream=None):
    """GQA KV-cache decode; sizes are read from the tensor shapes.

    q, o: bf16 or fp16 [B, sq, Hq, d]; k_cache, v_cache: same type [B, S_max, Hkv, d];
    seqlens_k: int32 [B]; lse: fp32 [B, Hq, sq] or None; workspace: a uint8 (or
    any) device tensor of at least attn_decode_workspace_size(...) bytes for the
    same num_splits, or None for one piece per KV head.
    """
    import torch
    et, f16 = _elem(q)
    _check(q, "q", et, 4)
    _check(k_cache, "k_cache", et, 4)
    _check(v_cache, "v_cache", et, 4)
    _check(seqlens_k, "seqlens_k", torch.int32, 1)
    _check(o, "o", et, 4)
    B, sq, Hq, d = q.shape
    _, S, Hkv, dk = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or dk != d or k_cache.shape[0] != B:
        raise ValueError("k_cache/v_cache must be [B, S_max, Hkv, d] matching q")
    if tuple(o.shape) != tuple(q.shape) or seqlens_k.shape[0] != B:
        raise ValueError("o must match q and seqlens_k must have B entries")
    if lse is not None:
        _check(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != (B, Hq, sq):
            raise ValueError("lse must be [B, Hq, sq]")
    wbytes = 0
    if workspace is not None:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous device memory")
        wbytes = workspace.numel() * workspace.element_size()
    fn = lib().attn_decode_f16 if f16 else lib().attn_decode_ex
    st = fn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k), _ptr(o), _ptr(lse), Hq, Hkv, d, sq, B, S,
            _ptr(workspace), wbytes, _stream_ptr(stream), int(num_splits))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode")


def _decode_shapes(q, k_cache, v_cache, seqlens_k, o, lse, et):
    import torch
    _check(q, "q", et, 4)
    _check(k_cache, "k_cache", et, 4)
    _check(v_cache, "v_cache", et, 4)
    _check(seqlens_k, "seqlens_k", torch.int32, 1)
    _check(o, "o", et, 4)
    B, sq, Hq, d = q.shape
    _, S, Hkv, dk = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or dk != d or k_cache.shape[0] != B:
        raise ValueError("k_cache/v_cache must be [B, S_max, Hkv, d] matching q")
    if tuple(o.shape) != tuple(q.shape) or seqlens_k.shape[0] != B:
        raise ValueError("o must match q and seqlens_k must have B entries")
    if lse is not None:
        _check(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != (B, Hq, sq):
            raise ValueError("lse must be [B, Hq, sq]")
    return B, sq, Hq, d, S, Hkv


def attn_decode_noalloc(q, k_cache, v_cache, seqlens_k, o, lse=None, num_splits=0, stream=None):
    """attn_decode (bf16) without a workspace: the library's fixed per-device scratch
    holds the partials (ATTN_NOALLOC_SCRATCH_BYTES); nothing is allocated. Calls that
    overlap on one device race on that scratch."""
    import torch
    B, sq, Hq, d, S, Hkv = _decode_shapes(q, k_cache, v_cache, seqlens_k, o, lse, torch.bfloat16)
    st = lib().attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k), _ptr(o), _ptr(lse),
                                   Hq, Hkv, d, sq, B, S, _stream_ptr(stream), int(num_splits))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_noalloc")


def attn_fwd(q, k, v, o, lse=None, causal=True, stream=None):
    """Prefill forward. q, o: bf16 or fp16 [B, Sq, Hq, d]; k, v: same type [B, Sk, Hkv, d];
    lse fp32 [B, Hq, Sq]."""
    import torch
    et, f16 = _elem(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check(t, nm, et, 4)
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or dk != d or k.shape[0] != B or tuple(o.shape) != tuple(q.shape):
        raise ValueError("shape mismatch among q, k, v, o")
    if lse is not None:
        _check(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != (B, Hq, Sq):
            raise ValueError("lse must be [B, Hq, Sq]")
    fn = lib().attn_fwd_f16 if f16 else lib().attn_fwd
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), 1 if causal else 0, B, Sq, Sk, Hq, Hkv, d,
            _stream_ptr(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd")


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, o, max_seqlen_q, lse=None, causal=True, stream=None):
    """Prefill forward over a packed variable-length batch. q, o: bf16 or fp16 [total_q, Hq, d];
    k, v: same type [total_k, Hkv, d]; cu_seqlens_q/k: int32 [B + 1] device offsets;
    lse: fp32 [Hq, total_q] or None; max_seqlen_q: at least the longest query length."""
    import torch
    et, f16 = _elem(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check(t, nm, et, 3)
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    tq, Hq, d = q.shape
    tk, Hkv, dk = k.shape
    B = cu_seqlens_q.shape[0] - 1
    if tuple(v.shape) != tuple(k.shape) or dk != d or tuple(o.shape) != tuple(q.shape):
        raise ValueError("shape mismatch among q, k, v, o")
    if cu_seqlens_k.shape[0] != B + 1 or B < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have B + 1 entries, B >= 1")
    if lse is not None:
        _check(lse, "lse", torch.float32, 2)
        if tuple(lse.shape) != (Hq, tq):
            raise ValueError("lse must be [Hq, total_q]")
    fn = lib().attn_fwd_varlen_f16 if f16 else lib().attn_fwd_varlen
    st = fn(_ptr(q), _ptr(k) if tk else None, _ptr(v) if tk else None, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
            _ptr(o), _ptr(lse), 1 if causal else 0, B, int(max_seqlen_q), tq, tk, Hq, Hkv, d, _stream_ptr(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_varlen")


def attn_bwd_workspace_size(batch, n_q_heads, seqlen_q) -> int:
    """Bytes of workspace attn_bwd needs (uninitialised memory is fine)."""
    return int(lib().attn_bwd_workspace_size(batch, n_q_heads, seqlen_q))


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal=True, stream=None):
    """Attention backward. q, o, dout, dq: bf16 or fp16 [B, Sq, Hq, d]; k, v, dk, dv: same
    type [B, Sk, Hkv, d]; lse: fp32 [B, Hq, Sq] from the forward; workspace: device memory
    of at least attn_bwd_workspace_size(B, Hq, Sq) bytes."""
    import torch
    et, f16 = _elem(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, nm, et, 4)
    _check(lse, "lse", torch.float32, 3)
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, dk_ = k.shape
    if tuple(v.shape) != tuple(k.shape) or dk_ != d or k.shape[0] != B:
        raise ValueError("k and v must be [B, Sk, Hkv, d] matching q")
    for t, nm in ((o, "o"), (dout, "dout"), (dq, "dq")):
        if tuple(t.shape) != tuple(q.shape):
            raise ValueError(f"{nm} must match q")
    for t, nm in ((dk, "dk"), (dv, "dv")):
        if tuple(t.shape) != tuple(k.shape):
            raise ValueError(f"{nm} must match k")
    if tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("lse must be [B, Hq, Sq]")
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous device memory")
    wbytes = workspace.numel() * workspace.element_size()
    fn = lib().attn_bwd_f16 if f16 else lib().attn_bwd
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
            1 if causal else 0, B, Sq, Sk, Hq, Hkv, d, _ptr(workspace), wbytes, _stream_ptr(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd")


def attn_bwd_varlen_workspace_size(n_q_heads, total_q) -> int:
    """Bytes of workspace attn_bwd_varlen needs (uninitialised memory is fine)."""
    return int(lib().attn_bwd_varlen_workspace_size(n_q_heads, total_q))


def attn_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    workspace, causal=True, stream=None):
    """Backward over a packed variable-length batch. q, o, dout, dq: [total_q, Hq, d]; k, v, dk, dv:
    [total_k, Hkv, d] (bf16 or fp16); lse fp32 [Hq, total_q]; cu_seqlens_q/k int32 [B + 1]."""
    import torch
    et, f16 = _elem(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, nm, et, 3)
    _check(lse, "lse", torch.float32, 2)
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    tq, Hq, d = q.shape
    tk, Hkv, dk_ = k.shape
    B = cu_seqlens_q.shape[0] - 1
    if tuple(v.shape) != tuple(k.shape) or dk_ != d or cu_seqlens_k.shape[0] != B + 1 or B < 1:
        raise ValueError("k, v must be [total_k, Hkv, d] and both offset arrays B + 1 long")
    for t, nm in ((o, "o"), (dout, "dout"), (dq, "dq")):
        if tuple(t.shape) != tuple(q.shape):
            raise ValueError(f"{nm} must match q")
    for t, nm in ((dk, "dk"), (dv, "dv")):
        if tuple(t.shape) != tuple(k.shape):
            raise ValueError(f"{nm} must match k")
    if tuple(lse.shape) != (Hq, tq):
        raise ValueError("lse must be [Hq, total_q]")
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous device memory")
    wbytes = workspace.numel() * workspace.element_size()
    fn = lib().attn_bwd_varlen_f16 if f16 else lib().attn_bwd_varlen
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), 1 if causal else 0, B, int(max_seqlen_q), int(max_seqlen_k),
            tq, tk, Hq, Hkv, d, _ptr(workspace), wbytes, _stream_ptr(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd_varlen")


def probe_stream_read(buf, out, grid, stream=None):
    """Measurement kernel: `grid` work-groups read all of `buf` (contiguous device memory, a
    multiple of 16 bytes) once; `out` (int32/uint32 device tensor) takes grid * 256 words."""
    nbytes = buf.numel() * buf.element_size()
    if not (buf.is_cuda and out.is_cuda and buf.is_contiguous() and out.is_contiguous()):
        raise ValueError("buf and out must be contiguous device tensors")
    if out.numel() * out.element_size() < grid * 256 * 4:
        raise ValueError("out needs grid * 256 words")
    st = lib().attn_probe_stream_read(_ptr(buf), nbytes, _ptr(out), int(grid), _stream_ptr(stream))
    if st != 0:
        raise RuntimeError(f"attn_probe_stream_read failed ({st})")


def probe_mfma_bf16(out, grid, iters, clk, stream=None):
    """Measurement kernel: `grid` work-groups of four waves issue `iters` rounds of four
    independent bf16 32x32x16 MFMAs each; `out` (float32) takes grid * 256 values, `clk`
    (int64, 4 entries) the shader and 100 MHz counters at the first wave's start and end."""
    import torch
    _check(out, "out", torch.float32)
    _check(clk, "clk", torch.int64)
    if out.numel() < grid * 256 or clk.numel() < 4:
        raise ValueError("out needs grid * 256 floats and clk 4 entries")
    st = lib().attn_probe_mfma_bf16(_ptr(out), int(grid), int(iters), _ptr(clk), _stream_ptr(stream))
    if st != 0:
        raise RuntimeError(f"attn_probe_mfma_bf16 failed ({st})")
