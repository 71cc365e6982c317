"""The C-ABI library: loads, exports every declared symbol, host-only logic.

CPU only: nothing here launches a kernel (validation failures return before
any device call; planning and workspace sizing are pure host functions).
"""
import ctypes
import math
import os
import re

import pytest

import attention_attn_decode_amd as aa
from tests._libload import ensure_built

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
HEADER = os.path.join(INCLUDE, "attn.h")
PROBE_HEADER = os.path.join(INCLUDE, "attn_probe.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = ensure_built()
    names = declared_functions()
    assert "attn_decode" in names and "attn_fwd" in names
    for nm in names:
        assert hasattr(L, nm), f"libattn.so does not export {nm}"
    assert sorted(aa.EXPORTS) == names
    probes = declared_functions(PROBE_HEADER)
    for nm in probes:
        assert hasattr(L, nm), f"libattn.so does not export {nm}"
    assert sorted(aa.PROBE_EXPORTS) == probes
    assert sorted(os.listdir(INCLUDE)) == ["attn.h", "attn_probe.h"]


def test_status_strings_and_version():
    ensure_built()
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        s = aa.status_string(code)
        assert s and s != "unknown status"
    assert aa.status_string(12345) == "unknown status"
    assert "gfx950" in aa.version()


def _expected_pieces(B, Hkv, d, S, req):
    """The automatic plan for a 256-CU part: 1024 workers at d = 64, 896 at d >= 128, and 1024 at d = 128 when
    a piece at 896 workers would hold fewer than 32 sub-blocks of 32 keys of capacity."""
    if req > 0:
        n = req
    else:
        workers = 1024 if d < 128 else 896
        if d == 128 and B * math.ceil(S / 32) < 32 * math.ceil(896 / Hkv):
            workers = 1024
        n = math.ceil(workers / Hkv)
    return max(1, min(n, aa.ATTN_MAX_PIECES))


@pytest.mark.parametrize("shape", [
    (1, 8, 1, 64, 1, 512), (32, 64, 8, 128, 1, 8192), (16, 32, 8, 64, 4, 4096),
    (4, 32, 8, 128, 1, 131072), (3, 4, 4, 128, 1, 1), (2, 16, 1, 64, 1, 1000),
])
@pytest.mark.parametrize("req", [0, 1, 2, 7, 64, 1000, 100000])
def test_decode_plan_and_workspace(shape, req):
    ensure_built()
    B, Hq, Hkv, d, sq, S = shape
    pieces, min_piece = aa.attn_decode_plan(B, Hq, Hkv, d, sq, S, req)
    assert pieces == _expected_pieces(B, Hkv, d, S, req)
    assert min_piece == aa.ATTN_MIN_PIECE
    ws = aa.attn_decode_workspace_size(B, Hq, Hkv, sq, d, S, req)
    assert ws == (0 if pieces == 1 else Hkv * (pieces + B) * 16 * (d + 2) * 4 + (B + 1) * 8)


def test_auto_plans_of_the_five_workloads():
    ensure_built()
    assert aa.attn_decode_plan(1, 8, 1, 64, 1, 512) == (1024, 64)
    assert aa.attn_decode_plan(32, 64, 8, 128, 1, 8192) == (112, 64)
    assert aa.attn_decode_plan(16, 32, 8, 64, 4, 4096) == (128, 64)
    assert aa.attn_decode_plan(4, 32, 8, 128, 1, 131072) == (112, 64)


def test_auto_plan_short_pieces():
    """d = 128 calls whose pieces would be short at 896 workers take 1024; d = 256 keeps 896."""
    ensure_built()
    assert aa.attn_decode_plan(1, 16, 2, 128, 1, 131072) == (512, 64)   # 4096 sub-blocks over 448 pieces
    assert aa.attn_decode_plan(1, 16, 1, 128, 1, 131072) == (1024, 64)
    assert aa.attn_decode_plan(32, 32, 1, 128, 1, 8192) == (1024, 64)  # MQA at the headline capacity
    assert aa.attn_decode_plan(1, 16, 2, 256, 1, 131072) == (448, 64)
    assert aa.attn_decode_plan(1, 16, 2, 64, 1, 131072) == (512, 64)
    # the threshold: 32 sub-blocks per piece at 112 pieces per KV head is 3584 sub-blocks of capacity
    assert aa.attn_decode_plan(14, 64, 8, 128, 1, 8192) == (112, 64)   # 3584: not below
    assert aa.attn_decode_plan(13, 64, 8, 128, 1, 8192) == (128, 64)   # 3328
    assert aa.attn_decode_plan(14, 64, 8, 128, 1, 8161) == (112, 64)   # ceil(8161 / 32) = 256: 3584
    assert aa.attn_decode_plan(14, 64, 8, 128, 1, 8160) == (128, 64)   # 255 sub-blocks each: 3570


def test_workspace_size_formula():
    ensure_built()
    assert aa.attn_decode_workspace_size(4, 32, 8, 1, 128, 131072) == 8 * (112 + 4) * 16 * 130 * 4 + 5 * 8
    assert aa.attn_decode_workspace_size(1, 8, 1, 1, 64, 100, 1) == 0
    assert aa.attn_decode_workspace_size(0, 8, 1, 1, 64, 100) == 0
    assert aa.attn_decode_workspace_size(1, 8, 1, 1, 64, 0) == 0
    assert aa.attn_decode_workspace_size(1, 8, 3, 1, 64, 10) == 0  # Hq % Hkv != 0
    # more than 16 packed rows: 32 columns per partial
    # 4 x 4096 sub-blocks of capacity over 896 pieces is under 32 per piece: 1024 pieces
    assert aa.attn_decode_workspace_size(4, 32, 1, 1, 128, 131072) == 1 * (1024 + 4) * 32 * 130 * 4 + 5 * 8
    assert aa.attn_decode_workspace_size(2, 16, 2, 4, 64, 4096) == 2 * (512 + 2) * 32 * 66 * 4 + 3 * 8
    assert aa.attn_decode_workspace_size(3, 16, 1, 1, 256, 70000) == 1 * (896 + 3) * 16 * 258 * 4 + 4 * 8


@pytest.mark.parametrize("args,status", [
    ((32, 8, 128, 1, 1, 64), aa.ATTN_OK),
    ((30, 8, 128, 1, 1, 64), aa.ATTN_ERR_INVALID),       # Hq % Hkv
    ((32, 8, 96, 1, 1, 64), aa.ATTN_ERR_UNSUPPORTED),    # d
    ((32, 8, 128, 5, 1, 64), aa.ATTN_OK),                # G * sq = 20: two column groups
    ((32, 8, 128, 9, 1, 64), aa.ATTN_ERR_UNSUPPORTED),   # G * sq = 36 > 32
    ((16, 1, 64, 1, 1, 64), aa.ATTN_OK),                 # G = 16, one column group
    ((32, 1, 128, 1, 1, 64), aa.ATTN_OK),                # G = 32, the widest group
    ((64, 1, 128, 1, 1, 64), aa.ATTN_ERR_UNSUPPORTED),   # G = 64
    ((16, 1, 256, 1, 1, 64), aa.ATTN_OK),                # d = 256, 16 packed rows
    ((8, 2, 256, 2, 1, 64), aa.ATTN_OK),                 # d = 256, G * sq = 8
    ((32, 1, 256, 1, 1, 64), aa.ATTN_ERR_UNSUPPORTED),   # d = 256 takes one column group
    ((32, 8, 256, 5, 1, 64), aa.ATTN_ERR_UNSUPPORTED),   # d = 256, G * sq = 20
    ((32, 8, 192, 1, 1, 64), aa.ATTN_ERR_UNSUPPORTED),   # d = 192
    ((32, 8, 128, 0, 1, 64), aa.ATTN_ERR_INVALID),       # sq = 0
    ((32, 8, 128, 1, 0, 64), aa.ATTN_ERR_INVALID),       # batch = 0
    ((32, 8, 128, 1, 8192, 64), aa.ATTN_OK),             # largest batch
    ((32, 8, 128, 1, 8193, 64), aa.ATTN_ERR_UNSUPPORTED),  # lengths no longer fit on chip
    ((32, 8, 128, 1, 1, 0), aa.ATTN_ERR_INVALID),        # max_seqlen_k = 0
])
def test_plan_validation(args, status):
    L = ensure_built()
    Hq, Hkv, d, sq, B, S = args
    ns, ch = ctypes.c_int(), ctypes.c_int()
    assert L.attn_decode_plan(B, Hq, Hkv, d, sq, S, 0, ctypes.byref(ns), ctypes.byref(ch)) == status


def test_null_pointers_are_rejected_before_any_device_work():
    L = ensure_built()
    fake = ctypes.c_void_p(0x1000)
    assert L.attn_decode(None, fake, fake, fake, fake, None, 8, 1, 64, 1, 1, 16, None, 0, None) == aa.ATTN_ERR_INVALID
    assert L.attn_decode(fake, fake, fake, None, fake, None, 8, 1, 64, 1, 1, 16, None, 0, None) == aa.ATTN_ERR_INVALID
    assert L.attn_fwd(fake, None, fake, fake, None, 1, 1, 16, 16, 8, 8, 64, None) == aa.ATTN_ERR_INVALID
    # shape errors are reported before alignment or launch
    assert L.attn_fwd(fake, fake, fake, fake, None, 1, 1, 16, 16, 8, 8, 80, None) == aa.ATTN_ERR_UNSUPPORTED
    assert L.attn_fwd(fake, fake, fake, fake, None, 1, 1, 16, 16, 8, 3, 64, None) == aa.ATTN_ERR_INVALID
    # misaligned pointers
    odd = ctypes.c_void_p(0x1002)
    assert L.attn_decode(odd, fake, fake, fake, fake, None, 8, 1, 64, 1, 1, 16, None, 0, None) == aa.ATTN_ERR_MISALIGNED
    assert L.attn_fwd(fake, fake, odd, fake, None, 1, 1, 16, 16, 8, 8, 64, None) == aa.ATTN_ERR_MISALIGNED
    # d = 256 passes the head-size check of the prefill (the alignment check comes next)
    assert L.attn_fwd(fake, fake, odd, fake, None, 1, 1, 16, 16, 8, 8, 256, None) == aa.ATTN_ERR_MISALIGNED
    assert L.attn_fwd(fake, fake, fake, fake, None, 1, 1, 16, 16, 8, 8, 192, None) == aa.ATTN_ERR_UNSUPPORTED
    # workspace too small for a multi-piece plan
    assert L.attn_decode_ex(fake, fake, fake, fake, fake, None, 8, 1, 64, 1, 1, 4096, fake, 16, None, 4) == aa.ATTN_ERR_WORKSPACE
    assert L.attn_decode_ex(fake, fake, fake, fake, fake, None, 8, 1, 64, 1, 1, 4096, fake, 16, None, -1) == aa.ATTN_ERR_INVALID


def test_backward_workspace_size_formula():
    ensure_built()
    for B, Hq, Sq in ((1, 1, 1), (2, 32, 8192), (3, 5, 129), (1, 64, 128)):
        pad = -(-Sq // 128) * 128
        assert aa.attn_bwd_workspace_size(B, Hq, Sq) == 2 * B * Hq * pad * 4
    assert aa.attn_bwd_workspace_size(0, 8, 16) == 0 and aa.attn_bwd_workspace_size(1, 8, -1) == 0


def test_backward_validation_before_any_device_work():
    L = ensure_built()
    f, odd = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1002)
    ws_ok = aa.attn_bwd_workspace_size(1, 8, 16)

    def call(q=f, k=f, v=f, o=f, lse=f, do=f, dq=f, dk=f, dv=f, causal=1, B=1, Sq=16, Sk=16, Hq=8, Hkv=8, d=64,
             ws=f, wsb=ws_ok, fn=L.attn_bwd):
        return fn(q, k, v, o, lse, do, dq, dk, dv, causal, B, Sq, Sk, Hq, Hkv, d, ws, wsb, None)

    for name in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "ws"):
        assert call(**{name: None}) == aa.ATTN_ERR_INVALID, name
    assert call(B=0) == aa.ATTN_ERR_INVALID and call(Sk=-1) == aa.ATTN_ERR_INVALID
    assert call(Hkv=3) == aa.ATTN_ERR_INVALID           # Hq % Hkv != 0
    assert call(d=96) == aa.ATTN_ERR_UNSUPPORTED
    assert call(d=256) == aa.ATTN_ERR_UNSUPPORTED        # the backward takes d = 64 and 128 only
    assert call(dk=odd) == aa.ATTN_ERR_MISALIGNED and call(lse=ctypes.c_void_p(0x1001)) == aa.ATTN_ERR_MISALIGNED
    assert call(wsb=ws_ok - 4) == aa.ATTN_ERR_WORKSPACE
    assert call(fn=L.attn_bwd_f16, d=80) == aa.ATTN_ERR_UNSUPPORTED


def test_varlen_validation_before_any_device_work():
    L = ensure_built()
    f, odd = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1002)

    def call(q=f, k=f, v=f, cq=f, ck=f, o=f, lse=None, causal=1, B=2, mq=16, tq=20, tk=20, Hq=8, Hkv=8, d=64,
             fn=L.attn_fwd_varlen):
        return fn(q, k, v, cq, ck, o, lse, causal, B, mq, tq, tk, Hq, Hkv, d, None)

    for name in ("q", "cq", "ck", "o"):
        assert call(**{name: None}) == aa.ATTN_ERR_INVALID, name
    assert call(k=None) == aa.ATTN_ERR_INVALID            # keys present but no k
    assert call(B=0) == aa.ATTN_ERR_INVALID and call(mq=0) == aa.ATTN_ERR_INVALID and call(tq=0) == aa.ATTN_ERR_INVALID
    assert call(Hkv=3) == aa.ATTN_ERR_INVALID and call(d=32) == aa.ATTN_ERR_UNSUPPORTED
    assert call(cq=ctypes.c_void_p(0x1001)) == aa.ATTN_ERR_MISALIGNED and call(o=odd) == aa.ATTN_ERR_MISALIGNED
    assert call(d=256, o=odd) == aa.ATTN_ERR_MISALIGNED   # d = 256 passes the head-size check
    assert call(fn=L.attn_fwd_varlen_f16, d=96) == aa.ATTN_ERR_UNSUPPORTED


def test_backward_varlen_validation_and_workspace():
    L = ensure_built()
    f = ctypes.c_void_p(0x1000)
    for Hq, tq in ((1, 1), (32, 35024), (8, 129)):
        pad = -(-(tq + 128) // 128) * 128
        assert aa.attn_bwd_varlen_workspace_size(Hq, tq) == 2 * Hq * pad * 4
    assert aa.attn_bwd_varlen_workspace_size(0, 5) == 0
    ws_ok = aa.attn_bwd_varlen_workspace_size(8, 20)

    def call(cq=f, ck=f, B=2, mq=16, mk=16, tq=20, tk=20, Hq=8, Hkv=8, d=64, ws=f, wsb=ws_ok, fn=L.attn_bwd_varlen):
        return fn(f, f, f, f, f, f, f, f, f, cq, ck, 1, B, mq, mk, tq, tk, Hq, Hkv, d, ws, wsb, None)

    assert call(cq=None) == aa.ATTN_ERR_INVALID and call(ws=None) == aa.ATTN_ERR_INVALID
    assert call(tk=0) == aa.ATTN_ERR_INVALID and call(mk=0) == aa.ATTN_ERR_INVALID
    assert call(d=80) == aa.ATTN_ERR_UNSUPPORTED and call(Hkv=3) == aa.ATTN_ERR_INVALID
    assert call(ck=ctypes.c_void_p(0x1002)) == aa.ATTN_ERR_MISALIGNED
    assert call(wsb=ws_ok - 1) == aa.ATTN_ERR_WORKSPACE
    assert call(fn=L.attn_bwd_varlen_f16, d=96) == aa.ATTN_ERR_UNSUPPORTED


def test_noalloc_decode_validation_before_any_device_work():
    """attn_decode_noalloc rejects NULL pointers, bad shapes and plans larger than its
    fixed scratch with no device call (the pointers below are never dereferenced)."""
    L = ensure_built()
    p = ctypes.c_void_p(0x10000)

    def call(q, B, Hq, Hkv, d, sq, S, ns=0):
        return L.attn_decode_noalloc(q, p, p, p, p, None, Hq, Hkv, d, sq, B, S, None, ns)

    assert call(None, 4, 8, 1, 64, 1, 512) == aa.ATTN_ERR_INVALID
    assert call(p, 4, 8, 3, 64, 1, 512) == aa.ATTN_ERR_INVALID          # Hq % Hkv != 0
    assert call(p, 4, 8, 1, 96, 1, 512) == aa.ATTN_ERR_UNSUPPORTED      # head size
    assert call(p, 4, 8, 1, 64, 1, 512, ns=-1) == aa.ATTN_ERR_INVALID
    big = (2048, 16, 8, 128, 1, 64)
    assert aa.attn_decode_workspace_size(big[0], big[1], big[2], big[4], big[3], big[5], 0) > \
        aa.ATTN_NOALLOC_SCRATCH_BYTES
    assert call(p, 2048, 16, 8, 128, 1, 64) == aa.ATTN_ERR_TOO_LARGE
    assert call(p, 64, 64, 8, 128, 1, 8192, ns=4096) == aa.ATTN_ERR_TOO_LARGE


def test_probe_validation_before_any_device_work():
    L = ensure_built()
    p = ctypes.c_void_p(0x10000)
    assert L.attn_probe_stream_read(None, 1 << 20, p, 4, None) == -1
    assert L.attn_probe_stream_read(p, 1000, p, 4, None) == -1          # not a multiple of 16
    assert L.attn_probe_stream_read(p, 1 << 20, p, 0, None) == -1
    assert L.attn_probe_mfma_bf16(p, 0, 10, p, None) == -1
    assert L.attn_probe_mfma_bf16(p, 4, 0, p, None) == -1
    assert L.attn_probe_mfma_bf16(None, 4, 10, p, None) == -1


def test_one_hip_runtime_whatever_is_imported_first():
    """Loading the library before torch must not leave two HIP runtimes in the process (torch ships its
    own copy; with two, launches on torch's tensors fail)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import attention_attn_decode_amd as aa\n"
            "aa.lib()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read()\n"
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))\n"
            ) % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == "1"


def test_c_caller_compiles_as_c99_without_warnings():
    """The C-ABI check program (and with it include/attn.h) compiles as C99 with -Wall -Wextra -Werror."""
    import shutil
    import subprocess
    from attention_attn_decode_amd import build as B
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(B.ROCM, "include"), "-I", B.INCLUDE, B.CAPI_SRC],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
