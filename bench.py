#!/usr/bin/env python3
"""Single-GPU benchmark of the attention hot path on MI355X.

A step is one pass of the whole path over one batch of synthetic input:
  * GQA decode on every decode workload, each through the C ABI (split-KV
    kernel + combine): the headline (batch 32, 64 query / 8 KV heads, d = 128,
    one new token, KV lengths uniform in [1024, 8192]), the small one (batch 1,
    8/1 heads, d = 64, 512 keys), multi-token decode (batch 16, 32/8 heads,
    d = 64, 4 causal new tokens over 4096 keys) and long-context decode
    (batch 4, 32/8 heads, d = 128, 131072 keys);
  * causal prefill (batch 2, 32 heads, d = 128, S = 8192) through attn_fwd;
  * the backward pass of that prefill (dQ, dK, dV from its O and LSE and a
    synthetic dO) through attn_bwd;
  * a packed variable-length causal prefill (16 sequences, lengths uniform in
    [256, 4096], 32 heads, d = 128) through attn_fwd_varlen.
Each workload's calls are captured once in a HIP graph and the steps replay
the graphs, one pair of HIP events around each replay on the stream the
kernels run on: a decode graph holds a few back-to-back calls (CALLS_PER_REPLAY),
the prefill, backward and packed-prefill graphs one call each, and a call's
time is its replay's time over its call count. Decode inputs rotate over
resident copies of at least 1 GiB in total (the Infinity Cache is 256 MB), so
no call reads K/V that an earlier call left in a cache. After the timed steps
every workload is also timed as plain launches, an event pair around each call
(`*_plain` fields), which adds the event markers' cost to every call.
The headline `value` is the headline decode's KV-read bandwidth: algorithmic
K+V bytes (sum_b L_b * Hkv * 4d) over the mean duration of its calls. Each
decode workload reports the same, prefill reports TFLOP/s over the exact
causal FLOPs (4 d per visible query-key pair), the backward TFLOP/s counted,
as the backward page does, as 2.5 times the forward FLOPs. After the timed
steps, two measurement kernels of the library give the device's practical
ceilings (a streaming read of 2 GiB, a bf16 MFMA loop with its clock; the
streaming read also over exactly each decode workload's K/V bytes, which a
decode call is compared with as `frac_of_bare_read`), and the
fp64 CPU oracle is timed on the host (the full headline decode; a sample of
the prefill).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-backward] [--no-varlen]
Prints one JSON line.

HBM traffic (`traffic` fields) comes from two rocprofv3 counter passes over
`bench.py --counter-run` (one 1 GiB device copy for calibration, then one call
of each decode workload, one prefill and one backward, nothing timed):
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT -o fetch -- python bench.py --counter-run
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT -o write -- python bench.py --counter-run
  python bench.py --ingest-counters OUT/fetch_counter_collection.csv OUT/write_counter_collection.csv
The last step (no GPU) scales each counter by what it read for the copy and
stores bytes per launch, keyed by a hash of the kernel code (comments and
layout excluded), in profiles/hbm_traffic_counters.json; a stale hash reports
traffic as null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
DECODE_SOURCES = ["attention_attn_decode_amd/csrc/decode.hip", "attention_attn_decode_amd/csrc/attn_device.h"]
FWD_SOURCES = ["attention_attn_decode_amd/csrc/fwd.hip", "attention_attn_decode_amd/csrc/attn_device.h"]
BWD_SOURCES = ["attention_attn_decode_amd/csrc/bwd.hip", "attention_attn_decode_amd/csrc/attn_device.h"]
COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic_counters.json")


def _code_only(text):
    """C/C++ source with comments removed and whitespace runs collapsed (string and
    character literals kept as written), so that comment edits do not count as a
    change of the kernel."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(paths):
    """Hash of the kernels' code (comments and layout excluded)."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def decode_kv_bytes(seqlens, n_kv_heads, d):
    """Algorithmic K+V bytes of one decode call: every visible key and value row once (bf16)."""
    return int(sum(int(L) for L in seqlens)) * n_kv_heads * 4 * d


def decode_problem_bytes(seqlens, B, Hq, Hkv, d, sq):
    """Effective problem bytes: Q, K, V and O each counted once."""
    return decode_kv_bytes(seqlens, Hkv, d) + 2 * (B * sq * Hq * d * 2)


def causal_flops(B, H, S, d):
    """Exact causal forward FLOPs: 2 GEMMs x 2 flop x d per visible (query, key) pair."""
    return 4 * d * B * H * (S * (S + 1) // 2)


def measured_traffic(kernel, src_hash, units):
    """HBM bytes per launch from stored rocprofv3 FETCH_SIZE/WRITE_SIZE runs, or None if stale."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 1 << 30
ROTATION_BYTES = 1 << 30     # each decode workload rotates over resident copies of at least this much K/V
# Back-to-back calls per graph replay (a replay costs ~10 us before its first kernel, spread over its
# calls). Calls cycle through the K/V copies (replay_plan), so between two reads of the same K/V bytes
# the run reads at least 1 GB of K/V, four times the 256 MB Infinity Cache.
CALLS_PER_REPLAY = {"gqa-decode": 8, "gqa-decode-small": 32, "multi-token-decode": 16, "long-context-decode": 4}
PLAIN_CALLS = 8              # plain-launch calls per workload after the timed steps

# Decode workloads timed in every step; the first (the headline) gives `value`
# and runs last in the step.
DECODE_LEGS = ["gqa-decode", "gqa-decode-small", "multi-token-decode", "long-context-decode"]
LEG_DESC = {
    "gqa-decode": "gqa-decode b=32 hq=64 hkv=8 d=128 sq=1 kv_len~U[1024,8192] (seed 1001)",
    "gqa-decode-small": "gqa-decode-small b=1 hq=8 hkv=1 d=64 sq=1 kv_len=512 (seed 1000)",
    "multi-token-decode": "multi-token-decode b=16 hq=32 hkv=8 d=64 sq=4 causal kv_len=4096 (seed 1002)",
    "long-context-decode": "long-context-decode b=4 hq=32 hkv=8 d=128 sq=1 kv_len=131072 (seed 1003)",
}
PREFILL_DESC = "causal-prefill b=2 h=32 d=128 s=8192 (seed 1004)"
BACKWARD_DESC = "causal-prefill backward b=2 h=32 d=128 s=8192 (seed 1004, dO seed 1005)"

# --counter-run dispatch order after the calibration copy: (stored key, kernel-name prefixes of its
# dispatches in order, sources, workload). Each decode call is a split kernel then one combine kernel.
COUNTER_LEGS = [(f"attn_decode:{w}", ("decode_stream<", "combine_"), DECODE_SOURCES, LEG_DESC[w]) for w in DECODE_LEGS] + [
    ("attn_fwd", ("fwd_",), FWD_SOURCES, PREFILL_DESC),
    ("attn_bwd", ("bwd_pre<", "bwd_dkdv<", "bwd_dq<"), BWD_SOURCES, BACKWARD_DESC),
]


def _short_name(name):
    name = name.replace("void ", "").replace("attn::(anonymous namespace)::", "")
    return name.split("(")[0].strip()


def ingest_counters(fetch_csv, write_csv):
    """Turn the FETCH_SIZE and WRITE_SIZE passes of `--counter-run` into bytes per launch.

    The dispatches after the 1 GiB calibration copy (the run's last copy) are matched, in
    dispatch order, to the calls `--counter-run` makes (COUNTER_LEGS; a decode call is its split
    kernel and, unless the grouped kernel served it, a combine kernel)."""
    import csv

    def read(path, counter):
        # the run ends with the calibration copy followed by the legs' dispatches
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        copies = [i for i, r in enumerate(rows) if "copyBuffer" in r["Kernel_Name"]]
        if not copies or copies[-1] + 1 >= len(rows):
            raise SystemExit(f"{path}: expected the calibration copy then the legs' dispatches at the end")
        kib = float(rows[copies[-1]]["Counter_Value"])
        seq = [(_short_name(r["Kernel_Name"]), float(r["Counter_Value"])) for r in rows[copies[-1] + 1:]]
        return COPY_BYTES / (kib * 1024.0), kib, seq

    fs, fcopy, fseq = read(fetch_csv, "FETCH_SIZE")
    ws, wcopy, wseq = read(write_csv, "WRITE_SIZE")
    out = {"note": "HBM bytes per launch: rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch, "
                   "separate passes over bench.py --counter-run), each scaled by the ratio of a "
                   "1 GiB device copy's true bytes to what the same counter read for it.",
           "calibration": {"copy_bytes": COPY_BYTES, "fetch_size_kib": fcopy, "write_size_kib": wcopy,
                           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)}}
    i = 0
    for key, prefixes, srcs, workload in COUNTER_LEGS:
        kern, fetch, write = {}, 0.0, 0.0
        for pre in prefixes:
            if i >= len(fseq) or i >= len(wseq):
                raise SystemExit(f"counter run ended before {key}")
            (nf, f), (nw, w) = fseq[i], wseq[i]
            if pre == "combine_" and not nf.startswith(pre):
                continue  # the grouped decode kernel has no combine
            if not (nf.startswith(pre) and nw == nf):
                raise SystemExit(f"dispatch {i} after the copy is {nf} / {nw}, expected {pre}... for {key}")
            kern[nf] = {"fetch_kib": round(f, 3), "write_kib": round(w, 3)}
            fetch += f * 1024.0 * fs
            write += w * 1024.0 * ws
            i += 1
        out[key] = {"source_hash": source_hash(srcs), "workload": workload, "kernels": kern,
                    "fetch_bytes": round(fetch), "write_bytes": round(write), "bytes_per_launch": round(fetch + write)}
    with open(COUNTERS, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps({k: v.get("bytes_per_launch") for k, v in out.items() if isinstance(v, dict) and k != "calibration"}))


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_decode(x, d):
    """Time the fp64 oracle on the full headline decode workload (all host cores for BLAS)."""
    import oracle
    from threadpoolctl import threadpool_limits
    ncores = host_cores()
    with threadpool_limits(limits=ncores):
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.attention(x.q, x.k, x.v, x.seqlens, True)
            reps += 1
            if time.perf_counter() - t0 > 10.0 or reps >= 5:
                break
        dt = (time.perf_counter() - t0) / reps
    kv = decode_kv_bytes(x.seqlens, x.k.shape[2], d)
    return {"value": round(kv / dt / 1e9, 3), "unit": "GB/s", "cores": ncores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"full headline decode workload, {reps} pass(es), {dt:.2f} s per pass, numpy fp64"}


def cpu_baseline_prefill(xp):
    """Time the fp64 oracle on the causal prefill: its (batch, head) pairs on the host
    threads (BLAS held to one thread each; about 30 s of CPU work in all), in TFLOP/s."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    B, S, H, d = xp.q.shape
    nthr = max(1, min(16, host_cores()))
    pairs = [(b, h) for b in range(B) for h in range(H)]

    def head(bh):
        b, h = bh
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        oracle.attention(xp.q[sl], xp.k[sl], xp.v[sl], None, True)

    with threadpool_limits(limits=1), ThreadPoolExecutor(nthr) as ex:
        t0 = time.perf_counter()
        list(ex.map(head, pairs))
        dt = time.perf_counter() - t0
    fl = causal_flops(1, len(pairs), S, d)
    return {"value": round(fl / dt / 1e12, 4), "unit": "TFLOP/s", "cores": nthr, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"all {len(pairs)} (batch, head) pairs of the causal prefill (S={S}, d={d}) on {nthr} "
                      f"threads, {dt:.2f} s, numpy fp64"}


def rotation_sets(set_bytes):
    """Resident K/V copies of one decode workload (one copy = K and V at capacity): at least
    ROTATION_BYTES in total, and at least two unless one copy alone is twice that."""
    return max(2 if set_bytes < 2 * ROTATION_BYTES else 1, -(-ROTATION_BYTES // set_bytes))


def replay_plan(nsets, reps, nreplays):
    """K/V copy each call of each captured graph reads: call r of graph g reads copy (g * reps + r) mod
    nsets, with as many graphs as it takes to visit every copy once but no more than the run's replays
    (replay i runs graph i mod the graph count)."""
    ngraphs = max(1, min(-(-nsets // reps), nreplays))
    return [[(g * reps + r) % nsets for r in range(reps)] for g in range(ngraphs)]


class DecodeLeg:
    """One decode workload on the device: q, seqlens, outputs, workspace, and K/V rotated over
    resident copies of at least ROTATION_BYTES (cache rows past each sequence end are zero)."""

    def __init__(self, aa, wl, name, num_splits, dev, to_dev):
        import torch
        self.aa, self.name, self.num_splits = aa, name, num_splits
        x = wl.decode_inputs(name, pad=wl.BF16_ZERO)
        B, sq, Hq, d = x.q.shape
        S, Hkv = x.k.shape[1], x.k.shape[2]
        self.shape = (B, sq, Hq, Hkv, d, S)
        self.seqlens = x.seqlens.copy()
        set_bytes = 2 * x.k.nbytes
        # at least two sets unless one set alone is at least twice the rotation footprint
        self.nsets = rotation_sets(set_bytes)
        self.q = to_dev(x.q)
        k0 = to_dev(x.k)
        self.K = torch.empty((self.nsets,) + tuple(k0.shape), dtype=k0.dtype, device=dev)
        self.K[:] = k0
        del k0
        v0 = to_dev(x.v)
        self.V = torch.empty_like(self.K)
        self.V[:] = v0
        del v0, x
        self.sl = torch.from_numpy(self.seqlens).to(dev)
        self.o = torch.empty((B, sq, Hq, d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, Hq, sq), dtype=torch.float32, device=dev)
        self.ws = torch.empty(max(16, aa.attn_decode_workspace_size(B, Hq, Hkv, sq, d, S, num_splits)),
                              dtype=torch.uint8, device=dev)
        self.pieces, _ = aa.attn_decode_plan(B, Hq, Hkv, d, sq, S, num_splits)
        self.kv_bytes = decode_kv_bytes(self.seqlens, Hkv, d)
        self.ms, self.ms_plain, self.reps, self.graphs = [], [], 1, []

    def call(self, i, stream):
        j = i % self.nsets
        self.aa.attn_decode(self.q, self.K[j], self.V[j], self.sl, self.o, self.lse, workspace=self.ws,
                            num_splits=self.num_splits, stream=stream)

    def capture(self, cap_stream, nreplays):
        """Graphs of back-to-back calls over the K/V copies replay_plan assigns them."""
        import torch
        self.reps = CALLS_PER_REPLAY[self.name]
        self.graphs = []
        for sets in replay_plan(self.nsets, self.reps, nreplays):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap_stream):
                for j in sets:
                    self.call(j, cap_stream)
            self.graphs.append(g)

    def replay(self, i):
        self.graphs[i % len(self.graphs)].replay()

    def report(self, read_peak, same_read_us=None):
        ms = self.ms
        mean = statistics.fmean(ms)
        thirds = [ms[k::3] for k in range(3)] if len(ms) >= 3 else [ms]
        gbps = self.kv_bytes / (mean * 1e-3) / 1e9
        B, sq, Hq, Hkv, d, S = self.shape
        r = {"workload": LEG_DESC[self.name], "kernel": "decode_stream + combine", "calls": len(ms) * self.reps,
             "calls_per_replay": self.reps, "graphs": len(self.graphs),
             "rotation_sets": self.nsets, "pieces_per_kv_head": self.pieces,
             "us_mean": round(mean * 1e3, 2), "us_median": round(statistics.median(ms) * 1e3, 2),
             "us_best_third_median": round(min(statistics.median(t) for t in thirds) * 1e3, 2),
             "us_min": round(min(ms) * 1e3, 2), "algorithmic_bytes_per_launch": self.kv_bytes,
             "kv_read_GBps": round(gbps, 1),
             "problem_GBps": round(decode_problem_bytes(self.seqlens, B, Hq, Hkv, d, sq) / (mean * 1e-3) / 1e9, 1),
             "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
             "traffic": measured_traffic(f"attn_decode:{self.name}", source_hash(DECODE_SOURCES), None)}
        if self.ms_plain:
            r["us_mean_plain"] = round(statistics.fmean(self.ms_plain) * 1e3, 2)
        if read_peak:
            r["frac_of_measured_read"] = round(gbps / read_peak, 4)
        if same_read_us:
            r["bare_read_same_bytes_us"] = round(same_read_us, 2)
            r["frac_of_bare_read"] = round(same_read_us / (mean * 1e3), 4)
        return r


def same_size_read_us(aa, dev, stream, nbytes):
    """Best time of the library's streaming-read kernel over exactly `nbytes` (8 back-to-back launches
    over copies rotated as the decode workloads rotate theirs, one event pair; best over grids)."""
    import torch
    ncopies = min(8, max(2, -(-ROTATION_BYTES // nbytes))) if nbytes < 2 * ROTATION_BYTES else 1
    bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(ncopies)]
    out = torch.empty(2048 * 256, dtype=torch.int32, device=dev)
    best = float("inf")
    for grid in (192, 256, 384, 512):
        for rep in range(3):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for r in range(8):
                aa.probe_stream_read(bufs[r % ncopies], out, grid, stream)
            ev[1].record(stream)
            torch.cuda.synchronize()
            if rep:
                best = min(best, ev[0].elapsed_time(ev[1]) / 8 * 1e3)
    del bufs, out
    return best


def measured_peaks(aa, dev, stream):
    """Practical ceilings of this device from the library's measurement kernels (not timed steps)."""
    import torch
    nbytes = 2 << 30
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device=dev)
    out = torch.empty(4096 * 256, dtype=torch.int32, device=dev)
    best, best_grid = 0.0, 0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for grid in (192, 256, 384, 512, 1024, 2048, 4096):
        for rep in range(3):
            ev[0].record(stream)
            aa.probe_stream_read(buf, out, grid, stream)
            ev[1].record(stream)
            torch.cuda.synchronize()
            if rep:
                gb = nbytes / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9
                if gb > best:
                    best, best_grid = gb, grid
    del buf, out
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    grid, iters = 2 * cus, 20000
    outf = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    clk = torch.zeros(4, dtype=torch.int64, device=dev)
    tf, ghz = 0.0, 0.0
    for rep in range(3):
        ev[0].record(stream)
        aa.probe_mfma_bf16(outf, grid, iters, clk, stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        t = grid * 4 * iters * 4 * 32768 / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e12
        c = clk.cpu().tolist()
        if rep and t > tf:
            tf, ghz = t, (c[1] - c[0]) / max(1, c[3] - c[2]) * 0.1
    return {"stream_read_GBps": round(best, 1), "stream_read_grid": best_grid,
            "stream_read_note": "2 GiB read once by attn_probe_stream_read (16-byte nontemporal loads, 256-thread "
                                "work-groups), best over grids and repetitions",
            "mfma_bf16_TFLOPs": round(tf, 1), "mfma_clock_GHz": round(ghz, 3),
            "mfma_note": f"attn_probe_mfma_bf16: {grid} work-groups x 4 waves, four independent "
                         "v_mfma_f32_32x32x16_bf16 chains per wave; clock from the shader-clock counter"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--num-splits", type=int, default=0, help="decode pieces per KV head (0 = automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--counter-run", action="store_true",
                    help="one copy, then one call of each decode workload, one prefill and one backward "
                         "(for rocprofv3 --pmc passes)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import attention_attn_decode_amd as aa
    import workloads as wl
    from attention_attn_decode_amd import build as _build

    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    aa.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    t0 = time.perf_counter()
    legs = [DecodeLeg(aa, wl, name, args.num_splits, dev, to_dev) for name in DECODE_LEGS]
    head = legs[0]
    xd = wl.decode_inputs("gqa-decode", pad=wl.BF16_ZERO) if not args.no_cpu_baseline else None

    # ---- prefill workload ----
    run_prefill = not args.no_prefill
    xp = None
    if run_prefill:
        pc = wl.PREFILL_CONFIGS["causal-prefill"]
        xp = wl.prefill_inputs(pc)
        qp, kp, vp = to_dev(xp.q), to_dev(xp.k), to_dev(xp.v)
        op = torch.empty_like(qp)
        lsep = torch.empty((pc.batch, pc.n_q_heads, pc.seqlen), dtype=torch.float32, device=dev)
        run_backward = not args.no_backward
        if run_backward:
            dop = to_dev(wl.make_grad_out(xp.q, 1005))
            dqp, dkp, dvp = torch.empty_like(qp), torch.empty_like(kp), torch.empty_like(vp)
            wsb = torch.empty(aa.attn_bwd_workspace_size(pc.batch, pc.n_q_heads, pc.seqlen), dtype=torch.uint8,
                              device=dev)
    else:
        run_backward = False
    run_varlen = not args.no_varlen and not args.counter_run
    if run_varlen:
        xv = wl.varlen_prefill_inputs()
        lens_v = np.diff(xv.cu_q).astype(np.int64)
        qv, kv_, vv = to_dev(xv.q), to_dev(xv.k), to_dev(xv.v)
        cqv = torch.from_numpy(xv.cu_q.copy()).to(dev)
        ckv = torch.from_numpy(xv.cu_k.copy()).to(dev)
        ov = torch.empty_like(qv)
        lsev = torch.empty((qv.shape[1], qv.shape[0]), dtype=torch.float32, device=dev)
        max_qv = int(lens_v.max())
        varlen_name = xv.meta["config"]
        del xv
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0

    stream = torch.cuda.current_stream()

    if args.counter_run:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        for leg in legs:
            leg.call(0, stream)
        if run_prefill:
            aa.attn_fwd(qp, kp, vp, op, lsep, causal=True, stream=stream)
        if run_backward:
            aa.attn_bwd(qp, kp, vp, op, lsep, dop, dqp, dkp, dvp, wsb, causal=True, stream=stream)
        torch.cuda.synchronize()
        print("counter run done", flush=True)
        return

    # Each workload's calls as a graph (one eager call of each first, outside any capture). Per step: the
    # prefill, its backward, the packed prefill, then every decode workload, the headline last; one event
    # pair around each replay on the launch stream. The steps are enqueued without waiting, so the host
    # runs ahead of the device and no replay's start event fires on an idle queue before the replay itself
    # is launched - except the first after the synchronize that opens the timed region, which is therefore
    # the long prefill (its host launch gap is then a fraction of a percent of it).
    def run_prefill_call(s):
        aa.attn_fwd(qp, kp, vp, op, lsep, causal=True, stream=s)

    def run_backward_call(s):
        aa.attn_bwd(qp, kp, vp, op, lsep, dop, dqp, dkp, dvp, wsb, causal=True, stream=s)

    def run_varlen_call(s):
        aa.attn_fwd_varlen(qv, kv_, vv, cqv, ckv, ov, max_qv, lse=lsev, causal=True, stream=s)

    single = [f for f, on in ((run_prefill_call, run_prefill), (run_backward_call, run_backward),
                              (run_varlen_call, run_varlen)) if on]
    for f in single:
        f(stream)
    for leg in legs:
        leg.call(0, stream)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    nreplays = args.warmup + args.steps
    for leg in legs:
        leg.capture(cap, nreplays)
    single_graphs = []
    for f in single:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            f(cap)
        single_graphs.append(g)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    nev = len(legs) + len(single_graphs)

    def step(i, evs=None):
        k = len(legs)
        for si, g in enumerate(single_graphs):
            if evs:
                evs[k + si][0].record(stream)
            g.replay()
            if evs:
                evs[k + si][1].record(stream)
        for li in reversed(range(len(legs))):
            if evs:
                evs[li][0].record(stream)
            legs[li].replay(i)
            if evs:
                evs[li][1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nev)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    for li, leg in enumerate(legs):
        leg.ms = [e[li][0].elapsed_time(e[li][1]) / leg.reps for e in events]
    k = len(legs)
    single_ms = [[e[k + si][0].elapsed_time(e[k + si][1]) for e in events] for si in range(len(single_graphs))]
    pre_ms = single_ms.pop(0) if run_prefill else []
    bwd_ms = single_ms.pop(0) if run_backward else []
    var_ms = single_ms.pop(0) if run_varlen else []

    # The same calls as plain launches, an event pair around each (not part of the timed steps).
    def plain(f, n):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for c in range(n):
            ev[c][0].record(stream)
            f(c)
            ev[c][1].record(stream)
        torch.cuda.synchronize()
        return [e[0].elapsed_time(e[1]) for e in ev]

    plain_ms = {}
    for f, name in zip(single, [n for n, on in (("prefill", run_prefill), ("backward", run_backward),
                                                 ("varlen_prefill", run_varlen)) if on]):
        plain_ms[name] = plain(lambda c, f=f: f(stream), 3)
    for leg in reversed(legs):
        leg.ms_plain = plain(lambda c, leg=leg: leg.call(c, stream), PLAIN_CALLS)

    peaks = None if args.no_peaks else measured_peaks(aa, dev, stream)
    read_peak = peaks["stream_read_GBps"] if peaks else None
    same_read = {} if args.no_peaks else {leg.name: same_size_read_us(aa, dev, stream, leg.kv_bytes) for leg in legs}
    mfma_peak = peaks["mfma_bf16_TFLOPs"] if peaks else None

    dec = head.report(read_peak, same_read.get(head.name))
    dec_mean_ms = dec["us_mean"] * 1e-3
    dec_gbps = head.kv_bytes / (statistics.fmean(head.ms) * 1e-3) / 1e9
    B, sq, Hq, Hkv, d, S = head.shape
    result = {
        "metric": "decode KV-read GB/s (% HBM peak); causal prefill fwd TFLOP/s (% MFMA peak)",
        "value": round(dec_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": LEG_DESC["gqa-decode"],
            "global_batch": B,
            "seq_len": int(S),
            "kv_tokens": int(head.seqlens.sum()),
            "pieces_per_kv_head": head.pieces,
            "other_decode_workloads": [LEG_DESC[w] for w in DECODE_LEGS[1:]],
            "prefill_workload": PREFILL_DESC if run_prefill else None,
            "backward_workload": BACKWARD_DESC if run_backward else None,
            "varlen_workload": varlen_name if run_varlen else None,
            "parallelism": "single-gpu",
            "device": props.name,
            "cus": props.multi_processor_count,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "attn_decode = decode_stream + combine_pieces",
            "achieved": round(dec_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
            "traffic": dec["traffic"],
            "algorithmic_bytes_per_launch": head.kv_bytes,
            "avg_launch_ms": round(dec_mean_ms, 5),
        },
        "decode": {w: leg.report(read_peak, same_read.get(w)) for w, leg in zip(DECODE_LEGS, legs)},
        "measured_peaks": peaks,
        "timing": ("HIP graph replays: each workload's calls captured once (decode: calls_per_replay back-to-back "
                   "calls per replay, K/V rotated over >= 1 GiB of resident copies; prefill, backward, packed "
                   "prefill: one call), one pair of HIP events around each replay on the launch stream; a call's "
                   "time = replay time / calls per replay; means over the timed steps. *_plain: the same calls "
                   "as plain launches with an event pair around each, after the timed steps"),
        "setup_s": round(setup_s, 1),
    }
    if run_prefill:
        pre_mean = statistics.fmean(pre_ms)
        fl = causal_flops(pc.batch, pc.n_q_heads, pc.seqlen, pc.d)
        tf = fl / (pre_mean * 1e-3) / 1e12
        result["prefill"] = {
            "bound": "mfma",
            "workload": PREFILL_DESC,
            "kernel": "fwd_persist (dense d = 128: one persistent work-group per CU)",
            "ms_mean": round(pre_mean, 5),
            "ms_median": round(statistics.median(pre_ms), 5),
            "ms_mean_plain": round(statistics.fmean(plain_ms["prefill"]), 5),
            "flops": fl,
            "achieved": round(tf, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "frac_of_measured_mfma": round(tf / mfma_peak, 4) if mfma_peak else None,
            "traffic": measured_traffic("attn_fwd", source_hash(FWD_SOURCES), None),
        }
    if run_backward:
        bwd_mean = statistics.fmean(bwd_ms)
        fl = 2.5 * causal_flops(pc.batch, pc.n_q_heads, pc.seqlen, pc.d)
        tf = fl / (bwd_mean * 1e-3) / 1e12
        result["backward"] = {
            "bound": "mfma",
            "workload": BACKWARD_DESC,
            "kernel": "attn_bwd = bwd_pre + bwd_dkdv + bwd_dq",
            "ms_mean": round(bwd_mean, 5),
            "ms_median": round(statistics.median(bwd_ms), 5),
            "ms_mean_plain": round(statistics.fmean(plain_ms["backward"]), 5),
            "flops": int(fl),
            "flops_note": "2.5 x the causal forward FLOPs (five products per visible pair)",
            "achieved": round(tf, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "frac_of_measured_mfma": round(tf / mfma_peak, 4) if mfma_peak else None,
            "traffic": measured_traffic("attn_bwd", source_hash(BWD_SOURCES), None),
        }
    if run_varlen:
        var_mean = statistics.fmean(var_ms)
        Hv, dv_ = qv.shape[1], qv.shape[2]
        fl = int(sum(4 * dv_ * Hv * (int(L) * (int(L) + 1) // 2) for L in lens_v))  # exact causal FLOPs
        tf = fl / (var_mean * 1e-3) / 1e12
        result["varlen_prefill"] = {
            "bound": "mfma",
            "kernel": "fwd_persist (packed d = 128: one persistent work-group per CU over the non-empty tiles)",
            "ms_mean": round(var_mean, 5),
            "ms_median": round(statistics.median(var_ms), 5),
            "ms_mean_plain": round(statistics.fmean(plain_ms["varlen_prefill"]), 5),
            "tokens": int(lens_v.sum()),
            "flops": fl,
            "achieved": round(tf, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4),
        }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_decode(xd, d)
        if xp is not None:
            result["cpu_baseline_prefill"] = cpu_baseline_prefill(xp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
