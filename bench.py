#!/usr/bin/env python3
"""Single-GPU benchmark of the attention hot path on MI355X.

A step is one pass of the whole path over one batch of synthetic input:
  * GQA decode on the headline workload (batch 32, 64 query / 8 KV heads,
    d = 128, one new token, KV lengths uniform in [1024, 8192]): split-KV
    kernel + combine, through the C ABI;
  * causal prefill (batch 2, 32 heads, d = 128, S = 8192) through attn_fwd;
  * the backward pass of that prefill (dQ, dK, dV from its O and LSE and a
    synthetic dO) through attn_bwd;
  * a packed variable-length causal prefill (16 sequences, lengths uniform in
    [256, 4096], 32 heads, d = 128) through attn_fwd_varlen.
The headline `value` is decode KV-read bandwidth: algorithmic K+V bytes
(sum_b L_b * Hkv * 4d) over the measured duration of the decode call, timed
with HIP events on the stream the kernels run on. Prefill TFLOP/s (exact causal
FLOPs, 4 d per visible query-key pair) is reported beside it, and backward
TFLOP/s counted, as the backward page does, as 2.5 times the forward FLOPs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-backward] [--no-varlen]
Prints one JSON line.

HBM traffic (roofline.traffic) comes from two rocprofv3 counter passes over
`bench.py --counter-run` (one 1 GiB device copy for calibration, then one
decode call, one prefill call and one backward call, nothing timed):
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT -o fetch -- python bench.py --counter-run
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT -o write -- python bench.py --counter-run
  python bench.py --ingest-counters OUT/fetch_counter_collection.csv OUT/write_counter_collection.csv
The last step (no GPU) scales each counter by what it read for the copy and
stores bytes per launch, keyed by a hash of the kernel sources, in
profiles/hbm_traffic_counters.json; a stale hash reports traffic as null.
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


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
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
TRAFFIC_KERNELS = {  # stored key -> (kernel-name prefixes, sources, workload)
    "attn_decode": (("decode_stream<", "combine_pieces<"), DECODE_SOURCES,
                    "gqa-decode b=32 hq=64 hkv=8 d=128 sq=1 kv_len~U[1024,8192] (seed 1001)"),
    "attn_fwd": (("fwd_persist<", "fwd_pp<"), FWD_SOURCES, "causal-prefill b=2 h=32 d=128 s=8192 (seed 1004)"),
    "attn_bwd": (("bwd_pre<", "bwd_dkdv<", "bwd_dq<"), BWD_SOURCES,
                 "causal-prefill backward b=2 h=32 d=128 s=8192 (seed 1004, dO seed 1005)"),
}


def _short_name(name):
    name = name.replace("void ", "").replace("attn::(anonymous namespace)::", "")
    return name.split("(")[0].strip()


def ingest_counters(fetch_csv, write_csv):
    """Turn the FETCH_SIZE and WRITE_SIZE passes of `--counter-run` into bytes per launch."""
    import csv

    def read(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not copies:
            raise SystemExit(f"{path}: no copy dispatch to calibrate {counter} against")
        scale = COPY_BYTES / (max(copies) * 1024.0)   # bytes per counted KiB
        per = {}
        for r in rows:
            per.setdefault(_short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return scale, max(copies), per

    fs, fcopy, fper = read(fetch_csv, "FETCH_SIZE")
    ws, wcopy, wper = read(write_csv, "WRITE_SIZE")
    out = {"note": "HBM bytes per launch: rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch, "
                   "separate passes over bench.py --counter-run), each scaled by the ratio of a "
                   "1 GiB device copy's true bytes to what the same counter read for it.",
           "calibration": {"copy_bytes": COPY_BYTES, "fetch_size_kib": fcopy, "write_size_kib": wcopy,
                           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)}}
    for key, (prefixes, srcs, workload) in TRAFFIC_KERNELS.items():
        kern, fetch, write = {}, 0.0, 0.0
        for nm in fper:
            if nm.startswith(prefixes):
                f = statistics.fmean(fper[nm])
                w = statistics.fmean(wper.get(nm, [0.0]))
                kern[nm] = {"fetch_kib": round(f, 3), "write_kib": round(w, 3), "dispatches": len(fper[nm])}
                fetch += f * 1024.0 * fs
                write += w * 1024.0 * ws
        if kern:
            out[key] = {"source_hash": source_hash(srcs), "workload": workload, "kernels": kern,
                        "fetch_bytes": round(fetch), "write_bytes": round(write),
                        "bytes_per_launch": round(fetch + write)}
    with open(COUNTERS, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps({k: v.get("bytes_per_launch") for k, v in out.items() if isinstance(v, dict)}))


def cpu_baseline_decode(x, d):
    """Time the fp64 oracle on the decode workload (full workload, one pass)."""
    import oracle
    try:
        ncores = len(os.sched_getaffinity(0))
    except AttributeError:
        ncores = os.cpu_count() or 1
    from threadpoolctl import threadpool_limits
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
            "sample": f"full decode workload, {reps} pass(es), {dt:.2f} s per pass, numpy fp64"}


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
    ap.add_argument("--counter-run", action="store_true",
                    help="one copy, one decode and one prefill dispatch for rocprofv3 --pmc passes")
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

    # ---- decode workload (cache at capacity, rows past each sequence end zero) ----
    dc = wl.DECODE_CONFIGS["gqa-decode"]
    t0 = time.perf_counter()
    xd = wl.decode_inputs(dc, pad=wl.BF16_ZERO)
    B, sq, Hq, d = xd.q.shape
    S, Hkv = xd.k.shape[1], xd.k.shape[2]
    sets = []
    q0, k0, v0 = to_dev(xd.q), to_dev(xd.k), to_dev(xd.v)
    sl = torch.from_numpy(xd.seqlens.copy()).to(dev)
    # two resident copies (2 x 1 GiB of cache) alternate so no step reads
    # K/V left in the 256 MB Infinity Cache by the previous one
    sets.append((q0, k0, v0))
    sets.append((q0.clone(), k0.clone(), v0.clone()))
    wsz = aa.attn_decode_workspace_size(B, Hq, Hkv, sq, d, S, args.num_splits)
    ws = torch.empty(wsz, dtype=torch.uint8, device=dev)
    od = torch.empty((B, sq, Hq, d), dtype=torch.bfloat16, device=dev)
    lsed = torch.empty((B, Hq, sq), dtype=torch.float32, device=dev)
    pieces, min_piece = aa.attn_decode_plan(B, Hq, Hkv, d, sq, S, args.num_splits)

    # ---- prefill workload ----
    run_prefill = not args.no_prefill
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
        del xp
    else:
        run_backward = False
    run_varlen = not args.no_varlen
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
    setup_s = time.perf_counter() - t0

    stream = torch.cuda.current_stream()

    if args.counter_run:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        q, k, v = sets[0]
        aa.attn_decode(q, k, v, sl, od, lsed, workspace=ws, num_splits=args.num_splits, stream=stream)
        if run_prefill:
            aa.attn_fwd(qp, kp, vp, op, lsep, causal=True, stream=stream)
        if run_backward:
            aa.attn_bwd(qp, kp, vp, op, lsep, dop, dqp, dkp, dvp, wsb, causal=True, stream=stream)
        torch.cuda.synchronize()
        print("counter run done", flush=True)
        return

    def step(i, evs=None):
        q, k, v = sets[i % 2]
        if evs:
            evs[0].record(stream)
        aa.attn_decode(q, k, v, sl, od, lsed, workspace=ws, num_splits=args.num_splits, stream=stream)
        if evs:
            evs[1].record(stream)
        if run_prefill:
            aa.attn_fwd(qp, kp, vp, op, lsep, causal=True, stream=stream)
        if evs:
            evs[2].record(stream)
        if run_backward:
            aa.attn_bwd(qp, kp, vp, op, lsep, dop, dqp, dkp, dvp, wsb, causal=True, stream=stream)
        if evs:
            evs[3].record(stream)
        if run_varlen:
            aa.attn_fwd_varlen(qv, kv_, vv, cqv, ckv, ov, max_qv, lse=lsev, causal=True, stream=stream)
        if evs:
            evs[4].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    dec_ms = [e[0].elapsed_time(e[1]) for e in events]
    pre_ms = [e[1].elapsed_time(e[2]) for e in events]
    bwd_ms = [e[2].elapsed_time(e[3]) for e in events]
    var_ms = [e[3].elapsed_time(e[4]) for e in events]
    dec_mean = statistics.fmean(dec_ms)
    pre_mean = statistics.fmean(pre_ms) if run_prefill else 0.0

    kv_bytes = decode_kv_bytes(xd.seqlens, Hkv, d)
    dec_gbps = kv_bytes / (dec_mean * 1e-3) / 1e9
    prob_gbps = decode_problem_bytes(xd.seqlens, B, Hq, Hkv, d, sq) / (dec_mean * 1e-3) / 1e9

    # plain device copy for context: practical HBM rate on this part
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record(stream)
    for _ in range(5):
        dst.copy_(src)
    ce[1].record(stream)
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * src.numel() / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e9
    del src, dst

    dec_hash = source_hash(DECODE_SOURCES)
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
            "workload": "gqa-decode b=32 hq=64 hkv=8 d=128 sq=1 kv_len~U[1024,8192] (seed 1001)",
            "global_batch": B,
            "seq_len": int(S),
            "kv_tokens": int(xd.seqlens.sum()),
            "pieces_per_kv_head": pieces,
            "prefill_workload": "causal-prefill b=2 h=32 d=128 s=8192 (seed 1004)" if run_prefill else None,
            "backward_workload": "backward of that prefill, dO seed 1005" if run_backward else None,
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
            "traffic": measured_traffic("attn_decode", dec_hash, kv_bytes),
            "algorithmic_bytes_per_launch": kv_bytes,
            "avg_launch_ms": round(dec_mean, 5),
        },
        "decode": {
            "ms_mean": round(dec_mean, 5),
            "ms_median": round(statistics.median(dec_ms), 5),
            "ms_min": round(min(dec_ms), 5),
            "kv_read_GBps": round(dec_gbps, 2),
            "problem_GBps": round(prob_gbps, 2),
            "frac_hbm_peak": round(dec_gbps / HBM_PEAK_GBPS, 4),
            "frac_of_device_copy": round(dec_gbps / copy_gbps, 4),
        },
        "device_copy_GBps": round(copy_gbps, 1),
        "setup_s": round(setup_s, 1),
    }
    if run_prefill:
        fl = causal_flops(pc.batch, pc.n_q_heads, pc.seqlen, pc.d)
        tf = fl / (pre_mean * 1e-3) / 1e12
        result["prefill"] = {
            "bound": "mfma",
            "kernel": "fwd_persist (dense d = 128: one persistent work-group per CU)",
            "ms_mean": round(pre_mean, 5),
            "ms_median": round(statistics.median(pre_ms), 5),
            "flops": fl,
            "achieved": round(tf, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("attn_fwd", source_hash(FWD_SOURCES), None),
        }
    if run_backward:
        bwd_mean = statistics.fmean(bwd_ms)
        fl = 2.5 * causal_flops(pc.batch, pc.n_q_heads, pc.seqlen, pc.d)
        tf = fl / (bwd_mean * 1e-3) / 1e12
        result["backward"] = {
            "bound": "mfma",
            "kernel": "attn_bwd = bwd_pre + bwd_dkdv + bwd_dq",
            "ms_mean": round(bwd_mean, 5),
            "ms_median": round(statistics.median(bwd_ms), 5),
            "flops": int(fl),
            "flops_note": "2.5 x the causal forward FLOPs (five products per visible pair)",
            "achieved": round(tf, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("attn_bwd", source_hash(BWD_SOURCES), None),
        }
    if run_varlen:
        var_mean = statistics.fmean(var_ms)
        Hv, dv_ = qv.shape[1], qv.shape[2]
        fl = int(sum(4 * dv_ * Hv * (int(L) * (int(L) + 1) // 2) for L in lens_v))  # exact causal FLOPs
        tf = fl / (var_mean * 1e-3) / 1e12
        result["varlen_prefill"] = {
            "bound": "mfma",
            "kernel": "fwd_pp (packed offsets, one work-group per tile)",
            "ms_mean": round(var_mean, 5),
            "ms_median": round(statistics.median(var_ms), 5),
            "tokens": int(lens_v.sum()),
            "flops": fl,
            "achieved": round(tf, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4),
        }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_decode(xd, d)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
