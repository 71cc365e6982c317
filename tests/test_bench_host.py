"""Host-side logic of bench.py that needs no GPU: the kernel-source hash that keys
the stored HBM counters, and the counter record lookup."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_only_drops_comments_and_layout_but_keeps_literals():
    b = _bench()
    src = ('int a = 1;  // trailing note\n/* block\n   comment */ const char *s = "x // y /* z */";\n'
           "char c = '\"';\tint   b ;\n")
    assert b._code_only(src) == 'int a = 1; const char *s = "x // y /* z */"; char c = \'"\'; int b ;'
    # A comment edit or a re-indent leaves the hash input unchanged; a code edit does not.
    assert b._code_only("x = 1; // one\n") == b._code_only("x  =  1;   /* two */")
    assert b._code_only("x = 1;") != b._code_only("x = 2;")


def test_source_hash_ignores_comment_edits(tmp_path, monkeypatch):
    b = _bench()
    f = tmp_path / "k.hip"
    f.write_text("__global__ void k() { int a = 0; } // v1\n")
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    h1 = b.source_hash(["k.hip"])
    f.write_text("// header\n__global__ void k() {\n  int a = 0;\n}\n")
    assert b.source_hash(["k.hip"]) == h1
    f.write_text("__global__ void k() { int a = 1; }\n")
    assert b.source_hash(["k.hip"]) != h1


def test_stored_traffic_is_reported_only_for_a_matching_hash(tmp_path, monkeypatch):
    b = _bench()
    counters = tmp_path / "c.json"
    counters.write_text('{"attn_fwd": {"source_hash": "abc", "bytes_per_launch": 123}}')
    monkeypatch.setattr(b, "COUNTERS", str(counters))
    assert b.measured_traffic("attn_fwd", "abc", None) == 123
    assert b.measured_traffic("attn_fwd", "def", None) is None
    assert b.measured_traffic("attn_bwd", "abc", None) is None


def test_replayed_decode_calls_never_find_their_kv_in_a_cache():
    """Every decode workload as the default run replays it (3 warm-up + 20 timed replays): between two reads
    of the same K/V bytes the run reads at least 1 GB of K/V (the copy's own call and every call between),
    so none of it can still sit in the 256 MB Infinity Cache."""
    import numpy as np
    import workloads as wl
    b = _bench()
    for name in b.DECODE_LEGS:
        c = wl.DECODE_CONFIGS[name]
        lens = wl.draw_lengths(c.seed, c.batch, c.len_lo, c.len_hi)
        call_bytes = b.decode_kv_bytes(np.asarray(lens), c.n_kv_heads, c.d)
        set_bytes = 2 * c.batch * c.max_seqlen_k * c.n_kv_heads * c.d * 2
        nsets = b.rotation_sets(set_bytes)
        assert nsets * set_bytes >= b.ROTATION_BYTES
        reps = b.CALLS_PER_REPLAY[name]
        plan = b.replay_plan(nsets, reps, 23)
        assert all(len(g) == reps and all(0 <= j < nsets for j in g) for g in plan)
        calls = [j for i in range(23) for j in plan[i % len(plan)]]
        last = {}
        for n, j in enumerate(calls):
            if j in last:
                between = n - last[j] - 1
                assert (1 + between) * call_bytes >= 1e9, (name, n, between)
            last[j] = n


def _counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, value) in enumerate(rows):
            f.write(f'{i + 1},"{name}",{counter},{value}\n')


def _counter_run_dispatches():
    """Kernel names of a --counter-run: a set-up copy, the 1 GiB calibration copy, then every leg."""
    names = ["__amd_rocclr_copyBuffer", "__amd_rocclr_copyBuffer"]
    for w in ("gqa-decode", "gqa-decode-small", "multi-token-decode", "long-context-decode"):
        names.append("void attn::(anonymous namespace)::decode_stream<128, false, 1, false>(int)")
        if w != "gqa-decode-small":  # the grouped kernel serves the small decode: no combine
            names.append("void attn::(anonymous namespace)::combine_pieces<128, false, 1>(int)")
    names += ["void attn::(anonymous namespace)::fwd_persist<128, false>(int)",
              "void attn::(anonymous namespace)::bwd_pre<128>(int)",
              "void attn::(anonymous namespace)::bwd_dkdv<128, false>(int)",
              "void attn::(anonymous namespace)::bwd_dq<128, false>(int)"]
    return names


def test_counter_ingest_scales_each_launch_by_the_calibration_copy(tmp_path, monkeypatch):
    b = _bench()
    names = _counter_run_dispatches()
    # FETCH_SIZE reads half of the copy's bytes (scale 2), WRITE_SIZE all of them (scale 1).
    fetch = [10.0, 512.0 * 1024] + [float(i + 1) for i in range(len(names) - 2)]
    write = [10.0, 1024.0 * 1024] + [float(100 + i) for i in range(len(names) - 2)]
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", list(zip(names, fetch)))
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", list(zip(names, write)))
    monkeypatch.setattr(b, "COUNTERS", str(tmp_path / "out.json"))
    b.ingest_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    import json
    out = json.load(open(tmp_path / "out.json"))
    assert out["calibration"]["fetch_scale"] == 2.0 and out["calibration"]["write_scale"] == 1.0
    # dispatch k after the calibration copy has FETCH k + 1 and WRITE 100 + k KiB
    expect, k = {}, 0
    for key, prefixes, _, _ in b.COUNTER_LEGS:
        n = 1 if key == "attn_decode:gqa-decode-small" else len(prefixes)
        expect[key] = sum((k + j + 1) * 1024 * 2 + (100 + k + j) * 1024 for j in range(n))
        k += n
    assert {key: out[key]["bytes_per_launch"] for key in expect} == expect
    assert list(out["attn_decode:gqa-decode-small"]["kernels"]) == ["decode_stream<128, false, 1, false>"]
    assert out["attn_bwd"]["source_hash"] == b.source_hash(b.BWD_SOURCES)


def test_counter_ingest_rejects_a_run_out_of_order(tmp_path, monkeypatch):
    b = _bench()
    names = _counter_run_dispatches()
    names[-1], names[-2] = names[-2], names[-1]  # bwd_dq before bwd_dkdv
    rows = [(n, 1024.0) for n in names]
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", rows)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", rows)
    monkeypatch.setattr(b, "COUNTERS", str(tmp_path / "out.json"))
    import pytest
    with pytest.raises(SystemExit):
        b.ingest_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    assert not (tmp_path / "out.json").exists()


def test_more_than_one_gpu_is_refused_with_a_message():
    import subprocess, sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
