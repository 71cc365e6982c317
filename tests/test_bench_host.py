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
