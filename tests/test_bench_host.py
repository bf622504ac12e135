"""Host logic of bench.py that needs no GPU: recorded counter figures are
reported only for the workload and the kernel source they were taken on, and
their traffic is the calibrated sum of the two byte counters."""
import hashlib
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_counters_only_for_recorded_workload_and_source(tmp_path):
    b = _bench()
    src = tmp_path / "kernel.hip"
    src.write_bytes(b"// some kernel source\n")
    rec = dict(b.COUNTERS["groups"]["cosine_gemm"])
    rec["source"] = str(src)  # absolute: os.path.join keeps it
    rec["sha256"] = hashlib.sha256(src.read_bytes()).hexdigest()
    b.COUNTERS["groups"]["probe"] = rec
    cfg = b.COUNTERS["config"]
    c = b.counters_for("probe", cfg)
    want = (rec["fetch_kib"] * b.COUNTERS["fetch_scale"] + rec["write_kib"] * b.COUNTERS["write_scale"]) * 1024 / 1e9
    assert c is not None and abs(c["traffic_gb"] - want) < 1e-9
    assert c["executed_tflop"] == rec["executed_tflop"] and c["mfma_busy"] == rec["mfma_busy"]
    # another workload, or a group never recorded: no figure
    assert b.counters_for("probe", cfg + 2) is None
    assert b.counters_for("no_such_group", cfg) is None
    # the source changed since: no figure
    src.write_bytes(b"// edited\n")
    assert b.counters_for("probe", cfg) is None
    # the source is missing: no figure
    rec["source"] = str(tmp_path / "missing.hip")
    assert b.counters_for("probe", cfg) is None


def test_recorded_groups_cover_the_step_kernels():
    b = _bench()
    g = b.COUNTERS["groups"]
    for name in ("cosine_gemm", "shared_attention", "gather_attention", "dense", "per_frame_gemm"):
        assert name in g and g[name]["fetch_kib"] > 0 and g[name]["write_kib"] > 0
    # the matrix-core groups executed at most the FLOP their launches could
    # hold, and the symmetric square makes the index GEMM execute less than
    # its algorithmic 2 (S P)^2 Df = 38.4 TFLOP at S = 100
    assert 0 < g["cosine_gemm"]["executed_tflop"] < 38.4
    assert 0 < g["shared_attention"]["mfma_busy"] < 1 and 0 < g["dense"]["mfma_busy"] < 1


def test_counters_keyed_on_every_listed_source(tmp_path):
    """A group recorded over two files (the kernel and the code that
    schedules its launches) loses its figures when either file changes."""
    b = _bench()
    a, s = tmp_path / "kernel.hip", tmp_path / "schedule.cpp"
    a.write_bytes(b"// kernel\n")
    s.write_bytes(b"// schedule\n")
    rec = dict(b.COUNTERS["groups"]["cosine_gemm"])
    rec["source"] = [str(a), str(s)]
    rec["sha256"] = hashlib.sha256(a.read_bytes() + s.read_bytes()).hexdigest()
    b.COUNTERS["groups"]["probe2"] = rec
    cfg = b.COUNTERS["config"]
    assert b.counters_for("probe2", cfg) is not None
    s.write_bytes(b"// another schedule\n")
    assert b.counters_for("probe2", cfg) is None
    s.write_bytes(b"// schedule\n")
    assert b.counters_for("probe2", cfg) is not None
    a.write_bytes(b"// another kernel\n")
    assert b.counters_for("probe2", cfg) is None

