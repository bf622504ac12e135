"""Host logic of bench.py that needs no GPU: recorded HBM counters are
reported only for the workload and the kernel source they were taken on."""
import hashlib
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_only_for_recorded_workload_and_source(tmp_path):
    b = _bench()
    src = tmp_path / "kernel.hip"
    src.write_bytes(b"// some kernel source\n")
    rec = dict(b.COSINE_GEMM_COUNTERS)
    rec["source"] = str(src)  # absolute: os.path.join keeps it
    rec["sha256"] = hashlib.sha256(src.read_bytes()).hexdigest()
    t = b.counters_traffic_gb(rec, rec["config"])
    want = (rec["fetch_kib_per_step"] * rec["fetch_scale"] + rec["write_kib_per_step"] * rec["write_scale"]) * 1024 / 1e9
    assert t is not None and abs(t - want) < 1e-9
    # another workload: no figure
    assert b.counters_traffic_gb(rec, rec["config"] + 2) is None
    # the source changed since: no figure
    src.write_bytes(b"// edited\n")
    assert b.counters_traffic_gb(rec, rec["config"]) is None
    # the source is missing: no figure
    rec["source"] = str(tmp_path / "missing.hip")
    assert b.counters_traffic_gb(rec, rec["config"]) is None
