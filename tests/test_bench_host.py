"""Host logic of bench.py that needs no GPU: the recorded HBM counters are
reported only for the workload and kernel source they were taken on."""
import copy
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_only_for_recorded_workload_and_source():
    b = _bench()
    rec = b.COSINE_GEMM_COUNTERS
    t = b.counters_traffic_gb(rec, rec["config"])
    assert t is not None and t > 0
    # the same figure from the record's own terms (KiB x calibration scale)
    want = (rec["fetch_kib_per_step"] * rec["fetch_scale"] + rec["write_kib_per_step"] * rec["write_scale"]) * 1024 / 1e9
    assert abs(t - want) < 1e-9
    # another workload: no figure
    assert b.counters_traffic_gb(rec, rec["config"] + 2) is None
    # another kernel source: no figure
    bad = copy.deepcopy(rec)
    bad["sha256"] = "0" * 64
    assert b.counters_traffic_gb(bad, rec["config"]) is None
