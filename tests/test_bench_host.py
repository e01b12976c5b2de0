"""Host-side checks of bench.py's contract (CPU only)."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""              # no JSON line for a refused run


@pytest.mark.parametrize("workload", ["video_dit_p4_s16384_h24_bf16", "wan_long_p4_s75600_h40_bf16"])
def test_traffic_profile_matches_the_kernel_source(workload):
    """The committed HBM counter runs were taken on the kernel source in the tree:
    otherwise bench.py reports traffic as null (a kernel changed since)."""
    bench = _bench()
    with open(os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)) as f:
        rec = json.load(f)
    assert rec["kernel_source_sha"] == bench.kernel_source_hash()
    assert bench.traffic_from_profiles(workload) == rec["hbm_bytes_per_launch"]
    # traffic is HBM bytes; within a few percent of the algorithmic bytes (the
    # cos/sin table, and for the padded sequence its pad rows) means no wasted re-reads
    assert 1.0 <= rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] < 1.03


def test_quantiles_and_spread():
    bench = _bench()
    t = sorted([1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0, 9.0, 10.0])
    assert bench.pick(t, 0.5) == 6.0 and bench.pick(t, 0.1) == 2.0 and bench.pick(t, 0.9) == 10.0
    s = bench.spread([0.1] * 20, 805306368, 1e9, "GB/s")
    assert s["samples"] == 20 and s["median_us"] == 100.0
    assert s["GB_s_at_median"] == round(805306368 / 1e-4 / 1e9, 2)


def test_bench_gates_and_defaults():
    """A/A drift beyond 2 % voids a record; at least 10 dominant launches are timed;
    the default run rotates over three buffer sets."""
    bench = _bench()
    assert bench.AA_MAX_DRIFT == 0.02 and bench.MIN_TIMED_LAUNCHES == 10
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert '"--sets", type=int, default=3' in src
