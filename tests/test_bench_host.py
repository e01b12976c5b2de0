"""Host-side checks of bench.py's contract (CPU only)."""
import importlib.util
import json
import os
import subprocess
import sys

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


def test_traffic_profile_matches_the_kernel_source():
    """The committed HBM counter run was taken on the kernel source in the tree:
    otherwise bench.py reports traffic as null (a kernel changed since)."""
    bench = _bench()
    with open(os.path.join(ROOT, "profiles", "traffic_video_dit_p4_s16384_h24_bf16.json")) as f:
        rec = json.load(f)
    assert rec["kernel_source_sha"] == bench.kernel_source_hash()
    assert bench.traffic_from_profiles("video_dit_p4_s16384_h24_bf16") == rec["hbm_bytes_per_launch"]
    # traffic is HBM bytes; within a few percent of the algorithmic bytes (the
    # cos/sin table adds 8 MiB) means no wasted re-reads
    assert 1.0 <= rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] < 1.03
