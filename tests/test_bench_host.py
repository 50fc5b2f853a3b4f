"""Host logic of bench.py (CPU only, no GPU call): the one-GPU guard, and the
rule that HBM traffic from the committed counter summary is reported only
while that summary was taken on the kernel source being measured."""

import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    for argv, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2, (argv, env, r.returncode, r.stderr)
        assert "one GPU" in r.stderr
        assert r.stdout == ""   # no JSON line


def test_traffic_only_for_the_measured_source(tmp_path):
    b = _bench()
    sha = b.kernel_source_sha()
    assert len(sha) == 16 and sha == b.kernel_source_sha()
    rec = {"source_sha": sha, "hbm_bytes_per_launch": 1234567}
    good = tmp_path / "good.txt"
    good.write_text("# comment line\n" + json.dumps(rec) + "\n")
    b.COUNTERS_FILE = str(good)
    assert b.traffic_from_counters() == 1234567
    stale = tmp_path / "stale.txt"
    stale.write_text(json.dumps({**rec, "source_sha": "0" * 16}))
    b.COUNTERS_FILE = str(stale)
    assert b.traffic_from_counters() is None
    b.COUNTERS_FILE = str(tmp_path / "missing.txt")
    assert b.traffic_from_counters() is None

