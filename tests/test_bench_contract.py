"""The benchmark's command-line contract, checked on the CPU: it measures one
GPU and says so when asked for more, and it reports the committed HBM
traffic figure only while the decode sources are the ones it was taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=env, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_exits_with_a_message(args, env):
    r = _run(args, env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    alg = 2785476608
    good = {"source_sha": bench.decode_source_hash(), "hbm_bytes_per_launch": 2814241382}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(alg) == 2814241382
    f.write_text(json.dumps(dict(good, source_sha="0" * 16)))
    assert bench.measured_traffic(alg) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic(alg) is None


def test_committed_traffic_file_matches_the_current_decode_sources():
    """The committed counter summary was taken on the decode sources in the
    tree (otherwise the bench line carries traffic = null)."""
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    assert t["source_sha"] == bench.decode_source_hash()
    assert 0.99 < t["hbm_bytes_per_launch"] / t["alg_bytes_per_launch"] < 1.1


def test_config_selector_names_known_sections_and_rejects_others():
    """--config picks one of the five workloads: each maps to component
    sections the bench knows (the decode step to none), and together they
    cover every section but the copy context."""
    assert set(bench.CONFIGS) == {"tiny", "llama7b", "sweep", "qjl", "decode"}
    named = set()
    for secs in bench.CONFIGS.values():
        assert set(secs) <= set(bench.SECTIONS)
        named |= set(secs)
    assert named == set(bench.SECTIONS) - {"copy"}
    r = _run(["--config", "nonesuch"])
    assert r.returncode == 2 and "invalid choice" in r.stderr
