"""bench.py's host-side contract (CPU): refusal of N > 1 and the traffic guard."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_is_null_once_a_kernel_source_changes(tmp_path, monkeypatch):
    import bench
    t = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))
    fake = dict(t, sources_sha256_16={k: "0" * 16 for k in t["sources_sha256_16"]})
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "hbm_traffic.json").write_text(json.dumps(fake))
    csrc = tmp_path / "memory_efficient_exact_tiled_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in t["sources_sha256_16"]:
        (csrc / name).write_text(open(os.path.join(ROOT, "memory_efficient_exact_tiled_amd", "csrc", name)).read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic() is None
