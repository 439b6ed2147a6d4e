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


def _tree(tmp_path, fingerprints):
    """A copy of the kernel sources under tmp_path with a traffic file whose
    stored code fingerprints are `fingerprints(name, text)`."""
    t = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))
    csrc = tmp_path / "memory_efficient_exact_tiled_amd" / "csrc"
    csrc.mkdir(parents=True)
    stored = {}
    for name in t["code_sha256_16"]:
        text = open(os.path.join(ROOT, "memory_efficient_exact_tiled_amd", "csrc", name)).read()
        (csrc / name).write_text(text)
        stored[name] = fingerprints(name, text)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "hbm_traffic.json").write_text(json.dumps(dict(t, code_sha256_16=stored)))
    return csrc


def test_traffic_is_null_once_a_kernel_changes(tmp_path, monkeypatch):
    import bench
    _tree(tmp_path, lambda name, text: "0" * 16)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic() is None


def test_traffic_survives_comment_edits_but_not_code_edits(tmp_path, monkeypatch):
    import bench
    csrc = _tree(tmp_path, lambda name, text: bench.kernel_code_hash(text))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic() is not None
    fwd = csrc / "fwd.hip"
    fwd.write_text("// a new comment line\n\n/* and a block\n   comment */\n" + fwd.read_text().replace("\n", "  // note\n", 3))
    assert bench.measured_traffic() is not None
    fwd.write_text(fwd.read_text() + "\nstatic const int kAnotherConstant = 1;\n")
    assert bench.measured_traffic() is None
