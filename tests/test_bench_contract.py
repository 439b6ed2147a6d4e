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


def _tree(tmp_path, stale=False):
    """A copy of the sources the traffic guard fingerprints under tmp_path, with
    a traffic file whose stored fingerprints are those of the copy (or zeros)."""
    import shutil

    import bench
    pkg = tmp_path / "memory_efficient_exact_tiled_amd"
    csrc = pkg / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.TRAFFIC_SOURCES:
        shutil.copy(os.path.join(ROOT, "memory_efficient_exact_tiled_amd", "csrc", name), csrc / name)
    shutil.copy(os.path.join(ROOT, "memory_efficient_exact_tiled_amd", "build.py"), pkg / "build.py")
    fp = bench.code_fingerprints(str(tmp_path))
    if stale:
        fp = {k: "0" * 16 for k in fp}
    prof = tmp_path / "profiles"
    prof.mkdir()
    t = {"code_sha256_16": fp, "fetch_factor": 2.0, "write_factor": 1.0,
         "kernels": {"fwd_kernelIDF16bLi64": {"fetch_bytes": 1.0, "write_bytes": 2.0, "dispatches": 1}}}
    (prof / "hbm_traffic.json").write_text(json.dumps(t))
    return pkg


def test_traffic_is_null_once_a_kernel_changes(tmp_path, monkeypatch):
    import bench
    _tree(tmp_path, stale=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic() is None


def test_traffic_survives_comment_edits_but_not_code_edits(tmp_path, monkeypatch):
    import bench
    pkg = _tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic() is not None
    fwd = pkg / "csrc" / "fwd.hip"
    fwd.write_text("// a new comment line\n\n/* and a block\n   comment */\n" + fwd.read_text().replace("\n", "  // note\n", 3))
    assert bench.measured_traffic() is not None
    fwd.write_text(fwd.read_text() + "\nstatic const int kAnotherConstant = 1;\n")
    assert bench.measured_traffic() is None


def test_traffic_is_null_after_a_host_side_or_flag_change(tmp_path, monkeypatch):
    """Kernel choice and tile height are made on the host (api.hip), launch
    parameters live in launch.hpp, and the code depends on the compiler flags."""
    import bench
    for target, edit in (("csrc/api.hip", lambda t: t + "\nstatic const int kTileChoice = 3;\n"),
                         ("csrc/launch.hpp", lambda t: t.replace("kDecodeMaxSplit = 1024", "kDecodeMaxSplit = 512")),
                         ("build.py", lambda t: t.replace('"-O3",', '"-O2",'))):
        sub = tmp_path / target.replace("/", "_").replace(".", "_")
        sub.mkdir()
        pkg = _tree(sub)
        monkeypatch.setattr(bench, "ROOT", str(sub))
        assert bench.measured_traffic() is not None, target
        f = pkg / target
        new = edit(f.read_text())
        assert new != f.read_text(), target
        f.write_text(new)
        assert bench.measured_traffic() is None, target
