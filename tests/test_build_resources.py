"""The compiler's resource report of the built kernels (CPU): no kernel spills
to scratch, and the occupancy each kernel is tuned for is reached.

build.py writes ``_build/resource_usage.json`` from hipcc's
``-Rpass-analysis=kernel-resource-usage`` remarks every time it compiles.
"""
import glob
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "memory_efficient_exact_tiled_amd")
REPORT = os.path.join(PKG, "_build", "resource_usage.json")


@pytest.fixture(scope="module")
def usage():
    if not os.path.exists(REPORT):
        pytest.skip("library not built (python memory_efficient_exact_tiled_amd/build.py)")
    newest = max(os.path.getmtime(p) for p in glob.glob(os.path.join(PKG, "csrc", "*")))
    assert os.path.getmtime(REPORT) >= newest, "kernel sources changed since the last build: rebuild"
    return json.load(open(REPORT))


def test_every_kernel_is_reported(usage):
    names = " ".join(usage)
    for k in ("fwd_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel", "bwd_prep_kernel", "decode_split_kernel",
              "decode_combine_kernel", "kv_append_kernel"):
        assert k in names, k


def test_no_scratch_spills(usage):
    spills = {k: v["ScratchSize [bytes/lane]"] for k, v in usage.items()
              if v.get("ScratchSize [bytes/lane]", "0") != "0" or v.get("VGPRs Spill", "0") != "0"}
    assert not spills, spills


def test_attention_kernels_keep_two_waves_per_simd(usage):
    """The forward and the D=64 backward rely on at least two waves per SIMD
    (one wave's softmax overlapping another's matrix-core work)."""
    for k, v in usage.items():
        occ = int(v["Occupancy [waves/SIMD]"])
        if "fwd_kernel" in k or ("Li64E" in k and ("bwd_dq" in k or "bwd_dkdv" in k)):
            assert occ >= 2, (k, occ)
