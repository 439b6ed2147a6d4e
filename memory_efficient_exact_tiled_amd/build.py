"""Builds libmea.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run ``python memory_efficient_exact_tiled_amd/build.py`` (by path: importing
the package would load the library being rebuilt), or call :func:`build`.
Objects go to ``_build/`` beside this file; the library is written next to
this file, where the binding loads it from. The compiler's per-kernel
resource report (registers, scratch, occupancy, LDS) is kept in
``_build/resource_usage.json``: every kernel here is designed to run without
scratch spills, and the tests check that it does.
"""
from __future__ import annotations

import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmea.so")
SOURCES = ["api.hip", "fwd.hip", "bwd.hip", "decode.hip", "kvcache.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
    "-Rpass-analysis=kernel-resource-usage",
]
RESOURCES = os.path.join(OBJDIR, "resource_usage.json")
_REMARK = re.compile(r"remark: ([^:]+): (.*?) \[-Rpass-analysis")


def _resources(text: str) -> dict:
    """Kernel resource remarks of one compile -> {kernel: {field: value}} (device pass only)."""
    out, cur = {}, None
    for m in _REMARK.finditer(text):
        field, value = m.group(1).strip(), m.group(2).strip()
        if field == "Function Name":
            cur = out.setdefault(value, {})
        elif cur is not None:
            cur[field] = value
    return out


def _compile(src: str, extra):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, _resources(r.stderr)


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compiles every source and links libmea.so; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        done = list(ex.map(lambda s: _compile(s, list(extra_flags)), SOURCES))
    objs = [o for o, _ in done]
    usage = {}
    for _, res in done:
        usage.update(res)
    with open(RESOURCES, "w") as f:
        json.dump(usage, f, indent=1, sort_keys=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        spills = [k for k, v in usage.items() if v.get("ScratchSize [bytes/lane]", "0") != "0"]
        print(f"built {LIB} ({len(usage)} kernels" + (f"; SCRATCH SPILLS in {spills}" if spills else "") + ")")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
