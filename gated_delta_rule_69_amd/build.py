"""Build libkda.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m gated_delta_rule_69_amd.build   (or call build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libkda.so")
OBJDIR = os.path.join(os.path.dirname(HERE), "_build", "libkda")
SOURCES = ["kda_api.hip", "kda_gate.hip", "kda_recurrent.hip", "kda_conv.hip", "kda_chunk.hip",
           "kda_chunk_bwd.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed FP32 VALU ops stay off (plain float code only)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-result", "-Wno-unused-variable",
        f"-I{INCLUDE}",
    ]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source to an object (in parallel), then link libkda.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()
    cmds = []
    for s in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o")
        cmds.append((s, [cc] + flags() + ["-c", "-o", obj, os.path.join(CSRC, s)], obj))
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda c: (c[0], c[1]) + _run(c[1]), cmds))
    for src, cmd, rc, out in results:
        if verbose:
            print(" ".join(cmd), flush=True)
            if out.strip():
                print(out)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{out}")
    tmp = LIB + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [c[2] for c in cmds]
    rc, out = _run(link)
    if verbose:
        print(" ".join(link), flush=True)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
