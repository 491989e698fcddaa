"""Build libmoe_q4.so (HIP, gfx950) in-tree with hipcc.

    python -m quantized_moe_expert_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_q4.so")
SOURCES = ["api.hip", "route.hip", "group.hip", "decode.hip", "prefill.hip", "shared.hip", "misc.hip"]
ARCH = os.environ.get("MOEQ4_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 instructions are kept out of the device code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", "-fvisibility=hidden"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip() and verbose:
        print(out)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source to an object (in parallel), then link the library."""
    from concurrent.futures import ThreadPoolExecutor
    import tempfile
    jobs = jobs or min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with tempfile.TemporaryDirectory(prefix="moeq4_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB + ".tmp"
        _run([HIPCC, *FLAGS, "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
