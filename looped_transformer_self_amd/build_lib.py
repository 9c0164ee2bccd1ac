"""Build libloopspec.so for gfx950 with hipcc (in-tree, next to this file)."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libloopspec.so")
SOURCES = ["mega.hip", "readout.hip", "verify.hip", "misc.hip", "loopspec_abi.hip", "stream.hip", "prefill.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         # packed fp32 arithmetic stays off: hipcc must not emit packed-fp32 instructions
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "warning: feature flag" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")


def build(verbose=False, jobs=None):
    """Compile every source to an object (in parallel), then link the shared library."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    inc = ["-I", os.path.join(HERE, "..", "include")]
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *FLAGS, *inc, "-c", os.path.join(SRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", OUT + ".tmp"], verbose)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
