"""Compile the HIP library ``libdensegemm.so`` for gfx950 with hipcc.

Every source is compiled in parallel with ``hipcc -c`` and linked into one
shared library next to this file.  The build always runs (no staleness check):
callers that only need a library that already exists load it directly.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdensegemm.so")
BUILD_DIR = os.path.join(ROOT, "_build")

# (source, object name, extra defines): tiled_inst.hip is compiled once per
# (element type, kernel variant, ladder family), so the instances build in
# parallel translation units
SOURCES = [("api.cpp", "api", []), ("select_tile.cpp", "select_tile", []), ("misc.hip", "misc", []),
           ("skinny.hip", "skinny", [])] + \
    [("tiled_inst.hip", f"tiled_d{d}_m{m}_f{f}",
      [f"-DDG_INST_DT={d}", f"-DDG_INST_MODE={m}", f"-DDG_INST_FAMILY={f}"])
     for d in (0, 1) for m in (0, 1, 2, 3) for f in (0, 1)]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()

    def compile_one(entry) -> str:
        src, name, defines = entry
        obj = os.path.join(BUILD_DIR, name + ".o")
        cmd = [cc, *FLAGS, *defines, *extra_flags, "-x", "hip", "-c", os.path.join(CSRC, src),
               "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {name}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
