"""Build the host programs the tests drive (test infrastructure, not the
product): tests/clients/gemm_client, a C-ABI client of libdensegemm.so that
runs a GEMM with no Python in between.  Host code only; hipcc supplies the
HIP runtime headers and library."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(os.path.dirname(_HERE))


def build(verbose: bool = False) -> str:
    libdir = os.path.join(_ROOT, "dense_gemm_linear_amd")
    out = os.path.join(_HERE, "gemm_client")
    tmp = out + ".tmp"
    cmd = ["/opt/rocm/bin/hipcc", "-O2", "-std=c++17", "-Wall", "-Wextra",
           "-I", os.path.join(_ROOT, "include"), os.path.join(_HERE, "gemm_client.cpp"),
           "-L", libdir, "-ldensegemm", f"-Wl,-rpath,{libdir}", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
