"""The C ABI from plain C: tests/clients/c_client.c, compiled with gcc against
include/densegemm.h alone and linked to libdensegemm.so, makes host-side
queries (tile selection, the launch plan, sizes, argument errors); its
answers must equal the Python binding's.  No device is needed."""
import os
import shutil
import subprocess

import pytest

import dense_gemm_linear_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.dirname(dg.lib._name)


def fields(t):
    return (f"kernel={t.kernel} tile_m={t.tile_m} tile_n={t.tile_n} tile_k={t.tile_k} "
            f"atom={t.atom} waves={t.waves} k_split={t.k_split} stages={t.lds_stages}")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_client_matches_binding(tmp_path):
    exe = tmp_path / "c_client"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "clients", "c_client.c"), "-L", LIBDIR, "-ldensegemm",
                    f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines()
    assert out[-1] == "ok"
    got = dict(line.split(" ", 1) for line in out[:-1])
    assert got["select_4096"] == fields(dg.select_tile(4096, 4096, 4096, "bf16", 256))
    assert got["select_decode"] == fields(dg.select_tile(1, 11008, 4096, "bf16", 256))
    t48 = dg.select_tile(48, 4096, 4096, "bf16", 256, workspace_bytes=64 << 20)
    assert got["select_ws_48"] == fields(t48)
    assert int(got["workspace_48"]) == dg.workspace_bytes(48, 4096, 4096, "bf16", t48)
    first, second, n1, m1 = dg.plan(1024, 50257, 512, "bf16", 256, 0)
    assert got["plan_first"] == fields(first) and got["plan_second"] == fields(second)
    assert int(got["plan_columns"]) == n1 and int(got["plan_rows"]) == m1 == 1024
    assert got["shuffle_bytes"] == f"{dg.shuffle_b_bytes(11008, 4096)} {dg.shuffle_b_bytes(4096, 4096, 'fp8')}"
    assert got["tile_check"] == f"{dg.GEMM_OK} {dg.GEMM_ERR_INVALID_VALUE}"
    assert got["errors"] == "GEMM_ERR_INVALID_VALUE GEMM_ERR_INVALID_VALUE GEMM_ERR_INVALID_VALUE"
