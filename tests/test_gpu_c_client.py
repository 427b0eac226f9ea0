"""The GEMM through the C ABI with no Python in between: tests/clients/
gemm_client (built by __graft_entry__.build()) allocates device memory with
the HIP runtime, preshuffles B and calls gemm_bf16 with the library's tile.
Inputs come from the seeded generators, expected values from the oracle:
bit-exact on small integers, the parity.py bounds otherwise."""
import os
import subprocess

import numpy as np
import pytest

import datagen
from parity import abs_bits, check_close, check_exact, oracle_full

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "clients", "gemm_client")


def run_client(tmp_path, A, B):
    assert os.path.exists(CLIENT), "tests/clients/gemm_client is missing: run __graft_entry__.build()"
    M, K = A.shape
    N = B.shape[0]
    pa, pb, pc = tmp_path / "a.bin", tmp_path / "b.bin", tmp_path / "c.bin"
    np.ascontiguousarray(A).tofile(pa)
    np.ascontiguousarray(B).tofile(pb)
    print(f"[gemm_client {M}x{N}x{K}]", flush=True)
    r = subprocess.run([CLIENT, str(M), str(N), str(K), str(pa), str(pb), str(pc)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return np.fromfile(pc, dtype=np.uint16).reshape(M, N)


@pytest.mark.parametrize("M,N,K", [(263, 270, 176), (8, 2000, 1024), (600, 700, 512)])
def test_c_client_gemm(tmp_path, M, N, K):
    A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=M + N)
    check_exact(run_client(tmp_path, A, B), oracle_full("bf16", A, B), f"C client {M}x{N}x{K}")
    A, B = datagen.make_bf16_pair(M, N, K, "normal", "normal", config=M + N + 1)
    check_close("bf16", run_client(tmp_path, A, B), oracle_full("bf16", A, B),
                oracle_full("bf16", abs_bits("bf16", A), abs_bits("bf16", B)), K,
                what=f"C client {M}x{N}x{K}")
