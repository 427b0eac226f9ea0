"""GEMMs captured in a HIP graph and replayed (the timed region of bench.py
replays such a graph).

One graph holds a tiled GEMM, a skinny (decode) GEMM, a split-K GEMM with its
reduction, a fused-epilogue GEMM and an e4m3 GEMM.  It is replayed several
times, with eager work and synchronizations of the program's own between the
replays (outputs overwritten with NaN, other GEMMs run eagerly), and every
replay must reproduce the eager results bit for bit (every kernel here sums in
a fixed order).  New inputs copied into the captured buffers must give the
eager results on those inputs: the graph reads the live buffers.  The oracle
pins the eager results themselves (bit-exact on small-integer inputs).
"""
import numpy as np
import pytest
import torch

import datagen
import dense_gemm_linear_amd as dg
from parity import check_exact, dev_bf16, dev_u8, host_bits, oracle_full

pytestmark = pytest.mark.gpu

NAN_BF16 = -1    # 0xFFFF: a NaN bit pattern the kernels never write


class Case:
    """One GEMM of the graph: device inputs, an output buffer and the call."""

    def __init__(self, name, dt, M, N, K, tile, cfg, epilogue=False, split=False):
        self.name, self.dt, self.M, self.N, self.K, self.tile = name, dt, M, N, K, tile
        self.cfg, self.epilogue = cfg, epilogue
        self.ws = None
        if split:
            nbytes = dg.workspace_bytes(M, N, K, dt, tile)
            assert nbytes > 0, f"{tile.name} does not split {M}x{N}x{K}"
            self.ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
        self.load(cfg)
        self.C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        if epilogue:
            g = torch.Generator().manual_seed(cfg)
            self.bias = dev_bf16(datagen_bits(torch.randint(-3, 4, (N,), generator=g)))
            self.mul = dev_bf16(datagen_bits(torch.randint(-2, 3, (M, N), generator=g)))

    def load(self, cfg):
        """(Re)fill the captured input buffers in place with a new seeded draw."""
        M, N, K = self.M, self.N, self.K
        if self.dt == "bf16":
            A, B = datagen.make_bf16_pair(M, N, K, "smallint", "smallint", config=cfg)
            Ad, Bd = dev_bf16(A), dev_bf16(B)
        else:
            A, B, _, _ = datagen.make_e4m3_pair(M, N, K, config=cfg, smallint=True)
            Ad, Bd = dev_u8(A), dev_u8(B)
        self.host = (A, B)
        Bs = dg.shuffle_b(Bd, dtype=self.dt)
        if not hasattr(self, "A"):
            self.A, self.Bs = Ad, Bs
            self.sa = torch.tensor([0.5], dtype=torch.float32, device="cuda")
            self.sb = torch.tensor([4.0], dtype=torch.float32, device="cuda")
        else:
            self.A.copy_(Ad)
            self.Bs.copy_(Bs)

    def call(self, out):
        kw = dict(bias=self.bias, mul=self.mul, activation="relu") if self.epilogue else {}
        if self.dt == "bf16":
            dg.gemm_bf16(self.A, self.Bs, self.N, out=out, tile=self.tile, workspace=self.ws, **kw)
        else:
            dg.gemm_fp8_scaled(self.A, self.Bs, self.N, self.sa, self.sb, out=out, tile=self.tile,
                               workspace=self.ws, **kw)

    def oracle(self):
        A, B = self.host
        return oracle_full(self.dt, A, B, *((0.5, 4.0) if self.dt == "fp8" else ()))


def datagen_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 bit patterns of small integers (exact in bf16)."""
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_cases():
    return [
        Case("tiled", "bf16", 530, 557, 192, dg.tiled_ab(256, 256, 8, 32), 101),
        Case("skinny", "bf16", 1, 2000, 1024, dg.skinny(16, 16), 102),
        Case("split_k", "bf16", 263, 270, 1040, dg.with_split(dg.tiled(128, 128, 4, 32), 3), 103,
             split=True),
        Case("epilogue", "bf16", 300, 272, 192, dg.tiled_pp(256, 256), 104, epilogue=True),
        Case("fp8", "fp8", 200, 333, 1088, dg.tiled_ab(256, 256, 8, 32), 105),
    ]


def test_graph_replays_match_eager():
    cases = make_cases()
    print("[graph: eager reference]", flush=True)
    eager = []
    for c in cases:
        c.call(c.C)
    torch.cuda.synchronize()
    for c in cases:
        eager.append(host_bits(c.C))
        if not c.epilogue:
            check_exact(eager[-1], c.oracle(), f"eager {c.name}")

    outs = [torch.full_like(c.C.view(torch.int16), NAN_BF16).view(torch.bfloat16) for c in cases]
    g = torch.cuda.CUDAGraph()
    print("[graph: capture]", flush=True)
    with torch.cuda.graph(g):
        for c, o in zip(cases, outs):
            c.call(o)
    torch.cuda.synchronize()

    for rep in range(3):
        print(f"[graph: replay {rep}]", flush=True)
        for o in outs:
            o.view(torch.int16).fill_(NAN_BF16)
        # eager work of the program's own between the replays
        scratch = torch.empty_like(cases[0].C)
        cases[0].call(scratch)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for c, o, want in zip(cases, outs, eager):
            assert np.array_equal(host_bits(o), want), f"replay {rep}: {c.name} differs from eager"

    # new inputs in the captured buffers: the replay reads them
    print("[graph: replay on new inputs]", flush=True)
    for c in cases:
        c.load(c.cfg + 50)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    fresh = []
    for c in cases:
        c.call(c.C)
    torch.cuda.synchronize()
    for c, o in zip(cases, outs):
        want = host_bits(c.C)
        assert np.array_equal(host_bits(o), want), f"{c.name}: replay on new inputs differs"
        if not c.epilogue:
            check_exact(want, c.oracle(), f"new inputs {c.name}")
        fresh.append(want)
    assert any(not np.array_equal(a, b) for a, b in zip(fresh, eager)), "inputs did not change"
    del g
