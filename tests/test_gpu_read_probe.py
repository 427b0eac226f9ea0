"""The streaming-read probe (gemm_read_probe) on the GPU: it reads every byte
of the buffer exactly once, so the XOR of its partials equals the XOR of all
32-bit words of the buffer computed on the host; and it covers sizes that are
not a multiple of its workgroup count, on both of its launch shapes (below
and above 64 MiB).  The probe's time is only a measurement aid; what is
tested here is that it reads what it claims to read."""
import numpy as np
import pytest
import torch

import dense_gemm_linear_amd as dg

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48, (33 << 20) + 16 * 7,
                                    (70 << 20) + 16 * 3])
def test_read_probe_xor_matches_host(nbytes):
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    want = int(np.bitwise_xor.reduce(words))
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    print(f"[read probe {nbytes} bytes]", flush=True)
    out = torch.full((dg.READ_PROBE_SLOTS,), -1, dtype=torch.int32, device="cuda")
    dg.read_probe(buf, out=out)
    torch.cuda.synchronize()
    parts = out.cpu().numpy().view(np.uint32)
    assert int(np.bitwise_xor.reduce(parts)) == want


def test_read_probe_binding_checks():
    buf = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        dg.read_probe(buf, out=torch.zeros(16, dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        dg.read_probe(buf[::2])
