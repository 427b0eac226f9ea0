"""The selector against the MI355X sweeps kept in the repository (host only:
select_tile is priced for 256 CUs, no device is touched).

- Calibrated shapes (calibration/mi355x_sweep.jsonl): with the measured-best
  table the pick is the fastest swept tile, regret 1.0.
- Held-out shapes (calibration/mi355x_holdout.jsonl, never fitted): the pick
  is one of the swept tiles and within 15 % of the fastest (measured:
  geometric mean 1.017, worst 1.047).
"""
import json
import os

import pytest

import bench
import dense_gemm_linear_amd as dg

CAL = os.path.join(os.path.dirname(dg.__file__), "calibration")
WS = bench.WORKSPACE_MIB << 20


def sweeps(name):
    res = {}
    with open(os.path.join(CAL, name)) as f:
        for line in f:
            if line.strip():
                d = json.loads(line)
                res.setdefault(d["sweep"], {})[d["tile"]] = d["kernel_us_median"]
    return res


CALIBRATED = sweeps("mi355x_sweep.jsonl")
HELD_OUT = sweeps("mi355x_holdout.jsonl")


@pytest.mark.parametrize("name", sorted(CALIBRATED))
def test_calibrated_shapes_pick_the_measured_best(name):
    M, N, K, dt = bench.WORKLOADS[name][:4]
    r = CALIBRATED[name]
    t = dg.select_tile(M, N, K, dt, bench.CUS, workspace_bytes=WS)
    assert r.get(t.name) == min(r.values()), (t.name, min(r, key=r.get))


@pytest.mark.parametrize("name", sorted(HELD_OUT))
def test_held_out_shapes_within_fifteen_percent(name):
    assert not set(HELD_OUT) & set(CALIBRATED), "held-out shapes must stay out of the fit"
    M, N, K, dt = bench.WORKLOADS[name][:4]
    r = HELD_OUT[name]
    t = dg.select_tile(M, N, K, dt, bench.CUS, workspace_bytes=WS)
    assert t.name in r, f"{t.name} was not swept"
    assert r[t.name] <= 1.15 * min(r.values()), (t.name, r[t.name], min(r, key=r.get), min(r.values()))
