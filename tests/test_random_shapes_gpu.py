"""Seeded random shapes across the scan's features, against the fp64 oracle.

Each case draws a state count (16, the tuned count, most often; also 1, 3,
8, 13, 24, 33, 64, 100), batch 1-3, 1-13 channels, a length from one of
three bands (1-300 tokens: only a partial block; 900-2200: one or two full
blocks and a partial one; 3000-6000: several), bf16 or fp32, the automatic
chunk plan or chunks of 1024 or 2048 tokens, the Euler or exact-ZOH input
term, with or without an initial state.  The forward is checked on y and
the final state; every second case of up to 2500 tokens also runs the
backward (every gradient).  Bars as elsewhere: 1e-4 for fp32, 2e-2 for
bf16 on the scaled error.
"""
import random

import pytest
import torch

import oracle
import selective_state_space_30_amd as ssm
import synthetic as syn
from parity_metrics import scaled_max_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = {"f32": 1e-4, "bf16": 2e-2}


def draw(rng, i):
    return dict(
        N=rng.choice([16, 16, 16, 1, 3, 8, 13, 16, 24, 33, 64, 100]),
        batch=rng.randint(1, 3), dim=rng.randint(1, 13),
        L=rng.choice([rng.randint(1, 300), rng.randint(900, 2200), rng.randint(3000, 6000)]),
        dtype=rng.choice(["f32", "bf16"]), chunk=rng.choice([0, 0, 1024, 2048]),
        zoh=rng.random() < 0.3, h0=rng.random() < 0.5, seed=1000 + i)


_rng = random.Random(12345)
CASES = [draw(_rng, i) for i in range(40)]


@pytest.mark.parametrize("c", CASES, ids=lambda c: "n%(N)d_b%(batch)d_d%(dim)d_l%(L)d_%(dtype)s_c%(chunk)d_z%(zoh)d" % c)
def test_random_shape(c):
    inp = syn.make_scan_inputs(syn.TINY, "cpu", batch=c["batch"], dim=c["dim"], dstate=c["N"],
                               seqlen=c["L"], dtype=c["dtype"], seed=c["seed"], with_h0=c["h0"])
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    tol = TOL[c["dtype"]]
    y, hf = ssm.ssm_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                             d["delta_bias"], True, d.get("h0"), chunk_len=c["chunk"],
                             zoh_b=c["zoh"])
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                               inp["z"], inp["delta_bias"], True, c["zoh"], inp.get("h0"))
    assert scaled_max_err(y, y_ref) <= tol, "y"
    assert scaled_max_err(hf, h_ref) <= tol, "h_final"
    if c["L"] > 2500 or c["seed"] % 2:
        return
    g = torch.Generator().manual_seed(c["seed"])
    dy = torch.randn(c["batch"], c["dim"], c["L"], generator=g).to(inp["u"].dtype)
    dhf = torch.randn(c["batch"], c["dim"], c["N"], generator=g)
    ref = oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                          inp["z"], inp["delta_bias"], True, inp.get("h0"), dy, dhf,
                          zoh_b=c["zoh"])
    got = ssm.ssm_scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                           d["delta_bias"], True, d.get("h0"), dy.to(DEV), dhf.to(DEV),
                           zoh_b=c["zoh"])
    torch.cuda.synchronize()
    for k, v in got.items():
        if v is not None and ref.get(k) is not None:
            assert scaled_max_err(v, ref[k]) <= tol, k
