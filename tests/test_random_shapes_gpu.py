"""Seeded random shapes across the scan's features, against the fp64 oracle
(the scan and its backward; the conv prologue with its backward; the decode
step; the Mamba-2 SSD form).

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


def draw_conv(rng, i):
    return dict(N=rng.choice([16, 16, 8, 24]), batch=rng.randint(1, 3), dim=rng.randint(1, 11),
                L=rng.choice([rng.randint(1, 300), rng.randint(900, 2600)]),
                dtype=rng.choice(["f32", "bf16"]), K=rng.randint(1, 4),
                cb=rng.random() < 0.7, seed=2000 + i)


_rng_c = random.Random(777)
CONV_CASES = [draw_conv(_rng_c, i) for i in range(12)]


@pytest.mark.parametrize("c", CONV_CASES, ids=lambda c: "n%(N)d_b%(batch)d_d%(dim)d_l%(L)d_%(dtype)s_k%(K)d_cb%(cb)d" % c)
def test_random_conv_shape(c):
    """The conv prologue (1-4 taps, with or without the conv bias): forward
    against the oracle's conv + scan, and the backward's x, tap and bias
    gradients against the oracle's chain rule."""
    inp = syn.make_conv_inputs(syn.TINY, "cpu", d_conv=c["K"], with_bias=c["cb"],
                               batch=c["batch"], dim=c["dim"], dstate=c["N"], seqlen=c["L"],
                               dtype=c["dtype"], with_h0=True, seed=c["seed"])
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    tol = TOL[c["dtype"]]
    u = oracle.causal_conv1d_silu(inp["x"], inp["conv_w"], inp["conv_b"])
    y_ref, h_ref = oracle.scan(u, inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                               inp["z"], inp["delta_bias"], True, False, inp["h0"])
    y, hf = ssm.ssm_conv_scan_fwd(d["x"], d["conv_w"], d["delta"], d["A"], d["B"], d["C"],
                                  d["D"], d["z"], d["delta_bias"], True, d["h0"],
                                  conv_b=d["conv_b"])
    torch.cuda.synchronize()
    assert scaled_max_err(y, y_ref) <= tol, "y"
    assert scaled_max_err(hf, h_ref) <= tol, "h_final"
    g = torch.Generator().manual_seed(c["seed"])
    dy = torch.randn(c["batch"], c["dim"], c["L"], generator=g).to(inp["x"].dtype)
    dhf = torch.randn(c["batch"], c["dim"], c["N"], generator=g)
    ref = oracle.scan_bwd(u, inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                          inp["delta_bias"], True, inp["h0"], dy, dhf)
    dx, dw, db = oracle.causal_conv1d_silu_bwd(inp["x"], inp["conv_w"], inp["conv_b"],
                                               ref["du"])
    got = ssm.ssm_conv_scan_bwd(d["x"], d["conv_w"], d["delta"], d["A"], d["B"], d["C"],
                                d["D"], d["z"], d["delta_bias"], True, d["h0"], dy.to(DEV),
                                dhf.to(DEV), conv_b=d["conv_b"])
    torch.cuda.synchronize()
    assert scaled_max_err(got["dx"], dx) <= tol, "dx"
    assert scaled_max_err(got["dconv_w"], dw) <= tol, "dconv_w"
    if c["cb"]:
        assert scaled_max_err(got["dconv_b"], db) <= tol, "dconv_b"
    for k in ("ddelta", "dA", "dB", "dC"):
        assert scaled_max_err(got[k], ref[k]) <= tol, k


def draw_decode(rng, i):
    return dict(N=rng.choice([16, 16, 4, 13, 32]), batch=rng.randint(1, 9),
                dim=rng.randint(1, 40), steps=rng.randint(1, 12),
                dtype=rng.choice(["f32", "bf16"]), seed=3000 + i)


_rng_d = random.Random(4242)
DECODE_CASES = [draw_decode(_rng_d, i) for i in range(10)]


@pytest.mark.parametrize("c", DECODE_CASES, ids=lambda c: "n%(N)d_b%(batch)d_d%(dim)d_s%(steps)d_%(dtype)s" % c)
def test_random_decode_shape(c):
    """Decode steps in sequence, each against the oracle's step, the ZOH term
    on every other step."""
    cfg = syn.DecodeConfig("random", c["batch"], c["dim"], c["N"], c["steps"], dtype=c["dtype"],
                           seed=c["seed"])
    inp = syn.make_decode_inputs(cfg, "cpu", with_h0=True)
    dinp = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    tol = TOL[c["dtype"]]
    state = dinp["h0"].clone()
    ref_state = inp["h0"].double().numpy().copy()
    for t in range(cfg.steps):
        zoh = t % 2 == 1
        s = syn.step_slice(dinp, t)
        y = ssm.ssm_state_update(state, s["x"], s["delta"], dinp["A"], s["B"], s["C"],
                                 dinp["D"], s["z"], dinp["delta_bias"], True, zoh_b=zoh)
        sh = syn.step_slice(inp, t)
        y_ref = oracle.step(ref_state, sh["x"], sh["delta"], inp["A"], sh["B"], sh["C"],
                            inp["D"], sh["z"], inp["delta_bias"], True, zoh)
        torch.cuda.synchronize()
        assert scaled_max_err(y, y_ref) <= tol, "y step %d" % t
        assert scaled_max_err(state, ref_state) <= tol, "state step %d" % t


def draw_ssd(rng, i):
    ngroups = rng.choice([1, 1, 2])
    return dict(batch=rng.randint(1, 2), nheads=ngroups * rng.randint(1, 4), ngroups=ngroups,
                N=rng.choice([64, 128, 128, 256]), L=rng.randint(1, 700),
                z=rng.random() < 0.8, D=rng.random() < 0.8, h0=rng.random() < 0.5,
                seed=4000 + i)


_rng_s = random.Random(99)
SSD_CASES = [draw_ssd(_rng_s, i) for i in range(10)]


@pytest.mark.parametrize("c", SSD_CASES, ids=lambda c: "b%(batch)d_h%(nheads)d_g%(ngroups)d_n%(N)d_l%(L)d" % c)
def test_random_ssd_shape(c):
    """The Mamba-2 SSD form (bf16) against its oracle: y and the final state."""
    inp = syn.make_ssd_inputs(syn.MAMBA2_LAYER, "cpu", batch=c["batch"], nheads=c["nheads"],
                              ngroups=c["ngroups"], dstate=c["N"], seqlen=c["L"],
                              with_z=c["z"], with_D=c["D"], with_h0=c["h0"], seed=c["seed"])
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    y_ref, h_ref = oracle.ssd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                              inp["z"], inp["dt_bias"], True, inp["h0"])
    y, hf = ssm.ssm_ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"],
                            d["dt_bias"], True, d["h0"])
    torch.cuda.synchronize()
    assert scaled_max_err(y, y_ref) <= TOL["bf16"], "y"
    assert scaled_max_err(hf, h_ref) <= TOL["bf16"], "h_final"
