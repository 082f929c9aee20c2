"""Parity of the Mamba-1 paths for state counts other than the tuned 16.

The S6 module takes d_state as a parameter ("Mamba & State Space Models -
Guide Complet", section 4: A is (d_model, d_state), B and C (batch, L,
d_state); section 5 gives 64-256 for the larger states of Mamba-2);
d_state = 16 runs the tuned instances, any other count up to 256 holds
state n in lane n % 64 of register n / 64 (one register up to 64 states,
four above).  Every case compares with the fp64 oracle, which
takes any N: the forward (whole sequence, split into chunks, exact ZOH, conv
prologue), the decode step (plain and with the conv window), and the
backward (whole sequence, split, and after the saving forward).  Counts
cover one state, odd counts (the last B/C staging phase holds one state), a
count above 16 that is not a multiple of 16 (the backward's adjoint
pre-pass works 16 states at a time), 64 (one full register) and counts
above it up to the maximum, 256.

Bars: fp32 activations 1e-4, bf16 2e-2 on the scaled error (as for N = 16).
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_30_amd as ssm
import synthetic as syn
from parity_metrics import report, scaled_max_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = {"f32": 1e-4, "bf16": 2e-2}


def check(got, ref, tol, what):
    err = scaled_max_err(got, ref)
    assert err <= tol, "%s: %s (tol %g)" % (what, report(got, ref), tol)


def to_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}


def scan_inputs(N, batch, dim, L, dt, seed, **kw):
    return syn.make_scan_inputs(syn.TINY, "cpu", batch=batch, dim=dim,
                                dstate=N, seqlen=L, dtype=dt, seed=seed, **kw)


FWD_CASES = [
    # (N, batch, dim, L, dtype)
    (1, 2, 9, 2100, "f32"),
    (5, 1, 6, 777, "f32"),     # odd count, unaligned rows
    (8, 2, 9, 2100, "bf16"),
    (13, 2, 5, 3000, "f32"),
    (32, 1, 8, 1500, "bf16"),
    (40, 1, 4, 1100, "f32"),
    (64, 2, 6, 2048, "f32"),
    (65, 1, 5, 1100, "f32"),   # one state in the second register
    (128, 2, 4, 1500, "bf16"),
    (200, 1, 3, 1300, "f32"),
    (256, 1, 3, 1024, "f32"),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "n%d_b%d_d%d_l%d_%s" % c)
def test_scan_other_state_counts(case):
    N, batch, dim, L, dt = case
    inp = scan_inputs(N, batch, dim, L, dt, 40 + N, with_h0=True)
    y_ref, h_ref = oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"],
                               inp["C"], inp["D"], inp["z"], inp["delta_bias"],
                               True, False, inp["h0"])
    d = to_dev(inp)
    y, hf = ssm.ssm_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"],
                             d["z"], d["delta_bias"], True, d["h0"])
    torch.cuda.synchronize()
    check(y, y_ref, TOL[dt], "y")
    check(hf, h_ref, TOL[dt], "h_final")


@pytest.mark.parametrize("N", [7, 64, 130])
def test_scan_other_state_counts_split_and_zoh(N):
    """A sequence split into 1024-token chunks (carry and fix-up over N
    states), and the exact ZOH input term."""
    inp = scan_inputs(N, 1, 6, 5000, "f32", 60 + N, with_h0=True)
    d = to_dev(inp)
    for zoh in (False, True):
        y_ref, h_ref = oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"],
                                   inp["C"], inp["D"], inp["z"],
                                   inp["delta_bias"], True, zoh, inp["h0"])
        y, hf = ssm.ssm_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"],
                                 d["D"], d["z"], d["delta_bias"], True, d["h0"],
                                 chunk_len=1024, zoh_b=zoh)
        torch.cuda.synchronize()
        check(y, y_ref, 1e-4, "y (zoh=%d)" % zoh)
        check(hf, h_ref, 1e-4, "h_final (zoh=%d)" % zoh)


def test_conv_scan_refuses_more_than_64_states():
    """The conv prologue over more than 64 states is refused: that case
    (96 states) gave intermittent wrong outputs near the start of the
    sequence in full test-suite runs, cause not found."""
    inp = to_dev(syn.make_conv_inputs(syn.TINY, "cpu", batch=2, dim=7, dstate=96,
                                      seqlen=1800, dtype="f32", with_h0=True, seed=176))
    with pytest.raises(ssm.SSMError, match="dstate <= 64"):
        ssm.ssm_conv_scan_fwd(inp["x"], inp["conv_w"], inp["delta"], inp["A"],
                              inp["B"], inp["C"], inp["D"], inp["z"],
                              inp["delta_bias"], True, inp["h0"], conv_b=inp["conv_b"])


@pytest.mark.parametrize("N", [4, 24, 64])
def test_conv_scan_other_state_counts(N):
    inp = syn.make_conv_inputs(syn.TINY, "cpu", batch=2, dim=7, dstate=N,
                               seqlen=1800, dtype="f32", with_h0=True,
                               seed=80 + N)
    u = oracle.causal_conv1d_silu(inp["x"], inp["conv_w"], inp["conv_b"])
    y_ref, h_ref = oracle.scan(u, inp["delta"], inp["A"], inp["B"], inp["C"],
                               inp["D"], inp["z"], inp["delta_bias"], True,
                               False, inp["h0"])
    d = to_dev(inp)
    y, hf = ssm.ssm_conv_scan_fwd(d["x"], d["conv_w"], d["delta"], d["A"],
                                  d["B"], d["C"], d["D"], d["z"],
                                  d["delta_bias"], True, d["h0"],
                                  conv_b=d["conv_b"])
    torch.cuda.synchronize()
    check(y, y_ref, 1e-4, "y")
    check(hf, h_ref, 1e-4, "h_final")


@pytest.mark.parametrize("case", [(1, "f32"), (8, "bf16"), (13, "f32"), (64, "f32"),
                                  (100, "f32"), (256, "bf16")],
                         ids=lambda c: "n%d_%s" % c)
def test_decode_other_state_counts(case):
    """Every step against the oracle's step, the ZOH term on the second
    half of the steps."""
    N, dt = case
    cfg = syn.DecodeConfig("small", 3, 37, N, 12, dtype=dt, seed=90 + N)
    inp = syn.make_decode_inputs(cfg, "cpu", with_h0=True)
    dinp = to_dev(inp)
    state = dinp["h0"].clone()
    ref_state = inp["h0"].double().numpy().copy()
    for t in range(cfg.steps):
        zoh = t >= cfg.steps // 2
        s = syn.step_slice(dinp, t)
        y = ssm.ssm_state_update(state, s["x"], s["delta"], dinp["A"], s["B"],
                                 s["C"], dinp["D"], s["z"], dinp["delta_bias"],
                                 True, zoh_b=zoh)
        sh = syn.step_slice(inp, t)
        y_ref = oracle.step(ref_state, sh["x"], sh["delta"], inp["A"], sh["B"],
                            sh["C"], inp["D"], sh["z"], inp["delta_bias"], True,
                            zoh)
        torch.cuda.synchronize()
        check(y, y_ref, TOL[dt], "y step %d" % t)
        check(state, ref_state, TOL[dt], "state step %d" % t)


@pytest.mark.parametrize("d_conv", [1, 4])
def test_conv_decode_other_state_counts(d_conv):
    """A fresh sequence fed token by token through the conv window gives
    the oracle's conv + scan over the same tokens, and the window ends as
    the last d_conv - 1 raw inputs."""
    N, T = 8, 30
    inp = syn.make_conv_inputs(syn.TINY, "cpu", batch=2, dim=5, dstate=N,
                               seqlen=T, dtype="f32", d_conv=d_conv,
                               with_h0=False, seed=70 + d_conv)
    u = oracle.causal_conv1d_silu(inp["x"], inp["conv_w"], inp["conv_b"])
    y_ref, h_ref = oracle.scan(u, inp["delta"], inp["A"], inp["B"], inp["C"],
                               inp["D"], inp["z"], inp["delta_bias"], True,
                               False, None)
    d = to_dev(inp)
    state = torch.zeros(2, 5, N, device=DEV)
    conv_state = torch.zeros(2, 5, max(d_conv - 1, 0), device=DEV)
    ys = []
    for t in range(T):
        ys.append(ssm.ssm_conv_state_update(
            state, conv_state, d["x"][..., t].contiguous(), d["conv_w"],
            d["delta"][..., t].contiguous(), d["A"], d["B"][..., t].contiguous(),
            d["C"][..., t].contiguous(), d["D"], d["z"][..., t].contiguous(),
            d["delta_bias"], True, conv_b=d["conv_b"]))
    torch.cuda.synchronize()
    check(torch.stack(ys, dim=-1), y_ref, 1e-4, "y")
    check(state, h_ref, 1e-4, "state")
    if d_conv > 1:
        assert torch.equal(conv_state, d["x"][..., T - (d_conv - 1):])


def bwd_inputs(N, batch, dim, L, dt, seed):
    inp = scan_inputs(N, batch, dim, L, dt, seed, with_h0=True)
    g = torch.Generator().manual_seed(seed + 7)
    inp["dy"] = torch.randn(batch, dim, L, generator=g).to(inp["u"].dtype)
    inp["dh_final"] = torch.randn(batch, dim, N, generator=g)
    return inp


def bwd_both(inp, zoh=False, **kw):
    ref = oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                          inp["D"], inp["z"], inp["delta_bias"], True, inp["h0"],
                          inp["dy"], inp["dh_final"], zoh_b=zoh)
    d = to_dev(inp)
    got = ssm.ssm_scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"],
                           d["z"], d["delta_bias"], True, d["h0"], d["dy"],
                           d["dh_final"], zoh_b=zoh, **kw)
    torch.cuda.synchronize()
    return ref, got, d


BWD_KEYS = ("du", "ddelta", "dA", "dB", "dC", "dh0", "dD", "ddelta_bias", "dz")


@pytest.mark.parametrize("case", [(1, "f32", 0), (5, "f32", 1), (8, "bf16", 0),
                                  (24, "f32", 0), (64, "f32", 1), (65, "f32", 1),
                                  (128, "bf16", 0), (256, "f32", 0)],
                         ids=lambda c: "n%d_%s_zoh%d" % c)
def test_bwd_other_state_counts(case):
    N, dt, zoh = case
    inp = bwd_inputs(N, 2, 11, 2100, dt, 100 + N)
    ref, got, _ = bwd_both(inp, zoh=bool(zoh))
    for k in BWD_KEYS:
        check(got[k], ref[k], TOL[dt], k)


@pytest.mark.parametrize("N", [8, 40, 130])
def test_bwd_other_state_counts_split_and_saved(N):
    """Few channels over 19000 tokens: the checkpoint pass and the sweep
    split; then the saving forward and the backward reusing its checkpoints
    (bitwise the recomputing backward)."""
    inp = bwd_inputs(N, 1, 6, 19000, "f32", 200 + N)
    ref, got, d = bwd_both(inp)
    for k in BWD_KEYS:
        check(got[k], ref[k], 1e-4, k)
    y, hf, ws = ssm.ssm_scan_fwd_save(d["u"], d["delta"], d["A"], d["B"], d["C"],
                                      d["D"], d["z"], d["delta_bias"], True,
                                      d["h0"])
    got2 = ssm.ssm_scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"],
                            d["z"], d["delta_bias"], True, d["h0"], d["dy"],
                            d["dh_final"], workspace=ws, saved=True)
    y_ref, h_ref = oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"],
                               inp["C"], inp["D"], inp["z"], inp["delta_bias"],
                               True, False, inp["h0"])
    torch.cuda.synchronize()
    check(y, y_ref, 1e-4, "y (saving forward)")
    check(hf, h_ref, 1e-4, "h_final (saving forward)")
    for k in got:
        assert torch.equal(got2[k], got[k]), k
