"""Parity of the scan with the fused conv prologue (ssm_conv_scan_fwd).

The oracle forms u = silu(conv_b + causal depthwise conv1d(x, conv_w)) in
fp64 and runs its scan on it; the HIP path forms u in registers inside the
scan kernel (it never reaches HBM).  Same bars as the plain scan: 1e-4 with
fp32 activations, 2e-2 with bf16.
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


def gpu_conv_scan(d, chunk_len=0):
    y, hf = ssm.ssm_conv_scan_fwd(d["x"], d["conv_w"], d["delta"], d["A"],
                                  d["B"], d["C"], d["D"], d["z"],
                                  d["delta_bias"], d["delta_softplus"],
                                  d["h0"], conv_b=d["conv_b"],
                                  chunk_len=chunk_len)
    torch.cuda.synchronize()
    return y, hf


def oracle_conv_scan(inp):
    u = oracle.causal_conv1d_silu(inp["x"], inp["conv_w"], inp["conv_b"])
    return oracle.scan(u, inp["delta"], inp["A"], inp["B"], inp["C"],
                       inp["D"], inp["z"], inp["delta_bias"],
                       inp["delta_softplus"], False, inp["h0"])


CASES = [
    # (batch, dim, L, dtype, d_conv, conv bias, h0, chunk)
    (1, 8, 256, "f32", 4, True, False, 0),       # one partial block
    (2, 13, 2048, "f32", 4, True, True, 0),      # history across blocks
    (2, 13, 2100, "f32", 3, False, True, 0),     # ragged tail, 3 taps
    (1, 6, 999, "f32", 2, True, False, 0),       # unaligned rows
    (2, 20, 3072, "bf16", 4, True, False, 0),
    (1, 9, 5000, "f32", 4, True, True, 1024),    # history across chunks
    (1, 9, 4500, "bf16", 4, True, True, 2048),
    (1, 4, 1, "f32", 4, True, True, 0),          # a single token
]


@pytest.mark.parametrize("case", CASES,
                         ids=lambda c: "b%d_d%d_l%d_%s_k%d_cb%d_h%d_c%d" % c)
def test_conv_scan_matches_oracle(case):
    batch, dim, L, dt, k, cbias, wh, chunk = case
    inp = syn.make_conv_inputs(syn.TINY, "cpu", d_conv=k, with_bias=cbias,
                               batch=batch, dim=dim, seqlen=L, dtype=dt,
                               with_h0=wh, seed=300 + L + k)
    y_ref, h_ref = oracle_conv_scan(inp)
    y, hf = gpu_conv_scan(to_dev(inp), chunk_len=chunk)
    check(y, y_ref, TOL[dt], "y")
    check(hf, h_ref, TOL[dt], "h_final")


def test_conv_scan_equals_conv_then_scan():
    """The fused prologue gives the scan of the explicit convolution."""
    inp = syn.make_conv_inputs(syn.TINY, "cpu", batch=2, dim=16, seqlen=3000,
                               dtype="f32", with_h0=True, seed=41)
    u = torch.from_numpy(oracle.causal_conv1d_silu(
        inp["x"], inp["conv_w"], inp["conv_b"])).float()
    d = to_dev(inp)
    y1, h1 = gpu_conv_scan(d)
    y2, h2 = ssm.ssm_scan_fwd(u.to(DEV), d["delta"], d["A"], d["B"], d["C"],
                              d["D"], d["z"], d["delta_bias"], True, d["h0"])
    torch.cuda.synchronize()
    check(y1, y2.double(), 1e-5, "y")
    check(h1, h2.double(), 1e-5, "h_final")


def test_conv_rejects_too_many_taps():
    inp = to_dev(syn.make_conv_inputs(syn.TINY, "cpu", d_conv=5, batch=1,
                                      dim=4, seqlen=64, seed=1))
    with pytest.raises(ssm.SSMError) as e:
        gpu_conv_scan(inp)
    assert e.value.status == 2


def test_mamba2p8b_workload_with_conv_sampled():
    cfg = syn.MAMBA_2P8B
    inp = syn.make_conv_inputs(cfg, DEV)
    y, hf = gpu_conv_scan(inp)
    r = np.random.default_rng(7)
    chans = sorted({(0, 0), (1, cfg.dim - 1)} |
                   {(int(r.integers(2)), int(r.integers(cfg.dim)))
                    for _ in range(14)})
    ys, hs = [], []
    for b, dd in chans:
        sl = (slice(b, b + 1), slice(dd, dd + 1))
        u = oracle.causal_conv1d_silu(inp["x"][sl], inp["conv_w"][dd:dd + 1],
                                      inp["conv_b"][dd:dd + 1])
        yr, hr = oracle.scan(u, inp["delta"][sl], inp["A"][dd:dd + 1],
                             inp["B"][b:b + 1], inp["C"][b:b + 1],
                             inp["D"][dd:dd + 1], inp["z"][sl],
                             inp["delta_bias"][dd:dd + 1], True, False, None)
        ys.append(yr[0, 0])
        hs.append(hr[0, 0])
    bi = torch.tensor([c[0] for c in chans], device=DEV)
    di = torch.tensor([c[1] for c in chans], device=DEV)
    check(y[bi, di], np.stack(ys), 2e-2, "y (sampled)")
    check(hf[bi, di], np.stack(hs), 2e-2, "h_final (sampled)")
    assert torch.isfinite(y.float()).all()
