"""Parity of the decode step (ssm_state_update through the C ABI).

The decode workload: batch=256, D=5120, N=16, fp32 state, bf16 x/delta/z
and B, C of shape (256, 16) per step; 64 consecutive steps.  Checked
against the fp64 oracle on every element (each step's y over all channels
and the state after 64 steps), and against the GPU's own scan over the same
64 tokens (the recurrent and the parallel form of one recurrence must agree
within the same tolerance).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_30_amd as ssm
import synthetic as syn
from parity_metrics import report, scaled_max_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def check(got, ref, tol, what):
    err = scaled_max_err(got, ref)
    assert err <= tol, "%s: %s (tol %g)" % (what, report(got, ref), tol)


def run_decode(inp, state):
    ys = []
    for t in range(inp["u"].shape[-1]):
        s = syn.step_slice(inp, t)
        ys.append(ssm.ssm_state_update(state, s["x"], s["delta"], inp["A"],
                                       s["B"], s["C"], inp["D"], s["z"],
                                       inp["delta_bias"], True))
    torch.cuda.synchronize()
    return torch.stack(ys, dim=-1)


@pytest.mark.parametrize("with_h0", [False, True])
def test_decode_workload_64_steps(with_h0):
    cfg = syn.DECODE
    inp = syn.make_decode_inputs(cfg, DEV, with_h0=with_h0)
    state = (inp["h0"].clone() if with_h0 else
             torch.zeros(cfg.batch, cfg.dim, 16, device=DEV))
    y_dec = run_decode(inp, state)
    # the scan over the same 64 tokens
    y_scan, h_scan = ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"],
                                      inp["B"], inp["C"], inp["D"], inp["z"],
                                      inp["delta_bias"], True, inp["h0"])
    torch.cuda.synchronize()
    check(state, h_scan.double(), 2e-2, "decode state vs scan h_final")
    check(y_dec, y_scan.double(), 2e-2, "decode y vs scan y")
    # the fp64 oracle over every channel (256 x 5120 channels, 64 tokens):
    # every step's y and the state after the last step
    y_ref, h_ref, _ = oracle.scan_threaded(
        inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
        inp["z"], inp["delta_bias"], True, False, inp["h0"],
        threads=min(16, os.cpu_count() or 1))
    check(y_dec, y_ref, 2e-2, "decode y vs oracle (all %d elements)" % y_ref.size)
    check(state, h_ref, 2e-2, "decode state vs oracle (all %d elements)" % h_ref.size)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_small_matches_oracle_every_step(dtype):
    cfg = syn.DecodeConfig("small", 3, 37, 16, 20, dtype=dtype, seed=21)
    inp = syn.make_decode_inputs(cfg, "cpu", with_h0=True)
    dinp = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}
    state = dinp["h0"].clone()
    ref_state = inp["h0"].double().numpy().copy()
    tol = 1e-4 if dtype == "f32" else 2e-2
    for t in range(cfg.steps):
        s = syn.step_slice(dinp, t)
        y = ssm.ssm_state_update(state, s["x"], s["delta"], dinp["A"], s["B"],
                                 s["C"], dinp["D"], s["z"],
                                 dinp["delta_bias"], True)
        sh = syn.step_slice(inp, t)
        y_ref = oracle.step(ref_state, sh["x"], sh["delta"], inp["A"],
                            sh["B"], sh["C"], inp["D"], sh["z"],
                            inp["delta_bias"], True, False)
        torch.cuda.synchronize()
        check(y, y_ref, tol, "y step %d" % t)
        check(state, ref_state, tol, "state step %d" % t)


def test_decode_without_optional_inputs():
    cfg = syn.DecodeConfig("bare", 2, 16, 16, 8, dtype="f32", seed=5)
    inp = syn.make_decode_inputs(cfg, "cpu")
    dinp = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}
    state = torch.zeros(2, 16, 16, device=DEV)
    ref_state = np.zeros((2, 16, 16))
    for t in range(cfg.steps):
        s = syn.step_slice(dinp, t)
        y = ssm.ssm_state_update(state, s["x"], s["delta"], dinp["A"], s["B"],
                                 s["C"], None, None, None, True)
        sh = syn.step_slice(inp, t)
        y_ref = oracle.step(ref_state, sh["x"], sh["delta"], inp["A"],
                            sh["B"], sh["C"], None, None, None, True, False)
        torch.cuda.synchronize()
        check(y, y_ref, 1e-4, "y step %d" % t)
    check(state, ref_state, 1e-4, "state")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_zoh_matches_oracle_every_step(dtype):
    cfg = syn.DecodeConfig("zoh", 2, 21, 16, 12, dtype=dtype, seed=33)
    inp = syn.make_decode_inputs(cfg, "cpu", with_h0=True)
    inp["A"][:, 5] = 0.0
    dinp = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}
    state = dinp["h0"].clone()
    ref_state = inp["h0"].double().numpy().copy()
    tol = 1e-4 if dtype == "f32" else 2e-2
    for t in range(cfg.steps):
        s = syn.step_slice(dinp, t)
        y = ssm.ssm_state_update(state, s["x"], s["delta"], dinp["A"], s["B"],
                                 s["C"], dinp["D"], s["z"],
                                 dinp["delta_bias"], True, zoh_b=True)
        sh = syn.step_slice(inp, t)
        y_ref = oracle.step(ref_state, sh["x"], sh["delta"], inp["A"],
                            sh["B"], sh["C"], inp["D"], sh["z"],
                            inp["delta_bias"], True, True)
        torch.cuda.synchronize()
        check(y, y_ref, tol, "y step %d" % t)
        check(state, ref_state, tol, "state step %d" % t)


def _offset_copy(t, offset):
    """t's values in a buffer that starts `offset` elements into a larger
    allocation: the data pointer loses its 8- and 16-byte alignment."""
    flat = torch.empty(t.numel() + offset, dtype=t.dtype, device=DEV)
    v = flat[offset:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("what", ["all", "B_only"])
def test_decode_unaligned_inputs(dtype, what):
    """Pointers without 16-byte alignment (the element-wise load path):
    every step against the oracle, odd batch and a channel count that is
    not a multiple of the workgroup's 64 channels."""
    cfg = syn.DecodeConfig("unaligned", 5, 70, 16, 6, dtype=dtype, seed=41)
    inp = syn.make_decode_inputs(cfg, "cpu", with_h0=True)
    dinp = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}
    state = (_offset_copy(dinp["h0"], 1) if what == "all"
             else dinp["h0"].clone())
    A = _offset_copy(dinp["A"], 1) if what == "all" else dinp["A"]
    ref_state = inp["h0"].double().numpy().copy()
    tol = 1e-4 if dtype == "f32" else 2e-2
    for t in range(cfg.steps):
        s = syn.step_slice(dinp, t)
        B = _offset_copy(s["B"], 1)
        C = _offset_copy(s["C"], 1) if what == "all" else s["C"]
        y = ssm.ssm_state_update(state, s["x"], s["delta"], A, B, C,
                                 dinp["D"], s["z"], dinp["delta_bias"], True)
        sh = syn.step_slice(inp, t)
        y_ref = oracle.step(ref_state, sh["x"], sh["delta"], inp["A"],
                            sh["B"], sh["C"], inp["D"], sh["z"],
                            inp["delta_bias"], True, False)
        torch.cuda.synchronize()
        check(y, y_ref, tol, "y step %d" % t)
        check(state, ref_state, tol, "state step %d" % t)


def test_decode_steps_replay_in_a_hip_graph():
    """Serving loops capture decode steps once and replay them: 8 bound
    steps captured into a graph (the library enqueues kernels only, no
    memsets), replayed three times with eager work between the replays;
    every replay gives the eager run's state and outputs bit for bit."""
    cfg = syn.DecodeConfig("graph", 4, 96, 16, 8, dtype="bf16", seed=51)
    inp = syn.make_decode_inputs(cfg, DEV, with_h0=True)
    steps = [syn.step_slice(inp, t) for t in range(cfg.steps)]
    side = torch.cuda.Stream()
    state = inp["h0"].clone()
    ys = [torch.empty(cfg.batch, cfg.dim, dtype=torch.bfloat16, device=DEV)
          for _ in steps]
    calls = [ssm.bind_state_update(state, s["x"], s["delta"], inp["A"],
                                   s["B"], s["C"], inp["D"], s["z"],
                                   inp["delta_bias"], True, y=ys[t],
                                   stream=side)
             for t, s in enumerate(steps)]
    torch.cuda.synchronize()
    for c in calls:
        c()
    side.synchronize()
    ref_state = state.clone()
    ref_ys = [y.clone() for y in ys]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for c in calls:
            c()
    for rep in range(3):
        state.copy_(inp["h0"])
        for y in ys:
            y.fill_(rep + 1)
        _ = (state * 2).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, ref_state), rep
        for t, (y, r) in enumerate(zip(ys, ref_ys)):
            assert torch.equal(y, r), (rep, t)


def test_decode_state_of_more_than_2_31_elements():
    """A state of 8200 x 16384 x 16 fp32 (2.15e9 elements, 8.6 GB): one
    step, checked against the oracle channel by channel on samples that
    include the last channel (indices past 2^31)."""
    cfg = syn.DecodeConfig("big", 8200, 16384, 16, 1, dtype="bf16", seed=61)
    assert cfg.batch * cfg.dim * 16 > 2 ** 31
    inp = syn.make_decode_inputs(cfg, DEV, with_h0=True)
    s = syn.step_slice(inp, 0)
    state = inp["h0"]
    h_before = {}
    r = np.random.default_rng(7)
    chans = sorted({(0, 0), (cfg.batch - 1, cfg.dim - 1)} |
                   {(int(r.integers(cfg.batch)), int(r.integers(cfg.dim)))
                    for _ in range(6)})
    for b, d in chans:
        h_before[b, d] = state[b:b + 1, d:d + 1].double().cpu().numpy().copy()
    y = ssm.ssm_state_update(state, s["x"], s["delta"], inp["A"], s["B"],
                             s["C"], inp["D"], s["z"], inp["delta_bias"], True)
    torch.cuda.synchronize()
    for b, d in chans:
        ref = h_before[b, d]
        y_ref = oracle.step(ref, s["x"][b:b + 1, d:d + 1], s["delta"][b:b + 1, d:d + 1],
                            inp["A"][d:d + 1], s["B"][b:b + 1], s["C"][b:b + 1],
                            inp["D"][d:d + 1], s["z"][b:b + 1, d:d + 1],
                            inp["delta_bias"][d:d + 1], True, False)
        check(y[b:b + 1, d:d + 1], y_ref, 2e-2, "y (b=%d, d=%d)" % (b, d))
        check(state[b:b + 1, d:d + 1], ref, 2e-2, "state (b=%d, d=%d)" % (b, d))


@pytest.mark.parametrize("shape", [(1, 1), (1, 65), (2, 1)],
                         ids=lambda s: "b%d_d%d" % s)
def test_decode_degenerate_shapes(shape):
    """Batch 1 (a thread's second batch entry is past the end) and a single
    channel (63 of the workgroup's 64 channels are past the end)."""
    batch, dim = shape
    cfg = syn.DecodeConfig("degenerate", batch, dim, 16, 4, dtype="bf16", seed=71)
    inp = syn.make_decode_inputs(cfg, "cpu", with_h0=True)
    dinp = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}
    state = dinp["h0"].clone()
    ref_state = inp["h0"].double().numpy().copy()
    for t in range(cfg.steps):
        s = syn.step_slice(dinp, t)
        y = ssm.ssm_state_update(state, s["x"], s["delta"], dinp["A"], s["B"],
                                 s["C"], dinp["D"], s["z"],
                                 dinp["delta_bias"], True)
        sh = syn.step_slice(inp, t)
        y_ref = oracle.step(ref_state, sh["x"], sh["delta"], inp["A"],
                            sh["B"], sh["C"], inp["D"], sh["z"],
                            inp["delta_bias"], True, False)
        torch.cuda.synchronize()
        check(y, y_ref, 2e-2, "y step %d" % t)
        check(state, ref_state, 2e-2, "state step %d" % t)
