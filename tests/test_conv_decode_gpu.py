"""Parity of the decode step with the fused conv prologue
(ssm_conv_state_update through the C ABI).

Each step takes one new input per channel, forms u = silu(conv_b + causal
depthwise conv1d) over the d_conv - 1 inputs kept in conv_state and the new
one, advances the state like ssm_state_update, and shifts the new input into
conv_state.  The oracle: its fp64 causal conv1d + SiLU over the kept window
followed by the new inputs (the first d_conv - 1 outputs, which would need
inputs before the window, are dropped), then its fp64 step per token.  A
fresh sequence (zero window) must also give what the conv scan gives over
the same tokens.  conv_state holds raw inputs, so after T steps it equals
the last d_conv - 1 of (window, inputs) bit for bit.  Bars: 1e-4 with fp32
activations, 2e-2 with bf16 (the same as the plain step's).
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


def gpu_steps(d, state, conv_state, zoh=False):
    """Feeds the sequence one token at a time; returns y (batch, dim, T)."""
    ys = []
    for t in range(d["u"].shape[-1]):
        s = syn.step_slice(d, t)
        ys.append(ssm.ssm_conv_state_update(
            state, conv_state, s["x"], d["conv_w"], s["delta"], d["A"],
            s["B"], s["C"], d["D"], s["z"], d["delta_bias"], True,
            conv_b=d["conv_b"], zoh_b=zoh))
    torch.cuda.synchronize()
    return torch.stack(ys, dim=-1)


def oracle_conv_input(inp):
    """fp64 u (batch, dim, T): the conv over (window, new inputs), with the
    outputs of the window's own positions dropped."""
    H = inp["conv_w"].shape[1] - 1
    xw = torch.cat([inp["conv_state0"], inp["u"]], dim=-1)
    return oracle.causal_conv1d_silu(xw, inp["conv_w"], inp["conv_b"])[:, :, H:]


def expected_window(inp):
    H = inp["conv_w"].shape[1] - 1
    return torch.cat([inp["conv_state0"], inp["u"]], dim=-1)[:, :, -H:] \
        if H > 0 else None


CASES = [
    # (dtype, d_conv, conv_b, kept window, steps)
    ("f32", 4, True, True, 9),
    ("bf16", 4, True, True, 9),
    ("f32", 4, False, False, 9),
    ("bf16", 3, True, True, 7),
    ("f32", 2, False, True, 7),
    ("bf16", 2, True, False, 5),
    ("f32", 1, True, False, 5),
    ("bf16", 1, False, False, 5),
    ("bf16", 4, True, True, 2),  # fewer tokens than the window holds
]


@pytest.mark.parametrize("case", CASES,
                         ids=lambda c: "%s_k%d_%s_%s_t%d" % (
                             c[0], c[1], "bias" if c[2] else "nobias",
                             "window" if c[3] else "fresh", c[4]))
def test_conv_decode_matches_oracle_every_step(case):
    dtype, K, with_bias, with_window, T = case
    cfg = syn.DecodeConfig("conv_small", 3, 37, 16, T, dtype=dtype, seed=41 + K)
    inp = syn.make_conv_decode_inputs(cfg, "cpu", d_conv=K, with_bias=with_bias,
                                      with_h0=True, with_window=with_window)
    d = to_dev(inp)
    state = d["h0"].clone()
    conv_state = d["conv_state0"].clone() if K > 1 else None
    y = gpu_steps(d, state, conv_state)
    u = oracle_conv_input(inp)
    ref_state = inp["h0"].double().numpy().copy()
    for t in range(T):
        sh = syn.step_slice(inp, t)
        y_ref = oracle.step(ref_state, u[:, :, t], sh["delta"], inp["A"],
                            sh["B"], sh["C"], inp["D"], sh["z"],
                            inp["delta_bias"], True, False)
        check(y[:, :, t], y_ref, TOL[dtype], "y step %d" % t)
    check(state, ref_state, TOL[dtype], "state after %d steps" % T)
    if K > 1:
        assert torch.equal(conv_state.cpu(), expected_window(inp))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_decode_zoh_matches_oracle(dtype):
    cfg = syn.DecodeConfig("conv_zoh", 2, 21, 16, 8, dtype=dtype, seed=53)
    inp = syn.make_conv_decode_inputs(cfg, "cpu", d_conv=4, with_h0=True,
                                      with_window=True)
    inp["A"][:, 5] = 0.0  # the exact input term's A -> 0 limit
    d = to_dev(inp)
    state = d["h0"].clone()
    conv_state = d["conv_state0"].clone()
    y = gpu_steps(d, state, conv_state, zoh=True)
    u = oracle_conv_input(inp)
    ref_state = inp["h0"].double().numpy().copy()
    for t in range(cfg.steps):
        sh = syn.step_slice(inp, t)
        y_ref = oracle.step(ref_state, u[:, :, t], sh["delta"], inp["A"],
                            sh["B"], sh["C"], inp["D"], sh["z"],
                            inp["delta_bias"], True, True)
        check(y[:, :, t], y_ref, TOL[dtype], "y step %d" % t)
    check(state, ref_state, TOL[dtype], "state")
    assert torch.equal(conv_state.cpu(), expected_window(inp))


def test_conv_decode_workload_matches_conv_scan_and_oracle():
    """The decode workload's shape (batch 256, D = 5120, N = 16, bf16) with a
    width-4 conv, 16 tokens from a fresh sequence: against the GPU conv scan
    over the same tokens everywhere, and the oracle on sampled channels."""
    cfg = syn.replace(syn.DECODE, steps=16)
    inp = syn.make_conv_decode_inputs(cfg, DEV, d_conv=4)
    state = torch.zeros(cfg.batch, cfg.dim, 16, device=DEV)
    conv_state = inp["conv_state0"].clone()
    y = gpu_steps(inp, state, conv_state)
    y_scan, h_scan = ssm.ssm_conv_scan_fwd(
        inp["u"], inp["conv_w"], inp["delta"], inp["A"], inp["B"], inp["C"],
        inp["D"], inp["z"], inp["delta_bias"], True, None,
        conv_b=inp["conv_b"])
    torch.cuda.synchronize()
    check(y, y_scan.double(), 2e-2, "decode y vs conv scan y")
    check(state, h_scan.double(), 2e-2, "decode state vs conv scan h_final")
    assert torch.equal(conv_state, inp["u"][:, :, -3:])
    r = np.random.default_rng(cfg.seed)
    chans = sorted({(0, 0), (cfg.batch - 1, cfg.dim - 1)} |
                   {(int(r.integers(cfg.batch)), int(r.integers(cfg.dim)))
                    for _ in range(62)})
    ys, hs = [], []
    for b, dd in chans:
        sl = (slice(b, b + 1), slice(dd, dd + 1))
        u = oracle.causal_conv1d_silu(inp["u"][sl], inp["conv_w"][dd:dd + 1],
                                      inp["conv_b"][dd:dd + 1])
        yr, hr = oracle.scan(u, inp["delta"][sl], inp["A"][dd:dd + 1],
                             inp["B"][b:b + 1], inp["C"][b:b + 1],
                             inp["D"][dd:dd + 1], inp["z"][sl],
                             inp["delta_bias"][dd:dd + 1], True, False, None)
        ys.append(yr[0, 0])
        hs.append(hr[0, 0])
    bi = torch.tensor([c[0] for c in chans], device=DEV)
    di = torch.tensor([c[1] for c in chans], device=DEV)
    check(y[bi, di], np.stack(ys), 2e-2, "decode y vs oracle (sampled)")
    check(state[bi, di], np.stack(hs), 2e-2, "decode state vs oracle (sampled)")


@pytest.mark.parametrize("shape", [(1, 1), (1, 65), (2, 1), (5, 129)],
                         ids=lambda s: "b%d_d%d" % s)
def test_conv_decode_degenerate_shapes(shape):
    """Batch 1 (a thread's second batch entry is past the end), a single
    channel (63 of the workgroup's 64 channels are past the end) and ragged
    sizes in both grid dimensions."""
    batch, dim = shape
    cfg = syn.DecodeConfig("conv_degenerate", batch, dim, 16, 5, dtype="bf16",
                           seed=77)
    inp = syn.make_conv_decode_inputs(cfg, "cpu", d_conv=4, with_h0=True,
                                      with_window=True)
    d = to_dev(inp)
    state = d["h0"].clone()
    conv_state = d["conv_state0"].clone()
    y = gpu_steps(d, state, conv_state)
    u = oracle_conv_input(inp)
    ref_state = inp["h0"].double().numpy().copy()
    for t in range(cfg.steps):
        sh = syn.step_slice(inp, t)
        y_ref = oracle.step(ref_state, u[:, :, t], sh["delta"], inp["A"],
                            sh["B"], sh["C"], inp["D"], sh["z"],
                            inp["delta_bias"], True, False)
        check(y[:, :, t], y_ref, 2e-2, "y step %d" % t)
    check(state, ref_state, 2e-2, "state")
    assert torch.equal(conv_state.cpu(), expected_window(inp))


def _offset_copy(t, offset):
    """t's values in a buffer that starts `offset` elements into a larger
    allocation: the data pointer loses its 8- and 16-byte alignment."""
    flat = torch.empty(t.numel() + offset, dtype=t.dtype, device=DEV)
    v = flat[offset:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_decode_unaligned_inputs(dtype):
    """B, the state, the taps and the window without 16-byte alignment (the
    element-wise instance of the kernel): every step against the oracle,
    with an odd batch and a ragged channel count."""
    cfg = syn.DecodeConfig("conv_unaligned", 5, 70, 16, 6, dtype=dtype, seed=61)
    inp = syn.make_conv_decode_inputs(cfg, "cpu", d_conv=4, with_h0=True,
                                      with_window=True)
    d = to_dev(inp)
    state = _offset_copy(d["h0"], 1)
    conv_state = _offset_copy(d["conv_state0"], 1)
    conv_w = _offset_copy(d["conv_w"], 1)
    u = oracle_conv_input(inp)
    ref_state = inp["h0"].double().numpy().copy()
    for t in range(cfg.steps):
        s = syn.step_slice(d, t)
        y = ssm.ssm_conv_state_update(
            state, conv_state, s["x"], conv_w, s["delta"], d["A"],
            _offset_copy(s["B"], 1), s["C"], d["D"], s["z"], d["delta_bias"],
            True, conv_b=d["conv_b"])
        sh = syn.step_slice(inp, t)
        y_ref = oracle.step(ref_state, u[:, :, t], sh["delta"], inp["A"],
                            sh["B"], sh["C"], inp["D"], sh["z"],
                            inp["delta_bias"], True, False)
        torch.cuda.synchronize()
        check(y, y_ref, TOL[dtype], "y step %d" % t)
    check(state, ref_state, TOL[dtype], "state")
    assert torch.equal(conv_state.cpu(), expected_window(inp))


def test_conv_decode_steps_replay_in_a_hip_graph():
    """Six conv decode steps captured into a graph (one kernel per step, no
    memsets), replayed three times with eager work between the replays;
    every replay gives the eager run's state, window and outputs bit for
    bit."""
    cfg = syn.DecodeConfig("conv_graph", 4, 96, 16, 6, dtype="bf16", seed=57)
    inp = syn.make_conv_decode_inputs(cfg, DEV, d_conv=4, with_h0=True,
                                      with_window=True)
    steps = [syn.step_slice(inp, t) for t in range(cfg.steps)]
    side = torch.cuda.Stream()
    state = inp["h0"].clone()
    window = inp["conv_state0"].clone()
    ys = [torch.empty(cfg.batch, cfg.dim, dtype=torch.bfloat16, device=DEV)
          for _ in steps]

    def enqueue():
        for t, s in enumerate(steps):
            ssm.ssm_conv_state_update(
                state, window, s["x"], inp["conv_w"], s["delta"], inp["A"],
                s["B"], s["C"], inp["D"], s["z"], inp["delta_bias"], True,
                conv_b=inp["conv_b"], y=ys[t], stream=side)
    torch.cuda.synchronize()
    enqueue()
    side.synchronize()
    ref_state, ref_window = state.clone(), window.clone()
    ref_ys = [y.clone() for y in ys]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        enqueue()
    for rep in range(3):
        state.copy_(inp["h0"])
        window.copy_(inp["conv_state0"])
        for y in ys:
            y.fill_(rep + 1)
        _ = (state * 2).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, ref_state), rep
        assert torch.equal(window, ref_window), rep
        for t, (y, r) in enumerate(zip(ys, ref_ys)):
            assert torch.equal(y, r), (rep, t)
