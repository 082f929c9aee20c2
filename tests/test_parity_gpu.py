"""Parity of the HIP scan (through the C ABI) with the fp64 oracle.

Bars: fp32 activations 1e-4, bf16 activations 2e-2, measured as
max |gpu - oracle| / (|oracle| + rms(oracle)) per output tensor (see
parity_metrics.py).  Small shapes are compared element by element over the
whole output; the full-size workloads run exactly as the benchmark launches
them: the 130M- and 2.8B-shaped layers over their whole output (the
threaded oracle), the long-context and ragged-length runs on sampled
channels, which the oracle computes one by one (channels are independent).
Besides the scaled bar, every comparison also bounds the plain relative
error over the elements with |oracle| >= rms(oracle) by the same tolerance.
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


def to_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}


def gpu_scan(inp, chunk_len=0, return_final_state=True):
    y, hf = ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"],
                             inp["C"], inp["D"], inp["z"], inp["delta_bias"],
                             inp["delta_softplus"], inp["h0"],
                             return_final_state=return_final_state,
                             chunk_len=chunk_len)
    torch.cuda.synchronize()
    return y, hf


def oracle_scan(inp):
    return oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                       inp["D"], inp["z"], inp["delta_bias"],
                       inp["delta_softplus"], False, inp["h0"])


def check(got, ref, tol, what):
    """Both bars: the scaled error and the plain relative error over the
    elements with |ref| >= rms(ref)."""
    r = report(got, ref)
    assert r["scaled_max"] <= tol and r["rel_over_rms"] <= tol, \
        "%s: %s (tol %g)" % (what, r, tol)
    return r["scaled_max"]


SMALL_CASES = [
    # (batch, dim, L, dtype, with_z, with_D, with_h0)
    (1, 64, 256, "f32", True, True, False),     # the tiny workload's shape
    (2, 37, 1000, "f32", True, True, True),     # ragged channels and tail
    (2, 37, 999, "f32", False, False, True),    # unaligned rows: scalar loads
    (1, 16, 1, "f32", True, True, True),        # a single token
    (1, 1, 300, "f32", True, True, False),      # a single channel
    (3, 20, 777, "bf16", True, True, False),    # unaligned bf16 rows
    (2, 48, 1536, "bf16", True, True, True),    # aligned bf16, 6 blocks
    (1, 5, 4096, "bf16", False, True, False),   # no gate
    (2, 37, 2048, "f32", True, True, True),     # aligned fp32, full blocks
    (1, 6, 3072, "bf16", True, False, True),    # 3 full blocks, no D
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: "b%d_d%d_l%d_%s_z%d_D%d_h%d" % c)
def test_small_shapes_match_oracle(case):
    batch, dim, L, dt, wz, wD, wh = case
    inp = syn.make_scan_inputs(syn.TINY, "cpu", batch=batch, dim=dim, seqlen=L,
                               dtype=dt, with_z=wz, with_D=wD, with_h0=wh,
                               seed=77 + L)
    y_ref, h_ref = oracle_scan(inp)
    y, hf = gpu_scan(to_dev(inp))
    check(y, y_ref, TOL[dt], "y")
    check(hf, h_ref, TOL[dt], "h_final")


def test_tiny_workload_exactly_as_specified():
    inp = syn.make_scan_inputs(syn.TINY, "cpu")
    y_ref, h_ref = oracle_scan(inp)
    y, hf = gpu_scan(to_dev(inp))
    check(y, y_ref, 1e-4, "y")
    check(hf, h_ref, 1e-4, "h_final")


CHUNK_CASES = [
    # (dtype, L, chunk, softplus, A kind); chunks are whole 1024-token blocks
    ("f32", 3000, 1024, True, "arange"),     # decays: fix-up stops early
    ("f32", 2049, 1024, True, "arange"),     # last chunk of one token
    ("f32", 5000, 2048, False, "arange"),    # softplus off: full fix-up
    ("f32", 3000, 1024, True, "positive"),   # an A > 0: full fix-up
    ("bf16", 8192, 2048, True, "arange"),
    ("bf16", 4500, 1024, True, "slow"),      # slow decay: long fix-up
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: "%s_l%d_c%d_sp%d_%s" % c)
def test_chunked_scan_matches_oracle(case):
    dt, L, chunk, sp, akind = case
    inp = syn.make_scan_inputs(syn.TINY, "cpu", batch=2, dim=24, seqlen=L,
                               dtype=dt, with_h0=True, seed=5 + L)
    if not sp:
        # a positive step used as given, small enough to stay stable
        inp["delta"] = (0.05 * inp["delta"].float().abs()).to(inp["delta"].dtype)
        inp["delta_softplus"] = False
        inp["delta_bias"] = None
    if akind == "positive":
        inp["A"][:, 0] = 0.002
    elif akind == "slow":
        inp["A"] = inp["A"] * 0.01
    assert ssm.ssm_scan_plan(2, 24, 16, L, chunk) == chunk
    y_ref, h_ref = oracle_scan(inp)
    y, hf = gpu_scan(to_dev(inp), chunk_len=chunk)
    check(y, y_ref, TOL[dt], "y")
    check(hf, h_ref, TOL[dt], "h_final")


def test_chunked_and_unsplit_agree():
    inp = to_dev(syn.make_scan_inputs(syn.TINY, "cpu", batch=1, dim=32,
                                      seqlen=5000, dtype="f32", seed=3))
    y1, h1 = gpu_scan(inp)
    y2, h2 = gpu_scan(inp, chunk_len=2048)
    check(y2, y1.double(), 1e-5, "y")
    check(h2, h1.double(), 1e-5, "h_final")


def test_resume_from_final_state():
    """Associativity: scanning [0, L1) and then [L1, L) from the first
    part's final state gives the whole scan."""
    L, L1 = 2000, 777
    inp = to_dev(syn.make_scan_inputs(syn.TINY, "cpu", batch=2, dim=40,
                                      seqlen=L, dtype="f32", with_h0=True,
                                      seed=11))
    y, hf = gpu_scan(inp)
    a = dict(inp)
    b = dict(inp)
    for k in ("u", "delta", "B", "C", "z"):
        a[k] = inp[k][..., :L1].contiguous()
        b[k] = inp[k][..., L1:].contiguous()
    ya, ha = gpu_scan(a)
    b["h0"] = ha
    yb, hb = gpu_scan(b)
    check(torch.cat([ya, yb], dim=-1), y.double(), 1e-5, "y")
    check(hb, hf.double(), 1e-5, "h_final")


def test_bitwise_deterministic():
    inp = to_dev(syn.make_scan_inputs(syn.MAMBA_130M, "cpu", batch=1, dim=64,
                                      seqlen=2048))
    y1, h1 = gpu_scan(inp)
    y2, h2 = gpu_scan(inp)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_zero_step_keeps_state_exactly():
    inp = syn.make_scan_inputs(syn.TINY, "cpu", batch=2, dim=20, seqlen=600,
                               dtype="f32", with_h0=True, seed=9)
    inp["delta"] = torch.zeros_like(inp["delta"])
    inp["delta_bias"] = None
    inp["delta_softplus"] = False
    y_ref, h_ref = oracle_scan(inp)
    y, hf = gpu_scan(to_dev(inp))
    assert torch.equal(hf.cpu(), inp["h0"])
    check(y, y_ref, 1e-4, "y")


def test_nan_propagates_forward():
    inp = syn.make_scan_inputs(syn.TINY, "cpu", batch=1, dim=16, seqlen=512,
                               dtype="f32", with_z=False, seed=4)
    inp["u"][0, 3, 300] = float("nan")
    y, hf = gpu_scan(to_dev(inp))
    y = y.cpu()
    assert torch.isfinite(y[0, 3, :300]).all()
    assert torch.isnan(y[0, 3, 300:]).all() and torch.isnan(hf[0, 3].cpu()).all()
    others = torch.cat([y[0, :3], y[0, 4:]])
    assert torch.isfinite(others).all()


def test_workspace_too_small_is_rejected_on_device():
    inp = to_dev(syn.make_scan_inputs(syn.TINY, "cpu", batch=1, dim=16,
                                      seqlen=2048, seed=2))
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ssm.SSMError) as e:
        ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                         chunk_len=1024, workspace=ws)
    assert e.value.status == 3


# ------------------------------------------------------- full workloads
HOST_THREADS = 16  # the host CPU share of a one-GPU machine


def sample_channels(batch, dim, k, seed):
    r = np.random.default_rng(seed)
    picks = {(0, 0), (batch - 1, dim - 1)}
    while len(picks) < k:
        picks.add((int(r.integers(batch)), int(r.integers(dim))))
    return sorted(picks)


def full_workload_check(cfg, k, tol):
    """The workload exactly as the benchmark launches it, checked on k
    sampled channels (the first, the last and random ones)."""
    inp = syn.make_scan_inputs(cfg, DEV)
    chans = sample_channels(cfg.batch, cfg.dim, k, cfg.seed)
    y, hf = gpu_scan(inp)
    check_channels(inp, y, hf, chans, tol)
    # Properties at full size: everything finite.
    assert torch.isfinite(y.float()).all() and torch.isfinite(hf).all()


def check_channels(inp, y, hf, chans, tol):
    y_ref, h_ref = oracle.scan_channels(
        inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
        inp["z"], inp["delta_bias"], inp["delta_softplus"], False, inp["h0"],
        channels=chans, threads=HOST_THREADS)
    bi = torch.tensor([c[0] for c in chans], device=DEV)
    di = torch.tensor([c[1] for c in chans], device=DEV)
    check(y[bi, di], y_ref, tol, "y (%d channels)" % len(chans))
    check(hf[bi, di], h_ref, tol, "h_final (%d channels)" % len(chans))


def whole_output_check(cfg, tol):
    """The workload exactly as the benchmark launches it, every element of
    y and h_final against the oracle over all channels."""
    inp = syn.make_scan_inputs(cfg, DEV)
    y, hf = gpu_scan(inp)
    y_ref, h_ref, _ = oracle.scan_threaded(
        inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
        inp["z"], inp["delta_bias"], inp["delta_softplus"], False, inp["h0"],
        threads=HOST_THREADS)
    check(y, y_ref, tol, "y (all %d elements)" % y_ref.size)
    check(hf, h_ref, tol, "h_final (all %d elements)" % h_ref.size)


def test_mamba130m_workload_whole_output():
    """The 130M-shaped layer: all 4 x 1536 channels x 2048 tokens."""
    whole_output_check(syn.MAMBA_130M, 2e-2)


def test_mamba2p8b_workload_whole_output():
    """The 2.8B-shaped layer (the benchmark's workload): all 2 x 5120
    channels x 4096 tokens and every final state."""
    whole_output_check(syn.MAMBA_2P8B, 2e-2)


@pytest.mark.parametrize("L", [4104, 4600, 4095, 100],
                         ids=lambda L: "l%d" % L)
def test_mamba2p8b_shape_ragged_lengths_sampled(L):
    """The 2.8B layer's width with lengths that end in a partial block of
    8, 504 and 1023 tokens (4 and 8 tokens per lane, and 16 with rows that
    are not 16-byte aligned: the element-wise instance) and a sequence
    shorter than one block; 64 sampled channels of 10240."""
    from dataclasses import replace
    full_workload_check(replace(syn.MAMBA_2P8B, seqlen=L), 64, 2e-2)


def test_long_context_workload_sampled():
    """The long-context workload (1536 channels x 2^20 tokens, fp32, split
    into chunks): 72 channels, 18 at each of the 4 wave positions of a
    workgroup, including the first and the last channel.  Every channel
    runs all the chunks (the first from h0 = 0, the others through the
    carry and the decay-bounded fix-up), so all chunk indices are covered
    on every sampled channel."""
    cfg = syn.LONG_1M
    chunk = ssm.ssm_scan_plan(cfg.batch, cfg.dim, 16, cfg.seqlen)
    assert chunk < cfg.seqlen
    r = np.random.default_rng(cfg.seed)
    chans = {(0, 0), (0, cfg.dim - 1)}
    for w in range(4):
        picks = r.choice(np.arange(w, cfg.dim, 4), size=17, replace=False)
        chans.update((0, int(d)) for d in picks)
    chans = sorted(chans)
    assert len(chans) >= 64 and {d % 4 for _, d in chans} == {0, 1, 2, 3}
    inp = syn.make_scan_inputs(cfg, DEV)
    y, hf = gpu_scan(inp)
    check_channels(inp, y, hf, chans, 1e-4)
    assert torch.isfinite(y).all() and torch.isfinite(hf).all()


def test_long_context_workload_whole_output():
    """The long-context workload on every element: all 1536 channels x 2^20
    tokens of y and every final state, against the oracle in ranges of 96
    channels (each range's inputs converted to fp64 on its own, so the
    host holds ~4 GB at a time; the scaled error takes each range's rms,
    over 1e8 elements of one distribution).  Every chunk boundary, fix-up
    length and wave position of the launch is covered."""
    cfg = syn.LONG_1M
    assert ssm.ssm_scan_plan(cfg.batch, cfg.dim, 16, cfg.seqlen) < cfg.seqlen
    inp = syn.make_scan_inputs(cfg, DEV)
    y, hf = gpu_scan(inp)
    step = 96
    worst = 0.0
    for d0 in range(0, cfg.dim, step):
        d1 = min(cfg.dim, d0 + step)
        sl = lambda t: None if t is None else t[:, d0:d1].contiguous()
        y_ref, h_ref, _ = oracle.scan_threaded(
            sl(inp["u"]), sl(inp["delta"]), inp["A"][d0:d1], inp["B"], inp["C"],
            inp["D"][d0:d1], sl(inp["z"]), inp["delta_bias"][d0:d1]
            if inp["delta_bias"] is not None else None,
            inp["delta_softplus"], False, sl(inp["h0"]), threads=HOST_THREADS)
        worst = max(worst, check(y[:, d0:d1], y_ref, 1e-4, "y channels %d..%d" % (d0, d1)))
        check(hf[:, d0:d1], h_ref, 1e-4, "h_final channels %d..%d" % (d0, d1))
    print("long context, whole output: worst scaled error %.3g" % worst)


def test_chunked_mixed_fixup_lengths_in_one_launch():
    """One launch with 8 chunks per channel in which some channels stop
    their fix-up early (A < 0, fast decay), some run it over the whole chunk
    (one A > 0) and some decay slowly (a long, partial fix-up); every
    channel and every chunk against the oracle."""
    L, chunk = 8 * 1024 - 300, 1024
    inp = syn.make_scan_inputs(syn.TINY, "cpu", batch=2, dim=24, seqlen=L,
                               dtype="f32", with_h0=True, seed=31)
    inp["A"][0::3, 5] = 0.002          # whole-chunk fix-up
    inp["A"][1::3] *= 0.01             # slow decay: long fix-up
    assert ssm.ssm_scan_plan(2, 24, 16, L, chunk) == chunk
    y_ref, h_ref = oracle_scan(inp)
    y, hf = gpu_scan(to_dev(inp), chunk_len=chunk)
    check(y, y_ref, 1e-4, "y")
    check(hf, h_ref, 1e-4, "h_final")


def test_more_than_2_31_elements():
    """2048 channels x 1,100,000 tokens (2.25e9 elements per activation
    tensor, 4.5 GB in bf16; a ragged last block; split into chunks): every
    element index past 2^31 must address the right element, checked on
    sampled channels including the last one."""
    from dataclasses import replace
    cfg = replace(syn.LONG_1M, dim=2048, seqlen=1_100_000, dtype="bf16")
    assert cfg.batch * cfg.dim * cfg.seqlen > 2 ** 31
    full_workload_check(cfg, 5, 2e-2)


# ------------------------------------------------ exact ZOH input term
ZOH_CASES = [
    # (batch, dim, L, dtype, chunk, A kind)
    (2, 24, 2048, "f32", 0, "arange"),
    (1, 13, 1500, "f32", 0, "zero_cols"),     # some A = 0: the Euler limit
    (2, 16, 3000, "bf16", 0, "arange"),
    (1, 8, 5000, "f32", 2048, "arange"),      # chunked
    (1, 5, 777, "f32", 0, "small"),           # |dt*A| mostly below 2^-5
    (2, 16, 2248, "f32", 0, "arange"),        # last block 200 tokens: 4 a lane
    (1, 8, 1124, "bf16", 0, "arange"),        # last block 100 tokens, bf16
    (1, 8, 1536, "bf16", 0, "arange"),        # last block 512 tokens: 8 a lane
]


@pytest.mark.parametrize("case", ZOH_CASES, ids=lambda c: "b%d_d%d_l%d_%s_c%d_%s" % c)
def test_zoh_scan_matches_oracle(case):
    batch, dim, L, dt, chunk, akind = case
    inp = syn.make_scan_inputs(syn.TINY, "cpu", batch=batch, dim=dim, seqlen=L,
                               dtype=dt, with_h0=True, seed=900 + L)
    if akind == "zero_cols":
        inp["A"][:, ::3] = 0.0
    elif akind == "small":
        inp["A"] = inp["A"] * 1e-3
    y_ref, h_ref = oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"],
                               inp["C"], inp["D"], inp["z"], inp["delta_bias"],
                               True, True, inp["h0"])
    d = to_dev(inp)
    y, hf = ssm.ssm_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"],
                             d["D"], d["z"], d["delta_bias"], True, d["h0"],
                             chunk_len=chunk, zoh_b=True)
    torch.cuda.synchronize()
    check(y, y_ref, TOL[dt], "y")
    check(hf, h_ref, TOL[dt], "h_final")
    # and the Euler result differs measurably (the flag is honoured)
    y_e, _ = gpu_scan(d)
    assert scaled_max_err(y_e, y_ref) > 10 * TOL[dt] or akind == "small"
