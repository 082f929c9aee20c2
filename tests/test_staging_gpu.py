"""The two ways the scan stages B and C give the same results, bit for bit.

Full blocks of fp32 rows whose starts are 16-byte aligned move B and C from
memory straight into the LDS tile; every other row goes through registers
(element loads when a row start is not 16-byte aligned).  The arithmetic is
the same, so one input read both ways must give identical outputs.  The
unaligned copy holds the same values 4 bytes past a 16-byte boundary, which
selects the element-wise instances for the whole call.  The aligned run is
also held to the fp64 oracle (fp32 bar 1e-4).  Cases: the tuned 16-state
instance (next block's tile requested during the last phase) with a
partial last block, whole blocks only, a sequence split into chunks, the
exact ZOH input term, the conv prologue, the saving forward; state counts
whose phase count ceil(N/2) is odd (13, 130) and even (64).
"""
import pytest
import torch

import oracle
import selective_state_space_30_amd as ssm
import synthetic as syn
from parity_metrics import scaled_max_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def unaligned(t):
    """Same values, storage starting one element past a 16-byte boundary."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


def scan_inputs(N, batch, dim, L, seed):
    inp = syn.make_scan_inputs(syn.TINY, "cpu", batch=batch, dim=dim, dstate=N,
                               seqlen=L, dtype="f32", seed=seed, with_h0=True)
    return inp, {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
                 for k, v in inp.items()}


CASES = [
    # (N, batch, dim, L, chunk_len)
    (16, 2, 9, 4100, 0),     # 4 full blocks and a partial one
    (16, 1, 6, 3072, 0),     # full blocks only
    (16, 1, 5, 5000, 1024),  # split into 1024-token chunks
    (13, 1, 6, 3000, 0),     # odd phase count
    (64, 1, 4, 2100, 0),
    (130, 1, 3, 2100, 0),    # odd phase count, two state registers
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "n%d_b%d_d%d_l%d_c%d" % c)
def test_direct_and_register_staging_agree(case):
    N, batch, dim, L, chunk = case
    inp, d = scan_inputs(N, batch, dim, L, 300 + N + L)
    for zoh in (False, True):
        args = (d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                d["delta_bias"], True, d["h0"])
        y, hf = ssm.ssm_scan_fwd(*args, chunk_len=chunk, zoh_b=zoh)
        yu, hfu = ssm.ssm_scan_fwd(d["u"], d["delta"], d["A"], unaligned(d["B"]),
                                   unaligned(d["C"]), d["D"], d["z"], d["delta_bias"],
                                   True, d["h0"], chunk_len=chunk, zoh_b=zoh)
        torch.cuda.synchronize()
        assert torch.equal(y, yu) and torch.equal(hf, hfu), "zoh=%d" % zoh
        y_ref, h_ref = oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"],
                                   inp["C"], inp["D"], inp["z"], inp["delta_bias"],
                                   True, zoh, inp["h0"])
        assert scaled_max_err(y, y_ref) <= 1e-4
        assert scaled_max_err(hf, h_ref) <= 1e-4


@pytest.mark.parametrize("N", [16, 13])
def test_direct_and_register_staging_agree_conv_and_saving(N):
    """The conv prologue's instances, and the saving forward (the backward's
    checkpoint instances) with the block states it saves."""
    inp = syn.make_conv_inputs(syn.TINY, "cpu", batch=2, dim=7, dstate=N,
                               seqlen=3100, dtype="f32", with_h0=True, seed=400 + N)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    y, hf = ssm.ssm_conv_scan_fwd(d["x"], d["conv_w"], d["delta"], d["A"], d["B"],
                                  d["C"], d["D"], d["z"], d["delta_bias"], True,
                                  d["h0"], conv_b=d["conv_b"])
    yu, hfu = ssm.ssm_conv_scan_fwd(d["x"], d["conv_w"], d["delta"], d["A"],
                                    unaligned(d["B"]), unaligned(d["C"]), d["D"],
                                    d["z"], d["delta_bias"], True, d["h0"],
                                    conv_b=d["conv_b"])
    torch.cuda.synchronize()
    assert torch.equal(y, yu) and torch.equal(hf, hfu)

    sinp, s = scan_inputs(N, 1, 6, 4100, 500 + N)
    y, hf, ws = ssm.ssm_scan_fwd_save(s["u"], s["delta"], s["A"], s["B"], s["C"],
                                      s["D"], s["z"], s["delta_bias"], True, s["h0"])
    yu, hfu, wsu = ssm.ssm_scan_fwd_save(s["u"], s["delta"], s["A"], unaligned(s["B"]),
                                         unaligned(s["C"]), s["D"], s["z"],
                                         s["delta_bias"], True, s["h0"])
    torch.cuda.synchronize()
    assert torch.equal(y, yu) and torch.equal(hf, hfu)
    # the workspace starts with the state entering every block (fp32)
    n_ck = 4 * 1 * 6 * ((4100 + 1023) // 1024) * N
    assert torch.equal(ws[:n_ck], wsu[:n_ck])
