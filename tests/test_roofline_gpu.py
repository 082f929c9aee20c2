"""The roofline microbenchmarks compute what they claim (so that their
timings measure the traffic and operations they are credited with)."""
import numpy as np
import pytest
import torch

import selective_state_space_30_amd as ssm

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_hbm_copy_rmw_read():
    n = 4 * ssm.SSM_ROOFLINE_HBM_QUANTUM // 4  # floats in 4 quanta
    g = torch.Generator(device=DEV).manual_seed(5)
    a = torch.randn(n, device=DEV, generator=g)
    b = torch.full_like(a, float("nan"))
    ssm.ssm_roofline_hbm("copy", a, b, repeats=2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = a.clone()
    ssm.ssm_roofline_hbm("rmw", a, repeats=3)
    torch.cuda.synchronize()
    for _ in range(3):
        ref = ref * 0.5 + 0.25
    assert torch.allclose(a, ref, rtol=1e-6, atol=1e-7)
    sink = torch.zeros(1, device=DEV)
    ssm.ssm_roofline_hbm("read", a, sink, repeats=1)
    torch.cuda.synchronize()
    assert sink.item() == 0.0  # the sink is written only for an impossible sum


@pytest.mark.parametrize("kind", ["exp", "fma", "mixed"])
def test_valu_chains(kind):
    threads = 4 * ssm.SSM_ROOFLINE_VALU_QUANTUM
    iters = 3
    out = torch.empty(threads, device=DEV)
    ssm.ssm_roofline_valu(kind, out, iters)
    torch.cuda.synchronize()
    lane = np.arange(threads) % 256
    ref = np.zeros(threads)
    for k in range(8):
        x = 0.5 + 0.0625 * ((lane + k) & 7)
        for _ in range(iters):
            is_exp = kind == "exp" or (kind == "mixed" and k % 2 == 0)
            x = 2.0 ** (-x) if is_exp else x * 0.999 + 0.001
        ref += x
    got = out.cpu().double().numpy()
    assert np.allclose(got, ref, rtol=1e-5), np.max(np.abs(got - ref) / ref)
