"""Calls on a stream other than torch's current one.

The binding allocates outputs and workspaces with torch; the kernels run on
the ``stream`` argument.  Those allocations must belong to that stream, or
the caching allocator may hand a workspace freed at the end of the call to
work on the current stream while the kernels still use it.
"""
import pytest
import torch

import selective_state_space_30_amd as ssm
import synthetic as syn

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inputs():
    inp = syn.make_scan_inputs(syn.TINY, "cpu", batch=2, dim=64, seqlen=16384,
                               dtype="f32", with_h0=True, seed=21)
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}


def _record_allocations(monkeypatch):
    seen = []
    real = torch.empty

    def empty(*a, **kw):
        t = real(*a, **kw)
        if t.is_cuda:
            seen.append(torch.cuda.current_stream(t.device).cuda_stream)
        return t
    monkeypatch.setattr(torch, "empty", empty)
    return seen


def test_allocations_belong_to_the_launch_stream(monkeypatch):
    inp = _inputs()
    side = torch.cuda.Stream()
    dy = torch.randn_like(inp["u"])
    seen = _record_allocations(monkeypatch)
    ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                     inp["D"], inp["z"], inp["delta_bias"], True, inp["h0"],
                     chunk_len=4096, stream=side)
    ssm.ssm_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                     inp["D"], inp["z"], inp["delta_bias"], True, inp["h0"],
                     dy, None, stream=side)
    torch.cuda.synchronize()
    assert seen and all(s == side.cuda_stream for s in seen), seen


def test_side_stream_results_survive_reuse_on_the_current_stream():
    inp = _inputs()
    dy = torch.randn_like(inp["u"])
    args = (inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
            inp["z"], inp["delta_bias"], True, inp["h0"])
    y_ref, h_ref = ssm.ssm_scan_fwd(*args, chunk_len=4096)
    g_ref = ssm.ssm_scan_bwd(*args, dy, None)
    torch.cuda.synchronize()
    ws = max(ssm.ssm_scan_workspace_size(2, 64, 16, 16384, 4096),
             ssm.ssm_scan_bwd_workspace_size(2, 64, 16, 16384, torch.float32))
    side = torch.cuda.Stream()
    # keep the side stream busy first, so its kernels run while the current
    # stream allocates and overwrites memory below
    big = torch.ones(1 << 26, device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(40):
            big.mul_(1.0001)
    y, h = ssm.ssm_scan_fwd(*args, chunk_len=4096, stream=side)
    g = ssm.ssm_scan_bwd(*args, dy, None, stream=side)
    for _ in range(20):
        t = torch.empty(ws, dtype=torch.uint8, device=DEV)
        t.fill_(0xFF)
        del t
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(h, h_ref)
    for k in g_ref:
        assert torch.equal(g[k], g_ref[k]), k
    del big
