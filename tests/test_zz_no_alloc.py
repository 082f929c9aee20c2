"""ssm_scan_fwd_noalloc (the entry point for callers that cannot allocate)
against ssm_scan_fwd on the same inputs, called through the C ABI.

Both run the same kernels with the same chunk plan, so the results must be
bitwise equal; the split cases put the chunk states in the library's fixed
scratch.  Two calls in a row, the second with a smaller input, check that
the scratch's leftover contents from the first call do not leak into the
second.
"""
import ctypes

import pytest
import torch

import selective_state_space_30_amd as ssm
import synthetic as syn

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc(inp, chunk_len=0, stream=None):
    lib = ssm.load_library()
    batch, dim, L = inp["u"].shape
    y = torch.empty_like(inp["u"])
    hf = torch.empty(batch, dim, 16, device=DEV)
    code = ssm.SSM_DTYPE_BF16 if inp["u"].dtype == torch.bfloat16 else ssm.SSM_DTYPE_F32
    flags = ssm.SSM_FLAG_DELTA_SOFTPLUS if inp["delta_softplus"] else 0
    s = stream or torch.cuda.current_stream(DEV)
    st = lib.ssm_scan_fwd_noalloc(
        _p(inp["u"]), _p(inp["delta"]), _p(inp["A"]), _p(inp["B"]), _p(inp["C"]),
        _p(inp["D"]), _p(inp["z"]), _p(inp["delta_bias"]), flags, _p(inp["h0"]),
        _p(y), _p(hf), batch, dim, 16, L, code, chunk_len,
        ctypes.c_void_p(s.cuda_stream))
    assert st == 0, lib.ssm_last_error().decode()
    return y, hf


def with_workspace(inp, chunk_len=0):
    return ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"],
                            inp["C"], inp["D"], inp["z"], inp["delta_bias"],
                            inp["delta_softplus"], inp["h0"],
                            chunk_len=chunk_len)


def to_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}


def test_two_calls_in_a_row_second_smaller():
    big = to_dev(syn.make_scan_inputs(syn.TINY, "cpu", batch=2, dim=96,
                                      seqlen=20000, dtype="f32", with_h0=True,
                                      seed=41))
    small = to_dev(syn.make_scan_inputs(syn.TINY, "cpu", batch=1, dim=24,
                                        seqlen=9000, dtype="bf16",
                                        with_h0=True, seed=42))
    # the big call's chunk states fill more of the scratch than the small
    # call writes
    assert (ssm.ssm_scan_workspace_size(2, 96, 16, 20000, 4096) >
            ssm.ssm_scan_workspace_size(1, 24, 16, 9000, 2048) > 0)
    y1, h1 = noalloc(big, chunk_len=4096)
    y2, h2 = noalloc(small, chunk_len=2048)
    torch.cuda.synchronize()
    r1 = with_workspace(big, chunk_len=4096)
    r2 = with_workspace(small, chunk_len=2048)
    torch.cuda.synchronize()
    assert torch.equal(y1, r1[0]) and torch.equal(h1, r1[1])
    assert torch.equal(y2, r2[0]) and torch.equal(h2, r2[1])


def test_long_context_workload_then_a_whole_sequence():
    """The long-context workload (split by the automatic plan into chunks
    whose states fill 1.6 MB of the scratch), then an unsplit call."""
    cfg = syn.LONG_1M
    assert 0 < ssm.ssm_scan_workspace_size(cfg.batch, cfg.dim, 16,
                                           cfg.seqlen) <= ssm.SCAN_SCRATCH_BYTES
    inp = syn.make_scan_inputs(cfg, DEV)
    y, h = noalloc(inp)
    torch.cuda.synchronize()
    ry, rh = with_workspace(inp)
    torch.cuda.synchronize()
    assert torch.equal(y, ry) and torch.equal(h, rh)
    del inp, y, h, ry, rh
    torch.cuda.empty_cache()
    small = to_dev(syn.make_scan_inputs(syn.TINY, "cpu", batch=2, dim=40,
                                        seqlen=3000, dtype="f32", seed=43))
    y, h = noalloc(small)
    torch.cuda.synchronize()
    ry, rh = with_workspace(small)
    torch.cuda.synchronize()
    assert torch.equal(y, ry) and torch.equal(h, rh)


def test_oversized_split_is_refused():
    lib = ssm.load_library()
    inp = to_dev(syn.make_scan_inputs(syn.TINY, "cpu", batch=1, dim=8,
                                      seqlen=2048, dtype="f32", seed=44))
    y, h = noalloc(inp, chunk_len=1024)  # fits
    torch.cuda.synchronize()
    ry, rh = with_workspace(inp, chunk_len=1024)
    torch.cuda.synchronize()
    assert torch.equal(y, ry) and torch.equal(h, rh)
    # a shape whose split needs more than the fixed scratch: refused before
    # any HIP call (the pointers are never dereferenced)
    fake = 0x7F0000000000
    st = lib.ssm_scan_fwd_noalloc(
        fake, fake + (1 << 40), fake + (2 << 40), fake + (3 << 40),
        fake + (4 << 40), None, None, None, 1, None, fake + (5 << 40), None,
        64, 1024, 16, 128 * 1024, ssm.SSM_DTYPE_F32, 1024, None)
    assert st == 3, lib.ssm_last_error().decode()
