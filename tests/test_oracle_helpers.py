"""The oracle's batch helpers against its plain entry point (CPU only).

``oracle.scan_channels`` checks every full-size GPU parity case (it scans
sampled channels one by one) and ``oracle.scan_threaded`` checks whole
outputs and produces the CPU baseline (it scans disjoint channel ranges on
threads).  Both only slice and view arrays before calling the same C loop
as ``oracle.scan``, so their results must equal ``oracle.scan`` bit for bit
on every channel; an indexing slip (a wrong batch row of B or C, a channel
range off by one, a per-channel parameter taken from the wrong channel, h0
or z of another channel) breaks that equality.  The shapes are ragged (no
dimension a multiple of the thread count or of the piece size) and every
optional input is tried present and absent.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle


def _inputs(seed, batch, dim, N, L, with_D, with_z, with_bias, with_h0):
    r = np.random.default_rng(seed)
    inp = {
        "u": r.normal(size=(batch, dim, L)),
        "delta": r.normal(size=(batch, dim, L)),
        # distinct values per channel and state, so that a parameter read
        # from the wrong channel changes the result
        "A": -r.uniform(0.1, 4.0, size=(dim, N)),
        "B": r.normal(size=(batch, N, L)),
        "C": r.normal(size=(batch, N, L)),
        "D": r.normal(size=dim) if with_D else None,
        "z": r.normal(size=(batch, dim, L)) if with_z else None,
        "delta_bias": (np.log(np.expm1(r.uniform(1e-3, 1e-1, size=dim)))
                       if with_bias else None),
        "h0": r.normal(size=(batch, dim, N)) if with_h0 else None,
    }
    return inp


OPTIONALS = list(itertools.product([False, True], repeat=4))


def _args(inp):
    return (inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
            inp["z"], inp["delta_bias"])


@pytest.mark.parametrize("opts", OPTIONALS,
                         ids=lambda o: "D%d_z%d_bias%d_h0%d" % o)
def test_scan_threaded_equals_scan_bitwise(opts):
    batch, dim, N, L = 3, 23, 16, 37
    inp = _inputs(11, batch, dim, N, L, *opts)
    for sp, zoh in ((True, False), (False, True)):
        if not sp:
            # softplus off: a small positive step used as given (delta +
            # bias > 0), so the state stays finite
            bias = (0.0 if inp["delta_bias"] is None
                    else inp["delta_bias"][None, :, None])
            inp = dict(inp, delta=0.05 * np.abs(inp["delta"]) + 0.01 - bias)
        y, hf = oracle.scan(*_args(inp), sp, zoh, inp["h0"])
        assert np.all(np.isfinite(y)) and np.all(np.isfinite(hf))
        for threads in (1, 3, 8):
            yt, ht, used = oracle.scan_threaded(*_args(inp), sp, zoh,
                                                inp["h0"], threads=threads)
            assert used == threads
            assert np.array_equal(yt, y), (opts, sp, zoh, threads)
            assert np.array_equal(ht, hf), (opts, sp, zoh, threads)


@pytest.mark.parametrize("opts", OPTIONALS,
                         ids=lambda o: "D%d_z%d_bias%d_h0%d" % o)
def test_scan_channels_equals_scan_bitwise(opts):
    batch, dim, N, L = 3, 23, 16, 37
    inp = _inputs(12, batch, dim, N, L, *opts)
    y, hf = oracle.scan(*_args(inp), True, False, inp["h0"])
    # first and last channel, a repeated channel, unsorted order
    chans = [(2, 22), (0, 0), (1, 7), (2, 0), (0, 22), (1, 7), (1, 13)]
    for threads in (1, 4):
        yc, hc = oracle.scan_channels(*_args(inp), True, False, inp["h0"],
                                      channels=chans, threads=threads)
        assert yc.shape == (len(chans), L) and hc.shape == (len(chans), N)
        for k, (b, d) in enumerate(chans):
            assert np.array_equal(yc[k], y[b, d]), (opts, b, d, threads)
            assert np.array_equal(hc[k], hf[b, d]), (opts, b, d, threads)


def test_scan_channels_reads_torch_bf16_rows_exactly():
    """The GPU tests hand it bf16 torch tensors; the selected rows must be
    widened exactly (the same values oracle.scan reads from the whole
    tensor)."""
    batch, dim, N, L = 2, 9, 16, 50
    inp = _inputs(13, batch, dim, N, L, True, True, True, True)
    t = {k: (torch.from_numpy(v).float().to(torch.bfloat16)
             if k in ("u", "delta", "B", "C", "z") and v is not None
             else (None if v is None else torch.from_numpy(v).float()))
         for k, v in inp.items()}
    y, hf = oracle.scan(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                        t["z"], t["delta_bias"], True, False, t["h0"])
    chans = [(1, 8), (0, 3)]
    yc, hc = oracle.scan_channels(t["u"], t["delta"], t["A"], t["B"], t["C"],
                                  t["D"], t["z"], t["delta_bias"], True, False,
                                  t["h0"], channels=chans, threads=2)
    for k, (b, d) in enumerate(chans):
        assert np.array_equal(yc[k], y[b, d]) and np.array_equal(hc[k], hf[b, d])


def test_scan_threaded_more_threads_than_channels():
    inp = _inputs(14, 1, 3, 16, 20, True, True, True, True)
    y, hf = oracle.scan(*_args(inp), True, False, inp["h0"])
    yt, ht, _ = oracle.scan_threaded(*_args(inp), True, False, inp["h0"],
                                     threads=16)
    assert np.array_equal(yt, y) and np.array_equal(ht, hf)
