"""Pins of the oracle's Mamba-2 SSD form (oracle.ssd, the O(L^2) masked
product y = (L o S) x) to things other than itself.

* The recurrence: a head with scalar decay A_h is the selective scan (the
  pinned Mamba-1 oracle, oracle.scan) on headdim channels that all carry
  the head's dt, bias and D, with A[d, n] = A_h for every state and the
  group's B and C.  The two oracles evaluate different formulas (a masked
  quadratic form vs a token-by-token recurrence) that must agree.
* Associativity: scanning [0, L) equals scanning [0, L1) and then [L1, L)
  from the first part's final state (checks the h0 and h_final terms).
* Attention form: with A = 0 and dt = 1 the decay mask is the plain causal
  mask, y = tril(C^T B) x (+ D x), a numpy matrix product.
"""
import numpy as np
import pytest

import oracle


def make(seed, batch, nheads, P, ngroups, N, L, softplus=True, with_D=True,
         with_z=True, with_bias=True, with_h0=True):
    r = np.random.default_rng(seed)
    return dict(
        x=r.normal(size=(batch, nheads, P, L)),
        dt=(r.normal(size=(batch, nheads, L)) if softplus
            else r.uniform(0.02, 0.3, size=(batch, nheads, L))),
        A=-r.uniform(0.2, 2.0, size=nheads),
        B=r.normal(size=(batch, ngroups, N, L)),
        C=r.normal(size=(batch, ngroups, N, L)),
        D=r.normal(size=nheads) if with_D else None,
        z=r.normal(size=(batch, nheads, P, L)) if with_z else None,
        dt_bias=r.normal(scale=0.5, size=nheads) if with_bias else None,
        h0=r.normal(size=(batch, nheads, P, N)) if with_h0 else None,
        dt_softplus=softplus)


def ssd(k, **over):
    a = dict(k)
    a.update(over)
    return oracle.ssd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"],
                      a["dt_bias"], a["dt_softplus"], a["h0"])


def as_scan(k):
    """The same computation laid out for the Mamba-1 oracle."""
    x = k["x"]
    batch, nheads, P, L = x.shape
    ngroups, N = k["B"].shape[1], k["B"].shape[2]
    hpg = nheads // ngroups
    u = x.reshape(batch, nheads * P, L)
    delta = np.repeat(k["dt"], P, axis=1)
    A = np.repeat(k["A"], P)[:, None] * np.ones((1, N))
    y = np.empty((batch, nheads * P, L))
    hf = np.empty((batch, nheads * P, N))
    for h in range(nheads):
        g = h // hpg
        sl = slice(h * P, (h + 1) * P)
        yh, hh = oracle.scan(
            u[:, sl], delta[:, sl], A[sl], k["B"][:, g], k["C"][:, g],
            None if k["D"] is None else np.full(P, k["D"][h]),
            None if k["z"] is None else k["z"][:, h],
            None if k["dt_bias"] is None else np.full(P, k["dt_bias"][h]),
            k["dt_softplus"], False,
            None if k["h0"] is None else k["h0"][:, h])
        y[:, sl] = yh
        hf[:, sl] = hh
    return y.reshape(x.shape), hf.reshape(batch, nheads, P, N)


def scaled(a, b):
    return float(np.max(np.abs(a - b) / (np.abs(b) + np.sqrt(np.mean(b * b)))))


VARIANTS = [
    dict(ngroups=1),
    dict(ngroups=2),
    dict(ngroups=1, softplus=False, with_D=False, with_z=False,
         with_bias=False, with_h0=False),
    dict(ngroups=4, with_h0=False),
]


@pytest.mark.parametrize("v", VARIANTS, ids=["g1", "g2", "bare", "g4"])
def test_quadratic_form_equals_recurrence(v):
    v = dict(v)
    ng = v.pop("ngroups")
    k = make(21, 2, 4, 3, ng, 8, 60, **v)
    y, hf = ssd(k)
    yr, hr = as_scan(k)
    assert scaled(y, yr) < 1e-11
    assert scaled(hf, hr) < 1e-11


def test_split_and_resume():
    k = make(22, 1, 2, 4, 1, 6, 50)
    y, hf = ssd(k)
    L1 = 23
    first = {**k, "x": k["x"][..., :L1], "dt": k["dt"][..., :L1],
             "B": k["B"][..., :L1], "C": k["C"][..., :L1], "z": k["z"][..., :L1]}
    y1, h1 = ssd(first)
    second = {**k, "x": k["x"][..., L1:], "dt": k["dt"][..., L1:],
              "B": k["B"][..., L1:], "C": k["C"][..., L1:], "z": k["z"][..., L1:],
              "h0": h1}
    y2, h2 = ssd(second)
    assert scaled(np.concatenate([y1, y2], axis=-1), y) < 1e-12
    assert scaled(h2, hf) < 1e-12


def test_no_decay_is_causal_attention():
    """A = 0, dt = 1: S = C^T B under the causal mask."""
    k = make(23, 1, 2, 3, 1, 5, 40, softplus=False, with_z=False,
             with_bias=False, with_h0=False)
    k["A"] = np.zeros(2)
    k["dt"] = np.ones_like(k["dt"])
    y, _ = ssd(k)
    Bm, Cm = k["B"][0, 0], k["C"][0, 0]          # (N, L)
    S = np.tril(Cm.T @ Bm)                       # (L, L): S[t, s] = C_t . B_s
    for h in range(2):
        ref = k["x"][0, h] @ S.T + k["D"][h] * k["x"][0, h]   # (P, L)
        assert scaled(y[0, h], ref) < 1e-12


def test_memoryless_limit():
    """A very negative: exp(A (cum_t - cum_s)) vanishes for s < t, so
    y_t = (C_t . B_t) dt_t x_t + D x_t."""
    k = make(24, 1, 1, 2, 1, 4, 30, softplus=False, with_z=False,
             with_bias=False, with_h0=False)
    k["A"] = np.array([-1e30])
    y, _ = ssd(k)
    cb = np.sum(k["C"][0, 0] * k["B"][0, 0], axis=0)           # (L,)
    ref = cb * k["dt"][0, 0] * k["x"][0, 0] + k["D"][0] * k["x"][0, 0]
    assert scaled(y[0, 0], ref) < 1e-14
