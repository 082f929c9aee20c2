"""Pins of the oracle's backward pass (oracle.scan_bwd) to things other than
itself.

* Central finite differences of the forward oracle (pinned on its own in
  test_oracle_pins.py): for a loss L = sum(dy * y) + sum(dh_final * h_final),
  every element of every input is nudged both ways and the slope compared
  with the analytic gradient.  A dropped chain-rule term, a wrong sign or a
  transposed index changes at least one slope.
* Exact linearity identities at a larger size, where differencing every
  element would be slow: with the steps, A, D and z held fixed, y and h_final
  are jointly linear in (u, h0), and jointly linear in (B, h0) and in C up to
  terms that do not depend on them, so L equals the inner product of those
  inputs with their gradients (Euler's theorem for homogeneous functions of
  degree one).
"""
import numpy as np
import pytest

import oracle


def loss(inp, dy, dhf):
    y, hf = oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                        inp["D"], inp["z"], inp["delta_bias"],
                        inp["delta_softplus"], inp.get("zoh_b", False),
                        inp["h0"])
    return float(np.sum(dy * y) + (np.sum(dhf * hf) if dhf is not None else 0.0))


def make(seed, batch, dim, N, L, softplus=True, with_z=True, with_D=True,
         with_bias=True, with_h0=True):
    r = np.random.default_rng(seed)
    inp = {
        "u": r.normal(size=(batch, dim, L)),
        "delta": (r.normal(size=(batch, dim, L)) if softplus
                  else r.uniform(0.05, 0.4, size=(batch, dim, L))),
        "A": -r.uniform(0.3, 3.0, size=(dim, N)),
        "B": r.normal(size=(batch, N, L)),
        "C": r.normal(size=(batch, N, L)),
        "D": r.normal(size=dim) if with_D else None,
        "z": r.normal(size=(batch, dim, L)) if with_z else None,
        "delta_bias": r.normal(scale=0.5, size=dim) if with_bias else None,
        "h0": r.normal(size=(batch, dim, N)) if with_h0 else None,
        "delta_softplus": softplus,
    }
    dy = r.normal(size=(batch, dim, L))
    dhf = r.normal(size=(batch, dim, N))
    return inp, dy, dhf


def grads(inp, dy, dhf):
    return oracle.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"],
                           inp["C"], inp["D"], inp["z"], inp["delta_bias"],
                           inp["delta_softplus"], inp["h0"], dy, dhf,
                           zoh_b=inp.get("zoh_b", False))


GRAD_OF = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC",
           "D": "dD", "z": "dz", "delta_bias": "ddelta_bias", "h0": "dh0"}

VARIANTS = [
    dict(softplus=True, with_z=True, with_D=True, with_bias=True, with_h0=True),
    dict(softplus=False, with_z=False, with_D=False, with_bias=False,
         with_h0=False),
    dict(softplus=True, with_z=True, with_D=False, with_bias=False,
         with_h0=True),
]


def _zoh_case(inp):
    """Exact zero-order hold, with an A = 0 column (the Euler limit, dc/dA =
    dt^2/2) and a column small enough that |dt*A| < 1e-3 (the series branch
    of dc/dA)."""
    inp["zoh_b"] = True
    inp["A"][:, 0] = 0.0
    inp["A"][:, 1] = -2e-4
    return inp


@pytest.mark.parametrize("variant,zoh", [(v, False) for v in VARIANTS] +
                         [(VARIANTS[0], True), (VARIANTS[1], True)],
                         ids=["all", "bare", "mixed", "zoh_all", "zoh_bare"])
def test_finite_differences_every_element(variant, zoh):
    inp, dy, dhf = make(11, 2, 3, 4, 6, **variant)
    if zoh:
        inp = _zoh_case(inp)
    g = grads(inp, dy, dhf)
    eps = 1e-5
    for name, gname in GRAD_OF.items():
        if inp[name] is None:
            assert gname not in g or name == "h0"
            continue
        x = inp[name]
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = loss(inp, dy, dhf)
            x[idx] = keep - eps
            lm = loss(inp, dy, dhf)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - g[gname]) / (1.0 + np.abs(g[gname])))
        assert err < 1e-7, "%s: max scaled error %.3g" % (name, err)


def test_finite_differences_without_final_state_gradient():
    inp, dy, _ = make(12, 1, 2, 3, 5)
    g = grads(inp, dy, None)
    eps = 1e-5
    for name in ("u", "delta", "A", "h0"):
        x = inp[name]
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = loss(inp, dy, None)
            x[idx] = keep - eps
            lm = loss(inp, dy, None)
            x[idx] = keep
            fd = (lp - lm) / (2 * eps)
            an = g[GRAD_OF[name]][idx]
            assert abs(fd - an) < 1e-7 * (1.0 + abs(an)), (name, idx, fd, an)


def _dot(a, b):
    return float(np.sum(a * b))


def test_linearity_in_u_and_h0():
    """L(u, h0) = <du, u> + <dh0, h0> with steps, A, B, C, D, z fixed."""
    inp, dy, dhf = make(13, 2, 6, 16, 200)
    g = grads(inp, dy, dhf)
    lhs = loss(inp, dy, dhf)
    rhs = _dot(g["du"], inp["u"]) + _dot(g["dh0"], inp["h0"])
    assert abs(lhs - rhs) <= 1e-10 * (abs(lhs) + 1.0)


def test_linearity_in_B_and_h0():
    """h is jointly linear in (B, h0); the D skip does not depend on them."""
    inp, dy, dhf = make(14, 2, 6, 16, 200)
    g = grads(inp, dy, dhf)
    y, _ = oracle.scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                       inp["D"], inp["z"], inp["delta_bias"], True, False,
                       inp["h0"])
    s = inp["z"] / (1.0 + np.exp(-inp["z"]))
    skip = _dot(dy * s, inp["D"][None, :, None] * inp["u"])
    lhs = loss(inp, dy, dhf) - skip
    rhs = _dot(g["dB"], inp["B"]) + _dot(g["dh0"], inp["h0"])
    assert abs(lhs - rhs) <= 1e-10 * (abs(lhs) + 1.0)


def test_linearity_in_C():
    """With no final-state gradient, y is linear in C plus the D skip."""
    inp, dy, _ = make(15, 2, 6, 16, 200)
    g = grads(inp, dy, None)
    s = inp["z"] / (1.0 + np.exp(-inp["z"]))
    skip = _dot(dy * s, inp["D"][None, :, None] * inp["u"])
    lhs = loss(inp, dy, None) - skip
    assert abs(lhs - _dot(g["dC"], inp["C"])) <= 1e-10 * (abs(lhs) + 1.0)


def test_gate_gradient_is_zero_where_output_vanishes():
    """C = 0 and D = 0 give y = 0 for every z, so dz = 0 and dC = gc * h."""
    inp, dy, _ = make(16, 1, 3, 4, 20)
    inp["C"][:] = 0.0
    inp["D"][:] = 0.0
    g = grads(inp, dy, None)
    assert np.all(g["dz"] == 0.0)
    assert np.all(g["du"] == 0.0) and np.all(g["dA"] == 0.0)


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
def test_zoh_linearity_in_u_and_h0(zoh):
    """The exact-ZOH input term is linear in u as well: L(u, h0) = <du, u>
    + <dh0, h0> with steps, A, B, C, D, z fixed (A with a zero column)."""
    inp, dy, dhf = make(17, 2, 5, 16, 150)
    if zoh:
        inp = _zoh_case(inp)
    g = grads(inp, dy, dhf)
    lhs = loss(inp, dy, dhf)
    rhs = _dot(g["du"], inp["u"]) + _dot(g["dh0"], inp["h0"])
    assert abs(lhs - rhs) <= 1e-10 * (abs(lhs) + 1.0)


def test_zoh_gradients_tend_to_euler_as_A_vanishes():
    """For A -> 0 the ZOH coefficient (exp(dt A) - 1)/A tends to the Euler
    coefficient dt, so every gradient but dA tends to the Euler one; at |A|
    = 1e-9 they agree to ~1e-9 (the first-order term dt^2 A / 2).  dA does
    not: the ZOH coefficient still depends on A there (dc/dA -> dt^2/2),
    which the finite-difference pin checks at A = 0 exactly."""
    inp, dy, dhf = make(18, 1, 3, 4, 30)
    inp["A"][:] = -1e-9
    ge = grads(inp, dy, dhf)
    gz = grads(dict(inp, zoh_b=True), dy, dhf)
    for k in ge:
        if k == "dA":
            continue
        scale = 1.0 + np.max(np.abs(ge[k]))
        assert np.max(np.abs(gz[k] - ge[k])) <= 1e-7 * scale, k


# ------------------------------------------------- conv prologue gradients
@pytest.mark.parametrize("K,with_bias", [(4, True), (3, False), (1, True)],
                         ids=["k4_bias", "k3", "k1_bias"])
def test_conv_bwd_finite_differences_every_element(K, with_bias):
    """oracle.causal_conv1d_silu_bwd against central differences of the
    forward conv oracle (pinned to numpy.convolve) for L = sum du * u."""
    r = np.random.default_rng(30 + K)
    batch, dim, L = 2, 3, 9
    x = r.normal(size=(batch, dim, L))
    w = r.normal(size=(dim, K))
    b = r.normal(size=dim) if with_bias else None
    du = r.normal(size=(batch, dim, L))
    dx, dw, db = oracle.causal_conv1d_silu_bwd(x, w, b, du)

    def f():
        return float(np.sum(du * oracle.causal_conv1d_silu(x, w, b)))
    eps = 1e-6
    for arr, grad in ((x, dx), (w, dw)) + (((b, db),) if with_bias else ()):
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + eps
            lp = f()
            arr[idx] = keep - eps
            lm = f()
            arr[idx] = keep
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * (1.0 + abs(grad[idx])), (idx, fd, grad[idx])
    if not with_bias:
        assert db is None


def test_conv_then_scan_chain_rule_finite_differences():
    """The whole Mamba prologue + scan: y = scan(u = silu(conv(x))); the
    gradient with respect to x, the taps and the conv bias is the conv
    backward applied to the scan backward's du, checked by central
    differences of the composed forward oracles."""
    r = np.random.default_rng(41)
    batch, dim, N, L, K = 1, 2, 4, 7, 4
    x = r.normal(size=(batch, dim, L))
    w = r.normal(size=(dim, K)) * 0.5
    cb = r.normal(size=dim) * 0.1
    inp, dy, dhf = make(42, batch, dim, N, L)

    def f():
        u = oracle.causal_conv1d_silu(x, w, cb)
        y, hf = oracle.scan(u, inp["delta"], inp["A"], inp["B"], inp["C"],
                            inp["D"], inp["z"], inp["delta_bias"], True, False,
                            inp["h0"])
        return float(np.sum(dy * y) + np.sum(dhf * hf))
    u = oracle.causal_conv1d_silu(x, w, cb)
    g = oracle.scan_bwd(u, inp["delta"], inp["A"], inp["B"], inp["C"],
                        inp["D"], inp["z"], inp["delta_bias"], True,
                        inp["h0"], dy, dhf)
    dx, dw, db = oracle.causal_conv1d_silu_bwd(x, w, cb, g["du"])
    eps = 1e-6
    for arr, grad in ((x, dx), (w, dw), (cb, db)):
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + eps
            lp = f()
            arr[idx] = keep - eps
            lm = f()
            arr[idx] = keep
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * (1.0 + abs(grad[idx])), (idx, fd, grad[idx])
