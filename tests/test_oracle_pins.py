"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test derives its expected values by a different route than the
oracle's token loop -- a library routine, a closed form, hand arithmetic or
brute-force products -- so that a dropped term, a wrong sign, a wrong index
or a transposed operand in the oracle fails at least one of them:

* convolution form of a time-invariant SSM (numpy.convolve and a direct
  O(L^2) sum): the johe.ru page, "SSM as Convolution"; the Guide Complet,
  section 2 (K = (CB, CAB, CA^2B, ...), y = K * u);
* a first-order IIR filter (scipy.signal.lfilter) for N = 1;
* A = 0 reduces the scan to a cumulative sum (numpy.cumsum);
* exp(dt*A) = 0 makes it memoryless;
* dt = 0 leaves the state unchanged (bitwise);
* C = 0 leaves only the gated skip D*u*silu(z) (scipy.special.expit);
* brute-force unrolling h_t = (prod a) h0 + sum (prod a) b with explicit
  products, the pscan contract of the Guide Complet's "Parallel Associative
  Scan" (h_k = A_k h_{k-1} + B_k);
* associativity: a split scan resumed from the first part's final state;
* L single steps equal one scan (the recurrent mode of "SSM as RNN");
* linearity in (u, h0) with the gate off;
* hand-worked examples in tests/golden/.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy import signal, special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def softplus_ref(x):
    return np.logaddexp(0.0, x)


# --------------------------------------------------------------- softplus
def test_softplus_matches_logaddexp():
    xs = np.concatenate([np.linspace(-60, 60, 2401),
                         [-800.0, -745.0, -40.0, -1e-8, 0.0, 1e-8, 40.0,
                          700.0, 800.0]])
    for x in xs:
        got = oracle.softplus(x)
        ref = float(softplus_ref(x))
        assert abs(got - ref) <= 4e-16 * max(abs(ref), 1e-300) or got == ref, x


def test_softplus_tiny_argument_keeps_precision():
    # log(1+e^x) = e^x - e^2x/2 + e^3x/3 - ... for x << 0; a naive
    # log(1 + exp(x)) returns 0 for all of these.
    for x in (-30.0, -50.0, -100.0, -700.0):
        e = math.exp(x)
        got = oracle.softplus(x)
        assert got > 0
        assert abs(got - (e - e * e / 2 + e ** 3 / 3)) <= 1e-15 * e


# ------------------------------------------------- time-invariant: conv form
def _time_invariant_case(seed, batch, dim, N, L, zoh=False, with_h0=True,
                         with_z=True):
    r = rng(seed)
    draw = r.normal(size=(dim,))                    # constant along t
    delta = np.repeat(draw[None, :, None], batch, 0).repeat(L, 2)
    bias = np.log(np.expm1(r.uniform(1e-3, 1e-1, size=dim)))
    A = -r.uniform(0.05, 3.0, size=(dim, N))
    Bv = r.normal(size=(batch, N))
    Cv = r.normal(size=(batch, N))
    B = np.repeat(Bv[:, :, None], L, 2)
    C = np.repeat(Cv[:, :, None], L, 2)
    u = r.normal(size=(batch, dim, L))
    D = r.normal(size=dim)
    z = r.normal(size=(batch, dim, L)) if with_z else None
    h0 = r.normal(size=(batch, dim, N)) if with_h0 else None
    return dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, delta_bias=bias,
                h0=h0, zoh=zoh, Bv=Bv, Cv=Cv, draw=draw)


def _conv_expected(case, method):
    u, A, D, z, h0 = case["u"], case["A"], case["D"], case["z"], case["h0"]
    batch, dim, L = u.shape
    N = A.shape[1]
    y = np.empty_like(u)
    for b in range(batch):
        for d in range(dim):
            dt = softplus_ref(case["draw"][d] + case["delta_bias"][d])
            abar = np.exp(dt * A[d])                              # (N,)
            if case["zoh"]:
                bbar = np.expm1(dt * A[d]) / A[d] * case["Bv"][b]
            else:
                bbar = dt * case["Bv"][b]
            powers = abar[None, :] ** np.arange(L + 1)[:, None]   # (L+1, N)
            K = powers[:L] @ (case["Cv"][b] * bbar)               # K_i
            if method == "convolve":
                yc = np.convolve(u[b, d], K)[:L]
            else:
                yc = np.array([sum(K[i] * u[b, d, t - i] for i in range(t + 1))
                               for t in range(L)])
            if h0 is not None:
                yc = yc + powers[1:] @ (case["Cv"][b] * h0[b, d])
            yc = yc + D[d] * u[b, d]
            if z is not None:
                yc = yc * z[b, d] * special.expit(z[b, d])
            y[b, d] = yc
    return y


@pytest.mark.parametrize("method", ["convolve", "direct"])
@pytest.mark.parametrize("zoh", [False, True])
def test_time_invariant_equals_convolution(method, zoh):
    case = _time_invariant_case(11 + zoh, batch=2, dim=3, N=5, L=64, zoh=zoh)
    y, _ = oracle.scan(case["u"], case["delta"], case["A"], case["B"],
                       case["C"], case["D"], case["z"], case["delta_bias"],
                       True, zoh, case["h0"])
    ref = _conv_expected(case, method)
    scale = np.abs(ref).max()
    assert np.max(np.abs(y - ref)) <= 1e-12 * scale


def test_time_invariant_final_state_closed_form():
    case = _time_invariant_case(5, batch=1, dim=2, N=4, L=40, with_z=False)
    _, hf = oracle.scan(case["u"], case["delta"], case["A"], case["B"],
                        case["C"], case["D"], None, case["delta_bias"], True,
                        False, case["h0"])
    L = case["u"].shape[2]
    for d in range(2):
        dt = softplus_ref(case["draw"][d] + case["delta_bias"][d])
        a = np.exp(dt * case["A"][d])
        ref = a ** L * case["h0"][0, d]
        for s in range(L):
            ref = ref + a ** (L - 1 - s) * dt * case["Bv"][0] * case["u"][0, d, s]
        assert np.allclose(hf[0, d], ref, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ N = 1: lfilter
def test_single_state_is_first_order_iir_filter():
    r = rng(3)
    L = 500
    u = r.normal(size=(1, 1, L))
    dt = 0.37
    a_cont = -1.3
    alpha, beta = math.exp(dt * a_cont), dt * 0.8
    A = np.array([[a_cont]])
    B = np.full((1, 1, L), 0.8)
    C = np.full((1, 1, L), -1.7)
    D = np.array([0.25])
    y, hf = oracle.scan(u, np.full((1, 1, L), dt), A, B, C, D, None, None,
                        False, False, None)
    h = signal.lfilter([beta], [1.0, -alpha], u[0, 0])
    ref = -1.7 * h + 0.25 * u[0, 0]
    assert np.max(np.abs(y[0, 0] - ref)) <= 1e-12 * np.abs(ref).max()
    assert abs(hf[0, 0, 0] - h[-1]) <= 1e-12 * abs(h).max()


# --------------------------------------------------------------- A = 0
def test_zero_A_is_cumulative_sum():
    r = rng(4)
    batch, dim, N, L = 2, 3, 4, 300
    u = r.normal(size=(batch, dim, L))
    draw = r.normal(size=(batch, dim, L))
    B = r.normal(size=(batch, N, L))
    C = r.normal(size=(batch, N, L))
    h0 = r.normal(size=(batch, dim, N))
    A = np.zeros((dim, N))
    y, hf = oracle.scan(u, draw, A, B, C, None, None, None, True, False, h0)
    dt = softplus_ref(draw)
    for b in range(batch):
        for d in range(dim):
            h = h0[b, d][:, None] + np.cumsum(dt[b, d] * B[b] * u[b, d], axis=1)
            ref = np.sum(C[b] * h, axis=0)
            assert np.allclose(y[b, d], ref, rtol=1e-12, atol=1e-12)
            assert np.allclose(hf[b, d], h[:, -1], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- memoryless dA = 0
def test_huge_negative_A_is_memoryless():
    r = rng(6)
    batch, dim, N, L = 2, 4, 16, 50
    u = r.normal(size=(batch, dim, L))
    draw = r.normal(size=(batch, dim, L))
    B = r.normal(size=(batch, N, L))
    C = r.normal(size=(batch, N, L))
    D = r.normal(size=dim)
    A = np.full((dim, N), -1e30)
    bias = np.full(dim, 1.0)
    h0 = r.normal(size=(batch, dim, N))
    y, hf = oracle.scan(u, draw, A, B, C, D, None, bias, True, False, h0)
    dt = softplus_ref(draw + 1.0)
    for b in range(batch):
        cb = np.sum(C[b] * B[b], axis=0)                 # (L,)
        for d in range(dim):
            ref = dt[b, d] * u[b, d] * cb + D[d] * u[b, d]
            assert np.allclose(y[b, d], ref, rtol=1e-13, atol=1e-14)
            assert np.allclose(hf[b, d], dt[b, d, -1] * B[b, :, -1] * u[b, d, -1],
                               rtol=1e-14, atol=1e-15)


# ----------------------------------------------------------- dt = 0 invariant
@pytest.mark.parametrize("mode", ["raw_zero", "softplus_underflow"])
def test_zero_step_keeps_state(mode):
    r = rng(7)
    batch, dim, N, L = 2, 3, 16, 40
    u = r.normal(size=(batch, dim, L))
    B = r.normal(size=(batch, N, L))
    C = r.normal(size=(batch, N, L))
    D = r.normal(size=dim)
    z = r.normal(size=(batch, dim, L))
    h0 = r.normal(size=(batch, dim, N))
    A = -np.arange(1, N + 1, dtype=float)[None].repeat(dim, 0)
    if mode == "raw_zero":
        draw, sp = np.zeros((batch, dim, L)), False
    else:
        draw, sp = np.full((batch, dim, L), -800.0), True
    y, hf = oracle.scan(u, draw, A, B, C, D, z, None, sp, False, h0)
    assert np.array_equal(hf, h0)
    for b in range(batch):
        for d in range(dim):
            ref = (h0[b, d] @ C[b] + D[d] * u[b, d]) * z[b, d] * special.expit(z[b, d])
            assert np.allclose(y[b, d], ref, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------ C = 0: gate
def test_zero_C_leaves_gated_skip():
    r = rng(8)
    batch, dim, N, L = 2, 5, 16, 33
    u = r.normal(size=(batch, dim, L))
    draw = r.normal(size=(batch, dim, L))
    z = 4 * r.normal(size=(batch, dim, L))
    D = r.normal(size=dim)
    A = -np.arange(1, N + 1, dtype=float)[None].repeat(dim, 0)
    B = r.normal(size=(batch, N, L))
    y, _ = oracle.scan(u, draw, A, B, np.zeros((batch, N, L)), D, z, None,
                       True, False, None)
    ref = D[None, :, None] * u * z * special.expit(z)
    assert np.allclose(y, ref, rtol=1e-15, atol=1e-15)


# ------------------------------------------------------- brute-force unroll
@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), batch=st.integers(1, 2),
       dim=st.integers(1, 4), N=st.sampled_from([1, 4, 16]),
       L=st.integers(1, 32), zoh=st.booleans(), gate=st.booleans())
def test_brute_force_products(seed, batch, dim, N, L, zoh, gate):
    r = rng(seed)
    u = r.normal(size=(batch, dim, L))
    draw = r.normal(size=(batch, dim, L))
    bias = r.normal(size=dim) - 2
    A = -r.uniform(0.01, 4.0, size=(dim, N))
    B = r.normal(size=(batch, N, L))
    C = r.normal(size=(batch, N, L))
    D = r.normal(size=dim)
    z = r.normal(size=(batch, dim, L)) if gate else None
    h0 = r.normal(size=(batch, dim, N))
    y, hf = oracle.scan(u, draw, A, B, C, D, z, bias, True, zoh, h0)
    for b in range(batch):
        for d in range(dim):
            dt = softplus_ref(draw[b, d] + bias[d])                  # (L,)
            a = np.exp(dt[:, None] * A[d][None, :])                   # (L, N)
            coef = (np.expm1(dt[:, None] * A[d][None, :]) / A[d][None, :]
                    if zoh else dt[:, None] * np.ones((1, N)))
            bb = coef * B[b].T * u[b, d][:, None]                     # (L, N)
            for t in range(L):
                h = np.prod(a[:t + 1], axis=0) * h0[b, d]
                for s in range(t + 1):
                    h = h + np.prod(a[s + 1:t + 1], axis=0) * bb[s]
                yt = np.dot(C[b, :, t], h) + D[d] * u[b, d, t]
                if gate:
                    yt *= z[b, d, t] * special.expit(z[b, d, t])
                assert abs(y[b, d, t] - yt) <= 1e-12 * (1 + abs(yt))
                if t == L - 1:
                    assert np.allclose(hf[b, d], h, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ associativity
@pytest.mark.parametrize("split", [1, 17, 99])
def test_split_scan_resumes_bitwise(split):
    r = rng(9)
    batch, dim, N, L = 2, 3, 16, 100
    u = r.normal(size=(batch, dim, L))
    draw = r.normal(size=(batch, dim, L))
    bias = r.normal(size=dim)
    A = -np.arange(1, N + 1, dtype=float)[None].repeat(dim, 0)
    B = r.normal(size=(batch, N, L))
    C = r.normal(size=(batch, N, L))
    D = r.normal(size=dim)
    z = r.normal(size=(batch, dim, L))
    h0 = r.normal(size=(batch, dim, N))
    y, hf = oracle.scan(u, draw, A, B, C, D, z, bias, True, False, h0)
    s0, s1 = slice(0, split), slice(split, L)
    y1, h1 = oracle.scan(u[..., s0], draw[..., s0], A, B[..., s0], C[..., s0],
                         D, z[..., s0], bias, True, False, h0)
    y2, h2 = oracle.scan(u[..., s1], draw[..., s1], A, B[..., s1], C[..., s1],
                         D, z[..., s1], bias, True, False, h1)
    assert np.array_equal(np.concatenate([y1, y2], axis=2), y)
    assert np.array_equal(h2, hf)


# -------------------------------------------------------- steps == one scan
@pytest.mark.parametrize("zoh", [False, True])
def test_single_steps_equal_scan(zoh):
    r = rng(10)
    batch, dim, N, L = 3, 4, 16, 24
    u = r.normal(size=(batch, dim, L))
    draw = r.normal(size=(batch, dim, L))
    bias = r.normal(size=dim)
    A = -np.arange(1, N + 1, dtype=float)[None].repeat(dim, 0)
    B = r.normal(size=(batch, N, L))
    C = r.normal(size=(batch, N, L))
    D = r.normal(size=dim)
    z = r.normal(size=(batch, dim, L))
    h0 = r.normal(size=(batch, dim, N))
    y, hf = oracle.scan(u, draw, A, B, C, D, z, bias, True, zoh, h0)
    state = h0.copy()
    for t in range(L):
        yt = oracle.step(state, u[:, :, t], draw[:, :, t], A, B[:, :, t],
                         C[:, :, t], D, z[:, :, t], bias, True, zoh)
        assert np.array_equal(yt, y[:, :, t])
    assert np.array_equal(state, hf)


# ---------------------------------------------------------------- linearity
def test_linear_in_input_and_initial_state():
    r = rng(12)
    batch, dim, N, L = 2, 3, 8, 60
    draw = r.normal(size=(batch, dim, L))
    A = -r.uniform(0.1, 2, size=(dim, N))
    B = r.normal(size=(batch, N, L))
    C = r.normal(size=(batch, N, L))
    D = r.normal(size=dim)
    u1, u2 = r.normal(size=(2, batch, dim, L))
    g1, g2 = r.normal(size=(2, batch, dim, N))
    al, be = 1.7, -0.6
    ya, ha = oracle.scan(al * u1 + be * u2, draw, A, B, C, D, None, None,
                         True, False, al * g1 + be * g2)
    y1, h1 = oracle.scan(u1, draw, A, B, C, D, None, None, True, False, g1)
    y2, h2 = oracle.scan(u2, draw, A, B, C, D, None, None, True, False, g2)
    assert np.allclose(ya, al * y1 + be * y2, rtol=1e-13, atol=1e-13)
    assert np.allclose(ha, al * h1 + be * h2, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------- NaN propagation
def test_nan_input_propagates_forward():
    r = rng(13)
    batch, dim, N, L = 1, 2, 4, 20
    u = r.normal(size=(batch, dim, L))
    u[0, 1, 7] = np.nan
    draw = r.normal(size=(batch, dim, L))
    A = -np.arange(1, N + 1, dtype=float)[None].repeat(dim, 0)
    B = r.normal(size=(batch, N, L))
    C = r.normal(size=(batch, N, L))
    y, hf = oracle.scan(u, draw, A, B, C, None, None, None, True, False, None)
    assert np.all(np.isfinite(y[0, 0])) and np.all(np.isfinite(y[0, 1, :7]))
    assert np.all(np.isnan(y[0, 1, 7:])) and np.all(np.isnan(hf[0, 1]))


# ------------------------------------------------------------ golden files
def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_golden_hand_worked_scan():
    g = _load_golden("hand_worked_n2_l3.json")
    i = g["inputs"]
    y, hf = oracle.scan(np.array(i["u"]), np.array(i["delta"]),
                        np.array(i["A"]), np.array(i["B"]), np.array(i["C"]),
                        np.array(i["D"]), None, None, i["delta_softplus"],
                        False, np.array(i["h0"]))
    tol = g["tolerance"]
    assert np.allclose(y, g["expected"]["y"], rtol=tol, atol=tol)
    assert np.allclose(hf, g["expected"]["h_final"], rtol=tol, atol=tol)
    # the same example one token at a time
    state = np.array(i["h0"], dtype=np.float64)
    for t in range(3):
        yt = oracle.step(state, np.array(i["u"])[:, :, t],
                         np.array(i["delta"])[:, :, t], np.array(i["A"]),
                         np.array(i["B"])[:, :, t], np.array(i["C"])[:, :, t],
                         np.array(i["D"]), None, None, False, False)
        assert abs(yt[0, 0] - g["expected"]["y"][0][0][t]) <= tol * 8


def test_golden_hand_worked_gate_and_zoh():
    g = _load_golden("hand_worked_gate_zoh.json")
    i = g["inputs"]
    y, hf = oracle.scan(np.array(i["u"]), np.array(i["delta"]),
                        np.array(i["A"]), np.array(i["B"]), np.array(i["C"]),
                        np.array(i["D"]), np.array(i["z"]), None,
                        i["delta_softplus"], i["zoh_b"], None)
    ln2, ln3 = math.log(2.0), math.log(3.0)
    ref_y = [0.0, (5 / (2 * ln2) + 2) * 0.75 * ln3]
    ref_h = 5 / (4 * ln2)
    tol = g["tolerance"]
    assert abs(y[0, 0, 0]) <= tol
    assert abs(y[0, 0, 1] - ref_y[1]) <= tol * abs(ref_y[1])
    assert abs(hf[0, 0, 0] - ref_h) <= tol * ref_h


# ------------------------------------------------------- argument checking
def test_oracle_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.scan(np.zeros((1, 2, 3)), np.zeros((1, 2, 4)), np.zeros((2, 4)),
                    np.zeros((1, 4, 3)), np.zeros((1, 4, 3)))


# ------------------------------------------ causal conv1d + SiLU prologue
@pytest.mark.parametrize("K", [1, 2, 4])
def test_causal_conv1d_silu_matches_numpy_convolve(K):
    r = rng(20 + K)
    batch, dim, L = 2, 5, 70
    x = r.normal(size=(batch, dim, L))
    w = r.normal(size=(dim, K))
    bias = r.normal(size=dim)
    u = oracle.causal_conv1d_silu(x, w, bias)
    for b in range(batch):
        for d in range(dim):
            # PyTorch-style cross-correlation with K-1 zeros of left padding
            # and the output trimmed to L is a full convolution with the
            # reversed taps, truncated to the first L samples.
            pre = np.convolve(x[b, d], w[d][::-1])[:L] + bias[d]
            ref = pre * special.expit(pre)
            assert np.allclose(u[b, d], ref, rtol=1e-13, atol=1e-14)


def test_causal_conv1d_is_causal_and_zero_padded():
    r = rng(31)
    x = r.normal(size=(1, 3, 40))
    w = r.normal(size=(3, 4))
    u1 = oracle.causal_conv1d_silu(x, w, None)
    x2 = x.copy()
    x2[..., 25:] = r.normal(size=(1, 3, 15))      # change only the future
    u2 = oracle.causal_conv1d_silu(x2, w, None)
    assert np.array_equal(u1[..., :25], u2[..., :25])
    # the first output sees only x[0] through the last tap
    pre0 = w[:, 3] * x[0, :, 0]
    assert np.allclose(u1[0, :, 0], pre0 * special.expit(pre0), rtol=1e-14)
