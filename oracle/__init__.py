"""fp64 CPU oracle for the selective SSM scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it shares no code
with them.

The arithmetic lives in plain C (``ssm_oracle.c``, fp64, one channel, token
and state at a time).  This module only marshals numpy arrays into it:

* :func:`scan` -- the full sequential scan, the per-token loop of the S6
  forward in "Mamba & State Space Models - Guide Complet", section 4, with the
  Euler input term of "SSM as RNN" on the johe.ru page (or exact ZOH from the
  Guide's section 1 when ``zoh_b=True``) and the ``y * silu(gate)`` output of
  that page's "Selective SSM" section.
* :func:`step` -- one token of the same recurrence, the recurrent (decoding)
  mode.
* :func:`causal_conv1d_silu` -- the depthwise causal convolution and SiLU
  that produce the scan's input u inside the Mamba block (the Guide
  Complet's section 4 architecture figure and section 7 block).
* :func:`causal_conv1d_silu_bwd` -- its gradients with respect to x, the
  taps and the conv bias.
* :func:`scan_bwd` -- gradients of :func:`scan` (Euler or exact-ZOH input
  term) by the chain rule through the recurrence, in reverse token order.
* :func:`ssd` -- the Mamba-2 "state space dual" form with one scalar decay
  per head: the masked matrix product y = (L o S) x of the Guide Complet's
  section 5, computed directly.
* :func:`scan_threaded` -- the same scan run on disjoint channel ranges from
  several Python threads (ctypes releases the GIL), used to time the oracle on
  all host cores.  It does not change the arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile ``ssm_oracle.c`` with gcc into ``liboracle.so`` (in-tree)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or (
                os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.oracle_scan_f64.argtypes = [P, P, P, P, P, P, P, P, I, I, P, P, P,
                                        I64, I64, I64, I64]
        lib.oracle_scan_f64.restype = I
        lib.oracle_step_f64.argtypes = [P, P, P, P, P, P, P, P, P, I, I, P,
                                        I64, I64, I64]
        lib.oracle_step_f64.restype = I
        lib.oracle_softplus.argtypes = [ctypes.c_double]
        lib.oracle_softplus.restype = ctypes.c_double
        lib.oracle_causal_conv1d_silu_f64.argtypes = [P, P, P, I64, P, I64,
                                                      I64, I64]
        lib.oracle_causal_conv1d_silu_f64.restype = I
        lib.oracle_causal_conv1d_silu_bwd_f64.argtypes = [P, P, P, I64, P, P,
                                                          P, P, I64, I64, I64]
        lib.oracle_causal_conv1d_silu_bwd_f64.restype = I
        lib.oracle_scan_bwd_f64.argtypes = [P] * 8 + [I, I] + [P] * 12 + [I64] * 4
        lib.oracle_scan_bwd_f64.restype = I
        lib.oracle_ssd_f64.argtypes = [P] * 8 + [I] + [P] * 3 + [I64] * 6
        lib.oracle_ssd_f64.restype = I
        _lib = lib
        return lib


def _f64(a, shape=None):
    if a is None:
        return None
    if hasattr(a, "detach"):  # a torch tensor: exact widening to fp64 on host
        a = a.detach().to("cpu").double().numpy()
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("oracle: expected shape %s, got %s" % (shape, a.shape))
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def softplus(x: float) -> float:
    return _load().oracle_softplus(float(x))


def causal_conv1d_silu(x, w, bias=None):
    """u = silu(bias + depthwise causal conv1d(x, w)); x (batch, dim, L),
    w (dim, K), bias (dim,) or None.  fp64 numpy result."""
    x = _f64(x)
    batch, dim, L = x.shape
    w = _f64(w)
    K = w.shape[1]
    w = _f64(w, (dim, K))
    bias = _f64(bias, (dim,))
    u = np.empty((batch, dim, L), np.float64)
    rc = _load().oracle_causal_conv1d_silu_f64(_ptr(x), _ptr(w), _ptr(bias),
                                               K, _ptr(u), batch, dim, L)
    if rc != 0:
        raise ValueError("oracle_causal_conv1d_silu_f64 rejected its arguments")
    return u


def causal_conv1d_silu_bwd(x, w, bias, du):
    """Gradients of :func:`causal_conv1d_silu` for a loss whose gradient
    with respect to u is ``du``.  Returns ``(dx, dw, db)`` (db None when
    ``bias`` is None) as fp64 arrays."""
    x = _f64(x)
    batch, dim, L = x.shape
    w = _f64(w)
    K = w.shape[1]
    w = _f64(w, (dim, K))
    bias = _f64(bias, (dim,))
    du = _f64(du, (batch, dim, L))
    dx = np.empty((batch, dim, L))
    dw = np.empty((dim, K))
    db = np.empty(dim) if bias is not None else None
    rc = _load().oracle_causal_conv1d_silu_bwd_f64(
        _ptr(x), _ptr(w), _ptr(bias), K, _ptr(du), _ptr(dx), _ptr(dw),
        _ptr(db), batch, dim, L)
    if rc != 0:
        raise ValueError("oracle_causal_conv1d_silu_bwd_f64 rejected its arguments")
    return dx, dw, db


def scan(u, delta, A, B, C, D=None, z=None, delta_bias=None,
         delta_softplus=True, zoh_b=False, h0=None):
    """Sequential fp64 scan.  Returns ``(y, h_final)`` as fp64 arrays.

    u, delta, z: (batch, dim, L); A: (dim, N); B, C: (batch, N, L);
    D, delta_bias: (dim,); h0: (batch, dim, N) or None (zero state).
    """
    u = _f64(u)
    if u.ndim != 3:
        raise ValueError("oracle: u must be (batch, dim, L)")
    batch, dim, L = u.shape
    A = _f64(A)
    N = A.shape[1]
    delta = _f64(delta, (batch, dim, L))
    A = _f64(A, (dim, N))
    B = _f64(B, (batch, N, L))
    C = _f64(C, (batch, N, L))
    D = _f64(D, (dim,))
    z = _f64(z, (batch, dim, L))
    delta_bias = _f64(delta_bias, (dim,))
    h0 = _f64(h0, (batch, dim, N))
    y = np.empty((batch, dim, L), np.float64)
    hf = np.empty((batch, dim, N), np.float64)
    rc = _load().oracle_scan_f64(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(delta_bias), int(bool(delta_softplus)), int(bool(zoh_b)),
        _ptr(h0), _ptr(y), _ptr(hf), batch, dim, N, L)
    if rc != 0:
        raise ValueError("oracle_scan_f64 rejected its arguments")
    return y, hf


def scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
             delta_softplus=True, h0=None, dy=None, dh_final=None, zoh_b=False):
    """Gradients of ``scan`` (Euler input term, or exact ZOH with ``zoh_b``)
    for a loss whose gradient is
    ``dy`` with respect to y and ``dh_final`` (or 0) with respect to the
    final state.  Returns a dict of fp64 arrays: du, ddelta, dA, dB, dC and,
    where the matching input is given, dD, ddelta_bias, dz; dh0 always."""
    u = _f64(u)
    batch, dim, L = u.shape
    A = _f64(A)
    N = A.shape[1]
    delta = _f64(delta, (batch, dim, L))
    B = _f64(B, (batch, N, L))
    C = _f64(C, (batch, N, L))
    D = _f64(D, (dim,))
    z = _f64(z, (batch, dim, L))
    delta_bias = _f64(delta_bias, (dim,))
    h0 = _f64(h0, (batch, dim, N))
    dy = _f64(dy, (batch, dim, L))
    dh_final = _f64(dh_final, (batch, dim, N))
    out = {"du": np.empty((batch, dim, L)), "ddelta": np.empty((batch, dim, L)),
           "dA": np.empty((dim, N)), "dB": np.empty((batch, N, L)),
           "dC": np.empty((batch, N, L)), "dh0": np.empty((batch, dim, N))}
    if D is not None:
        out["dD"] = np.empty(dim)
    if delta_bias is not None:
        out["ddelta_bias"] = np.empty(dim)
    if z is not None:
        out["dz"] = np.empty((batch, dim, L))
    rc = _load().oracle_scan_bwd_f64(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(delta_bias), int(bool(delta_softplus)), int(bool(zoh_b)),
        _ptr(h0), _ptr(dy), _ptr(dh_final), _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]),
        _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out.get("dD")),
        _ptr(out.get("ddelta_bias")), _ptr(out.get("dz")), _ptr(out["dh0"]),
        batch, dim, N, L)
    if rc != 0:
        raise ValueError("oracle_scan_bwd_f64 rejected its arguments")
    return out


def ssd(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=True,
        h0=None):
    """Mamba-2 SSD forward as the O(L^2) masked product.  x, z: (batch,
    nheads, headdim, L); dt: (batch, nheads, L); A, D, dt_bias: (nheads,);
    B, C: (batch, ngroups, N, L); h0: (batch, nheads, headdim, N).  Returns
    ``(y, h_final)`` as fp64 arrays."""
    x = _f64(x)
    batch, nheads, P, L = x.shape
    B = _f64(B)
    ngroups, N = B.shape[1], B.shape[2]
    B = _f64(B, (batch, ngroups, N, L))
    C = _f64(C, (batch, ngroups, N, L))
    dt = _f64(dt, (batch, nheads, L))
    A = _f64(A, (nheads,))
    D = _f64(D, (nheads,))
    z = _f64(z, (batch, nheads, P, L))
    dt_bias = _f64(dt_bias, (nheads,))
    h0 = _f64(h0, (batch, nheads, P, N))
    y = np.empty((batch, nheads, P, L))
    hf = np.empty((batch, nheads, P, N))
    rc = _load().oracle_ssd_f64(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
        _ptr(dt_bias), int(bool(dt_softplus)), _ptr(h0), _ptr(y), _ptr(hf),
        batch, nheads, P, ngroups, N, L)
    if rc != 0:
        raise ValueError("oracle_ssd_f64 rejected its arguments")
    return y, hf


def step(state, x, delta, A, B, C, D=None, z=None, delta_bias=None,
         delta_softplus=True, zoh_b=False):
    """One recurrent step.  ``state`` (batch, dim, N) fp64 numpy array is
    updated in place; returns y (batch, dim)."""
    if not (isinstance(state, np.ndarray) and state.dtype == np.float64
            and state.flags.c_contiguous):
        raise TypeError("oracle.step: state must be a C-contiguous fp64 array")
    batch, dim, N = state.shape
    x = _f64(x, (batch, dim))
    delta = _f64(delta, (batch, dim))
    A = _f64(A, (dim, N))
    B = _f64(B, (batch, N))
    C = _f64(C, (batch, N))
    D = _f64(D, (dim,))
    z = _f64(z, (batch, dim))
    delta_bias = _f64(delta_bias, (dim,))
    y = np.empty((batch, dim), np.float64)
    rc = _load().oracle_step_f64(
        _ptr(state), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
        _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)),
        int(bool(zoh_b)), _ptr(y), batch, dim, N)
    if rc != 0:
        raise ValueError("oracle_step_f64 rejected its arguments")
    return y


def scan_channels(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                  delta_softplus=True, zoh_b=False, h0=None, channels=None,
                  threads=1):
    """Scan only the listed ``(b, d)`` channels (the oracle is independent
    per channel).  Inputs are full-size arrays or tensors; only the selected
    rows are widened to fp64.  ``threads`` > 1 runs the channels on that
    many Python threads (ctypes releases the GIL); the arithmetic per
    channel is the same.  Returns ``(y[k, L], h_final[k, N])`` in the order
    of ``channels``."""
    channels = list(channels)

    def one(bd):
        b, d = bd
        sl = (slice(b, b + 1), slice(d, d + 1))
        y, hf = scan(u[sl], delta[sl], A[d:d + 1], B[b:b + 1], C[b:b + 1],
                     None if D is None else D[d:d + 1],
                     None if z is None else z[sl],
                     None if delta_bias is None else delta_bias[d:d + 1],
                     delta_softplus, zoh_b,
                     None if h0 is None else h0[sl])
        return y[0, 0], hf[0, 0]

    if threads > 1 and len(channels) > 1:
        with ThreadPoolExecutor(max_workers=int(threads)) as ex:
            res = list(ex.map(one, channels))
    else:
        res = [one(c) for c in channels]
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res])


def scan_threaded(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                  delta_softplus=True, zoh_b=False, h0=None, threads=None):
    """:func:`scan` over all channels, split into disjoint (b, d-range)
    pieces run on ``threads`` Python threads.  Same arithmetic per channel.
    Returns ``(y, h_final, threads_used)``."""
    u = _f64(u)
    batch, dim, L = u.shape
    A = _f64(A)
    N = A.shape[1]
    delta = _f64(delta, (batch, dim, L))
    B = _f64(B, (batch, N, L))
    C = _f64(C, (batch, N, L))
    D = _f64(D, (dim,))
    z = _f64(z, (batch, dim, L))
    delta_bias = _f64(delta_bias, (dim,))
    h0 = _f64(h0, (batch, dim, N))
    threads = max(1, int(threads or os.cpu_count() or 1))
    y = np.empty((batch, dim, L), np.float64)
    hf = np.empty((batch, dim, N), np.float64)
    lib = _load()
    pieces = []
    per = max(1, -(-batch * dim // (threads * 4)))
    for b in range(batch):
        for d0 in range(0, dim, per):
            pieces.append((b, d0, min(dim, d0 + per)))

    def run(piece):
        b, d0, d1 = piece
        k = d1 - d0

        def sub(a):
            return None if a is None else a[b:b + 1, d0:d1]
        views = [sub(u), sub(delta), A[d0:d1], B[b:b + 1], C[b:b + 1],
                 None if D is None else D[d0:d1], sub(z),
                 None if delta_bias is None else delta_bias[d0:d1], sub(h0),
                 y[b:b + 1, d0:d1], hf[b:b + 1, d0:d1]]
        ptrs = [None if v is None else v.ctypes.data for v in views]
        rc = lib.oracle_scan_f64(ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4],
                                 ptrs[5], ptrs[6], ptrs[7],
                                 int(bool(delta_softplus)), int(bool(zoh_b)),
                                 ptrs[8], ptrs[9], ptrs[10], 1, k, N, L)
        if rc != 0:
            raise ValueError("oracle_scan_f64 rejected its arguments")

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, pieces))
    return y, hf, threads
