"""Python binding of ``libssmscan.so`` -- the MI355X selective-scan library.

Argument marshalling only: tensors become device pointers, the current HIP
stream is passed along, and every step of the computation runs in the HIP
kernels behind the C ABI (``include/ssm_scan.h``).  There is no CPU or
PyTorch fallback: if the library cannot be loaded, or a call returns an error
status, these functions raise.

Names follow the C ABI:

* :func:`ssm_scan_fwd` -- whole-sequence selective scan (Mamba's S6 forward):
  dt = softplus(delta + bias), h_t = exp(dt*A) h_{t-1} + dt*B_t*u_t,
  y_t = (C_t . h_t + D*u_t) * silu(z_t).
* :func:`ssm_conv_scan_fwd` -- the same scan whose input u = silu(causal
  depthwise conv1d(x)) is formed inside the kernel (the Mamba block's
  convolution before the SSM).
* :func:`ssm_state_update` -- one decoding step on an in-place fp32 state.
* :func:`ssm_ssd_fwd` -- the Mamba-2 SSD form (one scalar decay per head,
  d_state 64-256) on the matrix cores; :func:`ssm_ssd_workspace_size`.
* :func:`ssm_conv_state_update` -- the decoding step with the conv
  prologue (its window kept per channel).
* :func:`ssm_scan_bwd` -- gradients of :func:`ssm_scan_fwd` (Euler or
  exact-ZOH input term) with respect to every input, recomputing the states from block
  checkpoints; :func:`ssm_scan_bwd_workspace_size`;
  :func:`ssm_scan_fwd_save`, the forward that keeps those checkpoints for
  the backward (which then skips its own checkpoint pass).
* :func:`ssm_conv_scan_bwd` -- gradients of :func:`ssm_conv_scan_fwd`,
  through the conv prologue as well; :func:`ssm_conv_scan_bwd_workspace_size`.
* :func:`ssm_scan_plan`, :func:`ssm_scan_workspace_size`,
  :func:`ssm_last_error`, :func:`ssm_abi_version`.
* :func:`ssm_roofline_hbm`, :func:`ssm_roofline_valu` -- microbenchmarks of
  the HBM and VALU-issue ceilings (``include/ssm_roofline.h``), used by the
  benchmark; not part of the method.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssmscan.so")

SSM_DTYPE_F32 = 0
SSM_DTYPE_BF16 = 1
SSM_FLAG_DELTA_SOFTPLUS = 1
SSM_FLAG_ZOH_B = 2
SSM_FLAG_BWD_SAVED = 4
STATUS = {0: "SSM_OK", 1: "SSM_ERR_INVALID_ARG", 2: "SSM_ERR_UNSUPPORTED",
          3: "SSM_ERR_WORKSPACE", 4: "SSM_ERR_HIP"}
EXPORTS = ("ssm_abi_version", "ssm_scan_plan", "ssm_scan_workspace_size",
           "ssm_scan_fwd", "ssm_conv_scan_fwd", "ssm_state_update",
           "ssm_conv_state_update",
           "ssm_scan_bwd_workspace_size", "ssm_scan_bwd_plan", "ssm_scan_fwd_save",
           "ssm_scan_bwd",
           "ssm_ssd_workspace_size", "ssm_ssd_fwd", "ssm_last_error",
           "ssm_roofline_hbm", "ssm_roofline_valu", "ssm_scan_fwd_noalloc",
           "ssm_conv_scan_bwd_workspace_size", "ssm_conv_scan_bwd")
SCAN_SCRATCH_BYTES = 16 << 20  # the fixed scratch of ssm_scan_fwd_noalloc
SSM_ROOFLINE_HBM_QUANTUM = 16384
SSM_ROOFLINE_VALU_QUANTUM = 256
ROOFLINE_HBM_KINDS = {"copy": 0, "rmw": 1, "read": 2}
ROOFLINE_VALU_KINDS = {"exp": 0, "fma": 1, "mixed": 2}

_lib = None
_lock = threading.Lock()


class SSMError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library (built in-tree by ``__graft_entry__.build()``).
    Raises if it is missing: there is no fallback."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                "libssmscan.so not found at %s; build it first "
                "(python -c 'import __graft_entry__ as g; g.build()')" % p)
        lib = ctypes.CDLL(p)
        P, I, I64, U = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                        ctypes.c_uint)
        lib.ssm_abi_version.argtypes = []
        lib.ssm_abi_version.restype = I
        lib.ssm_scan_plan.argtypes = [I64, I64, I64, I64, I64,
                                      ctypes.POINTER(I64)]
        lib.ssm_scan_plan.restype = I
        lib.ssm_scan_workspace_size.argtypes = [I64, I64, I64, I64, I64,
                                                ctypes.POINTER(ctypes.c_size_t)]
        lib.ssm_scan_workspace_size.restype = I
        lib.ssm_scan_fwd.argtypes = [P, P, P, P, P, P, P, P, U, P, P, P,
                                     I64, I64, I64, I64, I, I64, P,
                                     ctypes.c_size_t, P]
        lib.ssm_scan_fwd.restype = I
        lib.ssm_scan_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, U, P, P,
                                             P, I64, I64, I64, I64, I, I64, P]
        lib.ssm_scan_fwd_noalloc.restype = I
        lib.ssm_conv_scan_fwd.argtypes = [P, P, P, I, P, P, P, P, P, P, P, U,
                                          P, P, P, I64, I64, I64, I64, I, I64,
                                          P, ctypes.c_size_t, P]
        lib.ssm_conv_scan_fwd.restype = I
        lib.ssm_state_update.argtypes = [P, P, P, P, P, P, P, P, P, U, P,
                                         I64, I64, I64, I, P]
        lib.ssm_state_update.restype = I
        lib.ssm_conv_state_update.argtypes = [P, P, P, P, P, I, P, P, P, P, P,
                                              P, P, U, P, I64, I64, I64, I, P]
        lib.ssm_conv_state_update.restype = I
        lib.ssm_scan_bwd_workspace_size.argtypes = [
            I64, I64, I64, I64, I, ctypes.POINTER(ctypes.c_size_t)]
        lib.ssm_scan_bwd_workspace_size.restype = I
        lib.ssm_scan_bwd_plan.argtypes = [I64, I64, I64, I64, ctypes.POINTER(I64)]
        lib.ssm_scan_bwd_plan.restype = I
        lib.ssm_scan_bwd.argtypes = ([P] * 8 + [U] + [P] * 12 +
                                     [I64, I64, I64, I64, I, P,
                                      ctypes.c_size_t, P])
        lib.ssm_scan_bwd.restype = I
        lib.ssm_scan_fwd_save.argtypes = ([P] * 8 + [U] + [P] * 3 +
                                          [I64, I64, I64, I64, I, P,
                                           ctypes.c_size_t, P])
        lib.ssm_scan_fwd_save.restype = I
        lib.ssm_conv_scan_bwd_workspace_size.argtypes = [
            I64, I64, I64, I64, I, ctypes.POINTER(ctypes.c_size_t)]
        lib.ssm_conv_scan_bwd_workspace_size.restype = I
        lib.ssm_conv_scan_bwd.argtypes = ([P, P, P, I] + [P] * 7 + [U] +
                                          [P] * 14 + [I64] * 4 +
                                          [I, P, ctypes.c_size_t, P])
        lib.ssm_conv_scan_bwd.restype = I
        lib.ssm_ssd_workspace_size.argtypes = [
            I64, I64, I64, I64, ctypes.POINTER(ctypes.c_size_t)]
        lib.ssm_ssd_workspace_size.restype = I
        lib.ssm_ssd_fwd.argtypes = ([P] * 8 + [U] + [P] * 3 +
                                    [I64] * 6 + [I, P, ctypes.c_size_t, P])
        lib.ssm_ssd_fwd.restype = I
        lib.ssm_roofline_hbm.argtypes = [I, P, P, ctypes.c_size_t, I, P]
        lib.ssm_roofline_hbm.restype = I
        lib.ssm_roofline_valu.argtypes = [I, P, I64, I, P]
        lib.ssm_roofline_valu.restype = I
        lib.ssm_last_error.argtypes = []
        lib.ssm_last_error.restype = ctypes.c_char_p
        if path is None:
            _lib = lib
        return lib


def ssm_last_error() -> str:
    return load_library().ssm_last_error().decode()


def ssm_abi_version() -> int:
    return load_library().ssm_abi_version()


def _check(status):
    if status != 0:
        raise SSMError(status, ssm_last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SSM_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return SSM_DTYPE_BF16
    raise TypeError("activations must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t, name, dtype=None, shape=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s"
                         % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.device.type != "cuda":
        raise ValueError("%s must be a device (HIP) tensor" % name)
    return t.data_ptr()


def _stream_handle(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _on_stream(fn):
    """Runs the wrapper with ``stream`` (when given) as torch's current
    stream, so that the outputs and the workspace allocated inside belong to
    the stream the kernels run on: the caching allocator then cannot hand a
    freed workspace to work on another stream while these kernels still use
    it."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = sig.bind_partial(*args, **kwargs).arguments.get("stream")
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)
    return wrapper


def ssm_scan_plan(batch, dim, dstate, seqlen, requested_chunk=0) -> int:
    out = ctypes.c_int64(0)
    _check(load_library().ssm_scan_plan(batch, dim, dstate, seqlen,
                                        requested_chunk, ctypes.byref(out)))
    return out.value


def ssm_scan_workspace_size(batch, dim, dstate, seqlen, requested_chunk=0) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().ssm_scan_workspace_size(
        batch, dim, dstate, seqlen, requested_chunk, ctypes.byref(out)))
    return out.value


def _flags(delta_softplus, zoh_b):
    return ((SSM_FLAG_DELTA_SOFTPLUS if delta_softplus else 0) |
            (SSM_FLAG_ZOH_B if zoh_b else 0))


@_on_stream
def ssm_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                 delta_softplus=True, h0=None, return_final_state=True,
                 chunk_len=0, y=None, h_final=None, workspace=None,
                 stream=None, zoh_b=False):
    """Selective scan forward on device tensors.

    u, delta, z: (batch, dim, L); B, C: (batch, N, L) -- all one dtype
    (float32 or bfloat16).  A: (dim, N) fp32; D, delta_bias: (dim,) fp32;
    h0: (batch, dim, N) fp32 or None.  Returns ``(y, h_final)``
    (``h_final`` is None unless ``return_final_state``).  Outputs and the
    workspace are allocated here with torch unless passed in.  ``zoh_b``
    selects the exact zero-order-hold input term.
    """
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, L)")
    batch, dim, L = u.shape
    N = A.shape[-1] if A.dim() == 2 else 0
    dev = u.device
    act = u.dtype
    code = _dtype_code(u)
    pu = _ptr(u, "u", act, (batch, dim, L), dev)
    pd = _ptr(delta, "delta", act, (batch, dim, L), dev)
    pA = _ptr(A, "A", torch.float32, (dim, N), dev)
    pB = _ptr(B, "B", act, (batch, N, L), dev)
    pC = _ptr(C, "C", act, (batch, N, L), dev)
    pD = _ptr(D, "D", torch.float32, (dim,), dev)
    pz = _ptr(z, "z", act, (batch, dim, L), dev)
    pbias = _ptr(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    ph0 = _ptr(h0, "h0", torch.float32, (batch, dim, N), dev)
    if y is None:
        y = torch.empty((batch, dim, L), dtype=act, device=dev)
    py = _ptr(y, "y", act, (batch, dim, L), dev)
    if return_final_state and h_final is None:
        h_final = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    if not return_final_state:
        h_final = None
    ph = _ptr(h_final, "h_final", torch.float32, (batch, dim, N), dev)
    ws_bytes = ssm_scan_workspace_size(batch, dim, N, L, chunk_len)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    pws = workspace.data_ptr() if workspace is not None else None
    wsn = workspace.numel() * workspace.element_size() if workspace is not None else 0
    flags = _flags(delta_softplus, zoh_b)
    _check(load_library().ssm_scan_fwd(
        pu, pd, pA, pB, pC, pD, pz, pbias, flags, ph0, py, ph,
        batch, dim, N, L, code, chunk_len, pws, wsn,
        _stream_handle(dev, stream)))
    return y, h_final


@_on_stream
def ssm_conv_scan_fwd(x, conv_w, delta, A, B, C, D=None, z=None,
                      delta_bias=None, delta_softplus=True, h0=None,
                      conv_b=None, return_final_state=True, chunk_len=0,
                      y=None, h_final=None, workspace=None, stream=None,
                      zoh_b=False):
    """Scan with the fused conv prologue: u = silu(conv_b + causal depthwise
    conv1d(x, conv_w)) inside the kernel, then as :func:`ssm_scan_fwd`.
    x: (batch, dim, L) activation dtype; conv_w: (dim, d_conv) fp32 with
    d_conv <= 4; conv_b: (dim,) fp32 or None."""
    if x.dim() != 3:
        raise ValueError("x must be (batch, dim, L)")
    batch, dim, L = x.shape
    N = A.shape[-1] if A.dim() == 2 else 0
    dev = x.device
    act = x.dtype
    code = _dtype_code(x)
    if conv_w.dim() != 2:
        raise ValueError("conv_w must be (dim, d_conv)")
    d_conv = conv_w.shape[1]
    px = _ptr(x, "x", act, (batch, dim, L), dev)
    pw = _ptr(conv_w, "conv_w", torch.float32, (dim, d_conv), dev)
    pcb = _ptr(conv_b, "conv_b", torch.float32, (dim,), dev)
    pd = _ptr(delta, "delta", act, (batch, dim, L), dev)
    pA = _ptr(A, "A", torch.float32, (dim, N), dev)
    pB = _ptr(B, "B", act, (batch, N, L), dev)
    pC = _ptr(C, "C", act, (batch, N, L), dev)
    pD = _ptr(D, "D", torch.float32, (dim,), dev)
    pz = _ptr(z, "z", act, (batch, dim, L), dev)
    pbias = _ptr(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    ph0 = _ptr(h0, "h0", torch.float32, (batch, dim, N), dev)
    if y is None:
        y = torch.empty((batch, dim, L), dtype=act, device=dev)
    py = _ptr(y, "y", act, (batch, dim, L), dev)
    if return_final_state and h_final is None:
        h_final = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    if not return_final_state:
        h_final = None
    ph = _ptr(h_final, "h_final", torch.float32, (batch, dim, N), dev)
    ws_bytes = ssm_scan_workspace_size(batch, dim, N, L, chunk_len)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    pws = workspace.data_ptr() if workspace is not None else None
    wsn = workspace.numel() * workspace.element_size() if workspace is not None else 0
    flags = _flags(delta_softplus, zoh_b)
    _check(load_library().ssm_conv_scan_fwd(
        px, pw, pcb, d_conv, pd, pA, pB, pC, pD, pz, pbias, flags, ph0, py, ph,
        batch, dim, N, L, code, chunk_len, pws, wsn,
        _stream_handle(dev, stream)))
    return y, h_final


@_on_stream
def ssm_state_update(state, x, delta, A, B, C, D=None, z=None,
                     delta_bias=None, delta_softplus=True, y=None,
                     stream=None, zoh_b=False):
    """One decoding step: advances ``state`` (batch, dim, N) fp32 in place
    and returns y (batch, dim).  x, delta, z: (batch, dim); B, C:
    (batch, N), all one activation dtype."""
    if state.dim() != 3:
        raise ValueError("state must be (batch, dim, N)")
    batch, dim, N = state.shape
    dev = state.device
    act = x.dtype
    code = _dtype_code(x)
    ps = _ptr(state, "state", torch.float32, (batch, dim, N), dev)
    px = _ptr(x, "x", act, (batch, dim), dev)
    pd = _ptr(delta, "delta", act, (batch, dim), dev)
    pA = _ptr(A, "A", torch.float32, (dim, N), dev)
    pB = _ptr(B, "B", act, (batch, N), dev)
    pC = _ptr(C, "C", act, (batch, N), dev)
    pD = _ptr(D, "D", torch.float32, (dim,), dev)
    pz = _ptr(z, "z", act, (batch, dim), dev)
    pbias = _ptr(delta_bias, "delta_bias", torch.float32, (dim,), dev)
    if y is None:
        y = torch.empty((batch, dim), dtype=act, device=dev)
    py = _ptr(y, "y", act, (batch, dim), dev)
    flags = _flags(delta_softplus, zoh_b)
    _check(load_library().ssm_state_update(
        ps, px, pd, pA, pB, pC, pD, pz, pbias, flags, py, batch, dim, N,
        code, _stream_handle(dev, stream)))
    return y


@_on_stream
def ssm_conv_state_update(state, conv_state, x, conv_w, delta, A, B, C,
                          D=None, z=None, delta_bias=None, delta_softplus=True,
                          conv_b=None, y=None, stream=None, zoh_b=False):
    """One decoding step with the fused conv prologue: ``x`` (batch, dim)
    goes through the causal conv1d + SiLU over the window kept in
    ``conv_state`` (batch, dim, d_conv - 1; activation dtype; updated in
    place, zero for a fresh sequence), then advances ``state`` (batch, dim,
    N) fp32 in place like :func:`ssm_state_update`.  ``conv_w`` (dim,
    d_conv) and ``conv_b`` (dim,) fp32.  Returns y (batch, dim)."""
    if state.dim() != 3:
        raise ValueError("state must be (batch, dim, N)")
    batch, dim, N = state.shape
    dev = state.device
    act = x.dtype
    code = _dtype_code(x)
    K = conv_w.shape[-1] if conv_w.dim() == 2 else 0
    if y is None:
        y = torch.empty((batch, dim), dtype=act, device=dev)
    pcs = (_ptr(conv_state, "conv_state", act, (batch, dim, K - 1), dev)
           if K > 1 else None)
    _check(load_library().ssm_conv_state_update(
        _ptr(state, "state", torch.float32, (batch, dim, N), dev), pcs,
        _ptr(x, "x", act, (batch, dim), dev),
        _ptr(conv_w, "conv_w", torch.float32, (dim, K), dev),
        _ptr(conv_b, "conv_b", torch.float32, (dim,), dev), K,
        _ptr(delta, "delta", act, (batch, dim), dev),
        _ptr(A, "A", torch.float32, (dim, N), dev),
        _ptr(B, "B", act, (batch, N), dev),
        _ptr(C, "C", act, (batch, N), dev),
        _ptr(D, "D", torch.float32, (dim,), dev),
        _ptr(z, "z", act, (batch, dim), dev),
        _ptr(delta_bias, "delta_bias", torch.float32, (dim,), dev),
        _flags(delta_softplus, zoh_b),
        _ptr(y, "y", act, (batch, dim), dev),
        batch, dim, N, code, _stream_handle(dev, stream)))
    return y


@_on_stream
def bind_state_update(state, x, delta, A, B, C, D=None, z=None,
                      delta_bias=None, delta_softplus=True, y=None,
                      stream=None, zoh_b=False):
    """Checks and marshals the arguments of one decoding step once and
    returns a zero-argument callable that enqueues exactly that step (the
    same C call as :func:`ssm_state_update`, without per-call Python
    checks).  For launch-bound decode loops; the tensors must stay alive."""
    if state.dim() != 3:
        raise ValueError("state must be (batch, dim, N)")
    batch, dim, N = state.shape
    dev = state.device
    act = x.dtype
    code = _dtype_code(x)
    if y is None:
        y = torch.empty((batch, dim), dtype=act, device=dev)
    args = (_ptr(state, "state", torch.float32, (batch, dim, N), dev),
            _ptr(x, "x", act, (batch, dim), dev),
            _ptr(delta, "delta", act, (batch, dim), dev),
            _ptr(A, "A", torch.float32, (dim, N), dev),
            _ptr(B, "B", act, (batch, N), dev),
            _ptr(C, "C", act, (batch, N), dev),
            _ptr(D, "D", torch.float32, (dim,), dev),
            _ptr(z, "z", act, (batch, dim), dev),
            _ptr(delta_bias, "delta_bias", torch.float32, (dim,), dev),
            _flags(delta_softplus, zoh_b),
            _ptr(y, "y", act, (batch, dim), dev),
            batch, dim, N, code, _stream_handle(dev, stream))
    fn = load_library().ssm_state_update
    keep = (state, x, delta, A, B, C, D, z, delta_bias, y)

    def call():
        _check(fn(*args))
        return keep[-1]
    call.y = y
    return call


def ssm_scan_bwd_workspace_size(batch, dim, dstate, seqlen,
                                dtype=torch.bfloat16) -> int:
    out = ctypes.c_size_t(0)
    code = SSM_DTYPE_BF16 if dtype == torch.bfloat16 else SSM_DTYPE_F32
    _check(load_library().ssm_scan_bwd_workspace_size(
        batch, dim, dstate, seqlen, code, ctypes.byref(out)))
    return out.value


def ssm_scan_bwd_plan(batch, dim, dstate, seqlen) -> dict:
    """How :func:`ssm_scan_bwd` runs this shape: sweep and checkpoint-pass
    chunk lengths (seqlen = not split), dB/dC partial-sum rows per batch
    entry, and launches of the sweep kernel."""
    out = (ctypes.c_int64 * 4)()
    _check(load_library().ssm_scan_bwd_plan(batch, dim, dstate, seqlen, out))
    return {"sweep_chunk": out[0], "ckpt_chunk": out[1],
            "partial_rows": out[2], "sweep_launches": out[3]}


@_on_stream
def ssm_scan_fwd_save(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                      delta_softplus=True, h0=None, return_final_state=True,
                      y=None, h_final=None, workspace=None, stream=None,
                      zoh_b=False):
    """:func:`ssm_scan_fwd` (whole sequences) that also keeps, in the
    backward's workspace, the state entering every 1024-token block and the
    pre-gate output.  Returns ``(y, h_final, workspace)``; pass that
    workspace to :func:`ssm_scan_bwd` with ``saved=True`` (same inputs) to
    skip the backward's checkpoint pass."""
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, L)")
    batch, dim, L = u.shape
    N = A.shape[-1] if A.dim() == 2 else 0
    dev = u.device
    act = u.dtype
    code = _dtype_code(u)
    f32 = torch.float32
    if y is None:
        y = torch.empty((batch, dim, L), dtype=act, device=dev)
    if return_final_state and h_final is None:
        h_final = torch.empty((batch, dim, N), dtype=f32, device=dev)
    if not return_final_state:
        h_final = None
    ws_bytes = ssm_scan_bwd_workspace_size(batch, dim, N, L, act)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    wsn = workspace.numel() * workspace.element_size()
    _check(load_library().ssm_scan_fwd_save(
        _ptr(u, "u", act, (batch, dim, L), dev),
        _ptr(delta, "delta", act, (batch, dim, L), dev),
        _ptr(A, "A", f32, (dim, N), dev),
        _ptr(B, "B", act, (batch, N, L), dev),
        _ptr(C, "C", act, (batch, N, L), dev),
        _ptr(D, "D", f32, (dim,), dev),
        _ptr(z, "z", act, (batch, dim, L), dev),
        _ptr(delta_bias, "delta_bias", f32, (dim,), dev),
        _flags(delta_softplus, zoh_b),
        _ptr(h0, "h0", f32, (batch, dim, N), dev),
        _ptr(y, "y", act, (batch, dim, L), dev),
        _ptr(h_final, "h_final", f32, (batch, dim, N), dev),
        batch, dim, N, L, code, workspace.data_ptr(), wsn,
        _stream_handle(dev, stream)))
    return y, h_final, workspace


@_on_stream
def ssm_scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                 delta_softplus=True, h0=None, dy=None, dh_final=None,
                 want_dz=True, want_dh0=True, out=None, workspace=None,
                 stream=None, saved=False, zoh_b=False):
    """Gradients of :func:`ssm_scan_fwd` (Euler input term, or exact ZOH
    with ``zoh_b``) for a loss with
    gradient ``dy`` (batch, dim, L; activation dtype) with respect to y and
    ``dh_final`` (batch, dim, N; fp32, or None) with respect to the final
    state.  Returns a dict: du, ddelta (activation dtype), dA, dB, dC, dD,
    ddelta_bias, dh0 (fp32) and dz (activation dtype, when z is given).
    ``out`` may supply any of these tensors; the rest, and the workspace,
    are allocated here with torch.  ``saved``: ``workspace`` holds what
    :func:`ssm_scan_fwd_save` kept for these inputs (no checkpoint pass)."""
    if saved and workspace is None:
        raise ValueError("saved=True needs the workspace ssm_scan_fwd_save filled")
    if u.dim() != 3:
        raise ValueError("u must be (batch, dim, L)")
    batch, dim, L = u.shape
    N = A.shape[-1] if A.dim() == 2 else 0
    dev = u.device
    act = u.dtype
    code = _dtype_code(u)
    f32 = torch.float32
    if dy is None:
        raise ValueError("dy is required")
    out = dict(out or {})
    shapes = {"du": ((batch, dim, L), act), "ddelta": ((batch, dim, L), act),
              "dA": ((dim, N), f32), "dB": ((batch, N, L), f32),
              "dC": ((batch, N, L), f32), "dD": ((dim,), f32),
              "ddelta_bias": ((dim,), f32)}
    if z is not None and want_dz:
        shapes["dz"] = ((batch, dim, L), act)
    if want_dh0:
        shapes["dh0"] = ((batch, dim, N), f32)
    for k, (shp, dt) in shapes.items():
        if k not in out:
            out[k] = torch.empty(shp, dtype=dt, device=dev)
    p = {k: _ptr(out[k], k, shapes[k][1], shapes[k][0], dev) for k in shapes}
    ws_bytes = ssm_scan_bwd_workspace_size(batch, dim, N, L, act)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    wsn = workspace.numel() * workspace.element_size()
    _check(load_library().ssm_scan_bwd(
        _ptr(u, "u", act, (batch, dim, L), dev),
        _ptr(delta, "delta", act, (batch, dim, L), dev),
        _ptr(A, "A", f32, (dim, N), dev),
        _ptr(B, "B", act, (batch, N, L), dev),
        _ptr(C, "C", act, (batch, N, L), dev),
        _ptr(D, "D", f32, (dim,), dev),
        _ptr(z, "z", act, (batch, dim, L), dev),
        _ptr(delta_bias, "delta_bias", f32, (dim,), dev),
        _flags(delta_softplus, zoh_b) | (SSM_FLAG_BWD_SAVED if saved else 0),
        _ptr(h0, "h0", f32, (batch, dim, N), dev),
        _ptr(dy, "dy", act, (batch, dim, L), dev),
        _ptr(dh_final, "dh_final", f32, (batch, dim, N), dev),
        p["du"], p["ddelta"], p["dA"], p["dB"], p["dC"], p["dD"],
        p["ddelta_bias"], p.get("dz"), p.get("dh0"),
        batch, dim, N, L, code, workspace.data_ptr(), wsn,
        _stream_handle(dev, stream)))
    return {k: out[k] for k in shapes}


def ssm_conv_scan_bwd_workspace_size(batch, dim, dstate, seqlen,
                                     dtype=torch.bfloat16) -> int:
    out = ctypes.c_size_t(0)
    code = SSM_DTYPE_BF16 if dtype == torch.bfloat16 else SSM_DTYPE_F32
    _check(load_library().ssm_conv_scan_bwd_workspace_size(
        batch, dim, dstate, seqlen, code, ctypes.byref(out)))
    return out.value


@_on_stream
def ssm_conv_scan_bwd(x, conv_w, delta, A, B, C, D=None, z=None,
                      delta_bias=None, delta_softplus=True, h0=None, dy=None,
                      dh_final=None, conv_b=None, want_dz=True, want_dh0=True,
                      out=None, workspace=None, stream=None, zoh_b=False):
    """Gradients of :func:`ssm_conv_scan_fwd` for a loss with gradient
    ``dy`` with respect to y and ``dh_final`` with respect to the final
    state.  Returns a dict: dx, ddelta (activation dtype), dconv_w, dconv_b
    (when conv_b is given), dA, dB, dC, dD, ddelta_bias, dh0 (fp32) and dz
    (when z is given)."""
    if x.dim() != 3:
        raise ValueError("x must be (batch, dim, L)")
    if dy is None:
        raise ValueError("dy is required")
    batch, dim, L = x.shape
    N = A.shape[-1] if A.dim() == 2 else 0
    K = conv_w.shape[-1] if conv_w.dim() == 2 else 0
    dev = x.device
    act = x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    out = dict(out or {})
    shapes = {"dx": ((batch, dim, L), act), "ddelta": ((batch, dim, L), act),
              "dconv_w": ((dim, K), f32),
              "dA": ((dim, N), f32), "dB": ((batch, N, L), f32),
              "dC": ((batch, N, L), f32), "dD": ((dim,), f32),
              "ddelta_bias": ((dim,), f32)}
    if conv_b is not None:
        shapes["dconv_b"] = ((dim,), f32)
    if z is not None and want_dz:
        shapes["dz"] = ((batch, dim, L), act)
    if want_dh0:
        shapes["dh0"] = ((batch, dim, N), f32)
    for k, (shp, dt) in shapes.items():
        if k not in out:
            out[k] = torch.empty(shp, dtype=dt, device=dev)
    p = {k: _ptr(out[k], k, shapes[k][1], shapes[k][0], dev) for k in shapes}
    if workspace is None:
        workspace = torch.empty(
            ssm_conv_scan_bwd_workspace_size(batch, dim, N, L, act),
            dtype=torch.uint8, device=dev)
    wsn = workspace.numel() * workspace.element_size()
    _check(load_library().ssm_conv_scan_bwd(
        _ptr(x, "x", act, (batch, dim, L), dev),
        _ptr(conv_w, "conv_w", f32, (dim, K), dev),
        _ptr(conv_b, "conv_b", f32, (dim,), dev), K,
        _ptr(delta, "delta", act, (batch, dim, L), dev),
        _ptr(A, "A", f32, (dim, N), dev),
        _ptr(B, "B", act, (batch, N, L), dev),
        _ptr(C, "C", act, (batch, N, L), dev),
        _ptr(D, "D", f32, (dim,), dev),
        _ptr(z, "z", act, (batch, dim, L), dev),
        _ptr(delta_bias, "delta_bias", f32, (dim,), dev),
        _flags(delta_softplus, zoh_b),
        _ptr(h0, "h0", f32, (batch, dim, N), dev),
        _ptr(dy, "dy", act, (batch, dim, L), dev),
        _ptr(dh_final, "dh_final", f32, (batch, dim, N), dev),
        p["dx"], p["dconv_w"], p.get("dconv_b"), p["ddelta"], p["dA"],
        p["dB"], p["dC"], p["dD"], p["ddelta_bias"], p.get("dz"), p.get("dh0"),
        batch, dim, N, L, code, workspace.data_ptr(), wsn,
        _stream_handle(dev, stream)))
    return {k: out[k] for k in shapes}


def ssm_ssd_workspace_size(batch, ngroups, dstate, seqlen) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().ssm_ssd_workspace_size(batch, ngroups, dstate,
                                                 seqlen, ctypes.byref(out)))
    return out.value


@_on_stream
def ssm_ssd_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None,
                dt_softplus=True, h0=None, return_final_state=True, y=None,
                h_final=None, workspace=None, stream=None):
    """Mamba-2 SSD forward.  x, z: (batch, nheads, headdim, L) bf16; dt:
    (batch, nheads, L) bf16; A, D, dt_bias: (nheads,) fp32; B, C: (batch,
    ngroups, N, L) bf16; h0: (batch, nheads, headdim, N) fp32 or None.
    Returns ``(y, h_final)``."""
    if x.dim() != 4:
        raise ValueError("x must be (batch, nheads, headdim, L)")
    batch, nheads, P, L = x.shape
    if B.dim() != 4:
        raise ValueError("B must be (batch, ngroups, N, L)")
    ngroups, N = B.shape[1], B.shape[2]
    dev = x.device
    act = x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    if y is None:
        y = torch.empty((batch, nheads, P, L), dtype=act, device=dev)
    if return_final_state and h_final is None:
        h_final = torch.empty((batch, nheads, P, N), dtype=f32, device=dev)
    if not return_final_state:
        h_final = None
    if workspace is None:
        workspace = torch.empty(ssm_ssd_workspace_size(batch, ngroups, N, L),
                                dtype=torch.uint8, device=dev)
    wsn = workspace.numel() * workspace.element_size()
    _check(load_library().ssm_ssd_fwd(
        _ptr(x, "x", act, (batch, nheads, P, L), dev),
        _ptr(dt, "dt", act, (batch, nheads, L), dev),
        _ptr(A, "A", f32, (nheads,), dev),
        _ptr(B, "B", act, (batch, ngroups, N, L), dev),
        _ptr(C, "C", act, (batch, ngroups, N, L), dev),
        _ptr(D, "D", f32, (nheads,), dev),
        _ptr(z, "z", act, (batch, nheads, P, L), dev),
        _ptr(dt_bias, "dt_bias", f32, (nheads,), dev),
        _flags(dt_softplus, False),
        _ptr(h0, "h0", f32, (batch, nheads, P, N), dev),
        _ptr(y, "y", act, (batch, nheads, P, L), dev),
        _ptr(h_final, "h_final", f32, (batch, nheads, P, N), dev),
        batch, nheads, P, ngroups, N, L, code, workspace.data_ptr(), wsn,
        _stream_handle(dev, stream)))
    return y, h_final


def ssm_roofline_hbm(kind, a, b=None, repeats=1, stream=None):
    """``repeats`` passes of an HBM microbenchmark over the bytes of ``a``:
    kind "copy" (b = a, b the same size), "rmw" (a = a*0.5 + 0.25 in place)
    or "read" (b: a 1-element fp32 sink).  Enqueues only."""
    code = ROOFLINE_HBM_KINDS[kind]
    nbytes = a.numel() * a.element_size()
    pa = _ptr(a, "a")
    pb = _ptr(b, "b") if b is not None else None
    _check(load_library().ssm_roofline_hbm(code, pa, pb, nbytes, repeats,
                                           _stream_handle(a.device, stream)))


def ssm_roofline_valu(kind, out, iters, stream=None):
    """One VALU-issue microbenchmark pass: ``out.numel()`` threads each run
    ``iters`` iterations of 8 independent chains of kind "exp" (v_exp_f32),
    "fma" (v_fma_f32) or "mixed" (half of each); 8 lane-operations per
    thread and iteration.  Enqueues only."""
    code = ROOFLINE_VALU_KINDS[kind]
    _check(load_library().ssm_roofline_valu(
        code, _ptr(out, "out", torch.float32), out.numel(), iters,
        _stream_handle(out.device, stream)))
