"""Seeded synthetic inputs for the selective SSM scan and its decode step.

This module only draws random numbers and shapes them; it holds none of the
scan's arithmetic.  Both sides of every parity check -- the HIP library and
the fp64 oracle -- read the very tensors made here (the oracle after an exact
widening to fp64), so neither side's inputs come from the other.

Every tensor has its own ``torch.Generator`` seeded from ``(seed, tensor
index)``, so the same call on the same device always returns the same values.
Values are drawn in fp32 and rounded to bf16 (round-to-nearest-even, torch's
conversion) where the workload is bf16.

The named workloads are shaped like Mamba layers: d_state = 16 (the Mamba-1
hyper-parameter on the inferownia.pl page, "Zrob to sam"), channel counts of
the 130M and 2.8B checkpoints' inner dimension, and the S4D-real
initialisation A[d, n] = -(n + 1) of "Mamba & State Space Models - Guide
Complet", section 4 (A_log = log(1..N), A = -exp(A_log)).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class ScanConfig:
    name: str
    batch: int
    dim: int
    dstate: int
    seqlen: int
    dtype: str                  # "f32" or "bf16" (u, delta, B, C, z, y)
    a_init: str = "arange"      # "arange": -(n+1); "exp_log": -exp(log(n+1))
    delta_kind: str = "normal_bias"  # or "log_uniform"
    with_z: bool = True
    with_D: bool = True
    with_h0: bool = False
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def elements(self) -> int:
        return self.batch * self.dim * self.seqlen


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    dim: int
    dstate: int
    steps: int
    dtype: str = "bf16"
    seed: int = 0
    note: str = field(default="", compare=False)


# The five workloads.  The scan ones share one recipe: u, z ~ N(0,1);
# delta_raw ~ N(0,1) with a per-channel bias log(expm1(U[1e-3, 1e-1])) and
# softplus on; B, C ~ N(0,1) shaped (batch, N, L); D ~ N(0,1); zero initial
# state.  The long-context one instead draws the post-softplus step
# log-uniformly in [1e-3, 1e-1] and stores its softplus pre-image.
TINY = ScanConfig("tiny_b1_d64_l256_f32", 1, 64, 16, 256, "f32", seed=1000,
                  note="batch=1, D=64, N=16, L=256, fp32")
MAMBA_130M = ScanConfig("mamba130m_b4_d1536_l2048_bf16", 4, 1536, 16, 2048,
                        "bf16", seed=1001,
                        note="batch=4, D=1536, N=16, L=2048, bf16")
MAMBA_2P8B = ScanConfig("mamba2p8b_b2_d5120_l4096_bf16", 2, 5120, 16, 4096,
                        "bf16", a_init="exp_log", seed=1002,
                        note="batch=2, D=5120, N=16, L=4096, bf16")
LONG_1M = ScanConfig("long_b1_d1536_l1048576_f32", 1, 1536, 16, 1 << 20,
                     "f32", delta_kind="log_uniform", seed=1003,
                     note="batch=1, D=1536, N=16, L=1048576, fp32")
DECODE = DecodeConfig("decode_b256_d5120_n16_bf16", 256, 5120, 16, 64,
                      seed=1004,
                      note="batch=256, D=5120, N=16, 64 steps, bf16 x/dt/z")

SCAN_CONFIGS = {c.name: c for c in (TINY, MAMBA_130M, MAMBA_2P8B, LONG_1M)}


@dataclass(frozen=True)
class SsdConfig:
    """A Mamba-2 SSD layer: nheads heads of headdim rows (d_inner = nheads *
    headdim), dstate states, ngroups groups sharing B and C."""
    name: str
    batch: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    seqlen: int
    with_z: bool = True
    with_D: bool = True
    with_h0: bool = False
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def elements(self) -> int:
        return self.batch * self.nheads * self.headdim * self.seqlen


# d_inner 5120 (the 2.8B layer's inner width) as 80 heads of 64, d_state 128
# (inside the 64-256 the Guide Complet gives for Mamba-2), one group.
MAMBA2_LAYER = SsdConfig("mamba2_b2_h80_p64_n128_l4096_bf16", 2, 80, 64, 1, 128,
                         4096, seed=1005,
                         note="batch=2, 80 heads x 64, N=128, L=4096, bf16")


def make_ssd_inputs(cfg: SsdConfig, device="cpu", **over) -> dict:
    """Seeded SSD inputs (bf16 activations): x, z ~ N(0,1); dt_raw ~ N(0,1)
    with a per-head bias log(expm1(U[1e-3, 1e-1])) and softplus on (as the
    scan workloads); A[h] = -U[1, 16] (Mamba-2 keeps A = -exp(A_log) per
    head with A_log in [log 1, log 16]); B, C ~ N(0,1); D ~ N(0,1)."""
    if over:
        cfg = replace(cfg, **over)
    b, h, P, g, n, L, s = (cfg.batch, cfg.nheads, cfg.headdim, cfg.ngroups,
                           cfg.dstate, cfg.seqlen, cfg.seed)
    act = torch.bfloat16
    out = {}
    out["x"] = _normal((b, h, P, L), device, s, 1).to(act)
    out["dt"] = _normal((b, h, L), device, s, 2).to(act)
    target = _uniform((h,), 1e-3, 1e-1, device, s, 3)
    out["dt_bias"] = torch.log(torch.expm1(target)).contiguous()
    out["A"] = -_uniform((h,), 1.0, 16.0, device, s, 4)
    out["B"] = _normal((b, g, n, L), device, s, 5).to(act)
    out["C"] = _normal((b, g, n, L), device, s, 6).to(act)
    out["D"] = _normal((h,), device, s, 7) if cfg.with_D else None
    out["z"] = _normal((b, h, P, L), device, s, 8).to(act) if cfg.with_z else None
    out["h0"] = _normal((b, h, P, n), device, s, 9) if cfg.with_h0 else None
    out["dt_softplus"] = True
    return out


def ssd_bytes(cfg: SsdConfig) -> int:
    """Bytes the SSD forward must move: x, z read and y written (bf16), dt
    read (bf16), B and C read, A, D, bias read, the final state written (and
    the initial one read when given)."""
    e = cfg.elements
    by = e * 2 * (2 + (1 if cfg.with_z else 0))
    by += cfg.batch * cfg.nheads * cfg.seqlen * 2
    by += 2 * cfg.batch * cfg.ngroups * cfg.dstate * cfg.seqlen * 2
    by += 3 * cfg.nheads * 4
    st = cfg.batch * cfg.nheads * cfg.headdim * cfg.dstate * 4
    by += st * (2 if cfg.with_h0 else 1)
    return by


def ssd_flops(cfg: SsdConfig, chunk: int = 64) -> int:
    """Matrix-core flops of the chunked SSD form: per chunk and head the
    y products exp(A cum) S C (headdim x N x chunk) and X M^T (headdim x
    chunk x chunk) and the state update (X w) B^T (headdim x chunk x N);
    per chunk and group G = C^T B (chunk x N x chunk)."""
    nch = (cfg.seqlen + chunk - 1) // chunk
    P, N, T = cfg.headdim, cfg.dstate, chunk
    per_head = 2 * (P * N * T + P * T * T + P * T * N)
    per_group = 2 * T * N * T
    return nch * cfg.batch * (cfg.nheads * per_head + cfg.ngroups * per_group)


def torch_dtype(tag: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[tag]


def _gen(device, seed: int, idx: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + idx)
    return g


def _normal(shape, device, seed, idx):
    return torch.randn(shape, generator=_gen(device, seed, idx),
                       device=device, dtype=torch.float32)


def _uniform(shape, lo, hi, device, seed, idx):
    r = torch.rand(shape, generator=_gen(device, seed, idx), device=device,
                   dtype=torch.float32)
    return lo + (hi - lo) * r


def a_matrix(dim: int, dstate: int, kind: str = "arange",
             device="cpu") -> torch.Tensor:
    """S4D-real A, fp32 (dim, dstate).  ``arange``: -(n+1) exactly;
    ``exp_log``: -exp(log(n+1)) evaluated in fp32 as the S6 module writes it;
    ``zero``: all zeros."""
    n1 = torch.arange(1, dstate + 1, dtype=torch.float32, device=device)
    if kind == "arange":
        row = -n1
    elif kind == "exp_log":
        row = -torch.exp(torch.log(n1))
    elif kind == "zero":
        row = torch.zeros_like(n1)
    else:
        raise ValueError(kind)
    return row.unsqueeze(0).repeat(dim, 1).contiguous()


def make_scan_inputs(cfg: ScanConfig, device="cpu", **over) -> dict:
    """Inputs of one scan workload as torch tensors on ``device``.

    Keys: u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus.  Optional
    ones are None when the workload leaves them out.  ``over`` replaces
    fields of ``cfg`` (shape, dtype, flags) for parity cases of other sizes.
    """
    if over:
        cfg = replace(cfg, **over)
    b, d, n, L, s = cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen, cfg.seed
    act = torch_dtype(cfg.dtype)
    out = {}
    out["u"] = _normal((b, d, L), device, s, 1).to(act)
    if cfg.delta_kind == "normal_bias":
        out["delta"] = _normal((b, d, L), device, s, 2).to(act)
        target = _uniform((d,), 1e-3, 1e-1, device, s, 3)
        out["delta_bias"] = torch.log(torch.expm1(target)).contiguous()
    elif cfg.delta_kind == "log_uniform":
        lo, hi = math.log(1e-3), math.log(1e-1)
        target = torch.exp(_uniform((b, d, L), lo, hi, device, s, 2))
        out["delta"] = torch.log(torch.expm1(target)).to(act)
        out["delta_bias"] = None
    else:
        raise ValueError(cfg.delta_kind)
    out["A"] = a_matrix(d, n, cfg.a_init, device)
    out["B"] = _normal((b, n, L), device, s, 4).to(act)
    out["C"] = _normal((b, n, L), device, s, 5).to(act)
    out["D"] = _normal((d,), device, s, 6) if cfg.with_D else None
    out["z"] = _normal((b, d, L), device, s, 7).to(act) if cfg.with_z else None
    out["h0"] = _normal((b, d, n), device, s, 8) if cfg.with_h0 else None
    out["delta_softplus"] = True
    return out


def make_conv_inputs(cfg: ScanConfig, device="cpu", d_conv: int = 4,
                     with_bias: bool = True, **over) -> dict:
    """Inputs of the scan with the fused conv prologue: the scan workload's
    tensors with ``x`` (the pre-convolution activations, N(0,1), in place of
    u), ``conv_w`` ~ U(-1/sqrt(d_conv), 1/sqrt(d_conv)) of shape
    (dim, d_conv) and ``conv_b`` of the same distribution, both fp32 (the
    default initialisation range of a depthwise Conv1d)."""
    out = make_scan_inputs(cfg, device, **over)
    if over:
        cfg = replace(cfg, **over)
    out["x"] = out.pop("u")
    lim = 1.0 / math.sqrt(d_conv)
    out["conv_w"] = _uniform((cfg.dim, d_conv), -lim, lim, device, cfg.seed, 9)
    out["conv_b"] = (_uniform((cfg.dim,), -lim, lim, device, cfg.seed, 10)
                     if with_bias else None)
    return out


def make_decode_inputs(cfg: DecodeConfig, device="cpu", with_h0=False,
                       **over) -> dict:
    """A ``steps``-token sequence for the decode workload, laid out like a
    scan input (x, delta, z: (batch, dim, steps); B, C: (batch, N, steps)) so
    the same tensors can feed the scan; step t reads column t.  Same
    distributions as the scan workloads."""
    if over:
        cfg = replace(cfg, **over)
    b, d, n, T, s = cfg.batch, cfg.dim, cfg.dstate, cfg.steps, cfg.seed
    act = torch_dtype(cfg.dtype)
    out = {}
    out["u"] = _normal((b, d, T), device, s, 1).to(act)
    out["delta"] = _normal((b, d, T), device, s, 2).to(act)
    target = _uniform((d,), 1e-3, 1e-1, device, s, 3)
    out["delta_bias"] = torch.log(torch.expm1(target)).contiguous()
    out["A"] = a_matrix(d, n, "arange", device)
    out["B"] = _normal((b, n, T), device, s, 4).to(act)
    out["C"] = _normal((b, n, T), device, s, 5).to(act)
    out["D"] = _normal((d,), device, s, 6)
    out["z"] = _normal((b, d, T), device, s, 7).to(act)
    out["h0"] = _normal((b, d, n), device, s, 8) if with_h0 else None
    out["delta_softplus"] = True
    return out


def make_conv_decode_inputs(cfg: DecodeConfig, device="cpu", d_conv: int = 4,
                            with_bias: bool = True, with_h0: bool = False,
                            with_window: bool = False, **over) -> dict:
    """A decode sequence for the step with the fused conv prologue: the
    decode workload's tensors, ``u`` read as the pre-convolution input x,
    plus ``conv_w`` (dim, d_conv) and ``conv_b`` (dim,) drawn like the conv
    scan's, and ``conv_state0`` (batch, dim, d_conv - 1) in the activation
    dtype: N(0,1) (a sequence already under way) with ``with_window``, else
    zeros (a fresh one)."""
    out = make_decode_inputs(cfg, device, with_h0=with_h0, **over)
    if over:
        cfg = replace(cfg, **over)
    b, d, s = cfg.batch, cfg.dim, cfg.seed
    lim = 1.0 / math.sqrt(d_conv)
    out["conv_w"] = _uniform((d, d_conv), -lim, lim, device, s, 9)
    out["conv_b"] = (_uniform((d,), -lim, lim, device, s, 10)
                     if with_bias else None)
    H = d_conv - 1
    out["conv_state0"] = (_normal((b, d, H), device, s, 11) if with_window
                          else torch.zeros((b, d, H), device=device)
                          ).to(torch_dtype(cfg.dtype))
    return out


def step_slice(inputs: dict, t: int) -> dict:
    """Contiguous per-step tensors (x, delta, z: (batch, dim); B, C:
    (batch, N)) for token ``t`` of a decode sequence."""
    return {
        "x": inputs["u"][:, :, t].contiguous(),
        "delta": inputs["delta"][:, :, t].contiguous(),
        "z": inputs["z"][:, :, t].contiguous(),
        "B": inputs["B"][:, :, t].contiguous(),
        "C": inputs["C"][:, :, t].contiguous(),
    }


def algorithmic_bytes(cfg: ScanConfig, with_h0: bool | None = None) -> int:
    """Bytes the scan must move between HBM and the chip: u, delta, z read
    and y written once (``elem`` bytes each), B and C read once, A, D and the
    bias read once, the final state written (and the initial state read
    when given).  The discretised dA / dB*u never touch HBM."""
    elem = 2 if cfg.dtype == "bf16" else 4
    e = cfg.elements
    nbig = 2 + (1 if cfg.with_z else 0) + 1
    by = e * elem * nbig
    by += 2 * cfg.batch * cfg.dstate * cfg.seqlen * elem
    by += cfg.dim * cfg.dstate * 4
    by += cfg.dim * 4 * ((1 if cfg.with_D else 0) +
                         (1 if cfg.delta_kind == "normal_bias" else 0))
    by += cfg.batch * cfg.dim * cfg.dstate * 4
    if with_h0 if with_h0 is not None else cfg.with_h0:
        by += cfg.batch * cfg.dim * cfg.dstate * 4
    return by


def decode_step_bytes(cfg: DecodeConfig) -> int:
    """Per decode step: the fp32 state read and written once; x, delta, z
    read and y written (activation dtype); B, C (batch, N) read; A, D, bias
    read."""
    elem = 2 if cfg.dtype == "bf16" else 4
    bd = cfg.batch * cfg.dim
    by = 2 * bd * cfg.dstate * 4
    by += 4 * bd * elem
    by += 2 * cfg.batch * cfg.dstate * elem
    by += cfg.dim * cfg.dstate * 4 + 2 * cfg.dim * 4
    return by


def conv_decode_step_bytes(cfg: DecodeConfig, d_conv: int = 4) -> int:
    """Per decode step with the conv prologue: the plain step's bytes plus
    the kept window (d_conv - 1 inputs per channel, activation dtype) read
    and written, and the taps and conv bias (fp32) read."""
    elem = 2 if cfg.dtype == "bf16" else 4
    bd = cfg.batch * cfg.dim
    return (decode_step_bytes(cfg) + 2 * bd * (d_conv - 1) * elem
            + cfg.dim * (d_conv + 1) * 4)


def backward_bytes(cfg: ScanConfig) -> int:
    """Bytes the backward pass must move at least once: u, delta, z and dy
    read and du, ddelta, dz written (``elem`` bytes each); B and C read; dB
    and dC written (fp32); A, D, bias read and dA, dD, dbias written; the
    initial state read and its gradient written when given."""
    elem = 2 if cfg.dtype == "bf16" else 4
    e = cfg.elements
    nz = 1 if cfg.with_z else 0
    by = e * elem * (3 + 2 * nz + 2)   # u, delta, dy, (z, dz), du, ddelta
    bnl = cfg.batch * cfg.dstate * cfg.seqlen
    by += 2 * bnl * elem + 2 * bnl * 4
    by += 2 * cfg.dim * cfg.dstate * 4 + 4 * cfg.dim * 4
    if cfg.with_h0:
        by += 2 * cfg.batch * cfg.dim * cfg.dstate * 4
    return by
