#!/usr/bin/env python3
"""Throughput of the selective scan on one MI355X.

One step = one ``ssm_scan_fwd`` over the Mamba-2.8B-shaped layer workload
(batch=2, D=5120, N=16, L=4096, bf16 activations, fp32 state, gate and D
skip, final state returned) -- the whole hot path for that shape: B/C
staging, softplus, discretisation, scan, readout, gate and store in one
kernel.  Inputs are resident in HBM before the timed region; three input
sets are rotated so the 256 MB last-level cache cannot serve them.

Prints ONE JSON line.  ``value`` is GB/s of algorithmic traffic (bytes the
method must move: every input read once, y and the final state written
once).  ``roofline`` relates the algorithmic bytes of one launch of the scan
kernel to its average duration (HIP events around every step on the launch
stream, over the timed region) and to the 8 TB/s HBM peak; ``valu`` beside
it states the same launch against the VALU issue ceiling, which is what
actually bounds the kernel at 16 states.  Both ceilings are also measured in
the same run by hand-written microbenchmarks (include/ssm_roofline.h): a
non-temporal copy, read-modify-write and read over 1 GiB buffers, and chains
of v_exp_f32 and v_fma_f32.  They run before the timed steps, which also
gives the timed steps a GPU whose clocks have settled under sustained load.
``cpu_baseline`` is the fp64 oracle on the same inputs on the host cores.

Options beyond the contract: --no-cpu-baseline, --no-extra (skip the
other workloads: the 130M-shaped layer, long context, conv prologue, ZOH,
backward, SSD and decode figures), --only-scan (nothing but the timed steps;
for profiler runs), --only-ssd (only the Mamba-2 SSD figure, --steps calls;
for profiler runs), --only-decode (the decode workload, --steps passes of
its 64 steps), --only-bwd (the 2.8B-layer backward, --steps calls),
--summarize DIR (no GPU: turn the rocprofv3 CSV output
of the profiling commands below into the summaries under profiles/).

Profiling commands (run from /tmp with TMPDIR=/tmp; DIR = an output folder):
  rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace -o bench \
      -- python3 bench.py --no-cpu-baseline
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch -o fetch \
      -- python3 bench.py --steps 3 --warmup 1 --no-extra --no-cpu-baseline
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/write -o write \
      -- python3 bench.py --steps 3 --warmup 1 --no-extra --no-cpu-baseline
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/ssdfetch -o ssdfetch \
      -- python3 bench.py --only-ssd --steps 3
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/ssdwrite -o ssdwrite \
      -- python3 bench.py --only-ssd --steps 3
  (the same two passes with --only-decode into DIR/decodefetch and
  DIR/decodewrite, and with --only-bwd into DIR/bwdfetch and DIR/bwdwrite;
  and, for the SQ counters of those kernels, one pass each of
  --pmc SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_VALU_TRANS_F32
  SQ_WAIT_INST_LDS SQ_WAIT_ANY SQ_WAVE_CYCLES SQ_BUSY_CYCLES
  SQ_LDS_BANK_CONFLICT with --only-bwd, --only-ssd and --only-decode into
  DIR/bwdsq, DIR/ssdsq and DIR/decodesq)
  python3 bench.py --summarize DIR
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# fp32 vector peak without packed math (packed FP32 forms are disabled in
# this build): 256 CUs x 4 SIMDs x 16 lanes x 2 flop (FMA) x 2.4 GHz.
VALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
# Algorithmic flops: per state-update dt*A (1), exp (1), dt*u*B (1),
# h = dA*h + dBu (2), y += C*h (2); per element bias add, softplus (exp,
# log1p), dt*u, D*u + add, silu (exp, add, reciprocal, multiply), gate.
FLOP_PER_STATE_UPDATE = 7
FLOP_PER_ELEMENT = 13
TRAFFIC_FILE = os.path.join(ROOT, "profiles",
                            "scan_kernel_mamba2p8b_traffic.json")
SQ_FILE = os.path.join(ROOT, "profiles", "scan_kernel_mamba2p8b_sq_counters.txt")
KERNEL_SRC_DIRS = [os.path.join(ROOT, "selective_state_space_30_amd", "csrc"),
                   os.path.join(ROOT, "include")]


def kernel_source_hash() -> str:
    """sha256[:16] over every source the kernels are built from (all of
    csrc/ and include/, names and contents), so a profile taken before any
    change to them is recognised as stale."""
    h = hashlib.sha256()
    for d in KERNEL_SRC_DIRS:
        for name in sorted(os.listdir(d)):
            path = os.path.join(d, name)
            if os.path.isfile(path):
                h.update(name.encode() + b"\0")
                with open(path, "rb") as f:
                    h.update(f.read())
    return h.hexdigest()[:16]


def measured_valu_slots():
    """VALU issue slots (SQ_ACTIVE_INST_VALU: instructions plus the extra
    slots of transcendentals) per launch of the scan kernel, from the
    committed SQ-counter summary, or None if the sources changed since."""
    try:
        text = open(SQ_FILE).read()
    except OSError:
        return None
    if "sources sha256[:16] %s" % kernel_source_hash() not in text:
        return None
    for line in text.splitlines():
        if line.startswith("SQ_ACTIVE_INST_VALU"):
            return float(line.split()[1])
    return None


def profiled_launch_us():
    """Kernel-trace average duration (us) of the scan kernel over the 2.8B
    layer's dispatches in the committed profile, or None if the sources
    changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("kernel_trace_us_mean")


def measured_traffic(n_launch_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or
    None if the kernel source changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return int(t["hbm_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only-scan", action="store_true")
    ap.add_argument("--only-ssd", action="store_true")
    ap.add_argument("--only-decode", action="store_true")
    ap.add_argument("--only-bwd", action="store_true")
    ap.add_argument("--summarize", metavar="DIR")
    args = ap.parse_args()
    if args.summarize:
        summarize_profiles(args.summarize)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build runs the scan on a "
              "single MI355X (no collectives or sharding); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_30_amd as ssm
    import synthetic as syn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = ssm.load_library()
    only = {"only_ssd": (syn.MAMBA2_LAYER.name, ssd_measure),
            "only_decode": (syn.DECODE.name, decode_measure),
            "only_bwd": (syn.MAMBA_2P8B.name + "_backward", bwd_measure)}
    for flag, (name, measure) in only.items():
        if getattr(args, flag):
            stream = torch.cuda.current_stream(dev)
            r = measure(ssm, syn, dev, stream, args.steps,
                        lambda m: print("[bench] " + m, file=sys.stderr, flush=True))
            print(json.dumps({name: r}))
            return
    cfg = syn.MAMBA_2P8B
    E = cfg.elements
    nbytes = syn.algorithmic_bytes(cfg)

    def log(msg):
        print("[bench] " + msg, file=sys.stderr, flush=True)

    log("workload %s: generating 3 input sets on %s" % (cfg.name, dev))
    sets = []
    for i in range(3):
        inp = syn.make_scan_inputs(cfg, dev, seed=cfg.seed + 100 * i)
        inp["y"] = torch.empty_like(inp["u"])
        inp["h_final"] = torch.empty(cfg.batch, cfg.dim, 16, device=dev)
        sets.append(inp)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ceil = {} if args.only_scan else ceilings(torch, ssm, dev, stream, log)
    # The other workloads are measured before the headline's steps: after
    # an idle GPU the scan's step time first rises for some tens of steps
    # (the clocks settling under its sustained VALU load) before it comes
    # down to its steady value, so the headline is timed on a GPU that has
    # been busy for a while (its own warm-up count is unchanged).
    def step(i):
        s = sets[i % 3]
        ssm.ssm_scan_fwd(s["u"], s["delta"], s["A"], s["B"], s["C"], s["D"],
                         s["z"], s["delta_bias"], True, None,
                         y=s["y"], h_final=s["h_final"], stream=stream)

    extras = None
    if not (args.only_scan or args.no_extra):
        extras = extra_workloads(torch, ssm, syn, dev, stream, log, ceil)
        # the last of them: the headline step 300 times back to back, timed
        # per step, so the settling of the clock under this load is on
        # record (by position in the run); the headline's own warm-up and
        # timed steps follow it
        n_ss = 300
        log("consecutive steps: %d headline steps back to back" % n_ss)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_ss + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(n_ss):
            step(i)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        us = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n_ss)]

        def mean(v):
            return round(sum(v) / len(v), 1)
        extras[cfg.name + "_consecutive_steps"] = {
            "steps": n_ss, "us_mean_steps_0_19": mean(us[:20]),
            "us_mean_steps_20_99": mean(us[20:100]),
            "us_mean_steps_100_299": mean(us[100:]),
            "us_median": round(sorted(us)[n_ss // 2], 1), "us_min": round(min(us), 1),
            "note": "the headline step run back to back after the other "
                    "workloads, one event per step: the step time by position "
                    "shows the clock settling under the sustained load"}

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    # The K timed steps: one event before the first and one after the last,
    # on the launch stream (an event recorded after every step adds ~2 us
    # to each, measured on one box: 181.0-182.2 vs 178.8-179.7 us).
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    ms_wall = wall * 1e3 / args.steps
    # then K more with an event after every step, for the per-step median
    # and minimum (reported beside the mean; those include the events)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1])
                      for i in range(args.steps))
    ms_median = per_step[len(per_step) // 2]
    ms_min = per_step[0]
    sec = ms * 1e-3
    gbps = nbytes / sec / 1e9
    log("scan: %.1f us/step mean, %.1f median, %.1f min (events), %.1f "
        "(wall), %.0f GB/s" % (ms * 1e3, ms_median * 1e3, ms_min * 1e3,
                               ms_wall * 1e3, gbps))
    if args.only_scan:
        return

    flops = (E * cfg.dstate * FLOP_PER_STATE_UPDATE + E * FLOP_PER_ELEMENT)
    result = {
        "metric": "selective-scan HBM GB/s (% of peak) + elements/s, "
                  "D=5120 L=4096 N=16",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Mamba-2.8B-shaped layer)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "dim": cfg.dim,
                   "dstate": cfg.dstate, "seqlen": cfg.seqlen,
                   "activations": "bf16", "state": "fp32", "gate": True,
                   "D_skip": True, "final_state": True,
                   "A": "-exp(log(1..16)) fp32", "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "elements_per_s": round(E / sec),
        "state_updates_per_s": round(E * cfg.dstate / sec),
        "algorithmic_bytes_per_step": nbytes,
        "ms_per_step_median": round(ms_median, 5),
        "ms_per_step_min": round(ms_min, 5),
        "ms_per_step_wall": round(ms_wall, 5),
        # one step is one launch of the scan kernel (the sequence is not
        # split at this shape), so the per-launch duration is the step's
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(nbytes),
            "kernel": SCAN_KERNEL,
            "algorithmic_bytes_per_launch": nbytes,
            "launch_us_mean": round(ms * 1e3, 2),
            # the same kernel's average in the committed rocprofv3 trace
            # (another box; boxes differ by a few per cent)
            "profiled_launch_us_mean": profiled_launch_us(),
        },
    }
    result["valu"] = valu_block(ceil, E * cfg.dstate, flops, sec)
    if ceil:
        result["hbm_ceilings_GBps"] = {k: ceil[k] for k in
                                       ("copy", "rmw", "read")}
        result["copy_ceiling_GBps"] = ceil["copy"]
        result["pct_of_copy_ceiling"] = round(100 * gbps / ceil["copy"], 2)

    if extras is not None:
        result["other_workloads"] = extras

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(sets[0], cfg, nbytes, log)

    del sets
    print(json.dumps(result), flush=True)


def ceilings(torch, ssm, dev, stream, log):
    """The HBM and VALU-issue ceilings, measured by the library's
    microbenchmarks (include/ssm_roofline.h) on this GPU in this run.
    HBM: GB/s (bytes read plus bytes written) of a non-temporal copy, an
    in-place read-modify-write and a read-only pass over 1 GiB buffers (4x
    the 256 MB last-level cache), best of 5 timings of 10 passes each.
    VALU: lane-operations per second of chains of v_exp_f32, of v_fma_f32
    and of both interleaved, over 8 waves per SIMD, best of 5 timings of 20
    launches each (about a quarter of a second of sustained VALU issue in
    all, right before the scan's warm-up steps)."""
    log("ceilings: HBM copy / read-modify-write / read over 1 GiB, "
        "v_exp_f32 and v_fma_f32 issue rates")
    out = {}
    nb = 1 << 30
    a = torch.empty(nb // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    a.fill_(0.5)
    sink = torch.zeros(1, device=dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for kind, moved in (("copy", 2 * nb), ("rmw", 2 * nb), ("read", nb)):
        bb = b if kind == "copy" else (sink if kind == "read" else None)
        ssm.ssm_roofline_hbm(kind, a, bb, repeats=2, stream=stream)
        best = None
        for _ in range(5):
            e0.record(stream)
            ssm.ssm_roofline_hbm(kind, a, bb, repeats=10, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / 10
            best = t if best is None else min(best, t)
        out[kind] = round(moved / best / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    threads = 256 * 4 * 8 * 64      # 8 waves on each of the 1024 SIMDs
    iters = 4096
    launches = 20                   # per timing: ~10-20 ms of sustained issue
    vout = torch.empty(threads, device=dev)
    for kind in ("exp", "fma", "mixed"):
        ssm.ssm_roofline_valu(kind, vout, iters, stream=stream)
        best = None
        for _ in range(5):
            e0.record(stream)
            for _ in range(launches):
                ssm.ssm_roofline_valu(kind, vout, iters, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / launches
            best = t if best is None else min(best, t)
        out[kind + "_lane_ops_per_s"] = threads * iters * 8 / best
    # the mixed chains take half of each kind: if a transcendental overlapped
    # the FMAs, the mixed rate would approach the FMA rate; without overlap
    # the time is the sum of the two halves
    t_exp = 0.5 / out["exp_lane_ops_per_s"]
    t_fma = 0.5 / out["fma_lane_ops_per_s"]
    out["mixed_over_no_overlap"] = round(
        (1.0 / out["mixed_lane_ops_per_s"]) / (t_exp + t_fma), 3)
    log("ceilings: copy %.0f, rmw %.0f, read %.0f GB/s; exp %.3g, fma %.3g "
        "lane-ops/s (mixed / no-overlap time %.2f)"
        % (out["copy"], out["rmw"], out["read"], out["exp_lane_ops_per_s"],
           out["fma_lane_ops_per_s"], out["mixed_over_no_overlap"]))
    return out


def valu_block(ceil, state_updates, flops, sec):
    """The scan launch against the VALU issue ceiling: issue slots per
    launch (SQ_ACTIVE_INST_VALU from the committed counter summary, while
    the sources are unchanged) over the FMA issue rate measured in this run
    give the time the instruction stream needs at full issue; that over the
    launch's time is the fraction of the VALU ceiling reached.  The flop
    count of the older alu figure (7 per state-update, an exp counted as one
    flop although it takes two issue slots) is kept beside it, labelled."""
    slots = measured_valu_slots()
    out = {"what": "VALU issue: the ceiling that bounds this kernel at 16 "
                   "states (no packed fp32)",
           "alu_flops_per_launch_7_per_state_update": flops,
           "alu_frac_of_78.6_TFLOPs_nonpacked_fp32":
               round(flops / sec / 1e12 / VALU_PEAK_TFLOPS, 4)}
    if ceil:
        out["exp_lane_ops_per_s"] = float("%.4g" % ceil["exp_lane_ops_per_s"])
        out["fma_lane_ops_per_s"] = float("%.4g" % ceil["fma_lane_ops_per_s"])
        out["exp_issue_cost_in_fma_slots"] = round(
            ceil["fma_lane_ops_per_s"] / ceil["exp_lane_ops_per_s"], 2)
        out["mixed_over_no_overlap"] = ceil["mixed_over_no_overlap"]
    if slots is not None:
        lane_slots = slots * 64
        out["issue_slots_per_launch"] = lane_slots
        out["issue_slots_per_state_update"] = round(lane_slots / state_updates, 2)
        out["source"] = "profiles/scan_kernel_mamba2p8b_sq_counters.txt"
        if ceil:
            floor = lane_slots / ceil["fma_lane_ops_per_s"]
            out["issue_floor_us"] = round(floor * 1e6, 1)
            out["frac"] = round(floor / sec, 4)
    return out


SETTLE_MS = 30.0


def settle(torch, fn, stream, ms=SETTLE_MS):
    """Runs ``fn`` untimed for about ``ms`` of GPU time before a timed loop.
    Under a new sustained compute load the step time of these kernels drifts
    for some tens of milliseconds (the clocks settling; the headline's
    consecutive-steps record shows it) before it holds steady, so every
    compute-bound measurement below starts after this."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    for _ in range(int(ms / max(e0.elapsed_time(e1), 1e-3))):
        fn()
    torch.cuda.synchronize()


def extra_workloads(torch, ssm, syn, dev, stream, log, ceil):
    """The decode step, the SSD form, the backward, the long-context scan
    (chunked), the ZOH and conv-prologue variants and the 130M-shaped layer,
    each timed with events; reported beside the main line."""
    out = {}
    # the measurements end with the scan kernel itself (the long-context,
    # ZOH, conv-prologue and 130M-layer runs), right before the headline
    ccfg = syn.MAMBA_2P8B
    reps = 20
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    out[syn.DECODE.name] = decode_measure(ssm, syn, dev, stream, 1, log, ceil)
    torch.cuda.empty_cache()
    out[syn.MAMBA2_LAYER.name] = ssd_measure(ssm, syn, dev, stream, reps, log)
    torch.cuda.empty_cache()

    out[syn.MAMBA_2P8B.name + "_backward"] = bwd_measure(ssm, syn, dev, stream,
                                                         reps, log)
    torch.cuda.empty_cache()

    cfg = syn.LONG_1M
    log("long-context workload %s" % cfg.name)
    inp = syn.make_scan_inputs(cfg, dev)
    y = torch.empty_like(inp["u"])
    hf = torch.empty(cfg.batch, cfg.dim, 16, device=dev)
    ws_bytes = ssm.ssm_scan_workspace_size(cfg.batch, cfg.dim, 16, cfg.seqlen)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def run():
        ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["z"], inp["delta_bias"], True, None,
                         y=y, h_final=hf, workspace=ws, stream=stream)
    settle(torch, run, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nb = syn.algorithmic_bytes(cfg)
    out[cfg.name] = {
        "ms_per_call": round(ms, 4), "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
        "elements_per_s": round(cfg.elements / (ms * 1e-3)),
        "chunk_len": ssm.ssm_scan_plan(cfg.batch, cfg.dim, 16, cfg.seqlen),
        "algorithmic_bytes": nb}
    del y, hf, ws
    torch.cuda.empty_cache()

    # its backward (1536 channels: the sequence is split across waves)
    log("long-context backward %s" % cfg.name)
    g = torch.Generator(device=dev).manual_seed(cfg.seed + 9)
    dy = torch.randn(cfg.batch, cfg.dim, cfg.seqlen, generator=g, device=dev)
    bws = torch.empty(ssm.ssm_scan_bwd_workspace_size(cfg.batch, cfg.dim, 16,
                                                      cfg.seqlen, torch.float32),
                      dtype=torch.uint8, device=dev)
    grads = {}

    def brun():
        grads.update(ssm.ssm_scan_bwd(
            inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
            inp["z"], inp["delta_bias"], True, None, dy, None, workspace=bws,
            stream=stream))
        grads.clear()
    brun()
    torch.cuda.synchronize()
    reps = 3
    e0.record(stream)
    for _ in range(reps):
        brun()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nb = syn.backward_bytes(cfg)
    out[cfg.name + "_backward"] = {
        "ms_per_call": round(ms, 3), "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
        "algorithmic_bytes": nb,
        "note": "ssm_scan_bwd, no dh_final: checkpoint pass (split like the "
                "forward), adjoint pre-pass and carry, chunked sweep, "
                "reductions; gradient outputs allocated per call"}
    del inp, dy, bws
    torch.cuda.empty_cache()

    # the 2.8B layer with the exact zero-order-hold input term
    reps = 20
    log("ZOH input term on %s" % ccfg.name)
    zinp = syn.make_scan_inputs(ccfg, dev)
    zy = torch.empty_like(zinp["u"])
    zhf = torch.empty(ccfg.batch, ccfg.dim, 16, device=dev)

    def zrun():
        ssm.ssm_scan_fwd(zinp["u"], zinp["delta"], zinp["A"], zinp["B"],
                         zinp["C"], zinp["D"], zinp["z"], zinp["delta_bias"],
                         True, None, y=zy, h_final=zhf, stream=stream,
                         zoh_b=True)
    settle(torch, zrun, stream)
    e0.record(stream)
    for _ in range(reps):
        zrun()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nb = syn.algorithmic_bytes(ccfg)
    out[ccfg.name + "_zoh"] = {
        "ms_per_call": round(ms, 4), "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
        "elements_per_s": round(ccfg.elements / (ms * 1e-3)),
        "note": "exact zero-order-hold input term (flag)"}
    del zinp, zy, zhf
    torch.cuda.empty_cache()

    # the 2.8B layer with the fused conv prologue (x in place of u)
    ccfg = syn.MAMBA_2P8B
    log("conv-prologue workload %s" % ccfg.name)
    cinp = syn.make_conv_inputs(ccfg, dev)
    cy = torch.empty_like(cinp["x"])
    chf = torch.empty(ccfg.batch, ccfg.dim, 16, device=dev)

    def crun():
        ssm.ssm_conv_scan_fwd(cinp["x"], cinp["conv_w"], cinp["delta"],
                              cinp["A"], cinp["B"], cinp["C"], cinp["D"],
                              cinp["z"], cinp["delta_bias"], True, None,
                              conv_b=cinp["conv_b"], y=cy, h_final=chf,
                              stream=stream)
    settle(torch, crun, stream)
    reps = 20
    e0.record(stream)
    for _ in range(reps):
        crun()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nb = syn.algorithmic_bytes(ccfg) + ccfg.dim * 4 * 5  # + conv w, b
    out[ccfg.name + "_conv_prologue"] = {
        "ms_per_call": round(ms, 4), "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
        "elements_per_s": round(ccfg.elements / (ms * 1e-3)),
        "note": "x read in place of u; u = silu(conv1d(x)) formed in the kernel"}
    del cinp, cy, chf
    torch.cuda.empty_cache()

    # the 130M-shaped layer; three input sets rotated (305 MB, beyond the
    # last-level cache)
    scfg = syn.MAMBA_130M
    log("130M-layer workload %s" % scfg.name)
    ssets = []
    for i in range(3):
        s = syn.make_scan_inputs(scfg, dev, seed=scfg.seed + 100 * i)
        s["y"] = torch.empty_like(s["u"])
        s["h_final"] = torch.empty(scfg.batch, scfg.dim, 16, device=dev)
        ssets.append(s)

    def srun(i):
        s = ssets[i % 3]
        ssm.ssm_scan_fwd(s["u"], s["delta"], s["A"], s["B"], s["C"], s["D"],
                         s["z"], s["delta_bias"], True, None, y=s["y"],
                         h_final=s["h_final"], stream=stream)
    it = iter(range(1 << 30))
    settle(torch, lambda: srun(next(it)), stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 60
    e0.record(stream)
    for i in range(reps):
        srun(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nb = syn.algorithmic_bytes(scfg)
    out[scfg.name] = {
        "ms_per_call": round(ms, 4), "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
        "elements_per_s": round(scfg.elements / (ms * 1e-3)),
        "chunk_len": ssm.ssm_scan_plan(scfg.batch, scfg.dim, 16, scfg.seqlen),
        "algorithmic_bytes": nb}
    del ssets
    torch.cuda.empty_cache()

    return out


def bwd_measure(ssm, syn, dev, stream, reps, log):
    """Backward pass of the 2.8B layer (checkpoint pass, reverse sweep,
    channel-sum reductions); outputs and workspace allocated up front."""
    import torch
    ccfg = syn.MAMBA_2P8B
    log("backward on %s" % ccfg.name)
    binp = syn.make_scan_inputs(ccfg, dev)
    g = torch.Generator(device=dev).manual_seed(ccfg.seed + 9)
    bdy = torch.randn(ccfg.batch, ccfg.dim, ccfg.seqlen, generator=g,
                      device=dev).to(binp["u"].dtype)
    bws = torch.empty(ssm.ssm_scan_bwd_workspace_size(
        ccfg.batch, ccfg.dim, 16, ccfg.seqlen, binp["u"].dtype),
        dtype=torch.uint8, device=dev)
    bout = ssm.ssm_scan_bwd(binp["u"], binp["delta"], binp["A"], binp["B"],
                            binp["C"], binp["D"], binp["z"], binp["delta_bias"],
                            True, None, bdy, None, workspace=bws, stream=stream)

    def brun():
        ssm.ssm_scan_bwd(binp["u"], binp["delta"], binp["A"], binp["B"],
                         binp["C"], binp["D"], binp["z"], binp["delta_bias"],
                         True, None, bdy, None, out=bout, workspace=bws,
                         stream=stream)
    settle(torch, brun, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        brun()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps

    # a training step's pair: the forward that keeps the checkpoints, then
    # the backward that reuses them (no checkpoint pass)
    fy = torch.empty_like(binp["u"])
    fh = torch.empty(ccfg.batch, ccfg.dim, 16, device=dev)

    def frun():
        ssm.ssm_scan_fwd_save(binp["u"], binp["delta"], binp["A"], binp["B"],
                              binp["C"], binp["D"], binp["z"], binp["delta_bias"],
                              True, None, y=fy, h_final=fh, workspace=bws,
                              stream=stream)

    def srun():
        ssm.ssm_scan_bwd(binp["u"], binp["delta"], binp["A"], binp["B"],
                         binp["C"], binp["D"], binp["z"], binp["delta_bias"],
                         True, None, bdy, None, out=bout, workspace=bws,
                         stream=stream, saved=True)
    settle(torch, lambda: (frun(), srun()), stream)
    e0.record(stream)
    for _ in range(reps):
        frun()
        srun()
    e1.record(stream)
    torch.cuda.synchronize()
    pair_ms = e0.elapsed_time(e1) / reps

    def timed(fn):
        settle(torch, fn, stream)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # the same backward with the exact-ZOH input term
    zoh_ms = timed(lambda: ssm.ssm_scan_bwd(
        binp["u"], binp["delta"], binp["A"], binp["B"], binp["C"], binp["D"],
        binp["z"], binp["delta_bias"], True, None, bdy, None, out=bout,
        workspace=bws, stream=stream, zoh_b=True))
    # through the conv prologue (x in place of u, width 4)
    cinp = syn.make_conv_inputs(ccfg, dev)
    cws = torch.empty(ssm.ssm_conv_scan_bwd_workspace_size(
        ccfg.batch, ccfg.dim, 16, ccfg.seqlen, binp["u"].dtype),
        dtype=torch.uint8, device=dev)
    cout = ssm.ssm_conv_scan_bwd(cinp["x"], cinp["conv_w"], cinp["delta"],
                                 cinp["A"], cinp["B"], cinp["C"], cinp["D"],
                                 cinp["z"], cinp["delta_bias"], True, None,
                                 bdy, None, conv_b=cinp["conv_b"],
                                 workspace=cws, stream=stream)
    conv_ms = timed(lambda: ssm.ssm_conv_scan_bwd(
        cinp["x"], cinp["conv_w"], cinp["delta"], cinp["A"], cinp["B"],
        cinp["C"], cinp["D"], cinp["z"], cinp["delta_bias"], True, None, bdy,
        None, conv_b=cinp["conv_b"], out=cout, workspace=cws, stream=stream))
    del cinp, cws, cout
    nb = syn.backward_bytes(ccfg)
    return {"ms_per_call": round(ms, 4), "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
            "zoh_ms_per_call": round(zoh_ms, 4),
            "conv_prologue_ms_per_call": round(conv_ms, 4),
            "elements_per_s": round(ccfg.elements / (ms * 1e-3)),
            "algorithmic_bytes": nb, "workspace_bytes": bws.numel(),
            "fwd_save_plus_bwd_saved_ms": round(pair_ms, 4),
            "note": "gradients of u, delta, A, B, C, D, z, bias; states "
                    "recomputed from 1024-token checkpoints (ms_per_call: "
                    "the backward alone, with its own checkpoint pass; "
                    "fwd_save_plus_bwd_saved_ms: ssm_scan_fwd_save then "
                    "ssm_scan_bwd reusing its checkpoints; zoh_ms_per_call: "
                    "with the exact-ZOH input term; "
                    "conv_prologue_ms_per_call: ssm_conv_scan_bwd, x and the "
                    "width-4 conv in place of u)"}


N_DECODE_STATES = 8


def decode_measure(ssm, syn, dev, stream, passes, log, ceil=None):
    """The decode workload: ``passes`` times its 64 steps, each step one
    ssm_state_update call bound in advance.  Eight states (one per layer of
    a stack) take the steps in turn: 671 MB, so a state comes back after
    ~1.25 GB of other traffic, well past what the 256 MB last-level cache
    holds.  Stated against the read-modify-write ceiling measured in the
    same run (``ceil``)."""
    import torch
    dcfg = syn.DECODE
    log("decode workload %s" % dcfg.name)
    dinp = syn.make_decode_inputs(dcfg, dev)
    steps = [syn.step_slice(dinp, t) for t in range(dcfg.steps)]
    states = [torch.zeros(dcfg.batch, dcfg.dim, 16, device=dev)
              for _ in range(N_DECODE_STATES)]
    ys = [torch.empty(dcfg.batch, dcfg.dim, dtype=torch.bfloat16, device=dev)
          for _ in range(dcfg.steps)]
    calls = [ssm.bind_state_update(states[t % N_DECODE_STATES], s["x"], s["delta"], dinp["A"],
                                   s["B"], s["C"], dinp["D"], s["z"],
                                   dinp["delta_bias"], True, y=ys[t],
                                   stream=stream)
             for t, s in enumerate(steps)]
    for c in calls:
        c()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(passes):
        for c in calls:
            c()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (dcfg.steps * passes)

    # the same 64 steps captured once into a HIP graph and replayed (bound
    # to a side stream, the capture stream)
    side = torch.cuda.Stream()
    gcalls = [ssm.bind_state_update(states[t % N_DECODE_STATES], s["x"], s["delta"],
                                    dinp["A"], s["B"], s["C"], dinp["D"], s["z"],
                                    dinp["delta_bias"], True, y=ys[t], stream=side)
              for t, s in enumerate(steps)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for c in gcalls:
            c()
    graph.replay()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream(dev)
    e0.record(cur)
    for _ in range(passes):
        graph.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    us_graph = e0.elapsed_time(e1) * 1e3 / (dcfg.steps * passes)

    # the same steps with the width-4 conv prologue (ssm_conv_state_update),
    # each state with its own kept window, captured the same way
    cinp = syn.make_conv_decode_inputs(dcfg, dev, d_conv=4)
    windows = [cinp["conv_state0"].clone() for _ in range(N_DECODE_STATES)]
    torch.cuda.synchronize()
    cgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cgraph, stream=side):
        for t, s in enumerate(steps):
            ssm.ssm_conv_state_update(
                states[t % N_DECODE_STATES], windows[t % N_DECODE_STATES], s["x"], cinp["conv_w"],
                s["delta"], dinp["A"], s["B"], s["C"], dinp["D"], s["z"],
                dinp["delta_bias"], True, conv_b=cinp["conv_b"], y=ys[t],
                stream=side)
    cgraph.replay()
    torch.cuda.synchronize()
    e0.record(cur)
    for _ in range(passes):
        cgraph.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    us_conv = e0.elapsed_time(e1) * 1e3 / (dcfg.steps * passes)
    nb = syn.decode_step_bytes(dcfg)
    gbps = nb / (us * 1e-6) / 1e9
    out = {"us_per_step": round(us, 3), "GBps": round(gbps, 1),
           "bytes_per_step": nb, "states_rotated": N_DECODE_STATES,
           "state_bytes_rotated": N_DECODE_STATES * dcfg.batch * dcfg.dim * 16 * 4,
           "us_per_step_hip_graph": round(us_graph, 3),
           "us_per_step_conv4_hip_graph": round(us_conv, 3)}
    if ceil:
        out["rmw_ceiling_GBps"] = ceil["rmw"]
        out["frac_of_rmw_ceiling"] = round(gbps / ceil["rmw"], 4)
        out["frac_of_hbm_peak"] = round(gbps / HBM_PEAK_GBPS, 4)
    return out


def ssd_measure(ssm, syn, dev, stream, reps, log):
    """Mamba-2 SSD form (one scalar decay per head, matrix-core chunk
    products) on an 80-head layer; workspace and outputs allocated up front,
    inputs resident before the timed calls, three input sets rotated (the
    262 MB working set is about the size of the last-level cache)."""
    import torch
    scfg = syn.MAMBA2_LAYER
    log("SSD form on %s" % scfg.name)
    sets = [syn.make_ssd_inputs(scfg, dev, seed=scfg.seed + 100 * i)
            for i in range(3)]
    sws = torch.empty(ssm.ssm_ssd_workspace_size(
        scfg.batch, scfg.ngroups, scfg.dstate, scfg.seqlen),
        dtype=torch.uint8, device=dev)
    outs = [(torch.empty_like(s["x"]),
             torch.empty(scfg.batch, scfg.nheads, scfg.headdim, scfg.dstate,
                         device=dev)) for s in sets]

    def srun(i):
        s, (sy, shf) = sets[i % 3], outs[i % 3]
        ssm.ssm_ssd_fwd(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"],
                        s["z"], s["dt_bias"], True, None, y=sy, h_final=shf,
                        workspace=sws, stream=stream)
    it = iter(range(1 << 30))
    settle(torch, lambda: srun(next(it)), stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        srun(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nb, nf = syn.ssd_bytes(scfg), syn.ssd_flops(scfg)
    return {
        "ms_per_call": round(ms, 4), "GBps": round(nb / (ms * 1e-3) / 1e9, 1),
        "TFLOPs": round(nf / (ms * 1e-3) / 1e12, 1),
        "hbm_frac": round(nb / (ms * 1e-3) / 8.0e12, 4),
        "algorithmic_bytes": nb, "flops": nf,
        "workspace_bytes": sws.numel(),
        "note": "prep (causal C^T B as a bf16 pair, C^T) + chunked scan; "
                "bound by per-chunk latency, not by HBM or the matrix cores"}


def cpu_baseline(inp, cfg, nbytes, log):
    """The fp64 oracle, as it stands, over the whole workload on the host
    cores (disjoint channel ranges on threads), median of 3 runs; beside it
    one thread on a bounded sample."""
    import statistics
    import oracle
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    # the host CPU share of a one-GPU machine is 16 cores, whatever the machine
    # has in all
    threads = max(1, min(16, avail))
    log("cpu baseline: oracle on %d threads (%d usable, %s in the machine), "
        "median of 3" % (threads, avail, os.cpu_count()))
    host = {k: (v.detach().to("cpu").double().numpy() if hasattr(v, "detach")
                else v) for k, v in inp.items()
            if k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.scan_threaded(host["u"], host["delta"], host["A"], host["B"],
                             host["C"], host["D"], host["z"],
                             host["delta_bias"], True, False, None,
                             threads=threads)
        times.append(time.perf_counter() - t0)
    sec = statistics.median(times)
    # one thread on the first 256 channels of each batch entry (a bounded
    # sample of the same workload), median of 3
    nd = min(256, cfg.dim)
    part = {k: (v[:, :nd] if k in ("u", "delta", "z") else
                v[:nd] if k in ("A", "D", "delta_bias") else v)
            for k, v in host.items()}
    times1 = []
    for _ in range(3):
        t1 = time.perf_counter()
        oracle.scan_threaded(part["u"], part["delta"], part["A"], part["B"],
                             part["C"], part["D"], part["z"],
                             part["delta_bias"], True, False, None, threads=1)
        times1.append(time.perf_counter() - t1)
    sec1 = statistics.median(times1)

    # the 130M-shaped layer whole (median of 3) and a bounded sample of the
    # long-context workload (64 channels over all 2^20 tokens, once), on the
    # same threads
    import synthetic as syn

    def host_inputs(c, **over):
        t = syn.make_scan_inputs(c, "cpu", **over)
        return {k: (v.double().numpy() if hasattr(v, "double") else v)
                for k, v in t.items()}

    def run_oracle(h, th):
        t0 = time.perf_counter()
        oracle.scan_threaded(h["u"], h["delta"], h["A"], h["B"], h["C"], h["D"],
                             h["z"], h["delta_bias"], True, False, None,
                             threads=th)
        return time.perf_counter() - t0
    c1 = syn.MAMBA_130M
    h1 = host_inputs(c1)
    sec_c1 = statistics.median([run_oracle(h1, threads) for _ in range(3)])
    del h1
    c3 = syn.LONG_1M
    n3 = 64
    h3 = host_inputs(c3, dim=n3)
    sec_c3 = run_oracle(h3, threads)
    del h3
    e3 = c3.batch * n3 * c3.seqlen
    return {"value": round(nbytes / sec / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": "the whole workload (%d x %d channels x %d tokens), "
                      "fp64, median of 3 runs: %.2f s wall each (%.1f s of "
                      "CPU work in all)" % (cfg.batch, cfg.dim, cfg.seqlen, sec,
                                            sum(times) * threads),
            "elements_per_s": round(cfg.elements / sec),
            "host_cpus_usable": avail, "host_cpus_total": os.cpu_count(),
            "one_thread_elements_per_s": round(cfg.batch * nd * cfg.seqlen / sec1),
            "one_thread_sample": "%d x %d channels x %d tokens, median %.2f s" % (
                cfg.batch, nd, cfg.seqlen, sec1),
            c1.name: {"elements_per_s": round(c1.elements / sec_c1),
                      "GBps": round(syn.algorithmic_bytes(c1) / sec_c1 / 1e9, 4),
                      "sample": "whole workload, median of 3: %.2f s" % sec_c1},
            c3.name: {"elements_per_s": round(e3 / sec_c3),
                      "sample": "%d of its %d channels over all %d tokens, "
                                "once: %.2f s" % (n3, c3.dim, c3.seqlen, sec_c3)},
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# bf16 activations, vector loads, softplus on, no conv prologue, Euler input,
# not the checkpoint pass
SCAN_KERNEL = "scan_kernel<unsigned short, true, true, false, false, false, 16>"
CKPT_KERNEL = "scan_kernel<unsigned short, true, true, false, false, true, 16>"
# the Euler backward sweep (bf16, vector loads, softplus, no ZOH); the
# --only-bwd run also times the ZOH and conv-prologue backward, whose
# kernels are left out of that summary
BWD_KERNEL = "bwd_kernel<unsigned short, true, true, false, 1>"
COPY_KERNEL = "roof_copy_kernel"
COPY_BYTES = 1 << 30  # each calibration copy reads and writes 1 GiB


def _csvs(d, suffix):
    import glob
    return sorted(glob.glob(os.path.join(d, "**", "*" + suffix),
                            recursive=True))


def _kernel_key(name):
    # demangled names come with or without the "void " of the return type
    n = name.replace("void ", "", 1) if name.startswith("void ssm::") else name
    return n.replace("ssm::(anonymous namespace)::", "").split("(")[0]


def summarize_profiles(d):
    """Writes profiles/scan_kernel_mamba2p8b_{kernel_stats.txt,traffic.json,
    traffic.txt} from rocprofv3 CSVs under ``d`` (see the module doc)."""
    import csv
    import statistics
    cmd_trace = ("rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace "
                 "-o bench -- python3 bench.py "
                 "--no-cpu-baseline")
    cmd_pmc = ("rocprofv3 --pmc {c} --output-format csv -d DIR/{d} -o {d} -- "
               "python3 bench.py --steps 3 --warmup 1 --no-extra "
               "--no-cpu-baseline")
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    # kernel statistics
    rows = []
    for f in _csvs(os.path.join(d, "trace"), "_kernel_stats.csv"):
        rows += list(csv.DictReader(open(f)))
    lines = ["# rocprofv3 kernel statistics, Mamba-2.8B-shaped scan benchmark",
             "# command (from /tmp, TMPDIR=/tmp): " + cmd_trace,
             "# summarized by: python3 bench.py --summarize DIR",
             "# kernel | calls | average us | min us | max us | total ms"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[:12]:
        lines.append("%s | %s | %.2f | %.2f | %.2f | %.3f" % (
            _kernel_key(r["Name"])[:90], r["Calls"],
            float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6))
    # The same scan instance also runs the 130M-shaped layer among the
    # extras: per-dispatch durations from the trace, split by launch grid
    # (the 2.8B layer: ceil(D/4) workgroups of 256 threads by batch).
    import synthetic as syn
    c2 = syn.MAMBA_2P8B
    grid_c2 = ((c2.dim + 3) // 4 * 256, c2.batch, 1)
    by_grid = {}
    for f in _csvs(os.path.join(d, "trace"), "_kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            if _kernel_key(r["Kernel_Name"]) != SCAN_KERNEL:
                continue
            g = (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]),
                 int(r["Grid_Size_Z"]))
            by_grid.setdefault(g, []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if by_grid:
        lines.append("# %s per launch grid (threads), from the kernel trace:"
                     % SCAN_KERNEL)
        for g in sorted(by_grid, key=lambda g: -len(by_grid[g])):
            v = by_grid[g]
            lines.append("grid %dx%dx%d%s | %d | %.2f | %.2f | %.2f | %.3f" % (
                g + (" (Mamba-2.8B layer)" if g == grid_c2 else "",
                     len(v), statistics.mean(v), min(v), max(v),
                     sum(v) / 1e3)))
    with open(os.path.join(prof, "scan_kernel_mamba2p8b_kernel_stats.txt"),
              "w") as f:
        f.write("\n".join(lines) + "\n")

    # HBM traffic from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), scaled by
    # what the same counter reads for the 1 GiB calibration copy.
    def per_dispatch(sub, counter, stat=statistics.median):
        vals = {}
        for f in _csvs(os.path.join(d, sub), "_counter_collection.csv"):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                k = _kernel_key(r["Kernel_Name"])
                vals.setdefault(k, []).append(float(r["Counter_Value"]))
        return {k: stat(v) for k, v in vals.items()}
    fetch = per_dispatch("fetch", "FETCH_SIZE")
    write = per_dispatch("write", "WRITE_SIZE")
    for k in (SCAN_KERNEL, COPY_KERNEL):
        if k not in fetch or k not in write:
            raise SystemExit("summarize: no counters for %r; kernels seen: %s"
                             % (k, sorted(set(fetch) | set(write))))
    fetch_scale = COPY_BYTES / 1024 / fetch[COPY_KERNEL]
    write_scale = COPY_BYTES / 1024 / write[COPY_KERNEL]
    fb = fetch[SCAN_KERNEL] * fetch_scale * 1024
    wb = write[SCAN_KERNEL] * write_scale * 1024
    alg = syn.algorithmic_bytes(syn.MAMBA_2P8B)
    out = {"kernel": SCAN_KERNEL, "workload": syn.MAMBA_2P8B.name,
           "kernel_source_sha256_16": kernel_source_hash(),
           "fetch_kib_raw": fetch[SCAN_KERNEL], "write_kib_raw": write[SCAN_KERNEL],
           "copy_fetch_kib_raw": fetch[COPY_KERNEL],
           "copy_write_kib_raw": write[COPY_KERNEL],
           "fetch_scale": fetch_scale, "write_scale": write_scale,
           "hbm_read_bytes_per_launch": int(fb),
           "hbm_write_bytes_per_launch": int(wb),
           "hbm_bytes_per_launch": int(fb + wb),
           "algorithmic_bytes_per_launch": alg,
           "traffic_over_algorithmic": (fb + wb) / alg,
           # the kernel-trace average over the 2.8B-layer dispatches of the
           # same profiled sources, to set beside a live run's events
           "kernel_trace_us_mean": (round(statistics.mean(by_grid[grid_c2]), 2)
                                    if grid_c2 in by_grid else None),
           "commands": [cmd_pmc.format(c="FETCH_SIZE", d="fetch"),
                        cmd_pmc.format(c="WRITE_SIZE", d="write"),
                        "python3 bench.py --summarize DIR"]}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    txt = ["# HBM traffic of the scan kernel, Mamba-2.8B-shaped workload",
           "# commands (from /tmp, TMPDIR=/tmp):"] + ["#   " + c for c in out["commands"]]
    txt += ["calibration: %s reads+writes 1 GiB per dispatch; FETCH_SIZE reads "
            "%.0f KiB (scale %.3f), WRITE_SIZE %.0f KiB (scale %.3f)" % (
                COPY_KERNEL, fetch[COPY_KERNEL], fetch_scale,
                write[COPY_KERNEL], write_scale),
            "scan kernel per dispatch: FETCH_SIZE %.0f KiB -> %.1f MB read; "
            "WRITE_SIZE %.0f KiB -> %.1f MB written" % (
                fetch[SCAN_KERNEL], fb / 1e6, write[SCAN_KERNEL], wb / 1e6),
            "HBM bytes per launch %.1f MB vs algorithmic %.1f MB (ratio %.3f)" % (
                (fb + wb) / 1e6, alg / 1e6, (fb + wb) / alg),
            "sources sha256[:16] %s (all of csrc/ and include/)"
            % out["kernel_source_sha256_16"]]
    with open(os.path.join(prof, "scan_kernel_mamba2p8b_traffic.txt"), "w") as f:
        f.write("\n".join(txt) + "\n")

    # SQ counters (VALU issue, transcendentals, LDS), if that pass was run
    sq_counters = ["SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU",
                   "SQ_INSTS_VALU_TRANS_F32", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY",
                   "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT"]
    sq = {c: per_dispatch("sq", c).get(SCAN_KERNEL) for c in sq_counters}
    sq_txt = []
    if all(v is not None for v in sq.values()):
        upd = syn.MAMBA_2P8B.elements * syn.MAMBA_2P8B.dstate
        slots = sq["SQ_ACTIVE_INST_VALU"]
        sq_txt = [
            "# SQ counters of the scan kernel, Mamba-2.8B-shaped workload",
            "# kernel: " + SCAN_KERNEL,
            "# command (from /tmp, TMPDIR=/tmp): " + cmd_pmc.format(
                c=" ".join(sq_counters), d="sq"),
            "# median per dispatch over the timed calls"]
        sq_txt += ["%-24s %14.0f" % (c, sq[c]) for c in sq_counters]
        sq_txt += [
            "VALU instructions per state-update: %.2f (x64 lanes / %d)" % (
                sq["SQ_INSTS_VALU"] * 64 / upd, upd),
            "VALU issue slots per state-update: %.2f" % (slots * 64 / upd),
            "transcendentals per state-update: %.2f" % (
                sq["SQ_INSTS_VALU_TRANS_F32"] * 64 / upd),
            "VALU busy time at 2.4 GHz, 4 cycles per wave64 slot, 1024 SIMDs: "
            "%.1f us" % (slots * 4 / (1024 * 2.4e9) * 1e6),
            "sources sha256[:16] %s (all of csrc/ and include/)"
            % kernel_source_hash()]
        with open(os.path.join(prof, "scan_kernel_mamba2p8b_sq_counters.txt"),
                  "w") as f:
            f.write("\n".join(sq_txt) + "\n")
    extra_txt = summarize_extras(d, rows, per_dispatch, fetch_scale, write_scale,
                                 cmd_trace, prof)
    print("\n".join(lines + txt + sq_txt + extra_txt))


def summarize_workload(d, rows, per_dispatch, fetch_scale, write_scale,
                       cmd_trace, prof, *, title, fname, keys, tag, only,
                       alg_bytes, alg_note, per_call=None):
    """profiles/<fname>: the trace statistics (from the full benchmark run)
    of the kernels whose names start with one of ``keys``, and their HBM
    traffic per dispatch from the ``--<only> --steps 3`` counter passes under
    DIR/<tag>fetch and DIR/<tag>write, scaled by the same copy calibration
    as the scan kernel's.  A listed kernel runs once per call unless
    ``per_call`` gives its dispatches per call (then its figure is the mean
    dispatch times that count)."""
    import csv
    import statistics

    def match(k):
        return any(k.startswith(p) for p in keys)
    txt = ["# %s" % title,
           "# kernel statistics from: " + cmd_trace,
           "# kernel | calls | average us | min us | max us | total ms"]
    for r in rows:
        k = _kernel_key(r["Name"])
        if match(k):
            txt.append("%s | %s | %.2f | %.2f | %.2f | %.3f" % (
                k[:90], r["Calls"], float(r["AverageNs"]) / 1e3,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                float(r["TotalDurationNs"]) / 1e6))
    # a kernel that other workloads of the benchmark launch too (another
    # shape, the same instance): its dispatches by launch grid
    by = {}
    for f in _csvs(os.path.join(d, "trace"), "_kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            k = _kernel_key(r["Kernel_Name"])
            if match(k):
                g = (int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]),
                     int(r["Grid_Size_Z"]))
                by.setdefault(k, {}).setdefault(g, []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for k in sorted(by):
        if len(by[k]) < 2:
            continue
        txt.append("# %s per launch grid (threads), from the kernel trace:" % k[:90])
        for g in sorted(by[k], key=lambda g: -len(by[k][g])):
            v = by[k][g]
            txt.append("grid %dx%dx%d | %d | %.2f | %.2f | %.2f | %.3f" % (
                g + (len(v), statistics.mean(v), min(v), max(v), sum(v) / 1e3)))
    if not os.path.isdir(os.path.join(d, tag + "fetch")):
        return []
    per_call = per_call or {}
    fetch = per_dispatch(tag + "fetch", "FETCH_SIZE")
    write = per_dispatch(tag + "write", "WRITE_SIZE")
    if per_call:
        fetch.update({k: v * per_call[k] for k, v in per_dispatch(
            tag + "fetch", "FETCH_SIZE", statistics.mean).items() if k in per_call})
        write.update({k: v * per_call[k] for k, v in per_dispatch(
            tag + "write", "WRITE_SIZE", statistics.mean).items() if k in per_call})
    cmd = ("rocprofv3 --pmc {c} --output-format csv -d DIR/{d} -o {d} -- "
           "python3 bench.py --%s --steps 3" % only)
    txt += ["# HBM traffic per dispatch from (from /tmp, TMPDIR=/tmp):",
            "#   " + cmd.format(c="FETCH_SIZE", d=tag + "fetch"),
            "#   " + cmd.format(c="WRITE_SIZE", d=tag + "write"),
            "# scaled by the 1 GiB copy calibration (fetch x %.3f, write x %.3f)"
            % (fetch_scale, write_scale)]
    total = 0.0
    for k in sorted(fetch):
        if not match(k) or k not in write:
            continue
        fb = fetch[k] * fetch_scale * 1024
        wb = write[k] * write_scale * 1024
        total += fb + wb
        txt.append("%s: read %.1f MB, written %.1f MB%s" % (
            k, fb / 1e6, wb / 1e6,
            " (%d dispatches per call)" % per_call[k] if k in per_call else ""))
    txt.append("per call: %.1f MB vs algorithmic %.1f MB (ratio %.3f; %s)"
               % (total / 1e6, alg_bytes / 1e6, total / alg_bytes, alg_note))
    txt += summarize_sq(d, per_dispatch, rows, tag + "sq", only, match)
    with open(os.path.join(prof, fname), "w") as f:
        f.write("\n".join(txt) + "\n")
    return txt


SQ_COUNTERS = ["SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU_TRANS_F32",
               "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES",
               "SQ_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT"]


def summarize_sq(d, per_dispatch, rows, sub, only, match):
    """SQ counters per dispatch (mean over the --<only> --steps 3 run under
    DIR/<sub>) of the matching kernels, with the VALU issue time they imply
    (4 cycles per wave64 issue slot over 1024 SIMDs at 2.4 GHz) beside the
    kernel-trace average: how busy the VALU keeps each kernel."""
    import statistics
    if not os.path.isdir(os.path.join(d, sub)):
        return []
    vals = {c: per_dispatch(sub, c, statistics.mean) for c in SQ_COUNTERS}
    avg_us = {_kernel_key(r["Name"]): float(r["AverageNs"]) / 1e3 for r in rows}
    txt = ["# SQ counters per dispatch (mean), from (from /tmp, TMPDIR=/tmp):",
           "#   rocprofv3 --pmc %s --output-format csv -d DIR/%s -o %s -- "
           "python3 bench.py --%s --steps 3" % (" ".join(SQ_COUNTERS), sub, sub, only)]
    for k in sorted(vals["SQ_ACTIVE_INST_VALU"]):
        if not match(k) or any(k not in vals[c] for c in SQ_COUNTERS):
            continue
        txt.append("%s:" % k)
        txt += ["  %-24s %16.0f" % (c, vals[c][k]) for c in SQ_COUNTERS]
        busy_us = vals["SQ_ACTIVE_INST_VALU"][k] * 4 / (1024 * 2.4e9) * 1e6
        line = "  VALU issue time %.1f us" % busy_us
        if k in avg_us:
            line += " against a kernel-trace average of %.1f us (%.0f %% busy)" % (
                avg_us[k], 100.0 * busy_us / avg_us[k])
        txt.append(line)
        txt.append("  waiting share SQ_WAIT_ANY / SQ_WAVE_CYCLES %.2f" % (
            vals["SQ_WAIT_ANY"][k] / max(vals["SQ_WAVE_CYCLES"][k], 1.0)))
    return txt


def summarize_extras(d, rows, per_dispatch, fetch_scale, write_scale, cmd_trace,
                     prof):
    """The SSD, decode and backward summaries under profiles/."""
    import selective_state_space_30_amd as ssm
    import synthetic as syn
    scfg, dcfg, bcfg = syn.MAMBA2_LAYER, syn.DECODE, syn.MAMBA_2P8B
    out = []
    out += summarize_workload(
        d, rows, per_dispatch, fetch_scale, write_scale, cmd_trace, prof,
        title="Mamba-2 SSD form, workload " + scfg.name,
        fname="ssd_kernel_%s.txt" % scfg.name, keys=["ssd_"], tag="ssd",
        only="only-ssd", alg_bytes=syn.ssd_bytes(scfg),
        alg_note="x, z, dt, B, C read, y written once")
    out += summarize_workload(
        d, rows, per_dispatch, fetch_scale, write_scale, cmd_trace, prof,
        title="decode step, workload %s (one ssm_state_update call)" % dcfg.name,
        fname="step_kernel_%s.txt" % dcfg.name,
        keys=["step_kernel<unsigned short, true, false>"],
        tag="decode", only="only-decode", alg_bytes=syn.decode_step_bytes(dcfg),
        alg_note="fp32 state read and written, x, delta, z, B, C read, y "
                 "written")
    out += summarize_workload(
        d, rows, per_dispatch, fetch_scale, write_scale, cmd_trace, prof,
        title="decode step with a width-4 conv, workload %s (one "
              "ssm_conv_state_update call)" % dcfg.name,
        fname="step_conv4_kernel_%s.txt" % dcfg.name,
        keys=["step_kernel<unsigned short, true, true>"],
        tag="decode", only="only-decode",
        alg_bytes=syn.conv_decode_step_bytes(dcfg, 4),
        alg_note="the plain step's bytes, the 3-input window read and "
                 "written, taps and conv bias read")
    out += summarize_workload(
        d, rows, per_dispatch, fetch_scale, write_scale, cmd_trace, prof,
        title="backward, workload %s (checkpoint pass, sweep, reductions; "
              "Euler input term)" % bcfg.name,
        fname="bwd_kernels_%s.txt" % bcfg.name,
        keys=[BWD_KERNEL, "bwd_reduce", CKPT_KERNEL], tag="bwd", only="only-bwd",
        alg_bytes=syn.backward_bytes(bcfg),
        alg_note="inputs and dy read, gradients written once; the partial "
                 "sums of dB and dC (written by every sweep launch, read back "
                 "by the next and by the reduction) are extra by design",
        per_call={BWD_KERNEL: ssm.ssm_scan_bwd_plan(
            bcfg.batch, bcfg.dim, bcfg.dstate, bcfg.seqlen)["sweep_launches"]})
    return out

if __name__ == "__main__":
    main()
