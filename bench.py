"""Benchmark of the tiered activation-sparse decoding GEMV on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode7b] [--sparsity 0.5]
                    [--no-cpu-baseline] [--no-batched] [--no-separate] [--no-deterministic]
                    [--control none|full|skip]

Default workload (decode7b): one step is one token of a 32-layer 7B-shaped decoder: for each
layer and each projection group (q|k|v, o, gate|up, down) one TopK-Guided tier mask (s +-
0.01, approximate tier = 3/10 of the kept channels, two-bit groups of 128 rows) and one
tiered GEMV over the fused fp16 matrices, in order (layer-serial).  Weights are synthetic
(fp16 N(0, 0.02), drawn on the device from a seed) and packed by spax_pack_columns before
timing; activations are seeded Laplace(0, 1) vectors, one per (token, layer, group), resident
in HBM before the timed region.

Other workloads (one JSON line each, never printed by the default run):
  decode7b-int4 : the same stack with int4 base columns (g128) and two-bit approximations,
                  TopK 25% FULL / 35% APPROX / 40% skipped.
  linear512     : one 512x512 layer (TopK 20% / 30% / 50%, two-bit groups of 64 rows): the
                  latency of one mask + GEMV call on a blob that stays in the cache.
  mlp7b         : gate|up 4096->2x11008 and down 11008->4096, per-channel LogNormal(0, 0.5)
                  scaled Laplace activations, TopK 30% / 30% / 40%; five weight copies cycled
                  (one MLP pass per token) so the 256 MB last-level cache does not hold them.
  host8b        : Llama-3-8B shapes with the blobs in pinned host memory: device masks (TopK
                  20% / 30% / 50%), then spax_tiered_gemv_pinned (merged ranges over PCIe).

Prints one JSON line.  ``value`` is microseconds per token (lower is better).  The
``roofline`` object is for the fused mask+GEMV kernel (the only kernel of the default step):
algorithmic bytes = selected column records + activations + tier bytes + index lists + y,
per launch, over its average launch duration (the timed step's event time over its launches).
``cpu_baseline`` times the oracle (float64 NumPy) on a bounded sample of the same workload on
the host cores.  ``batched`` is the same step in the batched launch form (all masks in one
launch, all GEMVs in one), legal here only because the synthetic inputs are independent.
``separate`` is the same step through the two stand-alone kernels per phase, the mask kernel
of spax_build_tiers and the GEMV kernel of spax_tiered_gemv.  ``deterministic`` is the step
with SPAX_STEP_DETERMINISTIC (y identical bit for bit from run to run).
``token_us`` gives the median and 90th percentile over the timed tokens, each timed on its
own after the timed region.  ``--control full|skip`` replaces the tier rule by all-FULL or
all-SKIP masks: controls for the hardware byte counters.  ``read_probe`` gives what a plain
streaming read (spax_read_probe) gets: its rate on one large read (also reported in
``roofline`` as a measured second denominator) and the time of the step's launch pattern
when every launch only reads its selected byte count (a floor for the layer-serial form).
For linear512 and mlp7b ``cpu_baseline`` also holds a one-thread run of the oracle.
``dense_baseline`` (fp16 workloads) times the same step without tiers through torch's fp16
matrix-vector product on the same weights, as context for the speedup over dense decoding.
``--fit`` (decode7b) adds ``fixed_cost_fit``: the layer-serial step at s = 0.3, 0.5 and 0.7 and
the line t = a + b * MB per fused launch through them.  ``--tier-fit`` (decode workloads) adds
``tier_fit``: the step with FULL-only and with APPROX-only masks at three sizes each, and per
tier the line through the time against the bytes, so the cost of each tier's bytes shows apart.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "tiered sparse GEMV µs/token (7B projections); achieved GB/s vs HBM peak"
HBM_PEAK_GBS = 8000.0
SEED = 20261003
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_phase_kernel_decode7b_s05_traffic.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="decode7b",
                    choices=["decode7b", "decode7b-int4", "mlp7b", "linear512", "host8b"])
    ap.add_argument("--sparsity", type=float, default=0.5, help="decode7b TopK-Guided target s")
    ap.add_argument("--delta", type=float, default=0.01)
    ap.add_argument("--layers", type=int, default=None, help="override the workload's layers")
    ap.add_argument("--tokens", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip timing the batched step form")
    ap.add_argument("--no-separate", action="store_true",
                    help="skip timing the two-launch step form")
    ap.add_argument("--fit", action="store_true",
                    help="decode7b: also time the layer-serial step at s = 0.3, 0.5 and 0.7 and "
                         "fit the per-launch time against the bytes per launch")
    ap.add_argument("--tier-fit", action="store_true",
                    help="decode workloads: also time the step with FULL-only and APPROX-only "
                         "masks at three sizes each and fit the time against the bytes, per "
                         "tier (layer-serial and, unless --no-batched, batched form)")
    ap.add_argument("--no-deterministic", action="store_true",
                    help="skip timing the SPAX_STEP_DETERMINISTIC form")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the plain streaming-read ceiling and floor")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense fp16 baseline (torch matmul on the same weights)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="before the timed steps, run one elementwise kernel (bitwise_not) that "
                         "reads and writes this many MiB: known traffic for scaling hardware "
                         "byte counters (use more than the 256 MB last-level cache)")
    ap.add_argument("--cpu-layers", type=int, default=None,
                    help="layers the oracle runs for the CPU baseline")
    ap.add_argument("--control", default="none", choices=["none", "full", "skip"],
                    help="decode workloads: replace the tier rule by all-FULL (reads the dense "
                         "bytes) or all-SKIP (reads almost nothing), as byte-counter controls")
    ap.add_argument("--gap", type=int, default=0, help="host8b: range merging gap (columns)")
    ap.add_argument("--transfer", default="gather", choices=["memcpy", "gather", "hostgather"],
                    help="host8b: one hipMemcpyAsync per range, one copy kernel reading the "
                         "mapped blob, or host threads gathering the ranges for one copy")
    ap.add_argument("--sweep", action="store_true",
                    help="host8b: also time every transfer at range gaps 0, 4 and 8")
    ap.add_argument("--placement", default="channel", choices=["channel", "frequency"],
                    help="host8b: records in channel order, or ordered by calibrated "
                         "selection frequency (jointly selected columns placed together)")
    return ap.parse_args()


def workload_spec(args):
    """Shapes, formats and tier rule of the chosen workload."""
    s, delta = args.sparsity, args.delta
    if args.workload == "decode7b":
        spec = dict(shapes=synth.decoder_phases_7b(), fmt=0, G=128, tiers=("guided", s, delta),
                    channel_scaled=False, layers=32, tokens_per_step=1, cpu_layers=24,
                    desc=f"decode7b: 32 layers x (q|k|v 4096->3x4096, o 4096->4096, gate|up "
                         f"4096->2x11008, down 11008->4096), fp16 weights, TopK-Guided mask "
                         f"s={s}+-{delta}, approx tier 3/10 of kept, 2-bit G=128, batch 1, "
                         f"layer-serial")
    elif args.workload == "decode7b-int4":
        spec = dict(shapes=synth.decoder_phases_7b(), fmt=1, G=128, tiers=("topk", 0.25, 0.35),
                    channel_scaled=False, layers=32, tokens_per_step=1, cpu_layers=16,
                    desc="decode7b-int4: 32 layers of 7B shapes, int4 base (g128, fp16 s/z) + "
                         "2-bit approx (g128), TopK 25/35/40, batch 1, layer-serial")
    elif args.workload == "mlp7b":
        spec = dict(shapes=synth.mlp_phases_7b(), fmt=0, G=128, tiers=("topk", 0.3, 0.3),
                    channel_scaled=True, layers=5, tokens_per_step=5, cpu_layers=5,
                    desc="mlp7b: gate|up 4096->2x11008 + down 11008->4096, fp16, TopK 30/30/40, "
                         "LogNormal(0,0.5)-scaled Laplace x, 2-bit G=128; 5 weight copies, one "
                         "MLP pass per token")
    elif args.workload == "linear512":
        spec = dict(shapes=[("linear", 512, [512])], fmt=0, G=64, tiers=("topk", 0.2, 0.3),
                    channel_scaled=False, layers=1, tokens_per_step=1, cpu_layers=1,
                    desc="linear512: one 512x512 fp16 layer, TopK 20/30/50, 2-bit G=64, batch "
                         "1; the blob (0.6 MB) stays in the last-level cache, so this is a "
                         "latency figure per call, not a bandwidth one")
    else:
        raise ValueError(args.workload)
    if args.control != "none":
        if args.workload in ("mlp7b", "linear512"):
            raise ValueError("--control applies to the decode workloads")
        spec["tiers"] = ("topk", 1.0, 0.0) if args.control == "full" else ("topk", 0.0, 0.0)
        spec["desc"] += f"; CONTROL: all channels {args.control.upper()} (TopK " + \
            ("d/0/0)" if args.control == "full" else "0/0/d)")
    if args.layers is not None:
        spec["desc"] = spec["desc"].replace(f"{spec['layers']} layers", f"{args.layers} layers", 1)
        spec["layers"] = args.layers
        if args.workload == "mlp7b":
            spec["tokens_per_step"] = args.layers
    if args.cpu_layers is not None:
        spec["cpu_layers"] = args.cpu_layers
    spec["cpu_layers"] = min(spec["cpu_layers"], spec["layers"])
    return spec


def tier_params(spax, spec, d_in):
    kind = spec["tiers"][0]
    if kind == "guided":
        _, s, delta = spec["tiers"]
        lo, hi = spax.spax_guided_bounds(d_in, s, delta)
        return spax.guided_params(-math.log(1.0 - s), lo, hi, 3, 10)
    _, pf, pa = spec["tiers"]
    nf, na = spax.spax_counts_from_fractions(d_in, pf, pa)
    return spax.topk_params(nf, na)


class Stack:
    """Packed weights, per-token activations and per-phase output buffers on the device."""

    def __init__(self, spax, torch, dev, layers, tokens, s=0.5, delta=0.01, spec=None):
        if spec is None:  # the default decode workload
            spec = dict(shapes=synth.decoder_phases_7b(), fmt=0, G=128,
                        tiers=("guided", s, delta), channel_scaled=False)
        self.spax, self.torch, self.dev, self.spec = spax, torch, dev, spec
        self.shapes = spec["shapes"]
        self.layers, self.tokens = layers, tokens
        self.layouts, self.packed, self.params, self.bufs = [], [], [], []
        t0 = time.time()
        for l in range(layers):
            for k, (name, d_in, d_out) in enumerate(self.shapes):
                L = spax.spax_layout_init(d_in, d_out, spec["fmt"], 128, spec["G"])
                packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
                Ws = [synth.weights_device(SEED, d_in, r, dev, l, k, m) for m, r in enumerate(d_out)]
                spax.spax_pack_columns(L, Ws, packed)
                del Ws
                T = int(L.d_out_total)
                self.layouts.append(L)
                self.packed.append(packed)
                self.params.append(tier_params(spax, spec, d_in))
                self.bufs.append(dict(
                    tier=torch.empty(d_in, dtype=torch.uint8, device=dev),
                    f=torch.empty(d_in, dtype=torch.int32, device=dev),
                    a=torch.empty(d_in, dtype=torch.int32, device=dev),
                    c=torch.zeros(3, dtype=torch.int32, device=dev),
                    y=torch.empty(T, dtype=torch.float32, device=dev)))
        torch.cuda.synchronize()
        log(f"[bench] packed {layers} layers in {time.time() - t0:.1f} s, "
            f"{sum(int(L.total_bytes) for L in self.layouts) / 1e9:.2f} GB")
        # activations: one fp16 vector per (token, layer, group)
        self.x = []
        for t in range(tokens):
            row = []
            for l in range(layers):
                for k, (name, d_in, d_out) in enumerate(self.shapes):
                    row.append(torch.from_numpy(synth.activations(
                        SEED, d_in, t, l, k, channel_scaled=spec["channel_scaled"])).to(dev))
            self.x.append(row)
        self.phase_arrays = []
        for t in range(tokens):
            ph = [spax.make_phase(L, pk, x, p, b["tier"], b["f"], b["a"], b["c"], b["y"])
                  for L, pk, x, p, b in zip(self.layouts, self.packed, self.x[t], self.params, self.bufs)]
            self.phase_arrays.append(spax.phase_array(ph))
        self.ws = torch.zeros(spax.spax_step_workspace_bytes(self.phase_arrays[0]),
                              dtype=torch.uint8, device=dev)

    flags = 0

    def step(self, t):
        self.spax.spax_decode_step_projections(self.phase_arrays[t % self.tokens], self.ws,
                                               flags=self.flags)

    def algorithmic_bytes(self, i, counts):
        """Bytes phase i must move for a mask with these counts: the selected column
        records, x, the tier bytes, both index lists and y (read or written once each)."""
        L = self.layouts[i]
        nF, nA = int(counts[0]), int(counts[1])
        return (nF * int(L.rec_F) + nA * int(L.rec_A) + 2 * int(L.d_in) + int(L.d_in)
                + 4 * (nF + nA) + 4 * int(L.d_out_total))

    def timed_kernels(self, t):
        """The same decode step with events recorded by the library right before and after
        each phase's fused launch on the launch stream."""
        torch = self.torch
        n = len(self.layouts)
        if not hasattr(self, "events"):
            self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
            for e in self.events:   # creates the underlying HIP events
                e.record()
            torch.cuda.synchronize()
        self.spax.spax_decode_step_projections(self.phase_arrays[t % self.tokens], self.ws,
                                               events=self.events, flags=self.flags)
        torch.cuda.synchronize()
        counts = [b["c"].cpu().numpy() for b in self.bufs]
        ms = [self.events[2 * i].elapsed_time(self.events[2 * i + 1]) for i in range(n)]
        return ms, counts


# The sources the fused decode kernel is compiled from: its recorded byte counters stay valid
# while these are unchanged (comments aside).
KERNEL_SOURCES = [os.path.join(ROOT, "activation_sparse_tiered_amd", "csrc", f)
                  for f in ("decode.hip", "gemv_core.h", "mask_core.h", "common.h")] + \
                 [os.path.join(ROOT, "include", "spax.h")]


def _strip_c_comments(text: str) -> str:
    """C/C++ source without its comments (block and line; string literals kept), every run of
    white space reduced to one space, so that rewording or rewrapping a comment leaves it
    unchanged."""
    import re
    pat = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\])*"', re.S)
    code = pat.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
    return " ".join(code.split())


def _build_id():
    """Flags and compiler banner recorded by the build next to the library ('' if absent)."""
    path = os.path.join(ROOT, "activation_sparse_tiered_amd", "libspax.so.buildinfo")
    try:
        with open(path, encoding="utf-8") as fh:
            return " ".join(fh.read().split())
    except OSError:
        return ""


def sources_sha256():
    """sha256 over the fused kernel's sources without their comments (name, then text; in
    the order of KERNEL_SOURCES), then the build flags and compiler banner the build recorded:
    the recorded byte counters stay valid only for the same code built the same way."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_strip_c_comments(fh.read()).encode())
    h.update(_build_id().encode())
    return h.hexdigest()


def recorded_traffic(args):
    """HBM MB per fused launch from the committed FETCH_SIZE / WRITE_SIZE summary, scaled by
    its copy calibration; None unless this is the workload it was taken on and the kernel
    sources are unchanged since."""
    if (args.workload, args.sparsity, args.delta, args.layers, args.control) != \
            ("decode7b", 0.5, 0.01, None, "none") or not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if ":" in line and line.split(":")[0] in ("traffic_MB_per_launch", "sources_sha256"):
                k, v = line.split(":", 1)
                vals[k] = v.strip()
    if vals.get("sources_sha256") != sources_sha256() or "traffic_MB_per_launch" not in vals:
        return None
    return float(vals["traffic_MB_per_launch"])


def cpu_baseline(stack, layers, threads=None, min_seconds=2.0):
    """The oracle on `layers` layers of token 0, timed on the host, scaled to one token;
    the whole sample is repeated until it has taken at least `min_seconds` (small workloads)
    and the mean is reported.  Each phase's weights are drawn (on the device, as for the GPU
    run) and copied to the host right before it is timed, so only one phase is held in host
    memory at a time.  `threads`: BLAS threads (default: every core this process may run on)."""
    from oracle import gemv as ogemv
    from oracle import pack as opack
    from oracle import tiers as otiers
    spec = stack.spec
    cores = threads or len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        limiter = None
    dt = 0.0
    reps = 0
    while reps == 0 or dt < min_seconds:
        dt += _oracle_pass(stack, spec, layers, ogemv, opack, otiers)
        reps += 1
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    per_token_us = dt / reps / layers * stack.layers * 1e6 / spec["tokens_per_step"]
    return {"value": round(per_token_us, 1), "unit": "us/token", "cores": cores, "kind": "oracle",
            "sample": f"{layers} of {stack.layers} layers ({len(stack.shapes)} projection groups "
                      f"each) of one token, {reps} time(s): float64 NumPy tier mask + tiered "
                      f"GEMV, scaled to one token; {dt:.1f} s measured; BLAS threads = {cores}"}


def _oracle_pass(stack, spec, layers, ogemv, opack, otiers):
    """Seconds the oracle takes for `layers` layers of token 0 (weights drawn untimed)."""
    dt = 0.0
    for l in range(layers):
        for k, (name, d_in, d_out) in enumerate(stack.shapes):
            Ws = [synth.weights_device(SEED, d_in, r, stack.dev, l, k, m).cpu().numpy()
                  for m, r in enumerate(d_out)]
            O = opack.Layout(d_in, d_out, spec["fmt"], 128, spec["G"])
            x = synth.activations(SEED, d_in, 0, l, k, channel_scaled=spec["channel_scaled"])
            kind = spec["tiers"][0]
            t0 = time.perf_counter()
            if kind == "guided":
                _, s, delta = spec["tiers"]
                lo, hi = otiers.guided_bounds(d_in, s, delta)
                _, f, a, _ = otiers.build_tiers(x, otiers.MODE_TOPK_GUIDED, tau=-math.log(1 - s),
                                                n_lo=lo, n_hi=hi, num=3, den=10)
            else:
                nf, na = otiers.counts_from_fractions(d_in, spec["tiers"][1], spec["tiers"][2])
                _, f, a, _ = otiers.build_tiers(x, otiers.MODE_TOPK, n_full=nf, n_approx=na)
            ogemv.tiered_gemv(O, Ws, x, f, a)
            dt += time.perf_counter() - t0
            del Ws
    return dt


def read_probe(spax, torch, dev, launch_bytes, reps=8):
    """What a launch that only reads gets, with spax_read_probe (16-byte non-temporal loads
    over the whole GPU, nothing else): (1) the ceiling, its rate on one 2 GiB read; (2) the
    floor of the timed step's launch pattern, i.e. the same number of launches back to back
    on one stream, each reading as many bytes as that launch of the step selects (from
    consecutive places of the 2 GiB buffer, so the last-level cache does not hold them)."""
    big = 2 << 30
    buf = torch.empty(big, dtype=torch.uint8, device=dev)
    out = torch.zeros(8192, dtype=torch.int32, device=dev)
    f = spax.lib.spax_read_probe
    stream = torch.cuda.current_stream().cuda_stream
    base, outp = buf.data_ptr(), out.data_ptr()

    def run(ranges):
        # raw ctypes calls on precomputed pointers keep the host ahead of the GPU
        bad = 0
        for o, n in ranges:
            bad |= f(base + o, n, outp, 8192, None, stream)
        if bad:
            raise RuntimeError(f"spax_read_probe failed: {spax.lib.spax_last_error()}")

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(ranges):
        run(ranges)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            run(ranges)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps  # us per pass

    ceil_us = timed([(0, big)])
    ranges, off = [], 0
    for b in launch_bytes:
        n = int(b) // 16 * 16
        if off + n > big:
            off = 0
        ranges.append((off, n))
        off += (n + 4095) // 4096 * 4096
    floor_us = timed(ranges)
    total = sum(n for _, n in ranges)
    del buf, out
    return {"ceiling_GBps": round(big / (ceil_us * 1e-6) / 1e9, 1),
            "floor_us_per_step": round(floor_us, 2),
            "floor_GBps": round(total / (floor_us * 1e-6) / 1e9, 1),
            "launches_per_step": len(ranges),
            "what": "spax_read_probe (a plain streaming read, 16-byte non-temporal loads): "
                    "ceiling = one 2 GiB read; floor = the timed step's launches back to back, "
                    "each reading that launch's selected byte count"}


def time_form(stack, flags, args):
    """ms per step of the same step in another launch form (warm-up, then the timed steps
    between two events on the launch stream); the stack returns to the default form."""
    import torch
    stack.flags = flags
    try:
        for t in range(args.warmup):
            stack.step(t)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(args.steps):
            stack.step(args.warmup + t)
        e1.record()
        torch.cuda.synchronize()
    finally:
        stack.flags = 0
    return e0.elapsed_time(e1) / args.steps


def dense_baseline(stack, reps=10):
    """The same step without tiers, as context for the speedup over dense decoding: per phase
    one torch fp16 matrix-vector product (the vendor BLAS) of the phase's dense weights with
    the activation vector, W [sum d_out, d_in] (the matrices of a phase stacked, row-major:
    of the layouts and calls tried, torch.mv on this one was the fastest) times x [d_in]; the
    dense weights of every layer resident in HBM, phases in order on one stream."""
    torch, dev, spec = stack.torch, stack.dev, stack.spec
    Ws, xs = [], []
    for l in range(stack.layers):
        for k, (name, d_in, d_out) in enumerate(stack.shapes):
            Ws.append(torch.cat([synth.weights_device(SEED, d_in, r, dev, l, k, m)
                                 for m, r in enumerate(d_out)], dim=1).t().contiguous())
            xs.append(stack.x[0][l * len(stack.shapes) + k])
    dense_bytes = sum(w.numel() * 2 for w in Ws)

    def step():
        for w, x in zip(Ws, xs):
            torch.mv(w, x)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        step()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps / spec["tokens_per_step"]
    del Ws
    return {"value": round(us, 2), "unit": "us/token",
            "GBps": round(dense_bytes / spec["tokens_per_step"] / (us * 1e-6) / 1e9, 1),
            "dense_GB_per_token": round(dense_bytes / spec["tokens_per_step"] / 1e9, 4),
            "kind": "torch.mv in fp16 per phase (W [sum d_out, d_in] row-major times x), "
                    "dense weights in HBM, same shapes and weights, phases in order"}


def layer_serial_point(spax, torch, dev, spec, args):
    """One layer-serial measurement of a workload: (µs per launch, algorithmic MB per launch)
    over `args.steps` timed steps after `args.warmup`, bytes from the device counts of the
    timed tokens."""
    stack = Stack(spax, torch, dev, spec["layers"], args.tokens, spec=spec)
    for t in range(args.warmup):
        stack.step(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(args.steps):
        stack.step(args.warmup + t)
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / args.steps
    tok_bytes = {}
    for t in range(args.warmup, args.warmup + args.steps):
        key = t % stack.tokens
        if key not in tok_bytes:
            _, counts = stack.timed_kernels(t)
            tok_bytes[key] = sum(stack.algorithmic_bytes(i, c) for i, c in enumerate(counts))
    n = len(stack.layouts)
    step_bytes = float(np.mean([tok_bytes[t % stack.tokens]
                                for t in range(args.warmup, args.warmup + args.steps)]))
    del stack
    torch.cuda.empty_cache()
    return step_ms * 1e3 / n, step_bytes / n / 1e6


def fixed_cost_fit(spax, torch, dev, args, main_point):
    """The layer-serial decode7b step at s = 0.3, 0.5 and 0.7 (the timed run's point reused
    for its own s) and the least-squares line t = a + b * MB per launch."""
    points = []
    for s in (0.3, 0.5, 0.7):
        if abs(s - args.sparsity) < 1e-9:
            points.append((s,) + main_point)
            continue
        a2 = argparse.Namespace(**vars(args))
        a2.sparsity = s
        us, mb = layer_serial_point(spax, torch, dev, workload_spec(a2), args)
        log(f"[bench] fit point s={s}: {us:.3f} us, {mb:.3f} MB per launch")
        points.append((s, us, mb))
    mbs = np.array([p[2] for p in points])
    uss = np.array([p[1] for p in points])
    b, a = np.polyfit(mbs, uss, 1)
    return {"points": [{"s": p[0], "us_per_launch": round(p[1], 3), "MB_per_launch": round(p[2], 3)}
                       for p in points],
            "intercept_us": round(float(a), 3), "slope_us_per_MB": round(float(b), 5),
            "marginal_TBps": round(1.0 / float(b), 3) if b > 0 else None,  # MB/us = TB/s
            "what": "layer-serial fused launches: t = intercept + slope x algorithmic MB per "
                    "launch over the three skip targets"}


# One tier at a time: TopK masks that select only FULL columns, or only APPROX columns, for
# these fractions of the channels (the rest skipped).
TIER_FIT_POINTS = (("FULL", ((0.1, 0.0), (0.3, 0.0), (0.6, 0.0))),
                   ("APPROX", ((0.0, 0.2), (0.0, 0.4), (0.0, 0.7))))


def _line(xs, ys):
    b, a = np.polyfit(np.array(xs), np.array(ys), 1)
    return float(a), float(b)


def tier_fit(spax, torch, dev, args, spec):
    """The workload's step with one tier only, at three sizes per tier, and per tier the
    least-squares lines t = a + b * MB per fused launch (layer-serial form) and, unless
    --no-batched, t = a + b * GB per step (batched form): what each tier's bytes cost at the
    margin.  Bytes are the algorithmic ones, from the device counts of every token."""
    out = {}
    for tier, pts in TIER_FIT_POINTS:
        rows = []
        for f, a in pts:
            stack = Stack(spax, torch, dev, spec["layers"], args.tokens,
                          spec=dict(spec, tiers=("topk", f, a)))
            n = len(stack.layouts)
            ls_ms = time_form(stack, 0, args)
            bt_ms = None if args.no_batched else time_form(stack, spax.STEP_BATCHED, args)
            step_bytes = 0.0
            for t in range(stack.tokens):
                _, counts = stack.timed_kernels(t)
                step_bytes += sum(stack.algorithmic_bytes(i, c) for i, c in enumerate(counts))
            step_bytes /= stack.tokens
            del stack
            torch.cuda.empty_cache()
            row = {"full": f, "approx": a, "us_per_launch": round(ls_ms * 1e3 / n, 3),
                   "MB_per_launch": round(step_bytes / n / 1e6, 3),
                   "GB_per_step": round(step_bytes / 1e9, 4)}
            if bt_ms is not None:
                row["batched_us_per_step"] = round(bt_ms * 1e3, 1)
            log(f"[bench] tier fit {tier} {row}")
            rows.append(row)
        a0, b = _line([r["MB_per_launch"] for r in rows], [r["us_per_launch"] for r in rows])
        entry = {"points": rows,
                 "layer_serial": {"intercept_us": round(a0, 3), "slope_us_per_MB": round(b, 5),
                                  "marginal_TBps": round(1.0 / b, 3) if b > 0 else None}}
        if not args.no_batched:
            a1, b1 = _line([r["GB_per_step"] for r in rows],
                           [r["batched_us_per_step"] for r in rows])
            entry["batched"] = {"intercept_us": round(a1, 1), "slope_us_per_GB": round(b1, 2),
                                "marginal_TBps": round(1e3 / b1, 3) if b1 > 0 else None}
        out[tier] = entry
    out["what"] = ("the step with FULL-only or APPROX-only TopK masks: per tier, time against "
                   "algorithmic bytes (MB per fused launch, layer-serial; GB per step, batched)")
    return out


def device_bench(args, spax, torch, dev):
    spec = workload_spec(args)
    per_tok = spec["tokens_per_step"]
    stack = Stack(spax, torch, dev, spec["layers"], args.tokens, spec=spec)

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.bitwise_not(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- warmup, then exactly `steps` timed steps
    for t in range(args.warmup):
        stack.step(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record()
    for t in range(args.steps):
        stack.step(args.warmup + t)
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3
    step_ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] {args.workload} step: {step_ms * 1e3:.1f} us (event), "
        f"wall {wall_ms / args.steps:.3f} ms/step, {per_tok} token(s) per step")

    # ---- bytes: the masks of the timed tokens (deterministic per token) give the counts
    n_ph = len(stack.layouts)
    tok_bytes = {}
    per_phase = {}
    launch_bytes = None  # per launch, first timed token
    for t in range(args.warmup, args.warmup + args.steps):
        key = t % stack.tokens
        if key in tok_bytes:
            continue
        ms, counts = stack.timed_kernels(t)
        tb = 0
        lb = []
        for i, (m, c) in enumerate(zip(ms, counts)):
            b = stack.algorithmic_bytes(i, c)
            tb += b
            lb.append(b)
            pb = per_phase.setdefault(stack.shapes[i % len(stack.shapes)][0], [0, 0.0, 0])
            pb[0] += b
            pb[1] += m
            pb[2] += 1
        tok_bytes[key] = tb
        if launch_bytes is None:
            launch_bytes = lb
    timed_bytes = [tok_bytes[t % stack.tokens] for t in range(args.warmup, args.warmup + args.steps)]
    bytes_per_step = float(np.mean(timed_bytes))
    # The timed step is one fused launch per phase (plus one small clearing launch), back to
    # back on one stream: the kernel's average launch duration is the step time over the
    # launches, measured by the events around the timed region.
    avg_launch_ms = step_ms / n_ph
    avg_bytes = bytes_per_step / n_ph
    achieved = avg_bytes / (avg_launch_ms * 1e-3) / 1e9
    for name, (b, m, n) in per_phase.items():
        log(f"[bench]   {name:7s}: {b / n / 1e6:7.2f} MB per launch; event-bracketed launch "
            f"{m / n * 1e3:7.2f} us (includes the launch gap)")
    log(f"[bench] fused kernel: {avg_launch_ms * 1e3:.2f} us/launch, {avg_bytes / 1e6:.2f} MB/launch, "
        f"{achieved:.1f} GB/s; selected bytes/step {bytes_per_step / 1e9:.3f} GB")

    # ---- the masks of one timed token read from block storage (4 KiB blocks): selected bytes
    # against bytes physically read
    stack.step(args.warmup)
    torch.cuda.synchronize()
    lists = []
    for b in stack.bufs:
        cnt = b["c"].cpu().numpy()
        lists.append((b["f"].cpu().numpy()[:cnt[0]], b["a"].cpu().numpy()[:cnt[1]]))
    storage = storage_account(spax, stack.layouts, lists, 4096, 0)
    for k in ("selected_GB", "moved_GB", "read_GB"):
        storage[k] = round(storage[k] / per_tok, 4)
    log(f"[bench] storage ledger {storage}")

    # ---- per-token spread: the same steps again, each between its own pair of events
    # (outside the timed region above)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record()
    for t in range(args.steps):
        stack.step(args.warmup + t)
        ev[t + 1].record()
    torch.cuda.synchronize()
    tok_us = np.array([ev[t].elapsed_time(ev[t + 1]) * 1e3 / per_tok for t in range(args.steps)])
    token_us = {"median": round(float(np.median(tok_us)), 2),
                "p90": round(float(np.percentile(tok_us, 90)), 2), "n": int(args.steps)}
    log(f"[bench] per token: median {token_us['median']} us, p90 {token_us['p90']} us")

    # ---- the batched form of the same step (all masks in one launch, all GEMVs in one launch):
    # legal here only because the synthetic phase inputs are independent; reported beside the
    # layer-serial value, never as it
    batched = None
    if not args.no_batched:
        bt_ms = time_form(stack, spax.STEP_BATCHED, args)
        bgbs = bytes_per_step / (bt_ms * 1e-3) / 1e9
        batched = {"value": round(bt_ms * 1e3 / per_tok, 2), "unit": "us/token",
                   "achieved_GBps": round(bgbs, 1), "frac": round(bgbs / HBM_PEAK_GBS, 4),
                   "form": f"SPAX_STEP_BATCHED: all {n_ph} masks in one launch, then all GEMVs in "
                           "one persistent launch; valid only because the phase inputs are "
                           "independent"}
        log(f"[bench] batched step: {bt_ms * 1e3:.1f} us, {bgbs:.1f} GB/s")

    # ---- the two-launch form of the same step (per phase, the stand-alone mask kernel of
    # spax_build_tiers, then the stand-alone GEMV kernel of spax_tiered_gemv): what a caller
    # of those two entry points gets, reported beside the fused value
    separate = None
    if not args.no_separate:
        separate = {"value": round(time_form(stack, spax.STEP_SEPARATE, args) * 1e3 / per_tok, 2),
                    "unit": "us/token",
                    "form": f"SPAX_STEP_SEPARATE: per phase a build_tiers_kernel launch and a "
                            f"tiered_gemv_kernel launch ({2 * n_ph} launches per step), phases in order"}
        sgbs = bytes_per_step / (separate["value"] * per_tok * 1e-6) / 1e9
        separate["achieved_GBps"] = round(sgbs, 1)
        separate["frac"] = round(sgbs / HBM_PEAK_GBS, 4)
        log(f"[bench] two-launch step: {separate['value'] * per_tok:.1f} us, {sgbs:.1f} GB/s")

    # ---- the deterministic form (chunk partial sums in the workspace plus one fixed-order
    # reduce launch per phase that has several column chunks; waves keep to their own lists)
    deterministic = None
    if not args.no_deterministic:
        dt_ms = time_form(stack, spax.STEP_DETERMINISTIC, args)
        dgbs = bytes_per_step / (dt_ms * 1e-3) / 1e9
        deterministic = {"value": round(dt_ms * 1e3 / per_tok, 2), "unit": "us/token",
                         "achieved_GBps": round(dgbs, 1), "frac": round(dgbs / HBM_PEAK_GBS, 4),
                         "form": "SPAX_STEP_DETERMINISTIC: y identical bit for bit from run to "
                                 "run; the fused launch per phase plus a reduce launch"}
        log(f"[bench] deterministic step: {dt_ms * 1e3:.1f} us, {dgbs:.1f} GB/s")

    dense = None
    if not args.no_dense and spec["fmt"] == 0 and args.control == "none":
        dense = dense_baseline(stack)
        dense["speedup_layer_serial"] = round(dense["value"] / (step_ms * 1e3 / per_tok), 3)
        if batched is not None:
            dense["speedup_batched"] = round(dense["value"] / batched["value"], 3)
        log(f"[bench] dense baseline {dense}")

    probe = None
    if not args.no_read_probe:
        probe = read_probe(spax, torch, dev, launch_bytes)
        probe["floor_us_per_token"] = round(probe["floor_us_per_step"] / per_tok, 2)
        log(f"[bench] read probe {probe}")

    cpu = None
    fit = None
    if args.fit and args.workload == "decode7b" and args.control == "none":
        fit = fixed_cost_fit(spax, torch, dev, args, (avg_launch_ms * 1e3, avg_bytes / 1e6))
        log(f"[bench] fixed-cost fit {fit}")

    tfit = None
    if args.tier_fit and args.workload in ("decode7b", "decode7b-int4") and args.control == "none":
        tfit = tier_fit(spax, torch, dev, args, spec)

    if not args.no_cpu_baseline:
        cpu = cpu_baseline(stack, spec["cpu_layers"])
        if args.workload in ("linear512", "mlp7b"):
            one = cpu_baseline(stack, spec["cpu_layers"], threads=1)
            cpu["one_thread"] = {"value": one["value"], "unit": one["unit"], "cores": 1,
                                 "sample": one["sample"]}
        log(f"[bench] cpu baseline {cpu}")

    return {
        "metric": METRIC,
        "value": round(step_ms * 1e3 / per_tok, 2),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec["desc"], "layers": spec["layers"], "tokens": args.tokens,
                   "tokens_per_step": per_tok,
                   "selected_GB_per_token": round(bytes_per_step / per_tok / 1e9, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(args),
                     "traffic_source": (f"recorded: {os.path.relpath(TRAFFIC_FILE, ROOT)} "
                                        f"(rocprofv3 FETCH_SIZE/WRITE_SIZE runs of the same "
                                        f"sources, flags and compiler, sha256 "
                                        f"{sources_sha256()[:16]})"
                                        if recorded_traffic(args) is not None else None),
                     "traffic_unit": "MB per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "kernel": "fused_phase_kernel<%s>" % ("fp16" if spec["fmt"] == 0 else "int4"),
                     "avg_launch_us": round(avg_launch_ms * 1e3, 3),
                     "avg_algorithmic_MB": round(avg_bytes / 1e6, 3),
                     "measured_read_GBps": probe["ceiling_GBps"] if probe else None,
                     "frac_of_measured_read": (round(achieved / probe["ceiling_GBps"], 4)
                                               if probe else None)},
        "cpu_baseline": cpu,
        "batched": batched,
        "separate": separate,
        "deterministic": deterministic,
        "token_us": token_us,
        "read_probe": probe,
        "dense_baseline": dense,
        "storage_4KiB": storage,
        "fixed_cost_fit": fit,
        "tier_fit": tfit,
    }


def calibrated_order(spax, torch, dev, L, params, d_in, layer, group, tokens=16):
    """Record order from calibration masks (spax_placement_order over the masks of `tokens`
    calibration activations, distinct from the timed ones): channels by descending selected
    bytes.  Returns the order as a device int32 tensor (position p holds channel order[p])."""
    tier = torch.empty(d_in, dtype=torch.uint8, device=dev)
    f = torch.empty(d_in, dtype=torch.int32, device=dev)
    a = torch.empty(d_in, dtype=torch.int32, device=dev)
    c = torch.zeros(3, dtype=torch.int32, device=dev)
    masks = []
    for t in range(tokens):
        xc = torch.from_numpy(synth.activations(SEED, d_in, 1000 + t, 100 + layer, group,
                                                channel_scaled=True)).to(dev)
        spax.spax_build_tiers(xc, d_in, params, tier, f, a, c)
        masks.append(tier.cpu().numpy().copy())
    order = spax.spax_placement_order(L, np.stack(masks))
    return torch.from_numpy(order).to(dev)


def storage_account(spax, layouts, lists, block=4096, gap=0):
    """Bytes selected against bytes read from block storage (spax_storage_ledger, blocks of
    `block` bytes, each merged range one read request) summed over the phases of one token.
    ``lists``: per phase, (full_idx, approx_idx) host arrays."""
    sel = moved = read = ranges = 0
    for L, (f, a) in zip(layouts, lists):
        st = spax.spax_storage_ledger(L, f, a, gap, block)
        sel += st.selected_bytes
        moved += st.moved_bytes
        read += st.read_bytes
        ranges += st.n_ranges
    return {"block_bytes": block, "gap": gap, "selected_GB": round(sel / 1e9, 4),
            "moved_GB": round(moved / 1e9, 4), "read_GB": round(read / 1e9, 4),
            "read_over_selected": round(read / sel, 4) if sel else None,
            "read_requests": int(ranges),
            "what": "the token's masks read from block storage: each merged record range one "
                    "request rounded out to whole blocks of the blob (spax_storage_ledger)"}


HOST_TRANSFERS = {"memcpy": 0, "gather": 1, "hostgather": 2}


def host_bench(args, spax, torch, dev):
    """Llama-3-8B shapes, blobs in pinned host memory: per phase a device mask, then
    spax_tiered_gemv_pinned (ranges over PCIe).  Compared with the measured single-copy pinned
    host-to-device bandwidth.  Every layer distinct (32 by default); if pinned memory runs
    out, the layers that fit are timed and the result scaled to 32 (stated in the output)."""
    shapes = synth.decoder_phases_8b()
    want_layers = args.layers if args.layers is not None else 32
    t0 = time.time()
    phases = []
    alloc_note = None
    for l in range(want_layers):
        built = []
        try:
            for k, (name, d_in, d_out) in enumerate(shapes):
                L = spax.spax_layout_init(d_in, d_out, 0, 128, 128)
                nf, na = spax.spax_counts_from_fractions(d_in, 0.2, 0.3)
                params = spax.topk_params(nf, na)
                host = torch.empty(int(L.total_bytes), dtype=torch.uint8, pin_memory=True)
                dblob = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
                Ws = [synth.weights_device(SEED, d_in, r, dev, 100 + l, k, m)
                      for m, r in enumerate(d_out)]
                x = torch.from_numpy(synth.activations(SEED, d_in, 0, 100 + l, k,
                                                       channel_scaled=True)).to(dev)
                if args.placement == "frequency":
                    # Offline placement from calibration masks; the activations are permuted
                    # alike (a model does it once through the rows of the layer producing x).
                    perm = calibrated_order(spax, torch, dev, L, params, d_in, l, k)
                    spax.spax_pack_columns_placed(L, Ws, perm, dblob)
                    x = x[perm.long()].contiguous()
                else:
                    spax.spax_pack_columns(L, Ws, dblob)
                del Ws
                host.copy_(dblob)
                del dblob
                built.append(dict(L=L, host=host, x=x, p=params, d=d_in,
                                  f=torch.empty(d_in, dtype=torch.int32, device=dev),
                                  a=torch.empty(d_in, dtype=torch.int32, device=dev),
                                  c=torch.zeros(3, dtype=torch.int32, device=dev),
                                  y=torch.empty(int(L.d_out_total), dtype=torch.float32,
                                                device=dev)))
        except RuntimeError as e:  # pinned (or device) memory exhausted
            alloc_note = (f"allocation failed at layer {l} of {want_layers} "
                          f"({str(e).splitlines()[0][:120]}); {l} layers timed")
            log(f"[bench] host8b: {alloc_note}")
            del built
            torch.cuda.empty_cache()
            break
        phases.extend(built)
    n_layers = len(phases) // len(shapes)
    if n_layers == 0:
        raise RuntimeError(f"host8b: no layer fits in pinned memory ({alloc_note})")
    torch.cuda.synchronize()
    ws = torch.empty(max(spax.spax_pinned_workspace_bytes(ph["L"]) for ph in phases),
                     dtype=torch.uint8, device=dev)
    pinned_gb = sum(int(ph["L"].total_bytes) for ph in phases) / 1e9
    log(f"[bench] host8b: {n_layers} distinct layers in pinned memory ({pinned_gb:.2f} GB), "
        f"built in {time.time() - t0:.1f} s")

    # measured single-copy pinned host-to-device bandwidth (1 GiB)
    src = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h0.record()
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    h1.record()
    torch.cuda.synchronize()
    h2d = 3 * (1 << 30) / (h0.elapsed_time(h1) * 1e-3) / 1e9
    del src, dst

    def token(transfer, gap, account):
        # account=False: no byte account is asked for, so a call with the gather transfer
        # does not wait for the device (the host-merged transfers always read the lists back)
        moved = sel = ranges = 0
        for ph in phases:
            spax.spax_build_tiers(ph["x"], ph["d"], ph["p"], None, ph["f"], ph["a"], ph["c"])
            st = spax.spax_tiered_gemv_pinned(ph["L"], ph["host"], ph["x"], ph["f"], ph["a"],
                                              ph["c"], ph["y"], gap, ws, transfer=transfer,
                                              stats=account)
            if account:
                moved += st.moved_bytes + st.list_bytes
                sel += st.selected_bytes
                ranges += st.n_ranges
        torch.cuda.synchronize()
        return moved, sel, ranges

    def timed(transfer, gap, steps):
        moved, sel, ranges = token(transfer, gap, True)  # warm-up and the byte account
        t1 = time.perf_counter()
        for _ in range(steps):
            token(transfer, gap, False)
        return (time.perf_counter() - t1) / steps, moved, sel, ranges

    scale = 32 / n_layers
    steps = max(1, args.steps // 8)
    dt, moved, sel, ranges = timed(HOST_TRANSFERS[args.transfer], args.gap, steps)
    gbs = moved / dt / 1e9
    log(f"[bench] host8b: {dt * 1e3:.2f} ms for {n_layers} layers, {gbs:.2f} GB/s moved, "
        f"H2D copy {h2d:.2f} GB/s")

    sweep = None
    if args.sweep:
        sweep = []
        for name, tr in HOST_TRANSFERS.items():
            for gap in (0, 4, 8):
                d2, m2, s2, r2 = timed(tr, gap, 1)
                sweep.append({"transfer": name, "gap": gap,
                              "ms_per_token": round(d2 * scale * 1e3, 2),
                              "moved_GB_per_token": round(m2 * scale / 1e9, 4),
                              "ranges_per_token": int(r2 * scale),
                              "moved_GBps": round(m2 / d2 / 1e9, 2),
                              "frac_of_h2d": round(m2 / d2 / 1e9 / h2d, 4)})
                log(f"[bench] sweep {sweep[-1]}")

    # storage ledger of one token's masks (the same masks as the timed pass)
    token(HOST_TRANSFERS[args.transfer], args.gap, False)
    lists = []
    for ph in phases:
        cnt = ph["c"].cpu().numpy()
        lists.append((ph["f"].cpu().numpy()[:cnt[0]], ph["a"].cpu().numpy()[:cnt[1]]))
    storage = storage_account(spax, [ph["L"] for ph in phases], lists, 4096, args.gap)
    for k in ("selected_GB", "moved_GB", "read_GB"):
        storage[k] = round(storage[k] * scale, 4)
    storage["read_requests"] = int(storage["read_requests"] * scale)
    log(f"[bench] storage ledger {storage}")

    layers_note = (f"{n_layers} distinct layers timed (wall clock)" +
                   (f", scaled x{scale:g} to 32" if n_layers != 32 else "") +
                   (f"; {alloc_note}" if alloc_note else ""))
    return {
        "metric": "pinned-host tiered GEMV µs/token (Llama-3-8B shapes); moved GB/s vs measured "
                  "pinned host-to-device bandwidth",
        "value": round(dt * scale * 1e6, 1), "unit": "us/token", "n_gpus": 1,
        "steps": steps, "warmup": 1, "ms_per_step": round(dt * scale * 1e3, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"host8b: Llama-3-8B shapes (q|k|v 4096->4096+1024+1024, o, "
                               f"gate|up 4096->2x14336, down 14336->4096), fp16 blobs in pinned "
                               f"host memory ({pinned_gb:.1f} GB), TopK 20/30/50, range gap "
                               f"{args.gap}, transfer {args.transfer}, placement "
                               f"{args.placement}; {layers_note}",
                   "layers_timed": n_layers,
                   "selected_GB_per_token": round(sel * scale / 1e9, 4),
                   "moved_GB_per_token": round(moved * scale / 1e9, 4),
                   "ranges_per_token": int(ranges * scale)},
        "roofline": {"bound": "pcie", "achieved": round(gbs, 2), "peak": round(h2d, 2),
                     "unit": "GB/s", "frac": round(gbs / h2d, 4), "traffic": None,
                     "peak_note": "measured single 1 GiB pinned host-to-device copy"},
        "cpu_baseline": None,
        "transfer_sweep": sweep,
        "storage_4KiB": storage,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the path shards by "
                                   "output rows across GPUs but no multi-GPU run is built",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import activation_sparse_tiered_amd as spax
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "host8b":
        out = host_bench(args, spax, torch, dev)
    else:
        out = device_bench(args, spax, torch, dev)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
