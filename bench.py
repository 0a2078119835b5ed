"""Benchmark: one batch-one decode step over all projections of a 32-layer 7B-shaped decoder.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sparsity 0.5] [--no-cpu-baseline]

A step is one token: for each of 32 layers and each projection group (q|k|v, o, gate|up,
down) one TopK-Guided tier mask (s +- 0.01, approximate tier = 3/10 of the kept channels,
two-bit groups of 128 rows) and one tiered GEMV over the fused fp16 matrices, in order.
Weights are synthetic (fp16 N(0, 0.02), drawn on the device from a seed) and packed by
spax_pack_columns before timing; activations are seeded Laplace(0, 1) vectors, one per
(token, layer, group), resident in HBM before the timed region.

Prints one JSON line.  ``value`` is microseconds per token (lower is better).  The
``roofline`` object is for the fused mask+GEMV kernel (the only kernel of the default step):
algorithmic bytes = selected column records + activations + tier bytes + index lists + y,
per launch, over the kernel's average duration measured with HIP events that the library
records on the launch stream around each launch.  ``cpu_baseline`` times the oracle (float64
NumPy) on a bounded sample of the same workload on the host cores.
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--sparsity", type=float, default=0.5)
    ap.add_argument("--delta", type=float, default=0.01)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--tokens", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip timing the batched step form")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="before the timed steps, run one elementwise kernel (bitwise_not) that "
                         "reads and writes this many MiB: known traffic for scaling hardware "
                         "byte counters (use more than the 256 MB last-level cache)")
    ap.add_argument("--cpu-layers", type=int, default=24,
                    help="layers of one token the oracle runs for the CPU baseline")
    return ap.parse_args()


class Stack:
    """Packed weights, per-token activations and per-phase output buffers on the device."""

    def __init__(self, spax, torch, dev, layers, tokens, s, delta):
        self.spax, self.torch, self.dev = spax, torch, dev
        self.shapes = synth.decoder_phases_7b()
        self.layers, self.tokens = layers, tokens
        self.layouts, self.packed, self.params, self.bufs = [], [], [], []
        t0 = time.time()
        for l in range(layers):
            for k, (name, d_in, d_out) in enumerate(self.shapes):
                L = spax.spax_layout_init(d_in, d_out, spax.FMT_FP16, 128, 128)
                packed = torch.empty(int(L.total_bytes), dtype=torch.uint8, device=dev)
                Ws = [synth.weights_device(SEED, d_in, r, dev, l, k, m) for m, r in enumerate(d_out)]
                spax.spax_pack_columns(L, Ws, packed)
                del Ws
                lo, hi = spax.spax_guided_bounds(d_in, s, delta)
                p = spax.guided_params(-math.log(1.0 - s), lo, hi, 3, 10)
                T = int(L.d_out_total)
                self.layouts.append(L)
                self.packed.append(packed)
                self.params.append(p)
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
                    row.append(torch.from_numpy(synth.activations(SEED, d_in, t, l, k)).to(dev))
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


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_phase_kernel_decode7b_s05_traffic.md")


def sources_sha256():
    """sha256 over the kernel sources and the C header (name, then bytes; sorted by path)."""
    import glob
    import hashlib
    files = sorted(glob.glob(os.path.join(ROOT, "activation_sparse_tiered_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "spax.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(args):
    """HBM MB per fused launch from the committed FETCH_SIZE / WRITE_SIZE summary, scaled by
    its copy calibration; None unless this is the workload it was taken on and the kernel
    sources are unchanged since."""
    if (args.sparsity, args.delta, args.layers) != (0.5, 0.01, 32) or not os.path.exists(TRAFFIC_FILE):
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


def cpu_baseline(stack, layers, s, delta):
    """The oracle on `layers` layers of token 0, timed on the host, scaled to one token.
    Each phase's weights are drawn (on the device, as for the GPU run) and copied to the
    host right before it is timed, so only one phase is held in host memory at a time."""
    from oracle import gemv as ogemv
    from oracle import pack as opack
    from oracle import tiers as otiers
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        limiter = None
    bounds = {}
    dt = 0.0
    for l in range(layers):
        for k, (name, d_in, d_out) in enumerate(stack.shapes):
            Ws = [synth.weights_device(SEED, d_in, r, stack.dev, l, k, m).cpu().numpy()
                  for m, r in enumerate(d_out)]
            O = opack.Layout(d_in, d_out, 0, 128, 128)
            x = synth.activations(SEED, d_in, 0, l, k)
            if d_in not in bounds:
                bounds[d_in] = otiers.guided_bounds(d_in, s, delta)
            lo, hi = bounds[d_in]
            t0 = time.perf_counter()
            _, f, a, _ = otiers.build_tiers(x, otiers.MODE_TOPK_GUIDED, tau=-math.log(1 - s),
                                            n_lo=lo, n_hi=hi, num=3, den=10)
            ogemv.tiered_gemv(O, Ws, x, f, a)
            dt += time.perf_counter() - t0
            del Ws
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    per_token_us = dt / layers * stack.layers * 1e6
    return {"value": round(per_token_us, 1), "unit": "us/token", "cores": cores, "kind": "oracle",
            "sample": f"{layers} of {stack.layers} layers (4 projection groups each) of one token: "
                      f"float64 NumPy tier mask + tiered GEMV, scaled x{stack.layers / layers:g}; "
                      f"{dt:.1f} s measured; BLAS threads = cores"}


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
    s, delta = args.sparsity, args.delta
    stack = Stack(spax, torch, dev, args.layers, args.tokens, s, delta)

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.bitwise_not(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- warmup, then exactly `steps` timed decode steps
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
    log(f"[bench] decode step: {step_ms * 1e3:.1f} us/token (event), wall {wall_ms / args.steps:.3f} ms/step")

    # ---- bytes: the masks of the timed tokens (deterministic per token) give the counts
    n_ph = len(stack.layouts)
    tok_bytes = {}
    per_phase = {}
    for t in range(args.warmup, args.warmup + args.steps):
        key = t % stack.tokens
        if key in tok_bytes:
            continue
        ms, counts = stack.timed_kernels(t)
        tb = 0
        for i, (m, c) in enumerate(zip(ms, counts)):
            b = stack.algorithmic_bytes(i, c)
            tb += b
            pb = per_phase.setdefault(stack.shapes[i % 4][0], [0, 0.0, 0])
            pb[0] += b
            pb[1] += m
            pb[2] += 1
        tok_bytes[key] = tb
    timed_bytes = [tok_bytes[t % stack.tokens] for t in range(args.warmup, args.warmup + args.steps)]
    bytes_per_token = float(np.mean(timed_bytes))
    # The timed step is one fused launch per phase (plus one small clearing launch), back to
    # back on one stream: the kernel's average launch duration is the step time over the
    # launches, measured by the events around the timed region.
    avg_launch_ms = step_ms / n_ph
    avg_bytes = bytes_per_token / n_ph
    achieved = avg_bytes / (avg_launch_ms * 1e-3) / 1e9
    for name, (b, m, n) in per_phase.items():
        log(f"[bench]   {name:7s}: {b / n / 1e6:7.2f} MB per launch; event-bracketed launch "
            f"{m / n * 1e3:7.2f} us (includes the launch gap)")
    log(f"[bench] fused kernel: {avg_launch_ms * 1e3:.2f} us/launch, {avg_bytes / 1e6:.2f} MB/launch, "
        f"{achieved:.1f} GB/s; selected bytes/token {bytes_per_token / 1e9:.3f} GB")

    # ---- the batched form of the same step (all masks in one launch, all GEMVs in one launch):
    # legal here only because the synthetic phase inputs are independent; reported beside the
    # layer-serial value, never as it
    batched = None
    if not args.no_batched:
        stack.flags = spax.STEP_BATCHED
        for t in range(args.warmup):
            stack.step(t)
        torch.cuda.synchronize()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record()
        for t in range(args.steps):
            stack.step(args.warmup + t)
        b1.record()
        torch.cuda.synchronize()
        stack.flags = spax.STEP_DEFAULT
        bt_ms = b0.elapsed_time(b1) / args.steps
        bgbs = bytes_per_token / (bt_ms * 1e-3) / 1e9
        batched = {"value": round(bt_ms * 1e3, 2), "unit": "us/token",
                   "achieved_GBps": round(bgbs, 1), "frac": round(bgbs / HBM_PEAK_GBS, 4),
                   "form": "SPAX_STEP_BATCHED: all 128 masks in one launch, then all GEMVs in one "
                           "persistent launch; valid only because the phase inputs are independent"}
        log(f"[bench] batched step: {bt_ms * 1e3:.1f} us/token, {bgbs:.1f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(stack, min(args.cpu_layers, args.layers), s, delta)
        log(f"[bench] cpu baseline {cpu}")

    out = {
        "metric": METRIC,
        "value": round(step_ms * 1e3, 2),
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
        "config": {
            "workload": f"decode7b: {args.layers} layers x (q|k|v 4096->3x4096, o 4096->4096, "
                        f"gate|up 4096->2x11008, down 11008->4096), fp16 weights, "
                        f"TopK-Guided mask s={s}+-{delta}, approx tier 3/10 of kept, 2-bit G=128, "
                        f"batch 1, layer-serial",
            "sparsity": s, "layers": args.layers, "tokens": args.tokens,
            "selected_GB_per_token": round(bytes_per_token / 1e9, 4),
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(args),
                     "traffic_unit": "MB per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "kernel": "fused_phase_kernel<fp16>",
                     "avg_launch_us": round(avg_launch_ms * 1e3, 3),
                     "avg_algorithmic_MB": round(avg_bytes / 1e6, 3)},
        "cpu_baseline": cpu,
        "batched": batched,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
