#!/usr/bin/env python3
"""Decode-attention throughput of diagonal-aware sparse attention on one MI355X.

One step = one whole image decode: every decode token t = 0 .. L_dec-1 through
every layer in model order (append K/V, then the fused sparse decode launch),
for the whole batch, on synthetic grid-rotary inputs already resident in HBM.
The default workload is the Janus-Pro-7B shape (batch 96, 30 layers, 32 heads x
128, L_p 64, L_dec 576 on a 24x24 grid, N_r 288, N_att 29 = 95 % sparsity).

Printed: one JSON line with head-steps/s (batch x layers x heads x L_dec per
second) and HBM GB/s, the dense kernel at batch 32 beside it, the roofline of
the sparse kernel from per-launch HIP events, and the CPU oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E

# HBM bytes per sparse-decode launch from two rocprofv3 --pmc runs (FETCH_SIZE,
# then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads
# for a plain 1 GiB device copy (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0); the
# profiles/ summaries give the commands.  Keyed by workload and tied to the
# kernel source it was measured on: reported as null once that source changes.
TRAFFIC = {
    "janus_pro_7b": {"bytes_per_launch": 150.8e6, "kernel_sha256_16": "5ebed0da750676a7",
                     "launches": "sparse decode dispatches 12000-12299 (steps 400-409, phase 3)",
                     "algorithmic_bytes_same_launches": 150386688},
}


def kernel_sha16():
    import hashlib

    src = os.path.join(ROOT, "autoregressive_image_generation_amd", "csrc", "dsa_kernels.hip")
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(name):
    t = TRAFFIC.get(name)
    if not t or t["kernel_sha256_16"] != kernel_sha16():
        return None
    return t["bytes_per_launch"]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3, help="timed full decodes")
    p.add_argument("--warmup", type=int, default=1, help="untimed full decodes first")
    p.add_argument("--workload", default="janus_pro_7b")
    p.add_argument("--dense-batch", type=int, default=32, help="batch of the dense comparison (0: skip)")
    p.add_argument("--waves", type=int, default=0, help="wavefronts per lane (0: library's choice)")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-seconds of oracle work (0: skip)")
    p.add_argument("--layers", type=int, default=0, help="override the layer count (profiling only)")
    p.add_argument("--sweep", action="store_true", help="also time the sparsity sweep {0,.5,.8,.9,.95}")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB 5 times (HBM counter calibration) and exit")
    return p.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- byte model
def sparse_bytes_per_head_step(w, t):
    """Algorithmic HBM bytes of one lane at step t: the attended K|V rows (prompt,
    sinks, window; the current token's row comes from the appended input), the
    appended row written to the ring, q, the fp32 output and the index list."""
    import synth

    es = 2 if w.dtype == synth.BF16 else 4
    E = 2 * w.head_dim * es
    S = w.sink
    tw = t - S
    n_list = 0 if tw < 0 else min(tw + 1, w.N_att - S)
    n_sink = min(t + 1, S)
    rows = w.L_p + n_sink + n_list
    return rows * E + E + w.head_dim * es + 4 * w.head_dim + 2 * n_list


def dense_bytes_per_head_step(w, t):
    import synth

    es = 2 if w.dtype == synth.BF16 else 4
    E = 2 * w.head_dim * es
    return (w.L_p + t + 1) * E + E + w.head_dim * es + 4 * w.head_dim


# ----------------------------------------------------------------------------- inputs
class Inputs:
    """Per-layer device tensors: q, k, v [L_dec][B][H][D] and prompt k, v [B][L_p][H][D]."""

    def __init__(self, w, layers, dev):
        import numpy as np
        import torch

        import synth

        self.layers = []
        B, H, D, T, L = w.batch, w.heads, w.head_dim, w.L_dec, w.L_p
        host_dt = torch.int16 if w.dtype == synth.BF16 else torch.float32
        np_dt = np.uint16 if w.dtype == synth.BF16 else np.float32
        pin = {}
        for name, shape in (("q", (T, B, H, D)), ("k", (T, B, H, D)), ("v", (T, B, H, D)),
                            ("kp", (B, L, H, D)), ("vp", (B, L, H, D))):
            pin[name] = torch.empty(shape, dtype=host_dt, pin_memory=True)
        views = {n: pin[n].numpy().view(np_dt) for n in pin}
        t0 = time.perf_counter()
        for layer in range(layers):
            w.decode(layer, synth.Q, out=views["q"])
            w.decode(layer, synth.K, out=views["k"])
            w.decode(layer, synth.V, out=views["v"])
            if L:
                w.prompt(layer, synth.KP, out=views["kp"])
                w.prompt(layer, synth.VP, out=views["vp"])
            self.layers.append({n: pin[n].to(dev, non_blocking=False) for n in pin})
            if layer % 5 == 4 or layer == layers - 1:
                log("  inputs: %d/%d layers (%.1f s)" % (layer + 1, layers, time.perf_counter() - t0))
        torch.cuda.synchronize(dev)
        self.gen_seconds = time.perf_counter() - t0


# ----------------------------------------------------------------------------- runs
class SparseModel:
    """One sparse state per layer over caller-owned workspaces."""

    def __init__(self, w, inputs, layers, dev, waves, batch=None):
        import torch

        import autoregressive_image_generation_amd as dsa

        self.dsa, self.w, self.inputs, self.dev = dsa, w, inputs, dev
        self.B = batch or w.batch
        self.nbytes = dsa.dsa_state_workspace_bytes(self.B, w.L_p, w.N_r, w.N_att, w.heads, w.head_dim, w.sink,
                                                    w.dtype)
        self.ws = [torch.empty(self.nbytes, dtype=torch.uint8, device=dev) for _ in range(layers)]
        self.out = torch.empty((self.B, w.heads, w.head_dim), dtype=torch.float32, device=dev)
        self.waves = waves
        self.states = []

    def reset(self):
        """Fresh states with the prompt in the cache (the prefill's part; not timed)."""
        import torch

        dsa, w = self.dsa, self.w
        for st in self.states:
            dsa.dsa_state_destroy(st)
        self.states = []
        stream = torch.cuda.current_stream(self.dev)
        for layer, ws in enumerate(self.ws):
            st = dsa.dsa_state_init(self.B, w.L_p, w.N_r, w.N_att, w.heads, w.head_dim, w.sink, w.dtype, ws,
                                    self.nbytes, stream)
            dsa.dsa_set_waves(st, self.waves)
            x = self.inputs.layers[layer]
            dsa.dsa_append_prompt(st, x["kp"] if w.L_p else None, x["vp"] if w.L_p else None)
            self.states.append(st)
        torch.cuda.synchronize(self.dev)

    def decode(self):
        """All L_dec steps through all layers, in model order."""
        dsa, w = self.dsa, self.w
        q0 = self.inputs.layers[0]["q"]
        step_bytes = q0[0].numel() * q0.element_size()
        ptrs = [(x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr()) for x in self.inputs.layers]
        lib = dsa.library()
        out = self.out.data_ptr()
        for t in range(w.L_dec):
            off = t * step_bytes  # step t's first `B` sequences are contiguous in [B][H][D]
            for st, (qp, kp, vp) in zip(self.states, ptrs):
                rc = lib.dsa_append_kv(st, kp + off, vp + off)
                rc |= lib.dsa_decode_step(st, qp + off, out, None)
                if rc:
                    raise dsa.DsaError(rc, dsa.dsa_last_error())


class DenseModel(SparseModel):
    def __init__(self, w, inputs, layers, dev, waves, batch):
        import torch

        import autoregressive_image_generation_amd as dsa

        self.dsa, self.w, self.inputs, self.dev = dsa, w, inputs, dev
        self.B = batch
        self.nbytes = dsa.dense_state_workspace_bytes(batch, w.L_p, w.L_dec, w.heads, w.head_dim, w.dtype)
        self.ws = [torch.empty(self.nbytes, dtype=torch.uint8, device=dev) for _ in range(layers)]
        self.out = torch.empty((batch, w.heads, w.head_dim), dtype=torch.float32, device=dev)
        self.waves = waves
        self.states = []

    def reset(self):
        import torch

        dsa, w = self.dsa, self.w
        for st in self.states:
            dsa.dsa_state_destroy(st)
        self.states = []
        stream = torch.cuda.current_stream(self.dev)
        for layer, ws in enumerate(self.ws):
            st = dsa.dense_state_init(self.B, w.L_p, w.L_dec, w.heads, w.head_dim, w.dtype, ws, self.nbytes, stream)
            dsa.dsa_set_waves(st, self.waves)
            x = self.inputs.layers[layer]
            # the first `batch` sequences of the prompt: [B][L_p][H][D] keeps them contiguous
            dsa.dense_append_prompt(st, x["kp"] if w.L_p else None, x["vp"] if w.L_p else None)
            self.states.append(st)
        torch.cuda.synchronize(self.dev)

    def decode(self):
        dsa, w = self.dsa, self.w
        q0 = self.inputs.layers[0]["q"]
        step_bytes = q0[0].numel() * q0.element_size()
        ptrs = [(x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr()) for x in self.inputs.layers]
        lib = dsa.library()
        out = self.out.data_ptr()
        for t in range(w.L_dec):
            off = t * step_bytes  # step t's first `batch` sequences are contiguous in [B][H][D]
            for st, (qp, kp, vp) in zip(self.states, ptrs):
                rc = lib.dense_append_kv(st, kp + off, vp + off)
                rc |= lib.dense_decode_step(st, qp + off, out)
                if rc:
                    raise dsa.DsaError(rc, dsa.dsa_last_error())


def time_decodes(model, steps, warmup, dev):
    """Warm-up decodes, then `steps` timed decodes, each bracketed by a device
    synchronisation; returns (seconds per decode by host clock, by HIP events)."""
    import torch

    for _ in range(warmup):
        model.reset()
        model.decode()
    torch.cuda.synchronize(dev)
    wall = ev = 0.0
    for _ in range(steps):
        model.reset()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        start.record()
        model.decode()
        stop.record()
        torch.cuda.synchronize(dev)
        wall += time.perf_counter() - t0
        ev += start.elapsed_time(stop) * 1e-3
    return wall / steps, ev / steps


def kernel_durations(model, layers, dev):
    """One decode with an event pair around every sparse launch, on the stream the
    library launches on (torch's current stream).  Returns per-step lists of
    launch durations in seconds."""
    import torch

    model.reset()
    w = model.w
    n = w.L_dec * layers
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    dsa, lib = model.dsa, model.dsa.library()
    q0 = model.inputs.layers[0]["q"]
    step_bytes = q0[0].numel() * q0.element_size()
    ptrs = [(x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr()) for x in model.inputs.layers]
    out = model.out.data_ptr()
    i = 0
    for t in range(w.L_dec):
        off = t * step_bytes
        for st, (qp, kp, vp) in zip(model.states, ptrs):
            rc = lib.dsa_append_kv(st, kp + off, vp + off)
            evs[2 * i].record()
            rc |= lib.dsa_decode_step(st, qp + off, out, None)
            evs[2 * i + 1].record()
            if rc:
                raise dsa.DsaError(rc, dsa.dsa_last_error())
            i += 1
    torch.cuda.synchronize(dev)
    per_step = []
    for t in range(w.L_dec):
        per_step.append([evs[2 * (t * layers + l)].elapsed_time(evs[2 * (t * layers + l) + 1]) * 1e-3
                         for l in range(layers)])
    return per_step


def cpu_baseline(w, target_cpu_seconds):
    """The oracle as it stands on a bounded, seeded sample of lanes (all L_dec
    steps each), one lane per host thread; returns the JSON object.  Inputs are
    generated outside the timed parts, in chunks so host memory stays small."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    rng = np.random.default_rng(0)
    T = w.L_dec

    def run(ins):
        oracle.run_lane(w.L_p, w.N_r, w.N_att, w.sink, *ins)

    probe_in = oracle.lane_inputs(w, 0, 0, 0, T)
    t0 = time.perf_counter()
    run(probe_in)
    probe = time.perf_counter() - t0
    n = max(threads, int(math.ceil(target_cpu_seconds / max(probe, 1e-4))))
    n = min(n, 20000)
    lanes = [(int(rng.integers(w.layers)), int(rng.integers(w.batch)), int(rng.integers(w.heads))) for _ in range(n)]
    chunk = threads * 32
    wall = 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for i in range(0, n, chunk):
            inputs = [oracle.lane_inputs(w, *x, T) for x in lanes[i:i + chunk]]
            t0 = time.perf_counter()
            list(ex.map(run, inputs))
            wall += time.perf_counter() - t0
    rate = n * T / wall
    return {"value": rate, "unit": "head-steps/s", "cores": threads, "kind": "oracle",
            "sample": "%d seeded random (layer, batch, head) lanes x all %d decode steps of %s (fp64 C oracle, "
                      "one lane per thread, %.1f s wall, ~%.0f CPU-s; one lane alone %.4f s)"
                      % (n, T, w.name, wall, wall * threads, probe)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (lanes shard across GPUs "
              "with no exchange; see DESIGN.md). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import autoregressive_image_generation_amd as dsa
    import synth

    dsa.library()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        print(json.dumps({"calibrate_copy_bytes": n, "reads": n, "writes": n, "launches": 5}), flush=True)
        return

    w = synth.WORKLOADS[args.workload]
    layers = args.layers or w.layers
    log("bench: %s, %d layers, batch %d, generating inputs" % (w.name, layers, w.batch))
    inputs = Inputs(w, layers, dev)
    log("inputs ready in %.1f s" % inputs.gen_seconds)

    head_steps = w.batch * layers * w.heads * w.L_dec
    sparse = SparseModel(w, inputs, layers, dev, args.waves)
    sec, sec_ev = time_decodes(sparse, args.steps, args.warmup, dev)
    total_bytes = sum(sparse_bytes_per_head_step(w, t) for t in range(w.L_dec)) * w.batch * w.heads * layers
    log("sparse: %.1f ms per decode (events %.1f ms)" % (sec * 1e3, sec_ev * 1e3))

    # Roofline of the sparse kernel from the timed region's HIP events (torch's
    # current stream is the stream the library launches on): the launches run
    # back to back, so events / launches is the average launch duration,
    # inter-launch gaps included (rocprofv3's kernel trace agrees within ~1 %).
    n_launch = w.L_dec * layers
    launch_s = sec_ev / n_launch
    bytes_per_launch = total_bytes / n_launch
    achieved = bytes_per_launch / launch_s / 1e9
    log("sparse kernel: %.2f us per launch over %d launches, %.0f GB/s" % (launch_s * 1e6, n_launch, achieved))
    # per-phase latency from one decode with an event pair around every launch
    # (each pair adds ~2 us of event overhead; for the step profile only)
    durs = kernel_durations(sparse, layers, dev)
    phase_us = {}
    for name, lo, hi in (("phase1", 0, min(w.N_att - 1, w.L_dec)), ("phase2", max(w.N_att - 1, 0), min(w.N_r, w.L_dec)),
                         ("phase3", min(w.N_r, w.L_dec), w.L_dec)):
        if hi > lo:
            phase_us[name] = sum(sum(durs[t]) for t in range(lo, hi)) / ((hi - lo) * layers) * 1e6

    result = {
        "metric": "sparse decode-attn steps/s (batch x layers x heads) + HBM GB/s, Janus-Pro-7B shape",
        "value": head_steps / sec,
        "unit": "head-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == synth.BF16 else "fp32",
        "data": "synthetic grid-rotary Q/K/V + N(0,0.1) noise, seed 0, resident in HBM",
        "config": {"workload": w.name, "batch": w.batch, "layers": layers, "heads": w.heads,
                   "head_dim": w.head_dim, "L_p": w.L_p, "L_dec": w.L_dec, "N_r": w.N_r, "N_att": w.N_att,
                   "sink": w.sink, "sparsity": round(1 - w.N_att / w.L_dec, 4),
                   "step": "one full image decode: L_dec tokens x layers, all lanes",
                   "accumulation": "fp64 logits, fp32 softmax and PV"},
        "hbm_gbs": total_bytes / sec / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_for(w.name),
                     "kernel": "decode_kernel (sparse, bf16, head_dim 128)",
                     "avg_launch_us": launch_s * 1e6,
                     "bytes_per_launch": bytes_per_launch,
                     "event_pair_us_by_phase": phase_us},
        "events_ms_per_step": sec_ev * 1e3,
    }

    if args.dense_batch:
        db = min(args.dense_batch, w.batch)
        dense = DenseModel(w, inputs, layers, dev, args.waves, db)
        dsec, _ = time_decodes(dense, args.steps, args.warmup, dev)
        dsteps = db * layers * w.heads * w.L_dec
        dbytes = sum(dense_bytes_per_head_step(w, t) for t in range(w.L_dec)) * db * w.heads * layers
        sparse_b = SparseModel(w, inputs, layers, dev, args.waves, batch=db)
        ssec, _ = time_decodes(sparse_b, args.steps, args.warmup, dev)
        result["dense"] = {"batch": db, "value": dsteps / dsec, "unit": "head-steps/s", "hbm_gbs": dbytes / dsec / 1e9,
                           "ms_per_step": dsec * 1e3, "sparse_same_batch_value": dsteps / ssec,
                           "sparse_speedup": dsec / ssec,
                           "byte_ratio": dbytes / (sum(sparse_bytes_per_head_step(w, t) for t in range(w.L_dec))
                                                   * db * w.heads * layers)}
        log("dense b%d: %.1f ms per decode; sparse b%d %.1f ms -> %.2fx" % (db, dsec * 1e3, db, ssec * 1e3,
                                                                           dsec / ssec))
        del dense, sparse_b

    if args.sweep:
        sweep = []
        for sp in (0.0, 0.5, 0.8, 0.9, 0.95):
            n_att = synth.n_att_for(w.L_dec, sp)
            n_r = w.N_r if n_att <= w.N_r else w.L_dec
            ws = w.with_(N_att=n_att, N_r=n_r)
            m = SparseModel(ws, inputs, layers, dev, args.waves)
            s, _ = time_decodes(m, 1, 1, dev)
            b = sum(sparse_bytes_per_head_step(ws, t) for t in range(w.L_dec)) * w.batch * w.heads * layers
            sweep.append({"sparsity": sp, "N_r": n_r, "N_att": n_att, "value": head_steps / s,
                          "hbm_gbs": b / s / 1e9})
            log("sweep %.2f: %.1f ms" % (sp, s * 1e3))
            del m
        result["sweep"] = sweep

    if args.cpu_seconds > 0:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
