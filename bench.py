#!/usr/bin/env python3
"""Decode-attention throughput of diagonal-aware sparse attention on one MI355X.

One step = one whole image decode: every decode token t = 0 .. L_dec-1 through
every layer in model order (append K/V, then the fused sparse decode launch),
for the whole batch, on synthetic grid-rotary inputs already resident in HBM.
The headline workload is the Janus-Pro-7B shape (batch 96, 30 layers, 32 heads
x 128, L_p 64, L_dec 576 on a 24x24 grid, N_r 288, N_att 29 = 95 % sparsity).

Printed: one JSON line.  For the headline workload: head-steps/s (batch x
layers x heads x L_dec per second) and HBM GB/s of the decode split into two
micro-batch streams (`value`); the roofline of the sparse kernel (the same
decode on one stream, whole batch per launch, from HIP events on the launch
stream) and of the two-stream aggregate; the per-step launch time as the window
fills and slides; the dense kernel at the same batch and at batch 32, each
beside the sparse kernel at that batch; the last decode step alone, sparse at
90 % and 95 % against dense (attention only, batch 32); the sparse-KV
baselines at the same budget (SlidingWindow, StreamingLLM, TOVA, H2O); the
MXFP8 cache; the sparsity sweep; the attention-map characterization of one
layer; the device's HBM read ceiling from a plain read probe; and the CPU
oracle on a bounded sample of the same workload.  Then one leg per other
workload (Janus-Pro-1B, Lumina-mGPT 1024x1024, 8100 tokens + sink4), each with
its two-stream rate, one-stream roofline, per-step series, same-batch dense
comparison and CPU oracle sample.
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
    # one stream, dispatches 12480-12779 (steps 400-409, phase 3); algorithmic bytes of the same launches 150386688 (phase 2 window: counters / algorithmic 1.0034)
    ("janus_pro_7b", 1): {"bytes_per_launch": 150.8e6, "algorithmic_bytes_per_launch": 150386688, "kernel_sha256_16": "402cc1bfbc6d2ddc"},
    # one stream, dispatches 9984-10283 (steps 400-412, phase 3); algorithmic bytes of the same launches 32696320 (phase 2 window: counters / algorithmic 1.0054)
    ("janus_pro_1b", 1): {"bytes_per_launch": 32.86e6, "algorithmic_bytes_per_launch": 32696320, "kernel_sha256_16": "402cc1bfbc6d2ddc"},
    # one stream, dispatches 96512-96811 (steps 3000-3009, phase 3); algorithmic bytes of the same launches 79770624 (phase 2 window: counters / algorithmic 1.0033)
    ("lumina_mgpt_7b_1024", 1): {"bytes_per_launch": 80.01e6, "algorithmic_bytes_per_launch": 79770624, "kernel_sha256_16": "402cc1bfbc6d2ddc"},
    # one stream, dispatches 192512-192811 (steps 6000-6009, phase 3); algorithmic bytes of the same launches 119491584 (phase 2 window: counters / algorithmic 1.0018)
    ("hires_8100_sink4", 1): {"bytes_per_launch": 119.7e6, "algorithmic_bytes_per_launch": 119491584, "kernel_sha256_16": "402cc1bfbc6d2ddc"},
    # MXFP8 cache, two micro-batch streams (1536 lanes per launch), dispatches 24960-25259 of the
    # Mx8 decode kernel (steps 400-404, phase 3); algorithmic bytes 39386112 (phase 2 window,
    # steps 100-104: counters / algorithmic 1.0575)
    ("janus_pro_7b_mxfp8", 2): {"bytes_per_launch": 42.83e6, "algorithmic_bytes_per_launch": 39386112, "kernel_sha256_16": "402cc1bfbc6d2ddc"},
}

LEG_WORKLOADS = "janus_pro_1b,lumina_mgpt_7b_1024,hires_8100_sink4"


def kernel_sha16():
    import hashlib

    src = os.path.join(ROOT, "autoregressive_image_generation_amd", "csrc", "dsa_kernels.hip")
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(name, streams=1, ratio=False):
    """Counter bytes per launch of the workload's counter window (or, with
    ratio, their quotient by the algorithmic bytes of the same launches);
    None when not measured for the current kernel source."""
    t = TRAFFIC.get((name, streams))
    if not t or t["kernel_sha256_16"] != kernel_sha16():
        return None
    return t["bytes_per_launch"] / t["algorithmic_bytes_per_launch"] if ratio else t["bytes_per_launch"]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3, help="timed full decodes of the headline workload")
    p.add_argument("--warmup", type=int, default=1, help="untimed full decodes of the headline workload first")
    p.add_argument("--workload", default="janus_pro_7b", help="the headline workload")
    p.add_argument("--legs", default=LEG_WORKLOADS,
                   help="comma-separated further workloads, one leg each ('none': headline only)")
    p.add_argument("--leg-steps", type=int, default=3, help="timed decodes per leg and per comparison run")
    p.add_argument("--dense-batch", type=int, default=32,
                   help="batch of the extra dense comparison and of the last-step comparison (0: skip both)")
    p.add_argument("--no-dense-full", action="store_true", help="skip the dense kernel at each workload's batch")
    p.add_argument("--waves", type=int, default=0, help="wavefronts per lane (0: library's / measured choice)")
    p.add_argument("--streams", type=int, default=0,
                   help="micro-batches, each on its own stream (0: 2 when the batch is even, else 1)")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-seconds of oracle work per workload (0: skip)")
    p.add_argument("--layers", type=int, default=0, help="override the layer count (profiling only)")
    p.add_argument("--no-sweep", action="store_true", help="skip the sparsity sweep {0,.5,.8,.9,.95}")
    p.add_argument("--no-mxfp8", action="store_true", help="skip the MXFP8 KV-cache leg")
    p.add_argument("--no-ceiling", action="store_true", help="skip the HBM read-ceiling probe")
    p.add_argument("--no-series", action="store_true", help="skip the per-step series decode")
    p.add_argument("--profile-dist", type=int, default=48,
                   help="attention-map characterization of layer 0 up to this query distance (0: skip)")
    p.add_argument("--no-policies", action="store_true",
                   help="skip the baseline policies (SlidingWindow, StreamingLLM, TOVA, H2O) at equal N_att")
    p.add_argument("--summarize-trace", metavar="CSV",
                   help="only summarise a rocprofv3 run_kernel_trace.csv by kernel and launch shape, then exit")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB 5 times (HBM counter calibration) and exit")
    return p.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- byte model
def row_bytes(w):
    """Bytes of one cached K|V row: 2 d elements, or MXFP8 codes plus the 8-byte scale word
    (stored apart from the codes, read with them)."""
    import synth

    if w.dtype == synth.MXFP8:
        return 2 * w.head_dim + 8
    return 2 * w.head_dim * (2 if w.dtype == synth.BF16 else 4)


def sparse_bytes_per_head_step(w, t):
    """Algorithmic HBM bytes of one lane at step t: the attended K|V rows (prompt,
    sinks, window; the current token's row comes from the appended input), the
    appended row written to the ring, q, the fp32 output and the index list."""
    import synth

    es = 4 if w.dtype == synth.F32 else 2  # q (bf16 for an MXFP8 cache)
    E = row_bytes(w)
    S = w.sink
    tw = t - S
    n_list = 0 if tw < 0 else min(tw + 1, w.N_att - S)
    n_sink = min(t + 1, S)
    rows = w.L_p + n_sink + n_list
    return rows * E + E + w.head_dim * es + 4 * w.head_dim + 2 * n_list


POLICY_NAMES = ["diagonal", "diagonal_sink4", "sliding_window", "streaming_llm", "tova", "h2o"]


def policy_n_r(w, policy):
    """N_r argument of each policy at workload w: the ring for the diagonal
    policies, the cache size for SlidingWindow / StreamingLLM / TOVA, and for
    H2O the protected recent count (half the budget, rounded up)."""
    if policy <= 1:
        return w.N_r
    return w.N_att - w.N_att // 2 if policy == 5 else w.N_att


def policy_bytes_per_head_step(w, policy, t):
    """Algorithmic HBM bytes of one lane at step t under a policy.  Position
    policies are Algorithm 1 states (ring = N_att); TOVA / H2O read the attended
    slot rows, their slot metadata (4 + min(t, N_att) int32, 16-byte chunks) and
    write the new slot position and free slot (8 B); H2O also reads the cached
    entries' fp64 scores and writes them back with the new token's."""
    import synth

    if policy in (0, 1):
        return sparse_bytes_per_head_step(w.with_(sink=4 if policy == 1 else 0), t)
    if policy in (2, 3):
        return sparse_bytes_per_head_step(w.with_(N_r=w.N_att, sink=4 if policy == 3 else 0), t)
    es = 4 if w.dtype == synth.F32 else 2
    E = row_bytes(w)
    n = min(t + 1, w.N_att)
    n_meta = 4 + min(t, w.N_att)
    b = (w.L_p + n) * E + E + w.head_dim * es + 4 * w.head_dim + (n_meta + 3) // 4 * 16 + 8
    if policy == 5:
        b += 8 * (n - 1) + 8 * n
    return b


def dense_bytes_per_head_step(w, t):
    import synth

    es = 4 if w.dtype == synth.F32 else 2
    E = row_bytes(w)
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
        host_dt = torch.int16 if w.input_dtype == synth.BF16 else torch.float32
        np_dt = np.uint16 if w.input_dtype == synth.BF16 else np.float32
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
_STREAM_POOL = []


def micro_batch_streams(dev, n):
    """The process's micro-batch streams (default priority), created once and
    shared by every model.  Creating streams per model made every other model's
    pair share one hardware queue (GPU_MAX_HW_QUEUES = 4), which serialises it."""
    import torch

    while len(_STREAM_POOL) < n:
        _STREAM_POOL.append(torch.cuda.Stream(dev))
    return _STREAM_POOL[:n]


class SparseModel:
    """One sparse state per layer over caller-owned workspaces.

    With streams > 1 the batch is split into that many micro-batches, each with
    its own per-layer states on its own stream (default priority).  Every
    sequence still goes through the layers in model order; micro-batches are
    independent, so one's launch can overlap another's.
    """

    dense = False

    def __init__(self, w, inputs, layers, dev, waves, batch=None, streams=1, policy=None, splits=0):
        import torch

        import autoregressive_image_generation_amd as dsa

        self.dsa, self.w, self.inputs, self.dev = dsa, w, inputs, dev
        self.B = batch or w.batch
        if self.B % streams:
            raise ValueError("batch %d does not split into %d micro-batches" % (self.B, streams))
        self.S = streams
        self.Bc = self.B // streams
        self.policy = policy
        self.nbytes = self._workspace_bytes()
        self.ws = [[torch.empty(self.nbytes, dtype=torch.uint8, device=dev) for _ in range(layers)]
                   for _ in range(streams)]
        self.out = torch.empty((self.B, w.heads, w.head_dim), dtype=torch.float32, device=dev)
        self.streams = [torch.cuda.current_stream(dev)] if streams == 1 else micro_batch_streams(dev, streams)
        self.waves = waves
        self.splits = splits
        self.states = []  # [micro-batch][layer]

    def _workspace_bytes(self):
        w, dsa = self.w, self.dsa
        if self.policy is None:
            return dsa.dsa_state_workspace_bytes(self.Bc, w.L_p, w.N_r, w.N_att, w.heads, w.head_dim, w.sink, w.dtype)
        return dsa.dsa_policy_workspace_bytes(self.policy, self.Bc, w.L_p, policy_n_r(w, self.policy), w.N_att,
                                              w.heads, w.head_dim, w.dtype)

    def _init_state(self, ws, stream):
        w = self.w
        if self.policy is not None:
            return self.dsa.dsa_policy_state_init(self.policy, self.Bc, w.L_p, policy_n_r(w, self.policy), w.N_att,
                                                  w.heads, w.head_dim, w.dtype, ws, self.nbytes, stream)
        return self.dsa.dsa_state_init(self.Bc, w.L_p, w.N_r, w.N_att, w.heads, w.head_dim, w.sink, w.dtype, ws,
                                       self.nbytes, stream)

    def _append_prompt(self, st, x, c):
        w = self.w
        off = c * self.Bc * w.L_p * w.heads * w.head_dim * x["kp"].element_size()
        self.dsa.dsa_append_prompt(st, x["kp"].data_ptr() + off if w.L_p else None,
                                   x["vp"].data_ptr() + off if w.L_p else None)

    def reset(self):
        """Fresh states with the prompt in the cache (the prefill's part; not timed)."""
        import torch

        dsa = self.dsa
        for row in self.states:
            for st in row:
                dsa.dsa_state_destroy(st)
        self.states = []
        torch.cuda.synchronize(self.dev)
        for c in range(self.S):
            row = []
            for layer, ws in enumerate(self.ws[c]):
                st = self._init_state(ws, self.streams[c])
                dsa.dsa_set_waves(st, self.waves)
                if not self.dense:
                    dsa.dsa_set_splits(st, self.splits)
                self._append_prompt(st, self.inputs.layers[layer], c)
                row.append(st)
            self.states.append(row)
        torch.cuda.synchronize(self.dev)

    def free(self):
        for row in self.states:
            for st in row:
                self.dsa.dsa_state_destroy(st)
        self.states = []
        self.ws = None
        self.out = None

    def run(self, t0=0, t1=None, step_events=None):
        """Steps t0 .. t1-1 through all layers, in model order per micro-batch:
        one append-and-decode call per (step, layer, micro-batch).  With
        step_events (one stream only), event t - t0 is recorded on the launch
        stream before step t's launches and the last one after step t1 - 1."""
        dsa, w = self.dsa, self.w
        t1 = w.L_dec if t1 is None else t1
        q0 = self.inputs.layers[0]["q"]
        es = q0.element_size()
        step_bytes = q0[0].numel() * es
        chunk = self.Bc * w.heads * w.head_dim
        lib = dsa.library()
        call = lib.dense_append_decode_step if self.dense else lib.dsa_append_decode_step
        # per (layer, micro-batch), in launch order: state and its input / output addresses
        plan = []
        for layer, x in enumerate(self.inputs.layers):
            for c in range(self.S):
                off = c * chunk * es  # micro-batch c: contiguous in [B][H][D]
                plan.append((self.states[c][layer], x["k"].data_ptr() + off, x["v"].data_ptr() + off,
                             x["q"].data_ptr() + off, self.out.data_ptr() + c * chunk * 4))
        if step_events is not None and self.S != 1:
            raise ValueError("per-step events need one stream")
        for t in range(t0, t1):
            o = t * step_bytes
            if step_events is not None:
                step_events[t - t0].record(self.streams[0])
            if self.dense:
                for st, kp, vp, qp, op in plan:
                    rc = call(st, kp + o, vp + o, qp + o, op)
                    if rc:
                        raise dsa.DsaError(rc, dsa.dsa_last_error())
            else:
                for st, kp, vp, qp, op in plan:
                    rc = call(st, kp + o, vp + o, qp + o, op, None)
                    if rc:
                        raise dsa.DsaError(rc, dsa.dsa_last_error())
        if step_events is not None:
            step_events[t1 - t0].record(self.streams[0])


class DenseModel(SparseModel):
    """One dense state per layer (optionally per micro-batch and stream)."""

    dense = True

    def __init__(self, w, inputs, layers, dev, waves, batch, streams=1):
        super().__init__(w, inputs, layers, dev, waves, batch=batch, streams=streams)

    def _workspace_bytes(self):
        w = self.w
        return self.dsa.dense_state_workspace_bytes(self.Bc, w.L_p, w.L_dec, w.heads, w.head_dim, w.dtype)

    def _init_state(self, ws, stream):
        w = self.w
        return self.dsa.dense_state_init(self.Bc, w.L_p, w.L_dec, w.heads, w.head_dim, w.dtype, ws, self.nbytes,
                                         stream)

    def _append_prompt(self, st, x, c):
        w = self.w
        off = c * self.Bc * w.L_p * w.heads * w.head_dim * x["kp"].element_size()
        self.dsa.dense_append_prompt(st, x["kp"].data_ptr() + off if w.L_p else None,
                                     x["vp"].data_ptr() + off if w.L_p else None)


WARM_STEPS = 16  # a partial decode that loads the kernels and touches the workspaces


def time_decodes(model, steps, warmup, dev):
    """Warm-up decodes (warmup = 0: a partial decode of WARM_STEPS steps, so the
    timed decodes never pay first-launch costs), then `steps` timed decodes,
    each bracketed by a device synchronisation; returns (seconds per decode by
    host clock, by HIP events).  The events sit on the launch stream(s): with
    several micro-batch streams, every stream waits for the start event and the
    stop event waits for all."""
    import torch

    if warmup == 0:
        model.reset()
        model.run(0, min(WARM_STEPS, model.w.L_dec))
    for _ in range(warmup):
        model.reset()
        model.run()
    torch.cuda.synchronize(dev)
    wall = ev = 0.0
    per_stream = [0.0] * len(model.streams)
    main = torch.cuda.current_stream(dev)
    for _ in range(steps):
        model.reset()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ends = [torch.cuda.Event(enable_timing=True) for _ in model.streams]
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        start.record(main)
        for s in model.streams:
            if s != main:
                s.wait_event(start)
        model.run()
        for s, e in zip(model.streams, ends):
            e.record(s)
            if s != main:
                main.wait_event(e)
        stop.record(main)
        torch.cuda.synchronize(dev)
        wall += time.perf_counter() - t0
        ev += start.elapsed_time(stop) * 1e-3
        for i, e in enumerate(ends):
            per_stream[i] += start.elapsed_time(e) * 1e-3
    model.stream_seconds = [x / steps for x in per_stream]
    return wall / steps, ev / steps


def step_seconds(model, dev):
    """One decode on one stream (after a partial warm-up) with an event on the
    launch stream before every step and after the last: per step t, the time of
    its `layers` back-to-back launches.  One event per step, none around single
    launches, so the series carries no per-launch event overhead."""
    import torch

    if model.S != 1:
        return None
    w = model.w
    model.reset()
    model.run(0, min(WARM_STEPS, w.L_dec))
    model.reset()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(w.L_dec + 1)]
    model.run(step_events=evs)
    torch.cuda.synchronize(dev)
    return [evs[t].elapsed_time(evs[t + 1]) * 1e-3 for t in range(w.L_dec)]


def series_summary(w, per_step, layers):
    """Mean launch duration (us) per phase and at ~48 steps spread over the decode
    (plus the phase boundaries), from step_seconds."""
    phase_us = {}
    for name, lo, hi in (("phase1", 0, min(w.N_att - 1, w.L_dec)),
                         ("phase2", max(w.N_att - 1, 0), min(w.N_r, w.L_dec)),
                         ("phase3", min(w.N_r, w.L_dec), w.L_dec)):
        if hi > lo:
            phase_us[name] = sum(per_step[lo:hi]) / ((hi - lo) * layers) * 1e6
    marks = set(range(0, w.L_dec, max(1, w.L_dec // 48))) | {w.L_dec - 1}
    marks |= {t for t in (w.N_att - 2, w.N_att - 1, w.N_r - 1, w.N_r) if 0 <= t < w.L_dec}
    series = [[t, round(per_step[t] / layers * 1e6, 3)] for t in sorted(marks)]
    return phase_us, series


def library_waves(w, lanes, dtype=None):
    """The library's wavefront choice for a launch of `lanes` lanes (its
    choose_waves rule), used to size the launch-floor probe like the decode."""
    import synth

    dt = w.dtype if dtype is None else dtype
    ept = 4 if dt == synth.F32 else 16 if dt == synth.MXFP8 else 8
    gpw = 64 // (w.head_dim // ept)
    rows = w.L_p + w.N_att
    wv = 1
    while wv < 8 and lanes * 2 * wv < 3072 and rows >= (2 if lanes * 2 * wv >= 2048 else 4) * gpw * 2 * wv:
        wv *= 2
    return wv


def hbm_read_ceiling(dev, nbytes=4 << 30, reps=10):
    """Practical HBM read ceiling: the library's read probe (16-byte non-temporal
    loads, grid-stride) over a 4 GiB buffer, best of a few launch shapes."""
    import torch

    import autoregressive_image_generation_amd as dsa

    src = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    best = None
    for blocks in (1024, 2048, 4096, 8192):
        for threads in (256, 512):
            for unroll in (4, 8):
                def run():
                    dsa.dsa_hbm_read_probe(src, nbytes, blocks, threads, unroll, sink, stream)
                run()
                start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                start.record(stream)
                for _ in range(reps):
                    run()
                stop.record(stream)
                torch.cuda.synchronize(dev)
                gbs = nbytes * reps / (start.elapsed_time(stop) * 1e-3) / 1e9
                if best is None or gbs > best["GBs"]:
                    best = {"GBs": gbs, "blocks": blocks, "threads": threads, "unroll": unroll}
    if int(sink.item()) != 0:
        raise RuntimeError("read probe: the sink was written for a zero buffer")
    del src
    torch.cuda.empty_cache()
    return best


def launch_floor(dev, blocks, threads, nodes=48, reps=40):
    """Device time per launch of a near-empty kernel with the decode launch's
    grid (the read probe over 16 bytes per thread), back to back on one
    stream.  The launches are replayed from a captured graph: issued one by one
    from Python they would be bound by the host (~3.5 us per call), not by the
    device.  What any dependent kernel of that shape pays per launch here."""
    import torch

    import autoregressive_image_generation_amd as dsa

    nbytes = blocks * threads * 16
    src = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    side = torch.cuda.Stream(dev)
    with torch.cuda.stream(side):
        dsa.dsa_hbm_read_probe(src, nbytes, blocks, threads, 1, sink, side)
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _ in range(nodes):
            dsa.dsa_hbm_read_probe(src, nbytes, blocks, threads, 1, sink, torch.cuda.current_stream(dev))
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream(dev)
    start.record(stream)
    for _ in range(reps):
        graph.replay()
    stop.record(stream)
    torch.cuda.synchronize(dev)
    us = start.elapsed_time(stop) * 1e3 / (reps * nodes)
    if int(sink.item()) != 0:
        raise RuntimeError("read probe: the sink was written for a zero buffer")
    del graph
    return us


def characterize(w, inputs, dev, max_dist, reps=3):
    """Section 3.4 measurements (Figs. 8 and 10) on the dense decode map of
    layer 0, all lanes: mean mass split and vertical / diagonal similarity,
    with the time of the two kernels (HIP events on the launch stream)."""
    import numpy as np
    import torch

    import autoregressive_image_generation_amd as dsa

    x = inputs.layers[0]
    B, H, D, L, T = w.batch, w.heads, w.head_dim, w.L_p, w.L_dec
    lanes = B * H
    nbytes = dsa.dsa_profile_workspace_bytes(B, H, L, T, max_dist)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    mass = torch.empty((lanes, 3), dtype=torch.float64, device=dev)
    vert = torch.empty((lanes, max_dist), dtype=torch.float64, device=dev)
    diag = torch.empty((lanes, max_dist), dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        dsa.dsa_attention_profile(x["q"], x["k"], x["kp"] if L else None, B, H, D, L, T, w.input_dtype, max_dist, ws,
                                  nbytes, mass, vert, diag, stream)

    call()
    torch.cuda.synchronize(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        call()
    stop.record(stream)
    torch.cuda.synchronize(dev)
    ms = start.elapsed_time(stop) / reps
    m = mass.cpu().numpy().mean(axis=0)
    v = vert.cpu().numpy().mean(axis=0)
    g = diag.cpu().numpy().mean(axis=0)
    # algorithmic work of the map: one q.k per (query, causal key), the decode probabilities written once
    keys = T * L + T * (T + 1) // 2
    flops = 2.0 * D * keys * lanes
    map_bytes = 4.0 * (T * (T + 1) // 2) * lanes
    # ... and of the similarities: the vertical and the diagonal dot products of
    # every (i, i + d), i + 1 terms each (the prefix norms are running sums)
    band = sum((T - d) * (T - d + 1) // 2 for d in range(1, max_dist + 1))
    sim_flops = 2.0 * 2 * band * lanes
    picks = sorted({1, 2, w.grid_w, 2 * w.grid_w, max_dist} & set(range(1, max_dist + 1)))
    log("characterization: %.2f ms; mass prompt/local/middle %.3f/%.3f/%.3f" % (ms, *m))
    return {"layer": 0, "lanes": lanes, "T": T, "max_dist": max_dist, "ms": ms,
            "mass_prompt_local_middle": [float(a) for a in m],
            "vertical": {str(d): float(v[d - 1]) for d in picks},
            "diagonal": {str(d): float(g[d - 1]) for d in picks},
            "diagonal_minus_vertical_mean": float((g - v).mean()),
            "map_flop": flops, "map_prob_bytes": map_bytes, "similarity_flop": sim_flops,
            "note": "ms covers the three kernels (map: MFMA logits + softmax, writes the fp32 map; "
                    "similarity: banded MFMA Gram products; per-lane means)"}


def summarize_trace(path):
    """Per kernel and launch shape: dispatches and mean / min / max duration,
    plus the busy time (union of dispatch intervals) of each launch shape."""
    import csv
    from collections import defaultdict

    groups = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
            groups[key].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows = []
    for (name, grid, wg), iv in sorted(groups.items(), key=lambda kv: -sum(e - s for s, e in kv[1])):
        d = [e - s for s, e in iv]
        iv.sort()
        busy, cur_s, cur_e = 0, None, None
        for s0, e0 in iv:
            if cur_e is None or s0 > cur_e:
                if cur_e is not None:
                    busy += cur_e - cur_s
                cur_s, cur_e = s0, e0
            else:
                cur_e = max(cur_e, e0)
        busy += cur_e - cur_s
        rows.append({"kernel": name, "grid": grid, "workgroup": wg, "dispatches": len(d),
                     "mean_us": sum(d) / len(d) / 1e3, "min_us": min(d) / 1e3, "max_us": max(d) / 1e3,
                     "busy_us_per_dispatch": busy / len(d) / 1e3})
    for r in rows:
        print(json.dumps(r))


def cpu_baseline(w, target_cpu_seconds):
    """The oracle as it stands on a bounded, seeded sample of lanes (all L_dec
    steps each), one lane per host thread; returns the JSON object.  Inputs are
    generated outside the timed parts, in chunks so host memory stays small.
    Threads: the host's CPUs this process may use, at most 16 (the CPU share of
    one GPU on the boxes it runs on)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    threads = max(1, min(16, usable))
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
            "single_core_value": T / probe, "host_cpus": os.cpu_count(), "usable_cpus": usable,
            "sample": "%d seeded random (layer, batch, head) lanes x all %d decode steps of %s (fp64 C oracle, "
                      "one lane per thread on %d threads, %.1f s wall, ~%.0f CPU-s; one lane alone %.4f s)"
                      % (n, T, w.name, threads, wall, wall * threads, probe)}


def free_cuda():
    import gc

    import torch

    gc.collect()
    torch.cuda.empty_cache()


def measure_workload(w, dev, args, headline):
    """One workload: the sparse decode on S micro-batch streams (the rate) and on
    one stream (the kernel's roofline and its per-step series), and the dense
    kernel at the same batch.  Returns (result dict, inputs)."""
    import synth

    layers = args.layers or w.layers
    log("== %s: %d layers, batch %d, generating inputs" % (w.name, layers, w.batch))
    inputs = Inputs(w, layers, dev)
    log("inputs ready in %.1f s" % inputs.gen_seconds)
    head_steps = w.batch * layers * w.heads * w.L_dec
    S = args.streams if args.streams > 0 else (2 if w.batch % 2 == 0 else 1)
    waves = args.waves  # 0: the library's own choice
    steps, warmup = (args.steps, args.warmup) if headline else (args.leg_steps, 0)
    total_bytes = sum(sparse_bytes_per_head_step(w, t) for t in range(w.L_dec)) * w.batch * w.heads * layers
    n_launch = w.L_dec * layers  # launches per stream
    lanes = w.batch * w.heads

    # The whole job: the decode split into S micro-batches on S streams.
    sparse = SparseModel(w, inputs, layers, dev, waves, streams=S)
    sec, sec_ev = time_decodes(sparse, steps, warmup, dev)
    log("sparse (%d micro-batch streams): %.1f ms per decode (events %.1f ms)" % (S, sec * 1e3, sec_ev * 1e3))
    per_stream_launch_s = sum(sparse.stream_seconds) / S / n_launch

    # The kernel alone: the same decode on one stream.  Its launches run back
    # to back, so the timed region's HIP events (recorded on the stream the
    # library launches on) / the launches is the kernel's average launch
    # duration, gaps included, which is what rocprofv3's kernel trace reports
    # per dispatch.  With S streams, S launches overlap; the kernel trace
    # cannot follow that (the profiler serialises much of the overlap), so the
    # aggregate over streams is reported apart.
    if S > 1:
        sparse.free()
        del sparse
        free_cuda()
        single = SparseModel(w, inputs, layers, dev, args.waves, streams=1)
        s1, s1_ev = time_decodes(single, steps, warmup, dev)
        log("sparse, one stream: %.1f ms per decode" % (s1 * 1e3))
    else:
        single, s1, s1_ev = sparse, sec, sec_ev
    launch_s = s1_ev / n_launch
    bytes_per_launch = total_bytes / n_launch
    achieved = bytes_per_launch / launch_s / 1e9
    log("sparse kernel alone: %.2f us per launch over %d launches, %.0f GB/s" % (launch_s * 1e6, n_launch, achieved))
    wv = args.waves or library_waves(w, lanes)
    floor_us = launch_floor(dev, lanes, 64 * wv)
    log("launch floor (near-empty kernel, %d x %d threads, graph replay): %.2f us" % (lanes, 64 * wv, floor_us))
    phase_us, series = {}, None
    if not args.no_series:
        per_step = step_seconds(single, dev)
        phase_us, series = series_summary(w, per_step, layers)
    single.free()
    del single
    free_cuda()

    res = {
        "value": head_steps / sec,
        "unit": "head-steps/s",
        "ms_per_step": sec * 1e3,
        "steps": steps,
        "warmup": warmup if warmup else "partial decode of %d steps" % WARM_STEPS,
        "dtype": "bf16" if w.dtype == synth.BF16 else "fp32",
        "config": {"workload": w.name, "batch": w.batch, "layers": layers, "heads": w.heads,
                   "head_dim": w.head_dim, "L_p": w.L_p, "L_dec": w.L_dec, "N_r": w.N_r, "N_att": w.N_att,
                   "sink": w.sink, "sparsity": round(1 - w.N_att / w.L_dec, 4),
                   "step": "one full image decode: L_dec tokens x layers, all lanes",
                   "micro_batches": S,
                   "waves_per_lane": waves or "library choice",
                   "accumulation": "fp64 logits, fp32 softmax and PV"},
        "hbm_gbs": total_bytes / sec / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_for(w.name),
                     "traffic_over_algorithmic": traffic_for(w.name, ratio=True),
                     "kernel": "decode_kernel (sparse), whole batch per launch, one stream",
                     "avg_launch_us": launch_s * 1e6,
                     "bytes_per_launch": bytes_per_launch,
                     "launch_floor_us": floor_us,
                     "achieved_above_floor": bytes_per_launch / (launch_s - floor_us * 1e-6) / 1e9,
                     "us_per_launch_by_phase": phase_us,
                     "us_per_launch_by_step": series},
        "events_ms_per_step": sec_ev * 1e3,
    }
    if S > 1:
        agg = total_bytes / sec_ev / 1e9
        res["roofline_micro_batched"] = {
            "achieved": agg, "frac": agg / HBM_PEAK_GBS, "unit": "GB/s", "streams": S,
            "traffic": traffic_for(w.name, S),
            "avg_launch_us_per_stream": per_stream_launch_s * 1e6,
            "bytes_per_launch": total_bytes / n_launch / S,
            "note": "S launches of one micro-batch each in flight at once; all algorithmic bytes / event time"}
        res["single_stream"] = {"value": head_steps / s1, "ms_per_step": s1 * 1e3}

    if not args.no_dense_full:
        # the dense kernel at the same batch and in the same micro-batches; the
        # long decodes (L_dec > 576) are timed once, after a partial warm-up
        dsteps = args.leg_steps if w.L_dec <= 576 else 1
        dense = DenseModel(w, inputs, layers, dev, args.waves, w.batch, streams=S)
        dsec, _ = time_decodes(dense, dsteps, 0, dev)
        dense.free()
        del dense
        free_cuda()
        dbytes = sum(dense_bytes_per_head_step(w, t) for t in range(w.L_dec)) * w.batch * w.heads * layers
        res["dense_same_batch"] = {
            "batch": w.batch, "micro_batches": S, "value": head_steps / dsec, "unit": "head-steps/s",
            "ms_per_step": dsec * 1e3, "steps": dsteps, "hbm_gbs": dbytes / dsec / 1e9,
            "sparse_speedup": dsec / sec, "byte_ratio": dbytes / total_bytes,
            "budget_ratio": (w.L_p + w.N_r) / (w.L_p + w.N_att)}
        log("dense b%d: %.1f ms per decode -> sparse %.2fx (byte ratio %.2f)" % (
            w.batch, dsec * 1e3, dsec / sec, dbytes / total_bytes))
    return res, inputs


def headline_extras(w, inputs, res, dev, args):
    """What only the headline workload measures: the dense comparison at the
    extra batch, the last decode step alone, the policies, the MXFP8 cache, the
    characterization, the sweep and the read ceiling."""
    import synth

    layers = args.layers or w.layers
    S = args.streams if args.streams > 0 else (2 if w.batch % 2 == 0 else 1)
    waves = args.waves  # 0: the library's own choice
    head_steps = w.batch * layers * w.heads * w.L_dec
    sec = res["ms_per_step"] * 1e-3
    total_bytes = sum(sparse_bytes_per_head_step(w, t) for t in range(w.L_dec)) * w.batch * w.heads * layers
    ls = args.leg_steps

    if args.dense_batch and args.dense_batch < w.batch:
        db = args.dense_batch
        dS = S if db % S == 0 else 1
        wb = w.with_(batch=db)
        dense = DenseModel(wb, inputs, layers, dev, args.waves, db, streams=dS)
        dsec, _ = time_decodes(dense, ls, 0, dev)
        dense.free()
        del dense
        sparse_b = SparseModel(wb, inputs, layers, dev, args.waves, batch=db, streams=dS)
        ssec, _ = time_decodes(sparse_b, ls, 0, dev)
        sparse_b.free()
        del sparse_b
        free_cuda()
        dsteps = db * layers * w.heads * w.L_dec
        dbytes = sum(dense_bytes_per_head_step(w, t) for t in range(w.L_dec)) * db * w.heads * layers
        sbytes = sum(sparse_bytes_per_head_step(w, t) for t in range(w.L_dec)) * db * w.heads * layers
        res["dense_batch_%d" % db] = {
            "batch": db, "micro_batches": dS, "value": dsteps / dsec, "unit": "head-steps/s",
            "hbm_gbs": dbytes / dsec / 1e9, "ms_per_step": dsec * 1e3,
            "sparse_value": dsteps / ssec, "sparse_ms_per_step": ssec * 1e3, "sparse_hbm_gbs": sbytes / ssec / 1e9,
            "sparse_speedup": dsec / ssec, "byte_ratio": dbytes / sbytes,
            "budget_ratio": (w.L_p + w.N_r) / (w.L_p + w.N_att)}
        log("dense b%d: %.1f ms per decode; sparse b%d %.1f ms -> %.2fx" % (db, dsec * 1e3, db, ssec * 1e3,
                                                                           dsec / ssec))

        # The last decode step alone (attention only), one stream, batch db:
        # dense against sparse at 90 % and 95 % sparsity (N_att from the ratio),
        # the mean launch over the layers at t = L_dec - 1.
        last = {"batch": db, "t": w.L_dec - 1, "streams": 1}
        dense = DenseModel(wb, inputs, layers, dev, args.waves, db, streams=1)
        d_last = step_seconds(dense, dev)[-1] / layers
        dense.free()
        del dense
        last["dense_us"] = d_last * 1e6
        for sp in (0.9, 0.95):
            n_att = synth.n_att_for(w.L_dec, sp)
            ws_ = wb.with_(N_att=n_att)
            m = SparseModel(ws_, inputs, layers, dev, args.waves, batch=db, streams=1)
            s_last = step_seconds(m, dev)[-1] / layers
            m.free()
            del m
            rows_d = w.L_p + w.L_dec
            rows_s = w.L_p + n_att
            last["sparse_%g" % sp] = {"N_att": n_att, "us": s_last * 1e6, "speedup": d_last / s_last,
                                      "row_ratio": rows_d / rows_s}
            log("last step b%d: dense %.2f us, sparse %.2f (N_att %d) -> %.2fx" % (db, d_last * 1e6, s_last * 1e6,
                                                                                  n_att, d_last / s_last))
        free_cuda()
        res["last_step_attention_b%d" % db] = last

    if not args.no_policies:
        pol = []
        for policy in range(6):
            if policy in (1, 3) and w.N_att <= 4:
                continue
            m = SparseModel(w, inputs, layers, dev, waves, streams=S, policy=policy)
            s_p, _ = time_decodes(m, ls, 0, dev)
            b = sum(policy_bytes_per_head_step(w, policy, t) for t in range(w.L_dec)) * w.batch * w.heads * layers
            pol.append({"policy": POLICY_NAMES[policy], "N_r": policy_n_r(w, policy), "N_att": w.N_att,
                        "value": head_steps / s_p, "ms_per_step": s_p * 1e3, "hbm_gbs": b / s_p / 1e9,
                        "workspace_gb": m.nbytes * S * layers / 1e9})
            log("policy %s: %.1f ms per decode, %.0f GB/s" % (POLICY_NAMES[policy], s_p * 1e3, b / s_p / 1e9))
            m.free()
            del m
        free_cuda()
        res["policies"] = pol

    if not args.no_mxfp8 and w.dtype == synth.BF16:
        wm = w.with_(dtype=synth.MXFP8)
        m = SparseModel(wm, inputs, layers, dev, waves, streams=S)
        s_m, _ = time_decodes(m, ls, 0, dev)
        b = sum(sparse_bytes_per_head_step(wm, t) for t in range(w.L_dec)) * w.batch * w.heads * layers
        res["mxfp8_kv"] = {"value": head_steps / s_m, "unit": "head-steps/s", "ms_per_step": s_m * 1e3,
                           "hbm_gbs": b / s_m / 1e9, "speedup_vs_bf16_kv": sec / s_m,
                           "traffic_per_launch": traffic_for(w.name + "_mxfp8", S),
                           "traffic_over_algorithmic": traffic_for(w.name + "_mxfp8", S, ratio=True),
                           "algorithmic_bytes_per_launch": b / (w.L_dec * layers * S),
                           "byte_ratio": total_bytes / b, "workspace_gb": m.nbytes * S * layers / 1e9,
                           "kv": "MXFP8 (E4M3, E8M0 scale per 32), q/k/v bf16"}
        log("mxfp8 kv: %.1f ms per decode, %.0f GB/s, %.2fx the bf16 cache" % (s_m * 1e3, b / s_m / 1e9, sec / s_m))
        m.free()
        del m
        free_cuda()

    if args.profile_dist > 0:
        res["characterization"] = characterize(w, inputs, dev, args.profile_dist)

    if not args.no_sweep:
        sweep = []
        for sp in (0.0, 0.5, 0.8, 0.9, 0.95):
            n_att = synth.n_att_for(w.L_dec, sp)
            n_r = w.N_r if n_att <= w.N_r else w.L_dec
            ws_ = w.with_(N_att=n_att, N_r=n_r)
            m = SparseModel(ws_, inputs, layers, dev, args.waves, streams=S)
            s, _ = time_decodes(m, ls, 0, dev)
            b = sum(sparse_bytes_per_head_step(ws_, t) for t in range(w.L_dec)) * w.batch * w.heads * layers
            sweep.append({"sparsity": sp, "N_r": n_r, "N_att": n_att, "value": head_steps / s,
                          "ms_per_step": s * 1e3, "hbm_gbs": b / s / 1e9})
            log("sweep %.2f: %.1f ms" % (sp, s * 1e3))
            m.free()
            del m
        free_cuda()
        res["sweep"] = sweep

    if not args.no_ceiling:
        c = hbm_read_ceiling(dev)
        res["hbm_read_ceiling"] = {
            "kernel": "dsa_hbm_read_probe (16-byte non-temporal loads, grid-stride, 4 GiB, best launch shape)",
            "GBs": c["GBs"], "frac_of_peak": c["GBs"] / HBM_PEAK_GBS,
            "shape": {k: c[k] for k in ("blocks", "threads", "unroll")},
            "sparse_one_stream_frac_of_ceiling": res["roofline"]["achieved"] / c["GBs"],
            "sparse_micro_batched_frac_of_ceiling":
                res["roofline_micro_batched"]["achieved"] / c["GBs"] if "roofline_micro_batched" in res else None}
        log("hbm read ceiling: %.0f GB/s (%s)" % (c["GBs"], res["hbm_read_ceiling"]["shape"]))


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: no multi-GPU path is implemented (lanes would shard across "
              "GPUs with no exchange). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

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

    t_start = time.perf_counter()
    w = synth.WORKLOADS[args.workload]
    res, inputs = measure_workload(w, dev, args, headline=True)
    headline_extras(w, inputs, res, dev, args)
    del inputs
    free_cuda()
    if args.cpu_seconds > 0:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None

    legs = {}
    for name in [] if args.legs in ("", "none") else args.legs.split(","):
        if name == w.name:
            continue
        wl = synth.WORKLOADS[name]
        leg, leg_inputs = measure_workload(wl, dev, args, headline=False)
        del leg_inputs
        free_cuda()
        if args.cpu_seconds > 0:
            leg["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        legs[name] = leg
        log("leg %s: %.3g head-steps/s, one stream %.3f of peak, two streams %.3f" % (
            name, leg["value"], leg["roofline"]["frac"],
            leg.get("roofline_micro_batched", leg["roofline"])["frac"]))

    layers = args.layers or w.layers
    result = {
        "metric": "sparse decode-attn steps/s (batch x layers x heads) + HBM GB/s, Janus-Pro-7B shape",
        "value": res.pop("value"),
        "unit": res.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res.pop("dtype"),
        "data": "synthetic grid-rotary Q/K/V + N(0,0.1) noise, seed 0, resident in HBM",
        "config": res.pop("config"),
    }
    res.pop("steps")
    res.pop("warmup")
    result.update(res)
    result["legs"] = legs
    result["bench_seconds"] = time.perf_counter() - t_start
    assert layers == result["config"]["layers"]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
