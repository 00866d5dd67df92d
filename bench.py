#!/usr/bin/env python3
"""Benchmark: effective weight GB/s of the block-quantised decode hot path.

One *step* is one pass of the M = 1 hot path over one batch of synthetic
inputs, shaped like one decode step that streams many different weights
(the pages define effective bandwidth as bytes per token x tokens/s; the
metric is the M = 1 matvec's):

  1. qmv_q4_0           Q4_0 2048 x 2048, fp32 x
  2. qmv_q4_0_q8x       Q4_0 2048 x 2048, the same x quantised to Q8_0 in the
                        kernel's prologue (int path, own weight copy; the
                        codes and scales are written out too)
  3. qffn_gate_up_gelu  Q4_0 gate and up 8192 x 2048 -> h = G(gate x) * up x
  4. qmv_q4_0           Q4_0 down 2048 x 8192 against h
  5. qmv_q8_0           Q8_0 vocab 262144 x 2048 (0.57 GB of blocks), fp32 x

The prefill tile (qmm_tile_m, Q4_0 8192 x 2048 against M = 8, 16, 32 Q8_0
rows) is the path's other form; it is timed the same way in a loop of its
own right after the steps and reported as ``prefill_tiles`` (its bytes are
not M = 1 bytes, so they stay out of ``value``).

Every weight matrix is a distinct allocation, and ``--sets`` full copies of
the step's weights are rotated so nothing is served from the 256 MB
last-level cache between its uses. Inputs are resident in HBM before the
timed region. ``value`` = weight-block bytes streamed per step x steps /
wall time of the timed steps.

The roofline object is for the dominant kernel (the Q8_0 vocab matvec,
about 90 % of the step's bytes): algorithmic bytes per launch (weight
blocks + x + y) / its average duration from HIP events recorded on the
launch stream around its launch in every EVENT_EVERY-th step of the timed
region (launches_timed of them).

Also reported beside ``value`` (none of them replaces it):
  prefill_tiles        the three tiles per pass, timed like the steps
  chained              the steps recorded with gq_chain_*, CHAIN_STEPS
                       consecutive steps per chain (one graph launch), and
                       (one_step_per_replay) one step per chain
  read_stream_ceiling  best bandwidth of a plain 16-byte read-and-XOR kernel
                       (libgq_bench.so) over the 512 MiB vocab buffers;
                       breakdown rows give their % of it
  cpu_baseline[_threads]  the fp64 oracle on one thread / on T threads with
                       every matrix split by rows
  breakdown, extras    per-launch medians from HIP events
  per_config           each workload alone: launches over >= 2 GiB of rotated
                       weight copies, 7 timed repeats (median, min-max), the
                       host's issue time per launch, and 64-launch graph
                       figures over distinct copies and over one copy
                       (MALL-hot); the 64x256 Q8_0 config is a launch-latency
                       point, not a roofline point; Q4_K / Q5_K / Q6_K matvecs at
                       the 2048 x 2048, 8192 x 2048 and 262144 x 2048 shapes

Modes:
  python bench.py [--steps K --warmup W]    the benchmark (one JSON line)
  python bench.py --mode pmc                 vocab kernel + a calibration copy
                                             only, for rocprofv3 --pmc runs
  python bench.py --pmc-summary FETCH_DIR,WRITE_DIR [--write-profile]
                                             HBM bytes per launch from the two
                                             rocprofv3 counter runs
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective weight GB/s and % of HBM peak for Q4_0/Q8_0 matvec at M=1"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "qmv_q8_0_vocab_262144x2048_hbm_traffic.txt")
DOMINANT = "qmv_q8_0 262144x2048 (vocab)"
EVENT_EVERY = 4          # timed steps per event-bracketed dominant launch
CHAIN_STEPS = 8          # decode steps recorded per chain (one graph launch)
COPY_BYTES = 512 * 1024 * 1024        # calibration copy for the HBM counters


def kernel_source_hash(names=("gq_qmv.hip", "gq_device.hpp", "gq_launch.hpp")) -> str:
    """Hash of the sources a kernel is built from (default: the dominant one's)."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "gguf_block_quant_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------
# timing events
# ----------------------------------------------------------------------------

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
_hip = None


def _hip_runtime():
    """The HIP runtime torch has already loaded (resolved by its SONAME)."""
    global _hip
    if _hip is None:
        import ctypes

        import torch  # noqa: F401  (loads the runtime first)
        _hip = ctypes.CDLL("libamdhip64.so.7")
        _hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        _hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return _hip


class TimingEvent:
    """A HIP event used only for timing, created with
    hipEventDisableSystemFence: recording it does not write back and
    invalidate the caches (which a default event does, adding to the interval
    it brackets and slowing the work after it). Same interface as torch's
    timing events: record(stream), elapsed_time(end) in milliseconds."""

    def __init__(self):
        import ctypes
        self._ctypes = ctypes
        self.ev = ctypes.c_void_p()
        if _hip_runtime().hipEventCreateWithFlags(ctypes.byref(self.ev), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if _hip_runtime().hipEventRecord(self.ev, self._ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        ms = self._ctypes.c_float()
        if _hip_runtime().hipEventElapsedTime(self._ctypes.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        # (at interpreter exit the module globals may already be gone; the
        # runtime frees its events with the process then)
        try:
            if self.ev and _hip is not None:
                _hip.hipEventDestroy(self.ev)
        except Exception:
            pass


# ----------------------------------------------------------------------------
# workload
# ----------------------------------------------------------------------------

class Step:
    """The step's launches, with every pointer and size precomputed so the
    host issues each C-ABI call directly (a few microseconds each)."""

    def __init__(self, sets: int, log):
        import ctypes

        import numpy as np
        import torch

        import gguf_block_quant_amd as gq
        import synth

        self.torch = torch
        self.gq = gq
        L = gq.raw()
        dev = torch.device("cuda:0")
        # a stream of its own (default priority): the step can then also be
        # recorded as one chain, which the legacy default stream cannot
        self.stream = torch.cuda.Stream()
        sp = ctypes.c_void_p(self.stream.cuda_stream)
        self.sp = sp
        P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731

        def up(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to(dev)

        def pack(qtype, blocks, n, k):
            raw = up(synth.as_bytes(blocks).reshape(-1))
            qs, d = gq.pack(qtype, raw, n, k)
            torch.cuda.synchronize()
            del raw
            return qs, d

        t0 = time.time()
        c2 = synth.workload_q4_0_2048()
        c3 = synth.workload_ffn()
        c5 = synth.workload_tile()
        log("generated small workloads in %.1fs" % (time.time() - t0))
        t0 = time.time()
        c4 = synth.workload_vocab()
        log("generated vocab workload in %.1fs" % (time.time() - t0))
        self.host = {"c2": c2, "c3": c3, "c4": c4, "c5": c5}

        Q4, Q8 = gq.TYPE_Q4_0, gq.TYPE_Q8_0
        x2, x3, x4 = up(c2["x"]), up(c3["x"]), up(c4["x"])
        xq2 = torch.empty(2048, dtype=torch.int8, device=dev)
        xd2 = torch.empty(64, dtype=torch.int16, device=dev)
        y2a = torch.empty(2048, dtype=torch.float32, device=dev)
        y2b = torch.empty(2048, dtype=torch.float32, device=dev)
        h3 = torch.empty(8192, dtype=torch.float32, device=dev)
        y3 = torch.empty(2048, dtype=torch.float32, device=dev)
        y4 = torch.empty(262144, dtype=torch.float32, device=dev)
        acts = {m: (up(c5["acts"][m][0]), up(c5["acts"][m][1])) for m in (8, 16, 32)}
        yt = {m: torch.empty((m, 8192), dtype=torch.float32, device=dev) for m in (8, 16, 32)}
        self.keep = [x2, x3, x4, xq2, xd2, y2a, y2b, h3, y3, y4, acts, yt]
        self.outputs = {"y2a": y2a, "y2b": y2b, "h3": h3, "y3": y3, "y4": y4, "yt": yt}

        t0 = time.time()
        self.sets = []
        for s in range(sets):
            w2a = pack(Q4, c2["w"], 2048, 2048)
            w2b = pack(Q4, c2["w"], 2048, 2048)
            wg = pack(Q4, c3["wg"], 8192, 2048)
            wu = pack(Q4, c3["wu"], 8192, 2048)
            wd = pack(Q4, c3["wd"], 2048, 8192)
            wv = pack(Q8, c4["w"], 262144, 2048)
            wt = {m: pack(Q4, c5["w"], 8192, 2048) for m in (8, 16, 32)}
            self.keep.append((w2a, w2b, wg, wu, wd, wv, wt))
            self.vocab_qs = getattr(self, "vocab_qs", []) + [wv[0]]
            self.vocab_sets = getattr(self, "vocab_sets", []) + [wv]
            self.tile_weights = getattr(self, "tile_weights", []) + [wt]
            launches = [
                ("qmv_q4_0 2048x2048", L.gq_qmv_q4_0, (P(w2a[0]), P(w2a[1]), 2048, 2048, P(x2), P(y2a), sp),
                 2048 * 64 * 18, 8192 + 8192),
                ("qmv_q4_0_q8x 2048x2048 (quantise folded in)", L.gq_qmv_q4_0_q8x,
                 (P(w2b[0]), P(w2b[1]), 2048, 2048, P(x2), P(xq2), P(xd2), P(y2b), None, sp), 2048 * 64 * 18,
                 8192 + 2176 + 8192),
                ("qffn_gate_up_gelu 8192x2048", L.gq_qffn_gate_up_gelu,
                 (P(wg[0]), P(wg[1]), P(wu[0]), P(wu[1]), 8192, 2048, P(x3), P(h3), sp), 2 * 8192 * 64 * 18,
                 8192 + 32768),
                ("qmv_q4_0 2048x8192 (down)", L.gq_qmv_q4_0, (P(wd[0]), P(wd[1]), 2048, 8192, P(h3), P(y3), sp),
                 2048 * 256 * 18, 32768 + 8192),
                (DOMINANT, L.gq_qmv_q8_0, (P(wv[0]), P(wv[1]), 262144, 2048, P(x4), P(y4), sp),
                 262144 * 64 * 34, 8192 + 262144 * 4),
            ]
            tiles = []
            for m in (8, 16, 32):
                tiles.append(("qmm_tile_m 8192x2048 M=%d" % m, L.gq_qmm_tile_m,
                              (P(wt[m][0]), P(wt[m][1]), 8192, 2048, m, P(acts[m][0]), P(acts[m][1]),
                               P(yt[m]), None, sp), 8192 * 64 * 18, m * 2176 + m * 8192 * 4))
            self.sets.append(launches)
            self.tile_sets = getattr(self, "tile_sets", []) + [tiles]
            if s == 0:
                # entry points beyond the step (the folds around a projection,
                # the vocabulary head, a batched-decode tile), timed on their own
                rng = np.random.default_rng(1)
                g2 = up(rng.uniform(0.5, 1.5, 2048).astype(np.float32))
                res2 = up(rng.standard_normal(2048).astype(np.float32))
                y2c = torch.empty(2048, dtype=torch.float32, device=dev)
                logits = torch.empty(262144, dtype=torch.float32, device=dev)
                ws = torch.zeros(gq.argmax_workspace_bytes(), dtype=torch.uint8, device=dev)
                idx = torch.empty(1, dtype=torch.int32, device=dev)
                val = torch.empty(1, dtype=torch.float32, device=dev)
                xq4, xd4 = (up(c5["acts"][8][0][:4].copy()), up(c5["acts"][8][1][:4].copy()))
                y4t = torch.empty((4, 8192), dtype=torch.float32, device=dev)
                self.keep += [g2, res2, y2c, logits, ws, idx, val, xq4, xd4, y4t]
                self.extras = [
                    ("quantize_q8_0 2048 (standalone)", L.gq_quantize_q8_0, (P(x2), 1, 2048, P(xq2), P(xd2), sp), 0,
                     2048 * 4 + 2048 + 128),
                    ("qmv_q4_0_q8 2048x2048 (pre-quantised x)", L.gq_qmv_q4_0_q8,
                     (P(w2b[0]), P(w2b[1]), 2048, 2048, P(xq2), P(xd2), P(y2b), None, sp), 2048 * 64 * 18,
                     2176 + 8192),
                    ("qmv_q4_0_ex 2048x2048 (rmsnorm + residual)", L.gq_qmv_q4_0_ex,
                     (P(w2a[0]), P(w2a[1]), 2048, 2048, P(x2), P(g2), ctypes.c_float(1e-6), P(res2), P(y2c), sp),
                     2048 * 64 * 18, 8192 * 3 + 8192),
                    ("qffn_gate_up_gelu_ex 8192x2048 (rmsnorm)", L.gq_qffn_gate_up_gelu_ex,
                     (P(wg[0]), P(wg[1]), P(wu[0]), P(wu[1]), 8192, 2048, P(x3), P(g2), ctypes.c_float(1e-6),
                      P(h3), sp), 2 * 8192 * 64 * 18, 8192 * 2 + 32768),
                    ("qmv_q8_0_argmax 262144x2048 (rmsnorm + softcap 30 + argmax)", L.gq_qmv_q8_0_argmax,
                     (P(wv[0]), P(wv[1]), 262144, 2048, P(x4), P(g2), ctypes.c_float(1e-6), ctypes.c_float(30.0),
                      P(logits), P(ws), ws.numel(), P(idx), P(val), sp), 262144 * 64 * 34, 8192 * 2 + 262144 * 4),
                    ("qmm_tile_m 8192x2048 M=4 (batched decode)", L.gq_qmm_tile_m,
                     (P(wt[8][0]), P(wt[8][1]), 8192, 2048, 4, P(xq4), P(xd4), P(y4t), None, sp),
                     8192 * 64 * 18, 4 * 2176 + 4 * 8192 * 4),
                ]
        torch.cuda.synchronize()
        log("packed %d weight set(s) in %.1fs" % (sets, time.time() - t0))
        self.names = [l[0] for l in self.sets[0]]
        self.tile_names = [l[0] for l in self.tile_sets[0]]
        self.weight_bytes = {l[0]: l[3] for l in self.sets[0] + self.tile_sets[0]}
        self.other_bytes = {l[0]: l[4] for l in self.sets[0] + self.tile_sets[0]}
        self.step_weight_bytes = sum(self.weight_bytes[n] for n in self.names)
        self.tile_weight_bytes = sum(self.weight_bytes[n] for n in self.tile_names)

    def record_chains(self, steps_per_chain=1):
        """Recorded chains of steps_per_chain consecutive steps each (every
        weight set's steps in turn, as the eager loop runs them), enough
        chains for each to start on a different set when the count divides
        evenly; one chain is one graph launch."""
        self.chains = []
        n = len(self.sets) if steps_per_chain % len(self.sets) else 1
        for c0 in range(n):
            c = self.gq.Chain(self.stream)
            with c:
                for j in range(steps_per_chain):
                    self.run(c0 * steps_per_chain + j)
            self.chains.append(c)

    def close_chains(self):
        for c in self.chains:
            c.close()
        self.chains = []

    def replay(self, i):
        self.chains[i % len(self.chains)].launch(self.stream)

    def run(self, i, events=None, tiles=False):
        """Enqueue step i (or, with tiles, pass i of the prefill tiles);
        events maps a launch name to a list collecting (start, end) event
        pairs recorded around that launch."""
        sets = self.tile_sets if tiles else self.sets
        for name, fn, args, _, _ in sets[i % len(sets)]:
            if events is not None and name in events:
                a = TimingEvent()
                b = TimingEvent()
                a.record(self.stream)
                st = fn(*args)
                b.record(self.stream)
                events[name].append((a, b))
            else:
                st = fn(*args)
            if st != 0:
                raise self.gq.GQError(st, name)


def per_config(step, ceiling_gbps, log, rotate_bytes=2 << 30):
    """Each workload on its own, as a throughput measurement: enough packed
    copies of its weights to cover >= 2 GiB (so consecutive launches never
    find their weights in the 256 MB last-level cache), 10 warm-up launches,
    then 7 repeats of [event, L launches cycling through the copies, event]
    with L chosen so a repeat takes >= 20 ms; median and min-max per launch.
    Beside it: a graph figure (64 launches over distinct copies recorded as
    one chain and replayed, free of the host's per-call cost) and the same
    over one copy (MALL-hot, not an HBM figure)."""
    import ctypes
    import math

    import numpy as np
    import torch

    import synth

    gq = step.gq
    L = gq.raw()
    sp = step.sp
    dev = torch.device("cuda:0")
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    def copies(qtype, blocks, n, k, count):
        raw = up(synth.as_bytes(blocks).reshape(-1))
        out = [gq.pack(qtype, raw, n, k) for _ in range(count)]
        torch.cuda.synchronize()
        return out

    Q4, Q8 = gq.TYPE_Q4_0, gq.TYPE_Q8_0
    host = step.host
    c1 = synth.workload_q8_0_small()
    x1, y1 = up(c1["x"]), torch.empty(64, dtype=torch.float32, device=dev)
    x2, y2 = up(host["c2"]["x"]), torch.empty(2048, dtype=torch.float32, device=dev)
    xq2 = torch.empty(2048, dtype=torch.int8, device=dev)
    xd2 = torch.empty(64, dtype=torch.int16, device=dev)
    x3, h3 = up(host["c3"]["x"]), torch.empty(8192, dtype=torch.float32, device=dev)
    y3 = torch.empty(2048, dtype=torch.float32, device=dev)
    x4, y4 = up(host["c4"]["x"]), torch.empty(262144, dtype=torch.float32, device=dev)
    acts = {m: (up(host["c5"]["acts"][m][0]), up(host["c5"]["acts"][m][1])) for m in (8, 16, 32)}
    yt = {m: torch.empty((m, 8192), dtype=torch.float32, device=dev) for m in (8, 16, 32)}

    def ncopies(nbytes):
        return max(2, math.ceil(rotate_bytes / nbytes))

    rows = []
    w1 = copies(Q8, c1["w"], 64, 256, 64)
    rows.append(("C1 qmv_q8_0 64x256", 64 * 8 * 34, 1024 + 256,
                 [(L.gq_qmv_q8_0, (P(q), P(d), 64, 256, P(x1), P(y1), sp)) for q, d in w1]))
    w2 = copies(Q4, host["c2"]["w"], 2048, 2048, ncopies(2359296))
    rows.append(("C2 qmv_q4_0 2048x2048 fp32 x", 2359296, 8192 + 8192,
                 [(L.gq_qmv_q4_0, (P(q), P(d), 2048, 2048, P(x2), P(y2), sp)) for q, d in w2]))
    rows.append(("C2 qmv_q4_0_q8x 2048x2048 (Q8_0 x, quantised in the kernel)", 2359296, 8192 + 2176 + 8192,
                 [(L.gq_qmv_q4_0_q8x, (P(q), P(d), 2048, 2048, P(x2), P(xq2), P(xd2), P(y2), None, sp))
                  for q, d in w2]))
    nf = ncopies(3 * 9437184)
    wg = copies(Q4, host["c3"]["wg"], 8192, 2048, nf)
    wu = copies(Q4, host["c3"]["wu"], 8192, 2048, nf)
    wd = copies(Q4, host["c3"]["wd"], 2048, 8192, nf)
    gate_up = [(L.gq_qffn_gate_up_gelu, (P(g[0]), P(g[1]), P(u[0]), P(u[1]), 8192, 2048, P(x3), P(h3), sp))
               for g, u in zip(wg, wu)]
    down = [(L.gq_qmv_q4_0, (P(q), P(d), 2048, 8192, P(h3), P(y3), sp)) for q, d in wd]
    rows.append(("C3 qffn_gate_up_gelu 2x8192x2048", 2 * 9437184, 8192 + 32768, gate_up))
    rows.append(("C3 down qmv_q4_0 2048x8192", 9437184, 32768 + 8192, down))
    rows.append(("C3 FFN gate+up then down (pairs)", 3 * 9437184, 8192 + 2 * 32768 + 8192,
                 [pair for pair in zip(gate_up, down)]))
    rows.append(("C4 qmv_q8_0 262144x2048", 570425344, 8192 + 1048576,
                 [(L.gq_qmv_q8_0, (P(q), P(d), 262144, 2048, P(x4), P(y4), sp)) for q, d in step.vocab_sets]))
    # one GPU's share when the path is split over 8 GPUs (rows of the vocab
    # head; gate/up rows and down's k for the FFN, whose partial y would then
    # be summed across GPUs): the kernels at the shapes one GPU would run.
    # Row shards are contiguous views of the full copies; down's k shards
    # are packed on their own.
    y4s = torch.empty(32768, dtype=torch.float32, device=dev)
    rows.append(("C4/8 qmv_q8_0 32768x2048 (one GPU's rows of 8)", 71303168, 8192 + 131072,
                 [(L.gq_qmv_q8_0, (P(q[s * 32768:(s + 1) * 32768]), P(d[s * 32768:(s + 1) * 32768]), 32768, 2048,
                                   P(x4), P(y4s), sp)) for q, d in step.vocab_sets for s in range(8)]))
    wd_blocks = host["c3"]["wd"]
    wds = [copies(Q4, np.ascontiguousarray(wd_blocks[:, s * 32:(s + 1) * 32]), 2048, 1024, nf) for s in range(8)]
    h3s, y3s = torch.empty(1024, dtype=torch.float32, device=dev), torch.empty(2048, dtype=torch.float32, device=dev)
    gate_up8 = [(L.gq_qffn_gate_up_gelu, (P(g[0][s * 1024:(s + 1) * 1024]), P(g[1][s * 1024:(s + 1) * 1024]),
                                          P(u[0][s * 1024:(s + 1) * 1024]), P(u[1][s * 1024:(s + 1) * 1024]),
                                          1024, 2048, P(x3), P(h3s), sp))
                for g, u in zip(wg, wu) for s in range(8)]
    down8 = [(L.gq_qmv_q4_0, (P(q), P(d), 2048, 1024, P(h3s), P(y3s), sp)) for c in range(nf) for s in range(8)
             for q, d in [wds[s][c]]]
    rows.append(("C3/8 FFN gate+up 2x1024x2048 then down 2048x1024 (one GPU's share of 8, pairs)",
                 3 * 1179648, 8192 + 2 * 4096 + 8192, [pair for pair in zip(gate_up8, down8)]))
    w5 = copies(Q4, host["c5"]["w"], 8192, 2048, ncopies(9437184))
    for m in (8, 16, 32):
        rows.append(("C5 qmm_tile_m 8192x2048 M=%d" % m, 9437184, m * 2176 + m * 8192 * 4,
                     [(L.gq_qmm_tile_m, (P(q), P(d), 8192, 2048, m, P(acts[m][0]), P(acts[m][1]), P(yt[m]), None,
                                         sp)) for q, d in w5]))
    # the folds around a projection and the fused vocabulary head (RMSNorm
    # prologue, residual epilogue; soft cap and the two-stage greedy argmax),
    # on the same rotated weights as their plain rows above
    rngf = np.random.default_rng(1)
    gf = up(rngf.uniform(0.5, 1.5, 2048).astype(np.float32))
    resf = up(rngf.standard_normal(2048).astype(np.float32))
    y2f, h3f = torch.empty(2048, dtype=torch.float32, device=dev), torch.empty(8192, dtype=torch.float32, device=dev)
    logitsf = torch.empty(262144, dtype=torch.float32, device=dev)
    wsf = torch.zeros(gq.argmax_workspace_bytes(), dtype=torch.uint8, device=dev)
    idxf, valf = torch.empty(1, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.float32, device=dev)
    eps = ctypes.c_float(1e-6)
    rows.append(("F1 qmv_q4_0_ex 2048x2048 (rmsnorm + residual)", 2359296, 3 * 8192 + 8192,
                 [(L.gq_qmv_q4_0_ex, (P(q), P(d), 2048, 2048, P(x2), P(gf), eps, P(resf), P(y2f), sp))
                  for q, d in w2]))
    rows.append(("F1 qffn_gate_up_gelu_ex 2x8192x2048 (rmsnorm)", 2 * 9437184, 2 * 8192 + 32768,
                 [(L.gq_qffn_gate_up_gelu_ex, (P(g[0]), P(g[1]), P(u[0]), P(u[1]), 8192, 2048, P(x3), P(gf), eps,
                                               P(h3f), sp)) for g, u in zip(wg, wu)]))
    rows.append(("F2 qmv_q8_0_argmax 262144x2048 (rmsnorm + softcap 30 + argmax, two launches)", 570425344,
                 2 * 8192 + 4 * 262144,
                 [(L.gq_qmv_q8_0_argmax, (P(q), P(d), 262144, 2048, P(x4), P(gf), eps, ctypes.c_float(30.0),
                                          P(logitsf), P(wsf), wsf.numel(), P(idxf), P(valf), sp))
                  for q, d in step.vocab_sets]))
    fold_keep = [gf, resf, y2f, h3f, logitsf, wsf, idxf, valf]

    # K-quant matvecs (fp32 x, k = 2048): the decode shapes, and a
    # vocabulary-sized matrix that streams from HBM at the steady rate
    def kq_copies(qtype, blocks, n, k, count):
        raw = up(synth.as_bytes(blocks).reshape(-1))
        out = [gq.kq_pack(qtype, raw, n, k) for _ in range(count)]
        torch.cuda.synchronize()
        return out

    xk = up(synth.activations(np.random.default_rng(5), 2048))
    kq_keep = [xk]
    for qtype, tname, fn, sb_bytes in ((gq.TYPE_Q4_K, "Q4_K", L.gq_qmv_q4_k, 144),
                                      (gq.TYPE_Q5_K, "Q5_K", L.gq_qmv_q5_k, 176),
                                      (gq.TYPE_Q6_K, "Q6_K", L.gq_qmv_q6_k, 210)):
        for n in (2048, 8192, 262144):
            wbytes = n * 8 * sb_bytes
            kc = kq_copies(qtype, synth.weights(np.random.default_rng(n + qtype), qtype, n, 2048), n, 2048,
                           ncopies(wbytes))
            yk = torch.empty(n, dtype=torch.float32, device=dev)
            kq_keep += [kc, yk]
            rows.append(("K qmv_%s %dx2048" % (tname.lower(), n), wbytes, 8192 + 4 * n,
                         [(fn, (P(pk), n, 2048, P(xk), P(yk), sp)) for pk in kc]))
    keep = [w1, w2, wg, wu, wd, wds, w5, x1, y1, x2, y2, xq2, xd2, x3, h3, y3, x4, y4, y4s, h3s, y3s, acts, yt,
            kq_keep, fold_keep]

    def issue(launch):
        for fn, fargs in (launch if isinstance(launch[0], tuple) else (launch,)):
            if fn(*fargs) != 0:
                raise RuntimeError("launch failed in the per-config pass")

    out = {}
    for name, wbytes, obytes, launches in rows:
        nl = len(launches)
        for i in range(10):
            issue(launches[i % nl])
        torch.cuda.synchronize()
        # launches per repeat: >= 20 ms, from a first estimate
        a, b = TimingEvent(), TimingEvent()
        a.record(step.stream)
        for i in range(min(nl, 64)):
            issue(launches[i % nl])
        b.record(step.stream)
        torch.cuda.synchronize()
        est_us = a.elapsed_time(b) * 1e3 / min(nl, 64)
        per = max(nl, int(math.ceil(20000.0 / max(est_us, 0.5))))
        reps, host = [], []
        for _ in range(7):
            a, b = TimingEvent(), TimingEvent()
            a.record(step.stream)
            t0 = time.perf_counter()
            for i in range(per):
                issue(launches[i % nl])
            host.append((time.perf_counter() - t0) * 1e6 / per)
            b.record(step.stream)
            torch.cuda.synchronize()
            reps.append(a.elapsed_time(b) * 1e3 / per)
        reps.sort()
        med = reps[3]
        host_us = sorted(host)[3]
        def graph_us(pick):
            """64 launches recorded as one chain, replayed 7 times: per-launch
            device time without the host's per-call cost."""
            chain = gq.Chain(step.stream)
            with chain:
                for i in range(64):
                    issue(launches[pick(i)])
            chain.launch(step.stream)
            torch.cuda.synchronize()
            a, b = TimingEvent(), TimingEvent()
            a.record(step.stream)
            for _ in range(7):
                chain.launch(step.stream)
            b.record(step.stream)
            torch.cuda.synchronize()
            chain.close()
            return a.elapsed_time(b) * 1e3 / (7 * 64)

        graph_cold = graph_us(lambda i: i % nl)      # distinct copies
        graph_hot = graph_us(lambda i: 0)            # one copy: MALL-resident after the first
        out[name] = {
            "median_us": round(med, 3), "min_us": round(reps[0], 3), "max_us": round(reps[-1], 3),
            "launches_per_repeat": per, "copies_rotated": nl,
            "weight_GBps": round(wbytes / med / 1e3, 1), "total_GBps": round((wbytes + obytes) / med / 1e3, 1),
            "pct_of_8TBps": round(100.0 * wbytes / med / 1e3 / HBM_PEAK_GBPS, 1),
            "pct_of_read_ceiling": round(100.0 * (wbytes + obytes) / med / 1e3 / ceiling_gbps, 1),
            "calls_per_s": round(1e6 / med, 1),
            "tokens_per_s_at_0.783GB": round(wbytes / med / 1e3 / 0.783, 1),
            "graph_us_per_launch": round(graph_cold, 3), "graph_hot_MALL_us_per_launch": round(graph_hot, 3),
            # the host's own time to issue one launch through the C ABI; where
            # it reaches median_us the eager figure is host-bound and the graph
            # figure is the device's
            "host_issue_us": round(host_us, 3),
        }
        log("per-config %s: %.2f us (%.0f GB/s)" % (name, med, wbytes / med / 1e3))
    del keep
    torch.cuda.synchronize()
    return out


def _event_times(step, fn, fargs, reps):
    """Per-launch durations (us, sorted) from HIP events around each launch."""
    torch = step.torch
    evs = []
    for _ in range(reps):
        a = TimingEvent()
        b = TimingEvent()
        a.record(step.stream)
        if fn(*fargs) != 0:
            raise RuntimeError("launch failed")
        b.record(step.stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) * 1e3 for a, b in evs)


def read_stream_ceiling(step, log):
    """Best bandwidth of a plain 16-byte non-temporal read-and-XOR kernel
    (libgq_bench.so) over the rotated vocab quant buffers (512 MiB each, so
    consecutive launches never hit in the last-level cache)."""
    import ctypes

    torch = step.torch
    lib = ctypes.CDLL(os.path.join(ROOT, "gguf_block_quant_amd", "libgq_bench.so"))
    lib.gqb_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_void_p]
    lib.gqb_read_stream.restype = ctypes.c_int
    bufs = step.vocab_qs
    nbytes = bufs[0].numel() * bufs[0].element_size()
    grids = (256, 512, 1024, 2048)
    out = torch.empty(max(grids) * 256, dtype=torch.int32, device="cuda")
    best = (0.0, 0, 0)
    for g, pattern in [(g, pt) for g in grids for pt in (0, 1)]:
        def launch(i):
            return lib.gqb_read_stream(ctypes.c_void_p(bufs[i % len(bufs)].data_ptr()), nbytes,
                                       ctypes.c_void_p(out.data_ptr()), g, pattern, step.sp)
        for i in range(2):
            if launch(i) != 0:
                raise RuntimeError("read-stream launch failed")
        torch.cuda.synchronize()
        a = TimingEvent()
        b = TimingEvent()
        reps = 8
        a.record(step.stream)
        for i in range(reps):
            launch(i)
        b.record(step.stream)
        torch.cuda.synchronize()
        gbps = nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
        best = max(best, (gbps, g, pattern))
    log("read-stream ceiling %.0f GB/s (grid %d, shape %d)" % best)
    return {"GBps": round(best[0], 1), "grid": best[1],
            "shape": ("lane grid-stride", "wave 8 KiB chunks")[best[2]], "bytes_per_launch": nbytes,
            "kernel": "16-byte non-temporal loads, XOR-reduce, 256-thread workgroups; best of 4 grids x 2 "
                      "access shapes"}


# ----------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on the same inputs
# ----------------------------------------------------------------------------

def cpu_baseline(host, weight_bytes_per_step, seconds, log):
    import numpy as np

    import oracle

    c2, c3, c4 = host["c2"], host["c3"], host["c4"]
    Q4, Q8 = oracle.TYPE_Q4_0, oracle.TYPE_Q8_0

    def one_pass():
        oracle.matvec(Q4, c2["w"], 2048, 2048, c2["x"])
        xq, xd = oracle.quantize_q8_0(c2["x"])
        oracle.blockdots(Q4, c2["w"], 2048, 2048, xq, xd, want_s=False)
        f = oracle.ffn_gate_up(Q4, c3["wg"], c3["wu"], 8192, 2048, c3["x"])
        oracle.matvec(Q4, c3["wd"], 2048, 8192, f["h"])
        oracle.matvec(Q8, c4["w"], 262144, 2048, c4["x"])

    passes = 0
    t0 = time.perf_counter()
    while True:
        one_pass()
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    log("oracle: %d pass(es) in %.1fs" % (passes, el))
    return {
        "value": round(weight_bytes_per_step * passes / el / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "%d full pass(es) of the M=1 step's workload (every kernel once, same inputs) through the "
                  "single-threaded fp64 C oracle, %.1f s; weight-block bytes / time" % (passes, el),
        "seconds_per_step": round(el / passes, 3),
        "cpu": cpu_description(),
    }


def cpu_description():
    """Model name, sockets and logical CPUs of the host (from /proc/cpuinfo
    where it exists)."""
    model, sockets = None, set()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key = key.strip()
                if key == "model name" and model is None:
                    model = val.strip()
                elif key == "physical id":
                    sockets.add(val.strip())
    except OSError:
        pass
    model = model or platform.processor() or platform.machine()
    return "%s; %d socket(s), %d logical CPUs" % (model, max(1, len(sockets)), os.cpu_count() or 1)


def cpu_baseline_threads(host, weight_bytes_per_step, seconds, log):
    """The same oracle calls with every matrix split by rows into T contiguous
    chunks run on T threads (a chunk never splits a dot product; the C
    oracle runs without the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    c2, c3, c4 = host["c2"], host["c3"], host["c4"]
    Q4, Q8 = oracle.TYPE_Q4_0, oracle.TYPE_Q8_0
    T = max(1, min(os.cpu_count() or 1, 16))
    pool = ThreadPoolExecutor(T)

    def split(n):
        step = (n + T - 1) // T
        return [(r, min(n, r + step)) for r in range(0, n, step)]

    def rows(fn, w, n, *a):
        list(pool.map(lambda rr: fn(w[rr[0]:rr[1]], rr[1] - rr[0], *a), split(n)))

    def one_pass():
        rows(lambda w, n, k, x: oracle.matvec(Q4, w, n, k, x), c2["w"], 2048, 2048, c2["x"])
        xq, xd = oracle.quantize_q8_0(c2["x"])
        rows(lambda w, n, k: oracle.blockdots(Q4, w, n, k, xq, xd, want_s=False), c2["w"], 2048, 2048)
        hs = list(pool.map(lambda rr: oracle.ffn_gate_up(Q4, c3["wg"][rr[0]:rr[1]], c3["wu"][rr[0]:rr[1]],
                                                         rr[1] - rr[0], 2048, c3["x"])["h"], split(8192)))
        import numpy as np
        h = np.concatenate(hs)
        rows(lambda w, n, k: oracle.matvec(Q4, w, n, k, h), c3["wd"], 2048, 8192)
        rows(lambda w, n, k: oracle.matvec(Q8, w, n, k, c4["x"]), c4["w"], 262144, 2048)

    passes = 0
    t0 = time.perf_counter()
    while True:
        one_pass()
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    pool.shutdown()
    log("oracle on %d threads: %d pass(es) in %.1fs" % (T, passes, el))
    return {
        "value": round(weight_bytes_per_step * passes / el / 1e9, 4),
        "unit": "GB/s",
        "cores": T,
        "kind": "oracle",
        "sample": "%d full pass(es) of the step's workload through the fp64 C oracle, every matrix split "
                  "by rows over %d threads, %.1f s" % (passes, T, el),
        "seconds_per_step": round(el / passes, 3),
        "cpu": cpu_description(),
    }


# ----------------------------------------------------------------------------
# rocprofv3 counter runs
# ----------------------------------------------------------------------------

def pmc_mode(args, log):
    """Only the vocab kernel (3 launches) and a calibration copy of known
    size (3 launches), so a rocprofv3 --pmc pass stays short."""
    import torch

    step = Step(1, log)
    name, fn, fargs, _, _ = [l for l in step.sets[0] if l[0] == DOMINANT][0]
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        if fn(*fargs) != 0:
            raise RuntimeError("launch failed")
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("pmc pass done: 3 x %s, 3 x copy of %d bytes" % (name, COPY_BYTES))


def pmc_step_mode(args, log):
    """Three steps (every launch of the step, 3 times), then a calibration
    copy of known size (3 launches), for the per-kernel counter passes
    (VALU / MFMA, and HBM bytes). Prints the step's launches with their
    algorithmic bytes as one JSON line, in launch order."""
    import torch

    step = Step(1, log)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for i in range(3):
        step.run(i)
        step.run(i, tiles=True)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    launches = step.sets[0] + step.tile_sets[0]
    print(json.dumps({"step_launches": [[n, w, o] for n, _, _, w, o in launches], "steps": 3}), flush=True)
    log("pmc pass done: 3 steps of %d launches, 3 x copy of %d bytes" % (len(launches), COPY_BYTES))


def pmc_kq_mode(args, log):
    """The K-quant matvecs at 262144 x 2048 (3 launches each, Q4_K, Q5_K,
    then Q6_K), then a calibration copy of known size (3 launches), for the
    rocprofv3 --pmc passes of the K-quant kernels. Prints the launches with
    their algorithmic bytes as one JSON line."""
    import ctypes

    import numpy as np
    import torch

    import gguf_block_quant_amd as gq
    import synth

    L = gq.raw()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    n, k = 262144, 2048
    x = torch.from_numpy(synth.activations(np.random.default_rng(5), k)).cuda()
    launches, work = [], []
    for qtype, tname, fn, sb in ((gq.TYPE_Q4_K, "q4_k", L.gq_qmv_q4_k, 144), (gq.TYPE_Q5_K, "q5_k", L.gq_qmv_q5_k, 176),
                                 (gq.TYPE_Q6_K, "q6_k", L.gq_qmv_q6_k, 210)):
        raw = torch.from_numpy(synth.as_bytes(synth.weights(np.random.default_rng(n + qtype), qtype, n, k))
                               .reshape(-1)).cuda()
        pk = gq.kq_pack(qtype, raw, n, k)
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        work.append((fn, pk, y))
        launches.append(["qmv_%s %dx%d" % (tname, n, k), n * (k // 256) * sb, k * 4 + n * 4])
        del raw
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for fn, pk, y in work:
        for _ in range(3):
            if fn(P(pk), n, k, P(x), P(y), None) != 0:
                raise RuntimeError("launch failed")
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"kq_launches": launches, "reps": 3}), flush=True)
    log("pmc pass done: 3 x each K-quant matvec, 3 x copy of %d bytes" % COPY_BYTES)


# ----------------------------------------------------------------------------
# time against bytes: fixed cost and steady rate of each M = 1 kernel family
# ----------------------------------------------------------------------------

SWEEP_FILE = os.path.join(PROFILES, "matvec_fixed_cost_sweep.txt")
SWEEP_WARMUP = 8
SWEEP_GRAPH = 64
SWEEP_REPLAYS = 7

# (family, kernel-name key in the trace, shapes): every shape of a family
# runs the same kernel instantiation (the launch rules pick it by shape)
SWEEP_FAMILIES = [
    ("qmv_q4_0 fp32 x, k 2048 (the 2048x2048 kernel)", "qmv_kernel<2, 0, 1, 1, 1, false>",
     [1024, 2048, 4096, 8192, 12288]),
    ("qffn_gate_up_gelu, k 2048 (2 x n_ff rows)", "qmv_kernel<2, 2, 1, 1, 2, false>",
     [2048, 4096, 8192, 16384, 32768]),
    ("qmv_q4_0 fp32 x, k 8192 (the down projection)", "qmv_kernel<2, 0, 1, 4, 4, false>",
     [512, 1024, 2048, 4096, 8192]),
    ("qmv_q8_0 fp32 x, k 2048, tall (the vocab head)", "qmv_kernel<8, 0, 2, 1, 4, false>",
     [32768, 65536, 131072, 262144]),
    ("read stream (16-byte loads, 8 KiB per wave, 256 workgroups)", "wave_chunk_kernel",
     [8 << 20, 32 << 20, 128 << 20, 512 << 20]),
]


def sweep_mode(args, log):
    """Each M = 1 kernel family of the step at several sizes (one kernel
    instantiation per family), plus the plain read-stream kernel: per size,
    rotated copies of random weights covering >= 1 GiB (the 256 MB last-level
    cache never holds a launch's weights), SWEEP_WARMUP warm-up launches, then
    64 launches over distinct copies recorded as one chain and replayed
    1 + SWEEP_REPLAYS times, the last SWEEP_REPLAYS between events: the
    device's back-to-back time per launch, free of the host's per-call cost
    (which, at about 4 us through Python, would otherwise bound the short
    kernels). Prints one JSON line: the launch manifest in order (so a
    rocprofv3 kernel trace of this run can be cut into shapes) and the
    per-launch times."""
    import ctypes
    import math

    import torch

    import gguf_block_quant_amd as gq

    L = gq.raw()
    stream = torch.cuda.Stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    bench_lib = ctypes.CDLL(os.path.join(ROOT, "gguf_block_quant_amd", "libgq_bench.so"))
    bench_lib.gqb_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)

    def scales(nblocks):
        return (torch.rand(nblocks, device="cuda", generator=gen) * 9e-3 + 1e-3).half().view(torch.int16)

    def quants(nbytes):
        return torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=gen)

    manifest, event_us = [], {}
    read_out = torch.empty(256 * 256, dtype=torch.int32, device="cuda")
    for fam, _key, sizes in SWEEP_FAMILIES:
        for n in sizes:
            if fam.startswith("read stream"):
                wbytes, obytes = n, 0
                make = lambda: (quants(n),)  # noqa: E731
                call = lambda c: bench_lib.gqb_read_stream(P(c[0]), n, P(read_out), 256, 1, sp)  # noqa: E731
            elif fam.startswith("qffn"):
                k = 2048
                wbytes, obytes = 2 * n * k // 32 * 18, k * 4 + n * 4
                x = torch.randn(k, device="cuda", generator=gen)
                h = torch.empty(n, device="cuda")
                make = lambda: (quants(n * k // 2), scales(n * k // 32), quants(n * k // 2), scales(n * k // 32))  # noqa: E731
                call = lambda c: L.gq_qffn_gate_up_gelu(P(c[0]), P(c[1]), P(c[2]), P(c[3]), n, 2048, P(x), P(h), sp)  # noqa: E731
            else:
                q8 = "q8_0" in fam
                k = 8192 if "k 8192" in fam else 2048
                wbytes, obytes = n * k // 32 * (34 if q8 else 18), k * 4 + n * 4
                x = torch.randn(k, device="cuda", generator=gen)
                y = torch.empty(n, device="cuda")
                fn = L.gq_qmv_q8_0 if q8 else L.gq_qmv_q4_0
                make = lambda: (quants(n * k if q8 else n * k // 2), scales(n * k // 32))  # noqa: E731
                call = lambda c: fn(P(c[0]), P(c[1]), n, k, P(x), P(y), sp)  # noqa: E731
            ncopies = max(2, math.ceil((1 << 30) / wbytes))
            copies = [make() for _ in range(ncopies)]
            torch.cuda.synchronize()
            for i in range(SWEEP_WARMUP):
                if call(copies[i % ncopies]) != 0:
                    raise RuntimeError("launch failed: %s %d" % (fam, n))
            torch.cuda.synchronize()
            chain = gq.Chain(stream)
            with chain:
                for i in range(SWEEP_GRAPH):
                    if call(copies[i % ncopies]) != 0:
                        raise RuntimeError("launch failed: %s %d" % (fam, n))
            chain.launch(stream)
            torch.cuda.synchronize()
            a, b = TimingEvent(), TimingEvent()
            a.record(stream)
            for _ in range(SWEEP_REPLAYS):
                chain.launch(stream)
            b.record(stream)
            torch.cuda.synchronize()
            chain.close()
            launches = SWEEP_WARMUP + SWEEP_GRAPH * (1 + SWEEP_REPLAYS)
            label = "%s | %d" % (fam, n)
            manifest.append([fam, n, wbytes, obytes, launches, SWEEP_WARMUP + SWEEP_GRAPH])
            event_us[label] = a.elapsed_time(b) * 1e3 / (SWEEP_REPLAYS * SWEEP_GRAPH)
            log("sweep %s: %.2f us per launch back to back (%d copies)" % (label, event_us[label], ncopies))
            del copies
            torch.cuda.empty_cache()
    print(json.dumps({"sweep_manifest": manifest, "event_us": event_us}), flush=True)


def _fit(points):
    """Least-squares fit t = a + bytes / rate over (bytes, t_us) points:
    (a in us, rate in TB/s)."""
    n = len(points)
    mx = sum(b for b, _ in points) / n
    my = sum(t for _, t in points) / n
    sxx = sum((b - mx) ** 2 for b, _ in points)
    sxy = sum((b - mx) * (t - my) for b, t in points)
    slope = sxy / sxx                      # us per byte
    return my - slope * mx, 1.0 / slope / 1e6


def sweep_summary(args):
    """Fixed cost and steady rate per kernel family, from a rocprofv3
    --kernel-trace run of ``--mode sweep`` (kernel durations, median of each
    shape's timed launches) and from the same run's back-to-back event times."""
    run_dir, _, plain_log = args.sweep_summary.partition(",")
    run_dir = run_dir.rstrip("/")

    def sweep_line(path):
        found = None
        for line in open(path):
            if line.startswith('{"sweep_manifest"'):
                found = json.loads(line)
        if found is None:
            raise SystemExit("no sweep_manifest line in %s" % path)
        return found

    run = sweep_line(run_dir + ".log")
    # the back-to-back times from the same command without the profiler
    # (under it, every dispatch waits for its trace record)
    plain = sweep_line(plain_log) if plain_log else None
    if plain is not None and [m[:5] for m in plain["sweep_manifest"]] != [m[:5] for m in run["sweep_manifest"]]:
        raise SystemExit("the plain run's manifest differs from the traced run's")
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit("no kernel_trace.csv under %s" % run_dir)
    keys = [key for _, key, _ in SWEEP_FAMILIES]
    rows = []
    for r in csv.DictReader(open(files[0])):
        if any(k in r["Kernel_Name"] for k in ("qmv_kernel", "wave_chunk_kernel")):
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                         (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    rows.sort()
    pos = 0
    durations = {}
    for fam, n, wb, ob, launches, skip in run["sweep_manifest"]:
        part = rows[pos:pos + launches]
        pos += launches
        key = keys[[f for f, _, _ in SWEEP_FAMILIES].index(fam)]
        if len(part) != launches or any(key not in name for _, name, _ in part):
            raise SystemExit("trace does not match the manifest at %s %d" % (fam, n))
        d = sorted(t for _, _, t in part[skip:])
        durations[(fam, n)] = d[len(d) // 2]
    if pos != len(rows):
        raise SystemExit("trace has %d matvec dispatches, the manifest %d" % (len(rows), pos))
    lines = [
        "# Time against bytes per M = 1 kernel family (bench.py --mode sweep), MI355X: fixed cost per launch",
        "# and steady rate from a least-squares fit t = fixed + bytes / rate over the sizes of one kernel",
        "# instantiation (random weights, >= 1 GiB of rotated copies per size)",
        "# command (repository root R on the GPU host):",
        "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d $R/%s -o run \\" % run_dir,
        "#       --output-format csv -- python3 $R/bench.py --mode sweep > $R/%s.log" % run_dir,
        "#   cd $R && python3 bench.py --mode sweep > %s" % (plain_log or "(not given)"),
        "#   python3 bench.py --sweep-summary %s%s --write-profile" % (run_dir, "," + plain_log if plain_log else ""),
        "# kernel_us: median kernel duration in the trace (dispatch start to end; the replayed launches);",
        "# launch_us: device time per launch, back to back, in 64-launch graph replays over distinct copies",
        "# (the gap between dependent dispatches included), from the run without the profiler%s"
        % ("" if plain else " -- NOT GIVEN: these are the profiled run's, inflated by the tracing"),
        "# bytes = weight blocks + x + y (the read stream: its buffer)",
        "# kernel_source_hash = %s" % kernel_source_hash(),
    ]
    for fam, key, sizes in SWEEP_FAMILIES:
        lines.append("")
        lines.append("%s   [%s]" % (fam, key))
        lines.append("%10s %14s %10s %10s %9s" % ("size", "bytes", "kernel_us", "launch_us", "GB/s"))
        kp, lp = [], []
        for fam2, n, wb, ob, _, _ in run["sweep_manifest"]:
            if fam2 != fam:
                continue
            kt = durations[(fam, n)]
            lt = (plain or run)["event_us"]["%s | %d" % (fam, n)]
            kp.append((wb + ob, kt))
            lp.append((wb + ob, lt))
            lines.append("%10d %14d %10.2f %10.2f %9.0f" % (n, wb + ob, kt, lt, (wb + ob) / kt / 1e3))
        ka, kr = _fit(kp)
        la, lr = _fit(lp)
        lines.append("fit kernel: fixed %.2f us, steady %.2f TB/s;  back to back: fixed %.2f us, steady %.2f TB/s"
                     % (ka, kr, la, lr))
    text = "\n".join(lines) + "\n"
    print(text)
    if args.write_profile:
        with open(SWEEP_FILE, "w") as f:
            f.write(text)


KQ_TRAFFIC_FILE = os.path.join(PROFILES, "qmv_kquant_262144x2048_hbm_traffic.txt")


def kq_traffic_summary(args):
    """HBM bytes of the K-quant matvecs against their algorithmic bytes, from
    a FETCH_SIZE and a WRITE_SIZE run of ``--mode pmc-kq``, each counter
    scaled by its reading for the device copy of known size in the same run."""
    fetch_dir, write_dir = args.kq_traffic_summary.split(",")
    run = None
    for line in open(fetch_dir.rstrip("/") + ".log"):
        if line.startswith('{"kq_launches"'):
            run = json.loads(line)
    if run is None:
        raise SystemExit("no kq_launches line in %s.log" % fetch_dir.rstrip("/"))
    launches, reps = run["kq_launches"], run["reps"]
    per, factors = {}, {}
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_dispatches(run_dir, counter)
        work = [r for r in rows if "qmv_q4_k_kernel" in r[1] or "qmv_q6_k_kernel" in r[1]]
        if len(work) != reps * len(launches):
            raise SystemExit("%s: %d K-quant dispatches, expected %d" % (run_dir, len(work), reps * len(launches)))
        copies = [r for r in rows if "copy" in r[1].lower()]
        big = max(r[2] for r in copies)
        cal = [r[3] for r in copies if r[2] == big][-3:]
        factors[counter] = COPY_BYTES / (1024.0 * (sum(cal) / len(cal)))
        for i, r in enumerate(work):
            per.setdefault(launches[i // reps][0], {}).setdefault(counter, []).append(
                r[3] * 1024.0 * factors[counter])
    lines = [
        "# HBM traffic of the K-quant matvecs (fp32 x, 262144 x 2048; bench.py --mode pmc-kq), MI355X",
        "# commands (repository root R on the GPU host; one counter per run):",
        "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE -d $R/%s -o run \\" % fetch_dir,
        "#       --output-format csv -- python3 $R/bench.py --mode pmc-kq > $R/%s.log" % fetch_dir.rstrip("/"),
        "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE -d $R/%s -o run \\" % write_dir,
        "#       --output-format csv -- python3 $R/bench.py --mode pmc-kq > $R/%s.log" % write_dir.rstrip("/"),
        "#   python3 bench.py --kq-traffic-summary %s,%s --write-profile" % (fetch_dir, write_dir),
        "# each counter scaled by its reading for a %d-byte device copy in the same run (factors: FETCH_SIZE "
        "%.4f, WRITE_SIZE %.4f); bytes per launch, mean of %d launches"
        % (COPY_BYTES, factors["FETCH_SIZE"], factors["WRITE_SIZE"], reps),
        "# algorithmic = super-block bytes + x read + y written",
        "# kernel_source_hash = %s" % kernel_source_hash(("gq_kquant.hip", "gq_device.hpp", "gq_launch.hpp")),
        "%-24s %13s %11s %13s %8s" % ("launch", "fetch_B", "write_B", "algorithmic_B", "ratio"),
    ]
    for name, w, o in launches:
        f = sum(per[name]["FETCH_SIZE"]) / reps
        wr = sum(per[name]["WRITE_SIZE"]) / reps
        lines.append("%-24s %13.0f %11.0f %13d %8.3f" % (name, f, wr, w + o, (f + wr) / (w + o)))
    text = "\n".join(lines) + "\n"
    print(text)
    if args.write_profile:
        with open(KQ_TRAFFIC_FILE, "w") as f:
            f.write(text)


STEP_TRAFFIC_FILE = os.path.join(PROFILES, "decode_step_hbm_traffic.txt")


def _counter_dispatches(run_dir, counter):
    """(dispatch id, kernel, grid, value) of one counter, in dispatch order."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % run_dir)
    rows = []
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == counter:
                    rows.append((int(row["Dispatch_Id"]), row["Kernel_Name"], int(row["Grid_Size"]),
                                 float(row["Counter_Value"])))
    return sorted(rows)


def step_traffic_summary(args):
    """HBM bytes of every kernel of the step against its algorithmic bytes,
    from a FETCH_SIZE and a WRITE_SIZE run of ``--mode pmc-step``: the step's
    kernels are its matvec and tile dispatches in launch order (3 steps);
    each counter is scaled by its reading for the device copy of known size
    at the end of the same run."""
    fetch_dir, write_dir = args.step_traffic_summary.split(",")
    run = None
    for line in open(fetch_dir.rstrip("/") + ".log"):
        if line.startswith('{"step_launches"'):
            run = json.loads(line)
    if run is None:
        raise SystemExit("no step_launches line in %s.log" % fetch_dir.rstrip("/"))
    launches, steps = run["step_launches"], run["steps"]
    per = {}
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_dispatches(run_dir, counter)
        work = [r for r in rows if "qmv_kernel" in r[1] or "tile_kernel" in r[1]]
        if len(work) != steps * len(launches):
            raise SystemExit("%s: %d matvec/tile dispatches, expected %d" % (run_dir, len(work),
                                                                             steps * len(launches)))
        copies = [r for r in rows if "copy" in r[1].lower()]
        big = max(r[2] for r in copies)
        cal = [r[3] for r in copies if r[2] == big][-3:]
        factor = COPY_BYTES / (1024.0 * (sum(cal) / len(cal)))
        for i, r in enumerate(work):
            per.setdefault(launches[i % len(launches)][0], {}).setdefault(counter, []).append(
                r[3] * 1024.0 * factor)
        per.setdefault("_factor", {})[counter] = factor
    lines = [
        "# HBM traffic per kernel of one decode step (bench.py --mode pmc-step: 3 steps), MI355X",
        "# commands (repository root R on the GPU host; one counter per run):",
        "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE -d $R/%s -o run \\" % fetch_dir,
        "#       --output-format csv -- python3 $R/bench.py --mode pmc-step > $R/%s.log" % fetch_dir.rstrip("/"),
        "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE -d $R/%s -o run \\" % write_dir,
        "#       --output-format csv -- python3 $R/bench.py --mode pmc-step > $R/%s.log" % write_dir.rstrip("/"),
        "#   python3 bench.py --step-traffic-summary %s,%s --write-profile" % (fetch_dir, write_dir),
        "# each counter scaled by its reading for a %d-byte device copy in the same run (factors: FETCH_SIZE "
        "%.4f, WRITE_SIZE %.4f); bytes per launch, mean of %d launches"
        % (COPY_BYTES, per["_factor"]["FETCH_SIZE"], per["_factor"]["WRITE_SIZE"], steps),
        "# algorithmic = weight blocks + activations read + outputs written, as the benchmark counts them",
        "# kernel_source_hash = %s" % kernel_source_hash(),
        "%-46s %13s %11s %13s %8s" % ("launch", "fetch_B", "write_B", "algorithmic_B", "ratio"),
    ]
    for name, w, o in launches:
        f = sum(per[name]["FETCH_SIZE"]) / steps
        wr = sum(per[name]["WRITE_SIZE"]) / steps
        lines.append("%-46s %13.0f %11.0f %13d %8.3f" % (name[:46], f, wr, w + o, (f + wr) / (w + o)))
    text = "\n".join(lines) + "\n"
    print(text)
    if args.write_profile:
        with open(STEP_TRAFFIC_FILE, "w") as f:
            f.write(text)


COUNTERS_FILE = os.path.join(PROFILES, "decode_step_valu_mfma_counters.txt")
CU_NUM, SIMD_NUM, XCD_NUM = 256, 1024, 8


def counters_summary(args):
    """VALU busy and MFMA utilisation per kernel of the step from two
    rocprofv3 --pmc runs of ``--mode pmc-step``: run A with
    SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_I8 GRBM_GUI_ACTIVE, run B
    with SQ_ACTIVE_INST_VALU SQ_INSTS_VALU GRBM_GUI_ACTIVE. VALU busy =
    SQ_ACTIVE_INST_VALU / CU count / GRBM_GUI_ACTIVE; MFMA utilisation =
    SQ_VALU_MFMA_BUSY_CYCLES / (SIMD count x GRBM_GUI_ACTIVE), where the
    csv's GRBM_GUI_ACTIVE is summed over the 8 XCDs and so divided by 8 to get
    the busy cycles of one (the profiler's own derived metrics take the max
    over XCDs)."""
    dir_a, dir_b, *rest = args.counters_summary.split(",")
    out_file = os.path.join(PROFILES, rest[0]) if rest else COUNTERS_FILE
    mode = "pmc-kq" if rest and "kquant" in rest[0] else "pmc-step"

    def per_kernel(run_dir, names):
        out = {}
        for name in names:
            for kern, grid, val in _read_counter(run_dir, name):
                key = (kern, grid)
                out.setdefault(key, {}).setdefault(name, []).append(val)
        return out

    a = per_kernel(dir_a, ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_I8", "GRBM_GUI_ACTIVE"))
    b = per_kernel(dir_b, ("SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE"))
    avg = lambda v: sum(v) / len(v)  # noqa: E731
    lines = [
        "# VALU and MFMA counters per kernel (bench.py --mode %s), MI355X" % mode,
        "# commands (repository root R on the GPU host; one pass per run):",
        "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_I8 \\",
        "#       GRBM_GUI_ACTIVE -d $R/%s -o run --output-format csv -- python3 $R/bench.py --mode %s" % (dir_a, mode),
        "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc SQ_ACTIVE_INST_VALU SQ_INSTS_VALU GRBM_GUI_ACTIVE \\",
        "#       -d $R/%s -o run --output-format csv -- python3 $R/bench.py --mode %s" % (dir_b, mode),
        "#   python3 bench.py --counters-summary %s --write-profile" % args.counters_summary,
        "# valu_busy = SQ_ACTIVE_INST_VALU / %d CUs / G; mfma_util = SQ_VALU_MFMA_BUSY_CYCLES / (%d SIMDs x G);"
        % (CU_NUM, SIMD_NUM),
        "# G = GRBM_GUI_ACTIVE / %d (the csv sums it over the XCDs); mfma_i8_mops = SQ_INSTS_VALU_MFMA_MOPS_I8"
        % XCD_NUM,
        "# kernel_source_hash = %s" % kernel_source_hash(),
        "%-58s %6s %9s %9s %11s %12s" % ("kernel", "grid", "valu_busy", "mfma_util", "valu_insts", "mfma_i8_mops"),
    ]
    for key in sorted(set(a) | set(b), key=lambda kg: kg[0]):
        kern, grid = key
        label = next((lab for k, lab in KERNEL_LABELS if k in kern), kern[:58])
        va, vb = a.get(key, {}), b.get(key, {})
        busy = util = insts = mops = float("nan")
        if "SQ_ACTIVE_INST_VALU" in vb:
            busy = 100.0 * avg(vb["SQ_ACTIVE_INST_VALU"]) / CU_NUM / (avg(vb["GRBM_GUI_ACTIVE"]) / XCD_NUM)
            insts = avg(vb["SQ_INSTS_VALU"])
        if "SQ_VALU_MFMA_BUSY_CYCLES" in va:
            util = 100.0 * avg(va["SQ_VALU_MFMA_BUSY_CYCLES"]) / (SIMD_NUM * avg(va["GRBM_GUI_ACTIVE"]) / XCD_NUM)
            mops = avg(va["SQ_INSTS_VALU_MFMA_MOPS_I8"])
        lines.append("%-58s %6d %8.1f%% %8.2f%% %11.0f %12.0f" % (label, grid, busy, util, insts, mops))
    text = "\n".join(lines) + "\n"
    print(text)
    if args.write_profile:
        with open(out_file, "w") as f:
            f.write(text)


def _read_counter(run_dir, counter):
    """Per-dispatch values of one counter from a rocprofv3 counter_collection.csv."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % run_dir)
    rows = []
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == counter:
                    rows.append((row["Kernel_Name"], int(row["Grid_Size"]), float(row["Counter_Value"])))
    return rows


def pmc_summary(args):
    """Turn the FETCH_SIZE and WRITE_SIZE runs of ``--mode pmc`` into HBM bytes
    per launch of the dominant kernel. Each counter (KiB per dispatch) is
    scaled by what it reads for the 512 MiB device copy of the same run (the
    largest copy dispatch), so the result is in bytes."""
    fetch_dir, write_dir = args.pmc_summary.split(",")
    out = {}
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _read_counter(run_dir, counter)
        copies = [r for r in rows if "copy" in r[0].lower()]
        big = max(r[1] for r in copies)
        cal = [r[2] for r in copies if r[1] == big]
        factor = COPY_BYTES / (1024.0 * (sum(cal) / len(cal)))
        kern = [r[2] for r in rows if "qmv_kernel<8, 0," in r[0]]
        out[counter] = (sum(kern) / len(kern), factor, len(kern), sum(cal) / len(cal))
    fetch = out["FETCH_SIZE"][0] * 1024.0 * out["FETCH_SIZE"][1]
    write = out["WRITE_SIZE"][0] * 1024.0 * out["WRITE_SIZE"][1]
    alg = 262144 * 64 * 34 + 2048 * 4 + 262144 * 4
    lines = [
        "# HBM traffic of the Q8_0 vocab matvec (262144 x 2048, fp32 x), MI355X",
        "# commands (repository root R on the GPU host; one counter per run):",
        "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE -d $R/%s -o run \\" % fetch_dir,
        "#       --output-format csv -- python3 $R/bench.py --mode pmc",
        "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE -d $R/%s -o run \\" % write_dir,
        "#       --output-format csv -- python3 $R/bench.py --mode pmc",
        "#   python3 bench.py --pmc-summary %s,%s --write-profile" % (fetch_dir, write_dir),
        "# calibration: the same counter on a %d-byte device copy in the same run" % COPY_BYTES,
        "fetch_kib_per_launch_raw = %.3f" % out["FETCH_SIZE"][0],
        "fetch_copy_kib_raw = %.3f" % out["FETCH_SIZE"][3],
        "fetch_calibration_factor = %.5f" % out["FETCH_SIZE"][1],
        "write_kib_per_launch_raw = %.3f" % out["WRITE_SIZE"][0],
        "write_copy_kib_raw = %.3f" % out["WRITE_SIZE"][3],
        "write_calibration_factor = %.5f" % out["WRITE_SIZE"][1],
        "launches = %d" % out["FETCH_SIZE"][2],
        "fetch_bytes_per_launch = %.0f" % fetch,
        "write_bytes_per_launch = %.0f" % write,
        "algorithmic_bytes_per_launch = %d" % alg,
        "traffic_over_algorithmic = %.4f" % ((fetch + write) / alg),
        "kernel_source_hash = %s" % kernel_source_hash(),
    ]
    text = "\n".join(lines) + "\n"
    print(text)
    if args.write_profile:
        with open(TRAFFIC_FILE, "w") as f:
            f.write(text)


STATS_FILE = os.path.join(PROFILES, "decode_step_kernel_stats.txt")

# what each kernel instantiation is in the default run
KERNEL_LABELS = [
    ("qmv_q4_k_kernel<1, 4, false>", "qmv Q4_K fp32 x: k 2048 (8192, 262144 rows)"),
    ("qmv_q4_k_kernel<1, 2, false>", "qmv Q4_K fp32 x, 2 rows per step: 2048x2048"),
    ("qmv_q4_k_kernel<1, 4, true>", "qmv Q5_K fp32 x: k 2048 (8192, 262144 rows)"),
    ("qmv_q4_k_kernel<1, 2, true>", "qmv Q5_K fp32 x, 2 rows per step: 2048x2048"),
    ("qmv_q6_k_kernel<1, 4>", "qmv Q6_K fp32 x: k 2048 (8192, 262144 rows)"),
    ("qmv_q6_k_kernel<1, 2>", "qmv Q6_K fp32 x, 2 rows per step: 2048x2048"),
    ("kq_pack_kernel<12>", "pack Q4_K"),
    ("kq_pack_kernel<13>", "pack Q5_K"),
    ("kq_pack_kernel<14>", "pack Q6_K"),
    ("qmv_kernel<8, 0, 2, 1, 4, false>", "qmv Q8_0 fp32 x, tall: vocab 262144 (+1/8) x2048"),
    ("qmv_kernel<8, 0, 2, 1, 4, true>", "qmv Q8_0 + rmsnorm + softcap + argmax stage 1: vocab"),
    ("argmax_reduce_kernel", "argmax stage 2 (one workgroup)"),
    ("qmv_kernel<2, 2, 1, 1, 2, false>", "FFN gate+up GELU Q4_0: 2 x 8192 (+1/8) x2048"),
    ("qmv_kernel<2, 2, 1, 1, 2, true>", "FFN gate+up GELU + rmsnorm"),
    ("qmv_kernel<2, 0, 1, 4, 4, false>", "qmv Q4_0 fp32 x: down 2048x8192"),
    ("qmv_kernel<2, 0, 1, 1, 1, false>", "qmv Q4_0 fp32 x: 2048x2048 (+ down's 2048x1024 shard)"),
    ("qmv_kernel<2, 0, 1, 1, 1, true>", "qmv Q4_0 + rmsnorm + residual: 2048x2048"),
    ("qmv_kernel<2, 1, 1, 1, 1, false>", "qmv Q4_0 Q8_0 x: 2048x2048 (pre-quantised, extra)"),
    ("qmv_kernel<2, 1, 1, 1, 1, true>", "qmv Q4_0 Q8_0 x quantised in the prologue: 2048x2048"),
    ("qmv_kernel<8, 0, 1, 1, 1, false>", "qmv Q8_0 fp32 x: 64x256 (latency point)"),
    ("tile_kernel<1, true>", "tile M <= 8, paired blocks: 8192x2048 at M = 8 (and 4)"),
    ("tile_kernel<1, false>", "tile M <= 16: 8192x2048 at M = 16"),
    ("tile_kernel<2, false>", "tile M <= 32: 8192x2048 at M = 32"),
    ("quantize_q8_0_kernel", "quantize_q8_0 1x2048 (standalone, extra)"),
    ("pack_kernel<8>", "pack Q8_0 (vocab + small)"),
    ("pack_kernel<2>", "pack Q4_0 (all Q4_0 weights)"),
    ("lane_stride_kernel", "read-stream ceiling, lane grid-stride (bench helper)"),
    ("wave_chunk_kernel", "read-stream ceiling, wave chunks (bench helper)"),
    ("copyBuffer", "runtime copy"),
]


def _bench_line(path):
    """The JSON result line of a bench.py run's output file, or None."""
    if not path or not os.path.exists(path):
        return None
    found = None
    for line in open(path):
        if line.startswith("{"):
            found = json.loads(line)
    return found


def _timed_trace_average(run_dir, run):
    """Average duration (us) of the dominant kernel's dispatches inside the
    timed region, from the kernel trace: its launches in dispatch order are W
    warm-up steps, then the K timed steps."""
    if run is None:
        return None
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        return None
    durs = []
    for r in csv.DictReader(open(files[0])):
        if "qmv_kernel<8, 0, 2, 1, 4, false>" in r["Kernel_Name"]:
            durs.append((int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    durs.sort()
    w, k = run["warmup"], run["steps"]
    sel = [d for _, d in durs[w:w + k]]
    if len(sel) != k:
        return None
    every = run["roofline"].get("event_every", 1)
    bracketed = sel[::every]
    return sum(sel) / len(sel) / 1e3, sum(bracketed) / len(bracketed) / 1e3, every


def stats_summary(args):
    """Kernel table of a rocprofv3 --kernel-trace --stats run of the default
    benchmark, with the dominant kernel's rocprof average beside the live
    HIP-event average of the same run."""
    run_dir, _, bench_json = args.stats_summary.partition(",")
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit("no kernel_stats.csv under %s" % run_dir)
    rows = list(csv.DictReader(open(files[0])))
    lines = [
        "# rocprofv3 kernel statistics: the decode-step benchmark (bench.py, default arguments), MI355X (gfx950)",
        "# command (repository root R on the GPU host):",
        "#   cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d $R/%s -o run \\" % run_dir,
        "#       --output-format csv -- python3 $R/bench.py > $R/%s.log" % run_dir.rstrip("/"),
        "#   python3 bench.py --stats-summary %s --write-profile"
        % (run_dir + ("," + bench_json if bench_json else "")),
    ]
    if bench_json:
        lines.append("# (%s: the output of `python3 bench.py > %s`, the same command without the profiler)"
                     % (bench_json, bench_json))
    lines += [
        "# durations in microseconds; kernel_source_hash = %s" % kernel_source_hash(),
        "# calls cover the whole run: warm-up, the timed steps, the breakdown, the extras and the",
        "# per-config pass (eager and graph launches, MALL-hot), so an average mixes those contexts",
        "%-58s %6s %9s %9s %9s" % ("kernel", "calls", "avg_us", "min_us", "max_us"),
    ]
    dom = None
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        label = next((lab for key, lab in KERNEL_LABELS if key in r["Name"]), r["Name"][:58])
        lines.append("%-58s %6s %9.2f %9.2f %9.2f" % (label, r["Calls"], float(r["AverageNs"]) / 1e3,
                                                     float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
        if "qmv_kernel<8, 0, 2, 1, 4, false>" in r["Name"]:
            dom = float(r["AverageNs"]) / 1e3
    log_file = run_dir.rstrip("/") + ".log"
    run = _bench_line(log_file)
    trace = _timed_trace_average(run_dir, run)
    timed, timed_ev = (trace[0], trace[1]) if trace else (None, None)
    if dom is not None:
        alg = 262144 * 64 * 34 + 2048 * 4 + 262144 * 4
        lines.append("")
        # (the table's row for this kernel also counts the per-config pass's
        # launches at other shapes; the timed region holds only the vocab head)
        if timed is not None:
            lines.append("# dominant kernel (vocab), rocprof average over the timed region's launches (the kernel's "
                         "dispatches W+1..W+K in the trace): %d B / %.2f us = %.2f TB/s = %.1f%% of 8 TB/s"
                         % (alg, timed, alg / timed / 1e6, alg / timed / 1e6 / 8.0 * 100))
            if trace[2] > 1:
                lines.append("# over the event-bracketed ones only (one in %d of them, the launches the HIP events "
                             "time): %.2f us" % (trace[2], timed_ev))
        else:
            lines.append("# dominant kernel (vocab), rocprof average over all of the kernel's launches (no trace): "
                         "%d B / %.2f us = %.2f TB/s = %.1f%% of 8 TB/s"
                         % (alg, dom, alg / dom / 1e6, alg / dom / 1e6 / 8.0 * 100))
        if run is not None:
            ev = run["roofline"]["avg_launch_us"]
            lines.append("# the profiled run's live HIP-event average over the same launches: %.2f us (the events "
                         "bracket each launch, and under the profiler each dispatch waits for its trace record; "
                         "difference %.1f%%)" % (ev, (ev / (timed_ev or dom) - 1) * 100))
        plain = _bench_line(bench_json) if bench_json else None
        if plain is not None:
            ev = plain["roofline"]["avg_launch_us"]
            lines.append("# the same command without the profiler (%s): HIP-event average %.2f us, "
                         "roofline frac %.3f (difference %.1f%%)"
                         % (os.path.basename(bench_json), ev, plain["roofline"]["frac"],
                            (ev / (timed_ev or dom) - 1) * 100))
    text = "\n".join(lines) + "\n"
    print(text)
    if args.write_profile:
        with open(STATS_FILE, "w") as f:
            f.write(text)


# ----------------------------------------------------------------------------
# main
# ----------------------------------------------------------------------------

def load_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None if it is missing or was taken from other kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=2, help="rotated copies of the step's weights")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true", help="skip the per-workload throughput pass")
    ap.add_argument("--mode", choices=["bench", "pmc", "pmc-step", "pmc-kq", "sweep"], default="bench")
    ap.add_argument("--kq-traffic-summary", metavar="FETCH_DIR,WRITE_DIR",
                    help="FETCH_SIZE and WRITE_SIZE runs of --mode pmc-kq -> HBM bytes of the K-quant matvecs")
    ap.add_argument("--pmc-summary", default=None)
    ap.add_argument("--counters-summary", default=None,
                    help="A_DIR,B_DIR[,FILE] of the two --mode pmc-step (or, with FILE naming 'kquant', pmc-kq) "
                         "counter runs -> VALU / MFMA table (written to profiles/FILE)")
    ap.add_argument("--step-traffic-summary", metavar="FETCH_DIR,WRITE_DIR",
                    help="FETCH_SIZE and WRITE_SIZE runs of --mode pmc-step -> HBM bytes per kernel of the step")
    ap.add_argument("--stats-summary", default=None,
                    help="DIR[,BENCH_JSON]: rocprofv3 --kernel-trace --stats output dir of the default run "
                         "(its stdout in DIR.log) and optionally the JSON output of the same command run "
                         "without the profiler -> kernel table")
    ap.add_argument("--sweep-summary", default=None,
                    help="DIR[,PLAIN_LOG]: rocprofv3 --kernel-trace output dir of --mode sweep (its stdout in "
                         "DIR.log) and the stdout of the same command without the profiler -> fixed cost and "
                         "steady rate per kernel family")
    ap.add_argument("--write-profile", action="store_true",
                    help="with --pmc-summary: write the summary under profiles/")
    args = ap.parse_args()

    def log(msg):
        print("[bench] " + msg, file=sys.stderr, flush=True)

    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.stats_summary:
        stats_summary(args)
        return
    if args.counters_summary:
        counters_summary(args)
        return
    if args.step_traffic_summary:
        step_traffic_summary(args)
        return
    if args.kq_traffic_summary:
        kq_traffic_summary(args)
        return
    if args.sweep_summary:
        sweep_summary(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X and has no multi-GPU "
              "mode (asked for --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.mode == "pmc":
        pmc_mode(args, log)
        return
    if args.mode == "pmc-step":
        pmc_step_mode(args, log)
        return
    if args.mode == "pmc-kq":
        pmc_kq_mode(args, log)
        return
    if args.mode == "sweep":
        sweep_mode(args, log)
        return

    step = Step(args.sets, log)
    for i in range(args.warmup):
        step.run(i)
        step.run(i, tiles=True)
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides; an event
    # pair brackets the dominant launch of every EVENT_EVERY-th step (each
    # pair costs the step about 1.7 us of device time, so bracketing every
    # launch would add that much instrumentation to every step)
    ev = {DOMINANT: []}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step.run(i, ev if i % EVENT_EVERY == 0 else None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    value = step.step_weight_bytes * args.steps / elapsed / 1e9

    # the prefill tiles, timed the same way in a loop of their own
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step.run(i, tiles=True)
    torch.cuda.synchronize()
    tiles_s = (time.perf_counter() - t0) / args.steps
    prefill_tiles = {
        "value": round(step.tile_weight_bytes / tiles_s / 1e9, 2), "unit": "GB/s",
        "ms_per_pass": round(tiles_s * 1e3, 4), "passes_timed": args.steps,
        "weight_bytes_per_pass": step.tile_weight_bytes,
        "launches": step.tile_names,
        "hbm_frac": round(step.tile_weight_bytes / tiles_s / 1e9 / HBM_PEAK_GBPS, 4),
    }

    dom_ms = [a.elapsed_time(b) for a, b in ev[DOMINANT]]
    dom_avg_s = sum(dom_ms) / len(dom_ms) / 1e3
    dom_bytes = step.weight_bytes[DOMINANT] + step.other_bytes[DOMINANT]
    achieved = dom_bytes / dom_avg_s / 1e9

    # per-kernel breakdown (separate, untimed pass with events around every launch)
    bev = {n: [] for n in step.names + step.tile_names}
    nb = min(20, max(4, args.steps // 10))
    for i in range(nb):
        step.run(i, bev)
        step.run(i, bev, tiles=True)
    torch.cuda.synchronize()
    breakdown = {}
    for n in step.names + step.tile_names:
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in bev[n])
        med = us[len(us) // 2]
        wb = step.weight_bytes[n]
        breakdown[n] = {"median_us": round(med, 2), "weight_bytes": wb,
                        "weight_GBps": round(wb / med / 1e3, 1) if wb else None,
                        "total_GBps": round((wb + step.other_bytes[n]) / med / 1e3, 1)}

    # entry points beyond the step, each on its own (set-0 weights, MALL-cold
    # only to the extent the step's rotation left them)
    extras = {}
    for name, fn, fargs, wb, ob in step.extras:
        evs = []
        for _ in range(nb):
            a = TimingEvent()
            b = TimingEvent()
            a.record(step.stream)
            if fn(*fargs) != 0:
                raise RuntimeError("launch failed: " + name)
            b.record(step.stream)
            evs.append((a, b))
            step.run(0)        # stream other weights between repeats
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        med = us[len(us) // 2]
        extras[name] = {"median_us": round(med, 2), "weight_bytes": wb,
                        "weight_GBps": round(wb / med / 1e3, 1), "total_GBps": round((wb + ob) / med / 1e3, 1)}

    # the step recorded as chains and replayed: CHAIN_STEPS consecutive
    # steps per chain (one graph launch per CHAIN_STEPS steps), and one step
    # per chain (one graph launch per step)
    def time_chains(steps_per_chain):
        step.record_chains(steps_per_chain)
        replays = max(1, args.steps // steps_per_chain)
        for i in range(max(1, args.warmup // steps_per_chain)):
            step.replay(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(replays):
            step.replay(i)
        torch.cuda.synchronize()
        per_step = (time.perf_counter() - t0) / (replays * steps_per_chain)
        out = {"ms_per_step": round(per_step * 1e3, 4),
               "value": round(step.step_weight_bytes / per_step / 1e9, 2), "unit": "GB/s",
               "steps_per_replay": steps_per_chain, "launches_per_replay": step.chains[0].launches,
               "replays_timed": replays}
        step.close_chains()
        return out

    chained = time_chains(CHAIN_STEPS)
    chained["one_step_per_replay"] = time_chains(1)

    ceiling = read_stream_ceiling(step, log)
    for n, b in breakdown.items():
        if b["weight_GBps"]:
            b["pct_of_read_ceiling"] = round(100.0 * b["total_GBps"] / ceiling["GBps"], 1)
    configs = None if args.no_per_config else per_config(step, ceiling["GBps"], log)

    traffic = load_traffic()
    cpu = cpu_threads = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(step.host, step.step_weight_bytes, args.cpu_seconds, log)
        cpu_threads = cpu_baseline_threads(step.host, step.step_weight_bytes, args.cpu_seconds / 2, log)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "M=1 decode step over distinct weights: q4_0 2048x2048 (fp32 x; and q8_0 x quantised in "
                        "the kernel), ffn q4_0 gate+up 8192x2048 + down 2048x8192, q8_0 vocab 262144x2048 "
                        "(the prefill tile q4_0 8192x2048 at M=8,16,32 is timed apart: prefill_tiles)",
            "weight_bytes_per_step": step.step_weight_bytes,
            "weight_sets_rotated": args.sets,
            "launches_per_step": len(step.names),
        },
        "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "tokens_per_s_equiv": round(1e3 / ms_per_step, 1),
        "roofline": {
            "kernel": DOMINANT,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dom_bytes,
            "avg_launch_us": round(dom_avg_s * 1e6, 2),
            "launches_timed": len(dom_ms),
            "event_every": EVENT_EVERY,
        },
        "prefill_tiles": prefill_tiles,
        "cpu_baseline": cpu,
        "cpu_baseline_threads": cpu_threads,
        "chained": chained,
        "read_stream_ceiling": ceiling,
        "tokens_per_s_projection": {
            "value": round(value / 0.783, 1),
            "note": "effective GB/s / 0.783 GB per token (the byte budget per decoded token quoted "
                    "for the int2/int4/int8 Gemma-4-E2B port); context only"},
        "breakdown": breakdown,
        "extras": extras,
        "per_config": configs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
