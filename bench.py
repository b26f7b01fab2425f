#!/usr/bin/env python3
"""Benchmark of the ternary W1.58A8 hot path on one MI355X.

A step is one pass of the per-token path over a whole synthetic weight set:
per-token int8 quantization of every projection's activations (one
bt_quant_act_many launch) and every ternary product with its
rescale (one grouped launch, bt_gemm_grouped).  Packing is the offline
conversion step and runs before timing.  Inputs are resident in HBM when the
timed region starts.

Default workload: the 2B-shaped decode set at M=1 (30 layers x 7 projections,
0.52 GB of packed weights, larger than the 256 MB Infinity Cache).  Prints
one JSON line (rank 0, one GPU).  Unless --no-extra is given the line also
carries the other configurations: the single small GEMV (latency), batched
decode at M = 8/16/32 over the same weights, the M=512 prefill layer, the
8B-shaped set at M = 1 and 64, one launch per product beside the grouped
launch, the step as one launch that quantizes its own activations
(fused_step, 2B and 8B sets at M=1), the measured streaming-read ceiling,
the layer-chained decode and the format comparison.
--wave-timestamps prints instead where a streaming launch's time goes.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "W1.58A8 GEMV HBM GB/s (% of peak) at M=1; GEMM TOPS at M=512"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 matrix peak

WORKLOADS = {
    "decode_2b_m1": lambda: wl.decode_2b(1),
    "decode_2b_m2": lambda: wl.decode_2b(2),
    "decode_2b_m3": lambda: wl.decode_2b(3),
    "decode_2b_m4": lambda: wl.decode_2b(4),
    "decode_2b_m8": lambda: wl.decode_2b(8),
    "decode_2b_m16": lambda: wl.decode_2b(16),
    "decode_2b_m32": lambda: wl.decode_2b(32),
    "prefill_2b_m512": lambda: wl.prefill_2b(512),
    "decode_8b_m1": lambda: wl.decode_8b(1),
    "decode_8b_m64": lambda: wl.decode_8b(64),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_threads():
    return int(os.environ.get("OMP_NUM_THREADS", 0) or os.cpu_count() or 1)


def kernel_sources_sha():
    """Hash of the kernel sources and of the build script (its compiler
    flags shape the kernels too)."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "gemm_i2_bit_amd", "csrc",
                                           "*"))) + [
            os.path.join(ROOT, "gemm_i2_bit_amd", "build.py")]:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


class PackedSet:
    """Every (layer, projection) weight tensor of a workload's weight seed,
    packed on the GPU once and shared by the workloads that read the same
    weights (the decode set at every M, the chained decode).  The trits are
    drawn on several host threads (each tensor has its own generator, so the
    values do not depend on the threads).  The trits of the first
    `keep_layers` layers stay on the host for the CPU baseline."""

    def __init__(self, work: wl.Workload, torch, bt, keep_layers=1):
        self.work = work
        dev = torch.device("cuda:0")
        keys = [(p.layer, p.proj) for p in work.problems()]
        self.packed, self.s_w, self.trits = {}, {}, {}
        t0 = time.time()
        done = 0
        with ThreadPoolExecutor(max(1, min(16, host_threads()))) as ex:
            for i in range(0, len(keys), 32):
                batch = keys[i:i + 32]
                for key, (t, s_w) in zip(batch, ex.map(
                        lambda kk: work.weights(*kk), batch)):
                    self.packed[key] = bt.bt_pack_i2s(
                        torch.from_numpy(t).to(dev))
                    self.s_w[key] = float(s_w)
                    if key[0] < keep_layers:
                        self.trits[key] = t
                    del t
                done += len(batch)
                log(f"[bench] {work.name}: packed {done}/{len(keys)} tensors "
                    f"({time.time() - t0:.1f} s)")
        torch.cuda.synchronize()


class WorkSet:
    """Activations, outputs, plans and step functions of one workload over a
    PackedSet of its weights."""

    def __init__(self, work: wl.Workload, ps: PackedSet, torch, bt,
                 mode="grouped"):
        self.work, self.torch, self.bt, self.mode = work, torch, bt, mode
        dev = torch.device("cuda:0")
        probs = work.problems()
        m = work.m
        self.m = m
        ks = sorted({p.k for p in probs})
        rows = {k: m * sum(1 for p in probs if p.k == k) for k in ks}
        self.x = {k: torch.empty((rows[k], k), dtype=torch.float32,
                                 device=dev) for k in ks}
        self.xq = {k: torch.empty((rows[k], k), dtype=torch.int8, device=dev)
                   for k in ks}
        self.sa = {k: torch.empty(rows[k], dtype=torch.float32, device=dev)
                   for k in ks}
        off = {k: 0 for k in ks}
        self.problems = []
        for p in probs:
            key = (p.layer, p.proj)
            o = off[p.k]
            self.x[p.k][o:o + m].copy_(torch.from_numpy(
                work.activations(p.layer, p.proj)))
            off[p.k] += m
            self.problems.append(dict(
                packed=ps.packed[key], s_w=ps.s_w[key], n=p.n, k=p.k,
                x_q=self.xq[p.k][o:o + m], s_a=self.sa[p.k][o:o + m],
                x=self.x[p.k][o:o + m],
                y=torch.empty((m, p.n), dtype=torch.float32, device=dev)))
        torch.cuda.synchronize()
        self.ks = ks
        if mode == "fused":
            self.plan = bt.bt_grouped_plan_f32(self.problems)
        else:
            self.plan = bt.bt_grouped_plan(self.problems)

    # algorithmic bytes and ops -------------------------------------------
    def product_bytes(self, mode=None):
        """Packed weights + int8 activations + scales + fp32 outputs (fused:
        packed weights + fp32 activations + fp32 outputs)."""
        m = self.m
        if (mode or self.mode) == "fused":
            return sum(self.bt.bt_packed_bytes(p["n"], p["k"]) + 4 * m * p["k"]
                       + 4 * m * p["n"] for p in self.problems)
        return sum(self.bt.bt_packed_bytes(p["n"], p["k"]) + m * p["k"] + 4 * m
                   + 4 * m * p["n"] for p in self.problems)

    def quant_bytes(self):
        if self.mode == "fused":
            return 0
        return sum(5 * self.m * p["k"] + 4 * self.m for p in self.problems)

    def weight_bytes(self):
        return sum(self.bt.bt_packed_bytes(p["n"], p["k"])
                   for p in self.problems)

    def ops(self):
        return sum(2 * self.m * p["n"] * p["k"] for p in self.problems)

    # the step ------------------------------------------------------------
    def quant(self):
        if self.mode == "fused":
            return  # the product launch quantizes
        self.bt.bt_quant_act_many([self.x[k] for k in self.ks],
                                  [self.xq[k] for k in self.ks],
                                  [self.sa[k] for k in self.ks])

    def product(self):
        self.bt.bt_gemm_grouped(self.plan)

    def product_per_launch(self):
        for p in self.problems:
            self.bt.bt_gemm(p["packed"], p["s_w"], p["n"], p["k"], p["x_q"],
                            p["s_a"], y=p["y"])


def capture(torch, fn):
    """fn's launches as one HIP graph (captured after a warm-up call on a
    side stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# Untimed run-in before each timed section.  Launches that follow an idle
# GPU (bench.py packs weights and times the CPU oracle between sections)
# run slower while the GPU's clocks come up: the M=1 product took 92-96 us
# 5-10 ms after three idle seconds, 88-89 us at 10-20 ms and 87 us from
# 20 ms on (per-launch events, 3000 back-to-back launches).  A serving loop
# runs in the settled state, so every section first runs its own kernels,
# untimed, for SETTLE_MS of wall time; then its W warmup and K timed steps.
SETTLE_MS = 100.0


def settle(torch, fn, ms=SETTLE_MS):
    """Call fn back to back, untimed, for about `ms` of wall time."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_graph(torch, g, reps):
    """Average ms per replay of graph g over `reps` back-to-back replays
    (HIP events on the current stream, after the run-in and two untimed
    replays)."""
    settle(torch, g.replay)
    g.replay()
    g.replay()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_timed(ws: WorkSet, steps: int, warmup: int, torch):
    """Time `steps` whole steps (quantize + product); then time the product
    kernel alone over `steps` back-to-back launches (HIP events on the
    stream the kernels run on), so that its average matches a kernel trace
    (no gap after the quantization kernels).  Two untimed launches go
    first, so that the stream is busy when the start event is reached and
    the host's time to submit the first timed launch is not counted.
    The run-in (settle) goes before the warmup steps."""

    def step():
        ws.quant()
        ws.product()
    settle(torch, step)
    for _ in range(warmup):
        ws.quant()
        ws.product()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ws.quant()
        ws.product()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    ws.product()
    ws.product()
    e0.record()
    for _ in range(steps):
        ws.product()
    e1.record()
    torch.cuda.synchronize()
    return wall, e0.elapsed_time(e1) / steps


def fused_entry(work: wl.Workload, ps: PackedSet, torch, bt, steps, warmup,
                two_launch_ms):
    """The same step as one launch that quantizes its own activations
    (bt_grouped_plan_f32): ms per step beside the two-launch step's, and the
    fused kernel's rate over its own algorithmic bytes (packed weights, fp32
    activations, fp32 outputs)."""
    fws = WorkSet(work, ps, torch, bt, "fused")
    wall, kern = run_timed(fws, steps, warmup, torch)
    ms = wall / steps * 1e3
    out = {"ms_per_step": round(ms, 4),
           "two_launch_ms_per_step": round(two_launch_ms, 4),
           "speedup_vs_two_launch": round(two_launch_ms / ms, 4),
           "kernel_ms": round(kern, 5),
           "kernel_gb_s": round(fws.product_bytes() / (kern * 1e-3) / 1e9, 1)}
    del fws
    torch.cuda.empty_cache()
    return out


def per_launch_ms(ws: WorkSet, torch, reps=10):
    """One bt_gemm launch per product (the non-grouped mode), all of a pass
    captured in one HIP graph: ms per pass of the products alone (the
    activations are quantized once beforehand)."""
    ws.quant()
    g = capture(torch, ws.product_per_launch)
    ms = time_graph(torch, g, reps)
    del g
    return ms


def roofline(nbytes, ops, kern_ms, bound, traffic=None):
    if bound == "mfma":
        achieved = ops / (kern_ms * 1e-3) / 1e12
        return dict(bound="mfma", achieved=round(achieved, 2),
                    peak=INT8_PEAK_TOPS, unit="TFLOP/s",
                    frac=round(achieved / INT8_PEAK_TOPS, 4), traffic=traffic)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    return dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                traffic=traffic)


def config_entry(ws: WorkSet, torch, steps, warmup, ceiling=None,
                 with_per_launch=True, cpu_seconds=0.0, ps=None):
    """Figures of one configuration: the step (quantize + grouped product),
    the grouped product kernel against its roofline, one launch per product,
    and the oracle on a sample of the same workload."""
    wall, kern = run_timed(ws, steps, warmup, torch)
    ms_step = wall / steps * 1e3
    prefill = ws.m >= 128
    nbytes = ws.product_bytes()
    # counted HBM bytes per launch where profiles/ holds them for this
    # workload and the current kernel sources
    traffic = load_profile(f"traffic_{ws.work.name}.json",
                           kernel_sources_sha(), "hbm_bytes_per_launch")
    roof = roofline(nbytes, ws.ops(), kern, "mfma" if prefill else "hbm",
                    traffic)
    if ceiling and not prefill:
        roof["frac_of_measured_ceiling"] = round(
            roof["achieved"] / ceiling, 4)
    if not prefill:
        # the same against a probe that writes the launch's share of output
        # bytes between its reads
        wbytes = sum(4 * ws.m * p["n"] for p in ws.problems)
        mixed, shape = mixed_ceiling(torch, ws.bt, wbytes / (nbytes - wbytes))
        roof["write_share"] = round(wbytes / nbytes, 4)
        roof["measured_mixed_ceiling_gb_s"] = mixed
        roof["mixed_ceiling_best"] = shape
        roof["frac_of_mixed_ceiling"] = round(roof["achieved"] / mixed, 4)
    e = {"workload": ws.work.name, "m": ws.m,
         "ms_per_step": round(ms_step, 4),
         "product_kernel_ms": round(kern, 5),
         "algorithmic_bytes": nbytes,
         "weight_gb_s": round(ws.weight_bytes() / (kern * 1e-3) / 1e9, 1),
         "tops": round(ws.ops() / (kern * 1e-3) / 1e12, 2),
         "tokens_per_s_equiv": round(ws.m / (ms_step * 1e-3), 1),
         "roofline": roof}
    if with_per_launch:
        pl = per_launch_ms(ws, torch)
        e["per_launch"] = {
            "launches": len(ws.problems), "ms_per_pass": round(pl, 5),
            "gb_s": round(nbytes / (pl * 1e-3) / 1e9, 1),
            "tops": round(ws.ops() / (pl * 1e-3) / 1e12, 2),
            "frac": round((ws.ops() / (pl * 1e-3) / 1e12 / INT8_PEAK_TOPS)
                          if prefill else
                          (nbytes / (pl * 1e-3) / 1e9 / HBM_PEAK_GBS), 4)}
    # matrix-core and vector-ALU busy fractions where profiles/ holds
    # counters for this workload and the current kernel sources
    for key in ("mfma_busy", "valu_busy"):
        v = load_profile(f"counters_{ws.work.name}.json",
                         kernel_sources_sha(), key)
        if v is not None:
            e[key] = v
    if cpu_seconds > 0 and ps is not None:
        e["cpu_baseline"] = cpu_baseline(ws.work, ps, cpu_seconds,
                                         host_threads())
    return e


class ChainSet:
    """One token through the layer-chained decode of a workload's weights
    (workloads.CHAIN_PHASES): per layer, four dependent phases, each one
    quantization launch of the phase's input and one grouped launch of the
    products that read it (fused: one grouped launch that quantizes its fp32
    input itself).  Nothing runs ahead of its input."""

    def __init__(self, work: wl.Workload, torch, bt, layers=None,
                 fused=False, ps: PackedSet | None = None, norm=False,
                 persistent=False):
        self.torch, self.bt = torch, bt
        self.fused = fused or persistent
        fused = self.fused
        self.norm = norm
        self.persistent = persistent
        dev = torch.device("cuda:0")
        self.layers = work.layers if layers is None else layers
        self.x0 = torch.from_numpy(wl.chain_input(work)).to(dev)
        self.phases = []  # (input [1, k], x_q, s_a, plan, names, layer)
        self.y = []       # per layer: projection -> output [1, n]
        self.bytes = 0
        x = self.x0
        for l in range(self.layers):
            ys, packed = {}, {}
            for proj in wl.PROJ_NAMES:
                if ps is not None:
                    packed[proj] = (ps.packed[(l, proj)], ps.s_w[(l, proj)])
                    n = work.shapes[proj][1]
                else:
                    t, s_w = work.weights(l, proj)
                    packed[proj] = (bt.bt_pack_i2s(torch.from_numpy(t).to(dev)),
                                    float(s_w))
                    n = t.shape[0]
                    del t
                ys[proj] = torch.empty((1, n), dtype=torch.float32,
                                       device=dev)
            for ph, (src, dsts) in enumerate(wl.CHAIN_PHASES):
                xin = x if src == "x" else ys[src]
                k = xin.shape[1]
                x_q = torch.empty((1, k), dtype=torch.int8, device=dev)
                s_a = torch.empty(1, dtype=torch.float32, device=dev)
                gain = (torch.from_numpy(wl.norm_gain(work, l, ph)).to(dev)
                        if norm else None)
                probs = [dict(packed=packed[d][0], s_w=packed[d][1],
                              n=ys[d].shape[1], k=k, x_q=x_q, s_a=s_a,
                              x=xin, g=gain, eps=wl.NORM_EPS, y=ys[d])
                         for d in dsts]
                if fused:
                    plan = (bt.bt_grouped_plan_norm(probs) if norm
                            else bt.bt_grouped_plan_f32(probs))
                else:
                    plan = bt.bt_grouped_plan(probs)
                self.phases.append((xin, x_q, s_a, plan, dsts, l, gain))
                self.bytes += 5 * k + 4 + sum(
                    bt.bt_packed_bytes(p["n"], k) + k + 4 + 4 * p["n"]
                    for p in probs)
            self.y.append(ys)
            x = ys[wl.CHAIN_OUT]
        self.out = x
        self.chain = (bt.bt_chain_plan([ph[3] for ph in self.phases])
                      if persistent else None)
        torch.cuda.synchronize()

    def launches(self):
        if self.persistent:
            return 2  # the sync-word reset and the persistent launch
        return (1 if self.fused else 2) * len(self.phases)

    def step(self):
        if self.persistent:
            self.bt.bt_gemm_chain(self.chain)
            return
        for xin, x_q, s_a, plan, _, _, gain in self.phases:
            if not self.fused:
                if self.norm:
                    self.bt.bt_rmsnorm_quant(xin, gain, wl.NORM_EPS, x_q, s_a)
                else:
                    self.bt.bt_quant_act(xin, x_q, s_a)
            self.bt.bt_gemm_grouped(plan)

    def capture(self):
        """The token as one HIP graph."""
        return capture(self.torch, self.step)


def run_chain(cs: ChainSet, tokens: int, warmup: int, torch):
    """Per-token wall time of the chained decode, eager and graph-replayed
    (ms), each after the run-in (settle) and `warmup` untimed tokens."""
    settle(torch, cs.step)
    for _ in range(warmup):
        cs.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(tokens):
        cs.step()
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / tokens * 1e3
    if cs.persistent:  # one cooperative launch per token: no graph
        return eager, eager
    g = cs.capture()
    settle(torch, g.replay)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(tokens):
        g.replay()
    torch.cuda.synchronize()
    graph = (time.perf_counter() - t0) / tokens * 1e3
    return eager, graph


def format_ablation(torch, bt, reps=30):
    """Single-token products over the same random trits with the 2-bit
    format and packed dot products (bt_gemv), with the 2-bit format and
    lookup tables (bt_gemv_lut), and with five trits per byte (bt_gemv_b3):
    microseconds per call, averaged over back-to-back calls replayed from a
    HIP graph (so that the host's call rate does not set the time), and the
    weights per second each reaches."""
    dev = torch.device("cuda:0")
    shapes = [(2560, 2560), (6912, 2560), (2560, 6912), (131072, 4096)]
    out = {}
    for n, k in shapes:
        t = torch.randint(-1, 2, (n, k), dtype=torch.int8, device=dev)
        p2 = bt.bt_pack_i2s(t)
        p3 = bt.bt_pack_b3(t)
        del t
        x_q = torch.randint(-127, 128, (k,), dtype=torch.int8, device=dev)
        s_a = torch.ones(1, device=dev)
        y = torch.empty((1, n), device=dev)
        res = {}
        for name, fn, packed in (("dot4_us", bt.bt_gemv, p2),
                                 ("lut_us", bt.bt_gemv_lut, p2),
                                 ("b3_us", bt.bt_gemv_b3, p3)):
            def calls(fn=fn, packed=packed):
                for _ in range(reps):
                    fn(packed, 0.02, n, k, x_q, s_a, y=y)
            g = capture(torch, calls)
            res[name] = round(time_graph(torch, g, 1) / reps * 1e3, 2)
            del g
        res["bytes_2bit"] = p2.numel()
        res["bytes_b3"] = p3.numel()
        for name in ("dot4", "lut", "b3"):
            res[f"{name}_gweights_s"] = round(n * k / res[f"{name}_us"] / 1e3,
                                              1)
        out[f"{n}x{k}"] = res
        del p2, p3
    return out


def single_gemv(torch, bt, reps=200):
    """The small single GEMV (M=1, K=256, N=512, seed 0): latency of one
    bt_gemv call and of bt_quant_act followed by bt_gemv, averaged over
    back-to-back calls replayed from a HIP graph, and the host-side time of
    an eager call pair (enqueue to completion)."""
    dev = torch.device("cuda:0")
    t, s_w, x = wl.single_gemv()
    packed = bt.bt_pack_i2s(torch.from_numpy(t).to(dev))
    xd = torch.from_numpy(x).to(dev)
    x_q, s_a = bt.bt_quant_act(xd)
    y = torch.empty((1, t.shape[0]), device=dev)

    def gemv():
        for _ in range(reps):
            bt.bt_gemv(packed, s_w, t.shape[0], t.shape[1], x_q, s_a, y=y)

    def both():
        for _ in range(reps):
            bt.bt_quant_act(xd, x_q, s_a)
            bt.bt_gemv(packed, s_w, t.shape[0], t.shape[1], x_q, s_a, y=y)

    g1 = capture(torch, gemv)
    g2 = capture(torch, both)
    gemv_us = time_graph(torch, g1, 1) / reps * 1e3
    both_us = time_graph(torch, g2, 1) / reps * 1e3
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(50):
        bt.bt_quant_act(xd, x_q, s_a)
        bt.bt_gemv(packed, s_w, t.shape[0], t.shape[1], x_q, s_a, y=y)
        torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) / 50 * 1e6
    return {"workload": "single_gemv_m1_k256_n512",
            "gemv_us_graph": round(gemv_us, 3),
            "quant_plus_gemv_us_graph": round(both_us, 3),
            "quant_plus_gemv_us_eager_sync": round(eager_us, 2),
            "algorithmic_bytes": 32768 + 256 + 4 + 2048,
            "note": "L2-resident: a latency, not a bandwidth figure"}


def read_ceiling(torch, bt, nbytes=1 << 30, reps=20):
    """The streaming-read ceiling: bt_read_probe over a buffer larger than
    the 256 MB Infinity Cache, back-to-back launches timed with HIP events;
    GB/s for 4 and 8 waves per compute unit with 1 to 4 groups of four
    loads in flight per wave; the ceiling is the best of them."""
    dev = torch.device("cuda:0")
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    out = {"bytes": nbytes, "sweep": {}}
    settle(torch, lambda: bt.bt_read_probe(buf, sink, 8, 2))
    for wpc in (4, 8):
        for groups in (1, 2, 3, 4):
            for _ in range(3):
                bt.bt_read_probe(buf, sink, wpc, groups)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                bt.bt_read_probe(buf, sink, wpc, groups)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            out["sweep"][f"{wpc}w_{groups}g"] = round(
                nbytes / (ms * 1e-3) / 1e9, 1)
    best = max(out["sweep"], key=out["sweep"].get)
    out["gb_s"] = out["sweep"][best]
    out["best"] = best
    del buf, sink
    return out


def mixed_ceiling(torch, bt, write_frac, nbytes=1 << 30, reps=20):
    """The rate of a stream that writes `write_frac` of its bytes:
    bt_mix_probe reading 1 GiB once and writing write_frac of that once
    (1 KiB pieces spread through the reads in bursts of 1, 8 or 32),
    back-to-back launches timed with HIP events; GB/s of bytes read plus
    written, the best (and its shape) over 4 and 8 waves per compute unit
    with 2 load groups in flight and the three burst sizes."""
    dev = torch.device("cuda:0")
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    out_bytes = int(nbytes * write_frac) // 1024 * 1024
    out = torch.empty(max(out_bytes, 1024), dtype=torch.uint8,
                      device=dev)[:out_bytes]
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    settle(torch, lambda: bt.bt_mix_probe(buf, out, sink, 8, 2, 8))
    best, shape = 0.0, None
    for wpc in (4, 8):
        for burst in (1, 8, 32):
            for _ in range(3):
                bt.bt_mix_probe(buf, out, sink, wpc, 2, burst)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                bt.bt_mix_probe(buf, out, sink, wpc, 2, burst)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            gbs = (nbytes + out_bytes) / (ms * 1e-3) / 1e9
            if gbs > best:
                best, shape = gbs, f"{wpc}w_2g_burst{burst}"
    del buf, out, sink
    return round(best, 1), shape


def cpu_baseline(work: wl.Workload, ps: PackedSet, seconds: float,
                 threads: int):
    """The oracle, as it stands, on a bounded sample of the same workload:
    whole layers (all projections) of the trits kept on the host, repeated
    until about `seconds` of timed work (at least one layer pass); packing,
    the offline step, is not timed."""
    import oracle
    layers = sorted({l for l, _ in ps.trits})
    items = {}
    for l in layers:
        items[l] = []
        for proj in work.projs:
            t = ps.trits[(l, proj)]
            packed, _ = oracle.pack_i2s(t)
            items[l].append((packed, ps.s_w[(l, proj)], t.shape[0],
                             t.shape[1], work.activations(l, proj)))
    timed, nbytes, macs, passes = 0.0, 0, 0, 0
    while timed < seconds or passes == 0:
        l = layers[passes % len(layers)]
        t0 = time.perf_counter()
        for packed, s_w, n, k, x in items[l]:
            q, s_a = oracle.quant_act(x)
            oracle.gemm(packed, s_w, n, k, q, s_a, nthreads=threads)
        timed += time.perf_counter() - t0
        m = work.m
        nbytes += sum(p.size + 5 * m * k + 8 * m + 4 * m * n
                      for p, _, n, k, _ in items[l])
        macs += sum(m * n * k for _, _, n, k, _ in items[l])
        passes += 1
    return dict(value=round(nbytes / timed / 1e9, 4), unit="GB/s",
                cores=threads, kind="oracle",
                gmac_s=round(macs / timed / 1e9, 3),
                sample=f"{passes} layer passes (layers {layers[0]}-"
                       f"{layers[-1]} of {work.layers}, all "
                       f"{len(work.projs)} projections, M={work.m}; quantize "
                       f"+ product; {timed:.1f} s timed)")


def _bin_rates(lo_ns, hi_ns, nbytes, end_ns, bin_ns=250.0):
    """Aggregate read rate (GB/s, i.e. bytes per ns) in bins of bin_ns, each
    wave's bytes spread evenly over its [lo, hi) interval."""
    nb = int(np.ceil(end_ns / bin_ns)) + 1
    rate = np.zeros(nb)
    for a, b, by in zip(lo_ns, hi_ns, nbytes):
        if b <= a:
            continue
        r = by / (b - a)
        i0, i1 = int(a // bin_ns), int(b // bin_ns)
        for i in range(i0, min(i1, nb - 1) + 1):
            ov = min(b, (i + 1) * bin_ns) - max(a, i * bin_ns)
            if ov > 0:
                rate[i] += r * ov / bin_ns
    return rate


def _phases(lo_ns, hi_ns, nbytes, end_ns, bin_ns=250.0):
    """Ramp / steady / drain of one launch from its per-wave streaming
    intervals: the steady rate is the median of the middle half of the
    window; ramp and drain losses are the time lost against that rate in the
    first and second half (so that window = bytes / steady + ramp + drain)."""
    rate = _bin_rates(lo_ns, hi_ns, nbytes, end_ns, bin_ns)
    n = len(rate)
    steady = float(np.median(rate[n // 4:3 * n // 4]))
    loss = np.clip(1.0 - rate / steady, 0.0, None) * bin_ns
    return {"steady_gb_s": steady,
            "bytes_over_steady_us": float(np.sum(nbytes)) / steady / 1e3,
            "ramp_loss_us": float(loss[:n // 2].sum()) / 1e3,
            "drain_loss_us": float(loss[n // 2:].sum()) / 1e3,
            "rate_gb_s_per_us": [int(rate[i:i + 4].mean())
                                 for i in range(0, n, 4)]}


def _hw_xcd(hw):
    return (hw[:, 1] & 0xF).astype(np.int64)


def calibrate_xcd_shares(ws: WorkSet, torch, bt, rounds=2, launches=4):
    """Per-XCD shares for a streaming plan on a full grid, measured on this
    GPU: the plan is launched through the timing build (libbt_timing.so,
    include/bt_timing.h), each XCD's mean wave loop time is read from the
    per-wave timestamps, and each XCD's share is scaled by the mean loop
    time over its own (two rounds), so that the XCDs end their reads
    together.  The plan is then rebuilt with those shares
    (bt_grouped_plan_xcd); the outputs do not change.  Returns the shares
    (permille per XCD), or None where this does not apply."""
    import ctypes
    path = os.path.join(os.path.dirname(bt.LIB_PATH), "libbt_timing.so")
    host = ws.plan.host
    hdr = host[16:16 + 8 * 12].view(np.int64)
    kind = int(host[12:16].view(np.int32)[0])
    W = int(hdr[11])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if ws.mode != "grouped" or kind != 0 or W != 8 * cus or \
            not os.path.exists(path):
        return None
    V = ctypes.c_void_p
    T = ctypes.CDLL(path)
    T.bt_gemm_grouped.argtypes = [V, V, V]
    T.bt_gemm_grouped.restype = ctypes.c_int32
    T.bt_wave_timestamps.argtypes = [V, V]
    T.bt_wave_timestamps.restype = ctypes.c_int32
    stream = torch.cuda.current_stream().cuda_stream
    nx = 8
    shares = np.array([1000 if x % 2 == 0 else 900 for x in range(nx)],
                      np.float64)
    plan = ws.plan
    for _ in range(rounds):
        loops = []
        settle(torch, ws.product, ms=20.0)
        for _ in range(launches):
            for _ in range(3):
                if T.bt_gemm_grouped(plan.dev.data_ptr(), plan.host.ctypes.data,
                                     stream) != 0:
                    raise RuntimeError("timing build launch failed")
            torch.cuda.synchronize()
            ts = np.zeros((4096, 8), np.uint64)
            hw = np.zeros((4096, 2), np.uint32)
            if T.bt_wave_timestamps(ts.ctypes.data, hw.ctypes.data) != 0:
                raise RuntimeError("bt_wave_timestamps failed")
            ts = ts[:W].astype(np.int64)
            xcd = _hw_xcd(hw[:W])
            loop = (ts[:, 3] - ts[:, 1]).astype(np.float64)
            if set(np.unique(xcd)) != set(range(nx)):
                return None
            loops.append([loop[xcd == x].mean() for x in range(nx)])
        lx = np.median(np.array(loops), axis=0)
        shares = np.clip(shares * lx.mean() / lx, 500, 2000)
        plan = bt.bt_grouped_plan(ws.problems, xcd_shares=np.rint(shares))
    ws.plan = plan
    return [int(v) for v in np.rint(shares)]


def wave_timeline(ws: WorkSet, torch, bt, launches=8):
    """Per-wave timestamps of the streaming product launch and of the read
    probe over the same bytes, from the timing build (libbt_timing.so,
    include/bt_timing.h): where a launch's time goes (start, ramp, steady
    streaming, drain), per launch and summarized as medians."""
    import ctypes
    V = ctypes.c_void_p
    T = ctypes.CDLL(os.path.join(os.path.dirname(bt.LIB_PATH),
                                 "libbt_timing.so"))
    T.bt_gemm_grouped.argtypes = [V, V, V]
    T.bt_gemm_grouped.restype = ctypes.c_int32
    T.bt_read_probe.argtypes = [V, ctypes.c_int64, V, ctypes.c_int64,
                                ctypes.c_int32, ctypes.c_int32, V]
    T.bt_read_probe.restype = ctypes.c_int32
    for f in (T.bt_wave_timestamps, T.bt_probe_timestamps):
        f.argtypes = [V, V]
        f.restype = ctypes.c_int32
    host = ws.plan.host
    hdr = host[16:16 + 8 * 12].view(np.int64)
    kind = int(host[12:16].view(np.int32)[0])
    if kind != 0:
        raise SystemExit("--wave-timestamps needs a streaming plan (m <= 4 "
                         "with packed dot products)")
    total, start_off, W = int(hdr[7]), int(hdr[10]), int(hdr[11])
    if W > 0:  # the plan's own ranges
        tab = host[start_off:start_off + W * 128].reshape(W, 128)
        lo_c, hi_c = tab.view(np.int64)[:, 3], tab.view(np.int64)[:, 4]
    else:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        W = min(4 * min(2 * cus, (total + 15) // 16), total)
        lo_c = np.arange(W) * total // W
        hi_c = (np.arange(W) + 1) * total // W
    wpw = (8 if ws.mode == "grouped" and W == 8 *
           torch.cuda.get_device_properties(0).multi_processor_count else 4)
    stream = torch.cuda.current_stream().cuda_stream
    nbytes = ws.product_bytes()

    def launch():
        rc = T.bt_gemm_grouped(ws.plan.dev.data_ptr(), host.ctypes.data,
                               stream)
        if rc != 0:
            raise RuntimeError(f"timing build: status {rc}")
    # the timing build computes what the product library does, bit for bit
    outs = [p["y"] for p in ws.problems]
    for y in outs:
        y.fill_(float("nan"))
    ws.product()
    torch.cuda.synchronize()
    ref = torch.cat([y.flatten() for y in outs]).clone()
    for y in outs:
        y.fill_(float("nan"))
    launch()
    torch.cuda.synchronize()
    same = bool(torch.equal(ref, torch.cat([y.flatten() for y in outs])))

    def events(fn, reps=20):
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3
    settle(torch, launch)
    ev = {"product_library_us": [], "timing_build_us": []}
    for _ in range(3):
        ev["product_library_us"].append(round(events(ws.product), 2))
        ev["timing_build_us"].append(round(events(launch), 2))

    def med(rows, key):
        return round(float(np.median([r[key] for r in rows])), 2)
    kern = []
    for _ in range(launches):
        launch()
        launch()
        launch()
        torch.cuda.synchronize()
        ts = np.zeros((4096, 8), np.uint64)
        hw = np.zeros((4096, 2), np.uint32)
        if T.bt_wave_timestamps(ts.ctypes.data, hw.ctypes.data) != 0:
            raise RuntimeError("bt_wave_timestamps failed")
        ts = ts[:W].astype(np.int64)
        hw = hw[:W]
        t = (ts[:, :7] - ts[:, 0].min()) * 10.0  # ns
        by = (hi_c - lo_c) * 1024.0
        ph = _phases(t[:, 1], t[:, 3], by, t[:, 6].max())
        loop = (t[:, 3] - t[:, 1]) / 1e3
        slot = np.arange(W) % wpw
        xcd = _hw_xcd(hw)
        kern.append({
            "window_us": t[:, 6].max() / 1e3,
            "last_wave_start_us": t[:, 0].max() / 1e3,
            "start_us": float(np.median(t[:, 1] - t[:, 0])) / 1e3,
            "first_data_us": float(np.median(t[:, 2] - t[:, 1])) / 1e3,
            "loop_end_p10_us": float(np.percentile(t[:, 3], 10)) / 1e3,
            "loop_end_p50_us": float(np.median(t[:, 3])) / 1e3,
            "loop_end_max_us": t[:, 3].max() / 1e3,
            "handoff_us": float(np.median(t[:, 4] - t[:, 3])) / 1e3,
            "barrier_wait_us": float(np.median(t[:, 5] - t[:, 4])) / 1e3,
            "steady_gb_s": ph["steady_gb_s"],
            "bytes_over_steady_us": ph["bytes_over_steady_us"],
            "ramp_loss_us": ph["ramp_loss_us"],
            "drain_loss_us": ph["drain_loss_us"],
            "loop_us_by_slot": [float(loop[slot == j].mean())
                                for j in range(wpw)],
            "loop_us_by_xcd": [float(loop[xcd == x].mean()) if (xcd == x).any()
                               else None for x in range(8)],
            "rate": ph["rate_gb_s_per_us"]})
    # the read probe over the same bytes, best of its configurations
    pbytes = nbytes // 1024 * 1024
    buf = torch.ones(pbytes, dtype=torch.uint8, device="cuda:0")
    sink = torch.empty(1 << 16, dtype=torch.int32, device="cuda:0")

    def probe(wpc, g):
        rc = T.bt_read_probe(buf.data_ptr(), pbytes, sink.data_ptr(),
                             sink.numel(), wpc, g, stream)
        if rc != 0:
            raise RuntimeError(f"read probe: status {rc}")
    settle(torch, lambda: probe(8, 2))
    sweep = {(wpc, g): events(lambda wpc=wpc, g=g: probe(wpc, g))
             for wpc in (4, 8) for g in (1, 2, 3, 4)}
    best = min(sweep, key=sweep.get)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    PW = cus * best[0]
    steps = pbytes // 1024
    plo = np.arange(PW) * steps // PW
    phi = (np.arange(PW) + 1) * steps // PW
    prob = []
    for _ in range(launches):
        for _ in range(3):
            probe(*best)
        torch.cuda.synchronize()
        ts = np.zeros((4096, 4), np.uint64)
        hw = np.zeros((4096, 2), np.uint32)
        if T.bt_probe_timestamps(ts.ctypes.data, hw.ctypes.data) != 0:
            raise RuntimeError("bt_probe_timestamps failed")
        ts = ts[:PW].astype(np.int64)
        t = (ts[:, :3] - ts[:, 0].min()) * 10.0
        ph = _phases(t[:, 0], t[:, 2], (phi - plo) * 1024.0, t[:, 2].max())
        prob.append({
            "window_us": t[:, 2].max() / 1e3,
            "first_data_us": float(np.median(t[:, 1] - t[:, 0])) / 1e3,
            "loop_end_p10_us": float(np.percentile(t[:, 2], 10)) / 1e3,
            "loop_end_p50_us": float(np.median(t[:, 2])) / 1e3,
            "loop_end_max_us": t[:, 2].max() / 1e3,
            "steady_gb_s": ph["steady_gb_s"],
            "bytes_over_steady_us": ph["bytes_over_steady_us"],
            "ramp_loss_us": ph["ramp_loss_us"],
            "drain_loss_us": ph["drain_loss_us"]})
    keys_k = [k for k in kern[0] if not isinstance(kern[0][k], list)]
    keys_p = list(prob[0])
    return {
        "metric": "wave_timeline", "workload": ws.work.name,
        "mode": ws.mode,
        "bytes_per_launch": nbytes, "waves": W, "waves_per_workgroup": wpw,
        "launches": launches, "outputs_identical": same,
        "events_us": ev,
        "probe_config": {"waves_per_cu": best[0], "groups": best[1],
                         "events_us": round(sweep[best], 2)},
        "kernel": {k: med(kern, k) for k in keys_k},
        "kernel_loop_us_by_slot": [round(float(np.median(
            [r["loop_us_by_slot"][j] for r in kern])), 2) for j in range(wpw)],
        "kernel_loop_us_by_xcd": [round(float(np.median(
            [r["loop_us_by_xcd"][x] for r in kern])), 2)
            if kern[0]["loop_us_by_xcd"][x] is not None else None
            for x in range(8)],
        "kernel_rate_gb_s_per_us_first_launch": kern[0]["rate"],
        "probe": {k: med(prob, k) for k in keys_p}}


def device_info(torch):
    """The GPU the line was measured on (the rooflines assume an MI355X:
    256 CUs at 2.4 GHz)."""
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", None),
            "compute_units": pr.multi_processor_count,
            "memory_gib": round(pr.total_memory / 2**30, 1)}


def load_profile(name: str, sha: str, key: str):
    """A figure from a counter summary in profiles/ (null once the kernel
    sources have changed since the counters were taken)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sources_sha") != sha:
        return None
    return rec.get(key)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_2b_m1",
                    choices=sorted(WORKLOADS))
    ap.add_argument("--mode", default="grouped", choices=["grouped", "fused"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the selected workload (no other configuration)")
    ap.add_argument("--no-chain", action="store_true",
                    help="skip the chained-decode and lookup-table figures")
    ap.add_argument("--no-8b", action="store_true",
                    help="skip the 8B-shaped set")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--wave-timestamps", action="store_true",
                    help="instead of the benchmark line, print where a "
                         "streaming launch's time goes (ramp, steady, drain) "
                         "from the timing build's per-wave timestamps")
    ap.add_argument("--calibrate-xcd", action="store_true",
                    help="time the M=1 streaming plans with per-XCD shares "
                         "measured on this GPU (bt_grouped_plan_xcd)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 256 MiB device copy, so that a "
                         "counter run can scale FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the ternary product is measured "
              "on a single MI355X (no sharding, no collectives); "
              "use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemm_i2_bit_amd as bt
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bt.lib()  # fails loudly if the HIP library is missing
    sha = kernel_sources_sha()
    extra = not args.no_extra
    cpu = not args.no_cpu_baseline

    if args.wave_timestamps:
        work = WORKLOADS[args.workload]()
        ps = PackedSet(work, torch, bt)
        ws = WorkSet(work, ps, torch, bt, args.mode)
        ws.quant()
        print(json.dumps(wave_timeline(ws, torch, bt)), flush=True)
        return
    ceiling = read_ceiling(torch, bt) if extra else None
    work = WORKLOADS[args.workload]()
    log(f"[bench] workload {work.name}: {len(work.problems())} products, "
        f"{work.weight_bytes() / 1e6:.1f} MB packed weights")
    ps = PackedSet(work, torch, bt, keep_layers=2 if work.layers > 1 else 1)
    ws = WorkSet(work, ps, torch, bt, args.mode)
    xcd_shares = (calibrate_xcd_shares(ws, torch, bt) if args.calibrate_xcd
                  else None)
    wall, kern_avg = run_timed(ws, args.steps, args.warmup, torch)
    ms_step = wall / args.steps * 1e3
    step_bytes = ws.product_bytes() + ws.quant_bytes()
    prefill = work.m >= 128
    if prefill:
        value = ws.ops() / (ms_step * 1e-3) / 1e12
        unit = "TOPS"
    else:
        value = step_bytes / (ms_step * 1e-3) / 1e9
        unit = "GB/s"
    prof = "prefill_2b_m512" if prefill else work.name
    roof = roofline(ws.product_bytes(), ws.ops(), kern_avg,
                    "mfma" if prefill else "hbm",
                    load_profile(f"traffic_{prof}.json", sha,
                                 "hbm_bytes_per_launch"))
    if not prefill:
        # the same kernel time over the packed weight bytes alone
        wgbs = ws.weight_bytes() / (kern_avg * 1e-3) / 1e9
        roof["weight_gb_s"] = round(wgbs, 1)
        roof["weight_frac"] = round(wgbs / HBM_PEAK_GBS, 4)
        if ceiling:
            roof["weight_frac_of_measured_ceiling"] = round(
                wgbs / ceiling["gb_s"], 4)
    if ceiling and not prefill:
        roof["measured_ceiling_gb_s"] = ceiling["gb_s"]
        roof["frac_of_measured_ceiling"] = round(
            roof["achieved"] / ceiling["gb_s"], 4)
        # the same probe over as many bytes as one product launch moves: a
        # launch of this size pays the same ramp and drain as the kernel
        same = read_ceiling(torch, bt, nbytes=ws.product_bytes() // 1024 * 1024)
        roof["measured_ceiling_same_bytes_gb_s"] = same["gb_s"]
        roof["frac_of_ceiling_same_bytes"] = round(
            roof["achieved"] / same["gb_s"], 4)
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": unit,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": work.name, "m": work.m,
                   "layers": work.layers, "projections": len(work.projs),
                   "weight_bytes": ws.weight_bytes(),
                   "launch": args.mode,
                   "settle_ms": SETTLE_MS,
                   "xcd_shares": xcd_shares,
                   "product_kernel_ms": round(kern_avg, 5),
                   "tokens_per_s_equiv": round(work.m / (ms_step * 1e-3), 1),
                   "tops": round(ws.ops() / (kern_avg * 1e-3) / 1e12, 3)},
        "roofline": roof,
        "device": device_info(torch),
    }
    if extra and args.mode == "grouped":
        pl = per_launch_ms(ws, torch)
        out["per_launch"] = {
            "launches": len(ws.problems), "ms_per_pass": round(pl, 5),
            "gb_s": round(ws.product_bytes() / (pl * 1e-3) / 1e9, 1),
            "frac": round(ws.product_bytes() / (pl * 1e-3) / 1e9
                          / HBM_PEAK_GBS, 4)}
        if work.m <= 4:
            out["fused_step"] = fused_entry(work, ps, torch, bt, args.steps,
                                            args.warmup, ms_step)
    if cpu:
        log("[bench] timing the CPU oracle on a sample")
        cb = cpu_baseline(work, ps, args.cpu_seconds, host_threads())
        one = cpu_baseline(work, ps, args.cpu_seconds, 1)
        cb["value_1_thread"] = one["value"]
        cb["gmac_s_1_thread"] = one["gmac_s"]
        cb["sample_1_thread"] = one["sample"]
        out["cpu_baseline"] = cb
    del ws
    torch.cuda.empty_cache()

    if extra and work.name == "decode_2b_m1":
        out["read_ceiling"] = ceiling
        out["single_gemv"] = single_gemv(torch, bt)
        cpu_s = 3.0 if cpu else 0.0
        batched = {}
        for m in (8, 16, 32):
            bws = WorkSet(wl.decode_2b(m), ps, torch, bt)
            batched[f"m{m}"] = config_entry(bws, torch, 20, 3, ceiling["gb_s"],
                                            cpu_seconds=cpu_s, ps=ps)
            del bws
            torch.cuda.empty_cache()
        out["batched_decode_2b"] = batched
        pw = wl.prefill_2b(512)
        pps = PackedSet(pw, torch, bt)
        pws = WorkSet(pw, pps, torch, bt)
        pe = config_entry(pws, torch, 20, 3, cpu_seconds=cpu_s, ps=pps)
        pe["frac_int8_peak"] = pe["roofline"]["frac"]
        pe["traffic"] = load_profile("traffic_prefill_2b_m512.json", sha,
                                     "hbm_bytes_per_launch")
        pe["roofline"]["traffic"] = pe["traffic"]
        pe["mfma_busy"] = load_profile("counters_prefill_2b_m512.json", sha,
                                       "mfma_busy")
        out["prefill_m512"] = pe
        del pws, pps
        torch.cuda.empty_cache()
        if not args.no_chain:
            chained = {"workload": "decode_2b chained, M=1 (one token, every "
                                   "dependency kept)"}
            for norm in (False, True):
                for mode in ("two_launch", "fused", "persistent"):
                    cs = ChainSet(work, torch, bt, fused=mode == "fused",
                                  ps=ps, norm=norm,
                                  persistent=mode == "persistent")
                    eager, graph = run_chain(cs, 20, 3, torch)
                    if cs.persistent and bt.bt_chain_status(cs.chain) != 0:
                        raise RuntimeError("chained launch gave up waiting")
                    key = ("norm_" if norm else "") + mode
                    chained[key] = {
                        "layers": cs.layers,
                        "launches_per_token": cs.launches(),
                        "ms_per_token_eager": round(eager, 4),
                        "ms_per_token_graph": round(graph, 4),
                        "tokens_per_s_graph": round(1e3 / graph, 1)}
                    del cs
                    torch.cuda.empty_cache()
            out["chained_decode"] = chained
            out["format_ablation"] = format_ablation(torch, bt)
        del ps
        torch.cuda.empty_cache()
        if not args.no_8b:
            w8 = wl.decode_8b(1)
            ps8 = PackedSet(w8, torch, bt)
            d8 = {}
            for m in (1, 64):
                ws8 = WorkSet(wl.decode_8b(m), ps8, torch, bt)
                sh8 = (calibrate_xcd_shares(ws8, torch, bt)
                       if args.calibrate_xcd else None)
                d8[f"m{m}"] = config_entry(ws8, torch, 20, 3, ceiling["gb_s"],
                                           cpu_seconds=cpu_s, ps=ps8)
                if sh8 is not None:
                    d8[f"m{m}"]["xcd_shares"] = sh8
                if m == 1:
                    d8["m1"]["fused_step"] = fused_entry(
                        wl.decode_8b(1), ps8, torch, bt, 20, 3,
                        d8["m1"]["ms_per_step"])
                del ws8
                torch.cuda.empty_cache()
            out["decode_8b"] = d8
            del ps8
            torch.cuda.empty_cache()

    if args.calibrate_copy:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["calibration_copy_bytes"] = n
        # a second reference for the read counter: the read probe reads the
        # same 256 MiB once
        sink = torch.empty(1 << 16, dtype=torch.int32, device="cuda:0")
        bt.bt_read_probe(src, sink, 8, 2)
        torch.cuda.synchronize()
        out["calibration_read_probe_bytes"] = n
        del src, dst, sink

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
