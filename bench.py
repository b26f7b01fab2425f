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
one JSON line (rank 0, one GPU).
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

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


class WorkSet:
    """Device buffers, plan and step function for one workload."""

    def __init__(self, work: wl.Workload, torch, bt, mode="grouped"):
        self.work = work
        self.torch = torch
        self.bt = bt
        self.mode = mode
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
        t0 = time.time()
        for i, p in enumerate(probs):
            t, s_w = work.weights(p.layer, p.proj)
            packed = bt.bt_pack_i2s(torch.from_numpy(t).to(dev))
            del t
            x = work.activations(p.layer, p.proj)
            o = off[p.k]
            self.x[p.k][o:o + m].copy_(torch.from_numpy(x))
            off[p.k] += m
            y = torch.empty((m, p.n), dtype=torch.float32, device=dev)
            self.problems.append(dict(packed=packed, s_w=float(s_w), n=p.n,
                                      k=p.k, x_q=self.xq[p.k][o:o + m],
                                      s_a=self.sa[p.k][o:o + m], y=y))
            if (i + 1) % 50 == 0:
                log(f"[bench] prepared {i + 1}/{len(probs)} tensors "
                    f"({time.time() - t0:.1f} s)")
        torch.cuda.synchronize()
        self.plan = bt.bt_grouped_plan(self.problems)
        if mode == "fused":
            # the same products, quantizing the fp32 rows in the launch
            fprobs = []
            off = {k: 0 for k in ks}
            for p in self.problems:
                o = off[p["k"]]
                off[p["k"]] += m
                fprobs.append(dict(packed=p["packed"], s_w=p["s_w"], n=p["n"],
                                   k=p["k"], x=self.x[p["k"]][o:o + m],
                                   y=p["y"]))
            self.fplan = bt.bt_grouped_plan_f32(fprobs)
        self.ks = ks

    # algorithmic bytes and ops -------------------------------------------
    def product_bytes(self):
        """Packed weights + int8 activations + scales + fp32 outputs (fused:
        packed weights + fp32 activations + fp32 outputs)."""
        m = self.m
        if self.mode == "fused":
            return sum(self.bt.bt_packed_bytes(p["n"], p["k"]) + 4 * m * p["k"]
                       + 4 * m * p["n"] for p in self.problems)
        return sum(self.bt.bt_packed_bytes(p["n"], p["k"]) + m * p["k"] + 4 * m
                   + 4 * m * p["n"] for p in self.problems)

    def quant_bytes(self):
        if self.mode == "fused":
            return 0
        m = self.m
        return sum(5 * m * p["k"] + 4 * m for p in self.problems)

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
        if self.mode == "fused":
            self.bt.bt_gemm_grouped(self.fplan)
        elif self.mode == "grouped":
            self.bt.bt_gemm_grouped(self.plan)
        else:
            for p in self.problems:
                self.bt.bt_gemm(p["packed"], p["s_w"], p["n"], p["k"],
                                p["x_q"], p["s_a"], y=p["y"])


class ChainSet:
    """One token through the layer-chained decode of a workload's weights
    (workloads.CHAIN_PHASES): per layer, four dependent phases, each one
    quantization launch of the phase's input and one grouped launch of the
    products that read it (fused: one grouped launch that quantizes its fp32
    input itself).  Nothing runs ahead of its input."""

    def __init__(self, work: wl.Workload, torch, bt, layers=None,
                 fused=False):
        self.torch, self.bt = torch, bt
        self.fused = fused
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
                t, s_w = work.weights(l, proj)
                packed[proj] = (bt.bt_pack_i2s(torch.from_numpy(t).to(dev)),
                                float(s_w))
                ys[proj] = torch.empty((1, t.shape[0]), dtype=torch.float32,
                                       device=dev)
                del t
            for src, dsts in wl.CHAIN_PHASES:
                xin = x if src == "x" else ys[src]
                k = xin.shape[1]
                x_q = torch.empty((1, k), dtype=torch.int8, device=dev)
                s_a = torch.empty(1, dtype=torch.float32, device=dev)
                probs = [dict(packed=packed[d][0], s_w=packed[d][1],
                              n=ys[d].shape[1], k=k, x_q=x_q, s_a=s_a,
                              x=xin, y=ys[d]) for d in dsts]
                plan = (bt.bt_grouped_plan_f32(probs) if fused
                        else bt.bt_grouped_plan(probs))
                self.phases.append((xin, x_q, s_a, plan, dsts, l))
                self.bytes += 5 * k + 4 + sum(
                    bt.bt_packed_bytes(p["n"], k) + k + 4 + 4 * p["n"]
                    for p in probs)
            self.y.append(ys)
            x = ys[wl.CHAIN_OUT]
        self.out = x
        torch.cuda.synchronize()

    def launches(self):
        return (1 if self.fused else 2) * len(self.phases)

    def step(self):
        for xin, x_q, s_a, plan, _, _ in self.phases:
            if not self.fused:
                self.bt.bt_quant_act(xin, x_q, s_a)
            self.bt.bt_gemm_grouped(plan)

    def capture(self):
        """The token as one HIP graph (captured after a warm-up pass on a
        side stream)."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        torch.cuda.synchronize()
        return g


def run_chain(cs: ChainSet, tokens: int, warmup: int, torch):
    """Per-token wall time of the chained decode, eager and graph-replayed
    (ms)."""
    for _ in range(warmup):
        cs.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(tokens):
        cs.step()
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / tokens * 1e3
    g = cs.capture()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(tokens):
        g.replay()
    torch.cuda.synchronize()
    graph = (time.perf_counter() - t0) / tokens * 1e3
    return eager, graph


def lut_ablation(torch, bt, reps=30):
    """Single-token products with dot products (bt_gemv) and with lookup
    tables (bt_gemv_lut) on random packed weights: microseconds per call,
    averaged over back-to-back calls replayed from a HIP graph (so that the
    host's call rate does not set the time)."""
    dev = torch.device("cuda:0")
    shapes = [(2560, 2560), (6912, 2560), (2560, 6912), (131072, 4096)]
    out = {}
    for n, k in shapes:
        valid = torch.tensor([b for b in range(256)
                              if all((b >> (2 * j)) & 3 != 3 for j in range(4))],
                             dtype=torch.uint8, device=dev)  # no code 3
        packed = valid[torch.randint(0, valid.numel(),
                                     (bt.bt_packed_bytes(n, k),), device=dev)]
        x_q = torch.randint(-127, 128, (k,), dtype=torch.int8, device=dev)
        s_a = torch.ones(1, device=dev)
        y = torch.empty((1, n), device=dev)
        res = {}
        for name, fn in (("dot4_us", bt.bt_gemv), ("lut_us", bt.bt_gemv_lut)):
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for _ in range(3):
                    fn(packed, 0.02, n, k, x_q, s_a, y=y)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(reps):
                    fn(packed, 0.02, n, k, x_q, s_a, y=y)
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            res[name] = round(e0.elapsed_time(e1) / reps * 1e3, 2)
            del g
        res["weight_bytes"] = packed.numel()
        out[f"{n}x{k}"] = res
        del packed
    return out


def run_timed(ws: WorkSet, steps: int, warmup: int, torch):
    """Time `steps` whole steps (quantize + product); then time the product
    kernel alone over `steps` back-to-back launches (HIP events on the
    stream the kernels run on), so that its average matches a kernel trace
    (no gap after the quantization kernels).  Two untimed launches go
    first, so that the stream is busy when the start event is reached and
    the host's time to submit the first timed launch is not counted."""
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


def cpu_baseline(work: wl.Workload, seconds: float):
    """The oracle, as it stands, on a bounded sample of the same workload:
    whole layers (all projections), repeated until about `seconds` of timed
    work (packing, the offline step, is not timed)."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", 0) or os.cpu_count() or 1)
    timed = 0.0
    nbytes = 0
    passes = 0
    layer = 0
    items_cache = {}
    while timed < seconds:
        if layer not in items_cache:
            items = []
            for proj in work.projs:
                t, s_w = work.weights(layer, proj)
                packed, _ = oracle.pack_i2s(t)
                x = work.activations(layer, proj)
                items.append((packed, s_w, t.shape[0], t.shape[1], x))
                del t
            if len(items_cache) < 8:
                items_cache[layer] = items
        else:
            items = items_cache[layer]
        t0 = time.perf_counter()
        for packed, s_w, n, k, x in items:
            q, s_a = oracle.quant_act(x)
            oracle.gemm(packed, s_w, n, k, q, s_a, nthreads=threads)
        timed += time.perf_counter() - t0
        m = work.m
        nbytes += sum(p.size + 5 * m * k + 8 * m + 4 * m * n
                      for p, _, n, k, _ in items)
        passes += 1
        layer = (layer + 1) % min(work.layers, 8)
    return dict(value=round(nbytes / timed / 1e9, 3), unit="GB/s",
                cores=threads, kind="oracle",
                sample=f"{passes} layer passes (layers 0-{min(work.layers, 8) - 1} "
                       f"of {work.layers}, all {len(work.projs)} projections, "
                       f"M={work.m}; quantize + product; {timed:.1f} s timed)")


def load_traffic(workload: str, sha: str, launch_bytes: int):
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sources_sha") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_2b_m1",
                    choices=sorted(WORKLOADS))
    ap.add_argument("--mode", default="grouped",
                    choices=["grouped", "per-launch", "fused"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the M=512 prefill, chained-decode and "
                         "lookup-table figures")
    ap.add_argument("--no-chain", action="store_true",
                    help="skip the chained-decode and lookup-table figures "
                         "(keeps the M=512 prefill figure)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
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

    work = WORKLOADS[args.workload]()
    log(f"[bench] workload {work.name}: {len(work.problems())} products, "
        f"{work.weight_bytes() / 1e6:.1f} MB packed weights")
    ws = WorkSet(work, torch, bt, args.mode)
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
    launch_bytes = ws.product_bytes()
    sha = kernel_sources_sha()
    if prefill:
        achieved = ws.ops() / (kern_avg * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2),
                    peak=INT8_PEAK_TOPS, unit="TFLOP/s",
                    frac=round(achieved / INT8_PEAK_TOPS, 4),
                    traffic=load_traffic(args.workload, sha, launch_bytes))
    else:
        achieved = launch_bytes / (kern_avg * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=load_traffic(args.workload, sha, launch_bytes))
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
                   "product_kernel_ms": round(kern_avg, 5),
                   "tokens_per_s_equiv": round(work.m / (ms_step * 1e-3), 1),
                   "tops": round(ws.ops() / (ms_step * 1e-3) / 1e12, 3)},
        "roofline": roof,
    }
    del ws
    torch.cuda.empty_cache()

    if not args.no_extra and not prefill:
        pw = wl.prefill_2b(512)
        pws = WorkSet(pw, torch, bt, "grouped")
        pwall, pk_avg = run_timed(pws, 20, 3, torch)
        tops_k = pws.ops() / (pk_avg * 1e-3) / 1e12
        out["prefill_m512"] = {
            "workload": pw.name, "ms_per_step": round(pwall / 20 * 1e3, 4),
            "product_kernel_ms": round(pk_avg, 5),
            "tops_step": round(pws.ops() / (pwall / 20) / 1e12, 2),
            "tops_kernel": round(tops_k, 2),
            "frac_int8_peak": round(tops_k / INT8_PEAK_TOPS, 4),
            "traffic": load_traffic(pw.name, sha, pws.product_bytes())}
        del pws
        torch.cuda.empty_cache()
        if work.name.startswith("decode_2b_m1") and not args.no_chain:
            chained = {"workload": "decode_2b chained, M=1 (one token, every "
                                   "dependency kept)"}
            for fused in (False, True):
                cs = ChainSet(work, torch, bt, fused=fused)
                eager, graph = run_chain(cs, 20, 3, torch)
                chained["fused" if fused else "two_launch"] = {
                    "layers": cs.layers, "launches_per_token": cs.launches(),
                    "ms_per_token_eager": round(eager, 4),
                    "ms_per_token_graph": round(graph, 4),
                    "tokens_per_s_graph": round(1e3 / graph, 1)}
                del cs
                torch.cuda.empty_cache()
            out["chained_decode"] = chained
            out["lut_ablation"] = lut_ablation(torch, bt)

    if args.calibrate_copy:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["calibration_copy_bytes"] = n
        del src, dst

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(work, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
