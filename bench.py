#!/usr/bin/env python3
"""MoE expert-FFN forward+backward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral]
                    [--extra-workloads deepseek_v3,token_drop] [--fp8] [--fused-wi] [--graph]

A step is one pass of the whole path over one batch of synthetic input:
router GEMM, top-k routing, permute, the up-projection grouped GEMMs,
SwiGLU, the down-projection grouped GEMM and the weighted combine, then the
hand-derived backward (combine backward, grouped GEMMs with the rhs
transposed, transposed grouped GEMMs for the expert weight gradients,
SwiGLU backward, permute backward, routing backward and the router GEMM
backward).  Inputs are resident in HBM before the timed region starts.

`value` is expert-FFN TFLOP/s of the headline workload (Mixtral-8x7B
shape by default): 18 * R * d_model * d_ff algorithmic flops per step
(R = kept routed rows; padding rows and the router GEMM excluded) divided
by the step time, which is taken over K steps with no other events in the
stream (with --graph, K replays of one step captured into a HIP graph).
A second pass of the same steps brackets every expert GEMM and
memory-bound call with events, each after a 1 GiB scratch write that
evicts the 256 MB memory-side cache, and classifies each kind of call by
its own roofline: MFMA-bound when flops / peak exceeds algorithmic bytes /
HBM bandwidth, else HBM-bound.  Extra workloads (the DeepSeek-V3 shape and
the token-dropping shape by default) are measured the same way and
reported under "workloads"; a workload with a capacity is also run in the
capacity-padded batched layout (every expert owns C rows) on the same
inputs, with the ratio of the two step times and, for context, the
forward's three GEMMs through the vendor batched GEMM (torch.bmm).
Prints ONE JSON line on stdout; everything else goes to stderr.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE FFN fwd+bwd grouped-GEMM TFLOP/s and % of bf16 MFMA peak, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
FLUSH_BYTES = 1 << 30          # scratch written before each bracketed call (> 256 MB MALL)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--kernel-steps", type=int, default=5,
                   help="steps of the second pass that times each call after a cache flush")
    p.add_argument("--workload", default="mixtral")
    p.add_argument("--extra-workloads", default="deepseek_v3,token_drop",
                   help="comma-separated workloads reported under 'workloads' ('' = none)")
    p.add_argument("--cpu-tokens", type=int, default=0,
                   help="tokens of the headline workload the CPU oracle runs on (0 = all)")
    p.add_argument("--fused-wi", action="store_true",
                   help="one [E, D, 2F] up-projection weight [wi_0 | wi_1]")
    p.add_argument("--fp8", action="store_true",
                   help="FP8 expert GEMMs (e4m3 forward, e5m2 backward, current scaling)")
    p.add_argument("--graph", action="store_true",
                   help="time the steps as replays of one step captured into a HIP graph")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-kernel-events", action="store_true",
                   help="skip the per-call pass (only the step timing runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain row copy of known size (for scaling HBM counters)")
    p.add_argument("--traffic-summary", nargs=5,
                   metavar=("WORKLOAD", "BENCH_FETCH", "BENCH_WRITE", "COPY_FETCH", "COPY_WRITE"),
                   help="turn four rocprofv3 --pmc counter_collection.csv files into "
                        "profiles/<workload>_traffic.json and exit")
    return p.parse_args()


class _Bracket:
    """Context manager: optional cache flush, then a start and an end event
    around the launches inside it."""

    __slots__ = ("rec", "kind", "flops", "nbytes", "s")

    def __init__(self, rec, kind, flops, nbytes):
        self.rec, self.kind, self.flops, self.nbytes = rec, kind, flops, nbytes

    def __enter__(self):
        rec = self.rec
        if rec.active:
            if rec.flush is not None:
                rec.flush.fill_(float(len(rec.items) & 1023))
            self.s = rec.torch.cuda.Event(enable_timing=True)
            self.s.record(rec.torch.cuda.current_stream())

    def __exit__(self, *exc):
        rec = self.rec
        if rec.active:
            e = rec.torch.cuda.Event(enable_timing=True)
            e.record(rec.torch.cuda.current_stream())
            rec.items.append((self.kind, self.flops, self.nbytes, self.s, e))
        return False


class LaunchRecorder:
    """Brackets launches with events on the stream they are issued on."""

    def __init__(self, flush=None):
        import torch
        self.torch = torch
        self.items = []
        self.active = False
        self.flush = flush

    def __call__(self, kind, flops=0.0, nbytes=0.0):
        return _Bracket(self, kind, flops, nbytes)

    def summary(self, peak_tflops):
        agg = {}
        for kind, flops, nbytes, s, e in self.items:
            ms = s.elapsed_time(e)
            a = agg.setdefault(kind, dict(launches=0, ms=0.0, flops=0.0, bytes=0.0))
            a["launches"] += 1
            a["ms"] += ms
            a["flops"] += flops
            a["bytes"] += nbytes
        for a in agg.values():
            sec = a["ms"] * 1e-3
            a["avg_ms"] = a["ms"] / a["launches"]
            a["tflops"] = a["flops"] / sec / 1e12
            a["gbs"] = a["bytes"] / sec / 1e9
            # the roofline that bounds this kind of call: the larger of its
            # compute time at the MFMA peak and its traffic time at the HBM peak
            t_mfma = a["flops"] / (peak_tflops * 1e12)
            t_hbm = a["bytes"] / (PEAK_HBM_GBS * 1e9)
            a["bound"] = "mfma" if t_mfma >= t_hbm else "hbm"
            a["frac"] = max(t_mfma, t_hbm) / sec if sec > 0 else 0.0
        return agg


# Kernel symbols behind a recorded launch kind, per workload (for the
# rocprofv3 summaries and the PMC traffic): each is launched once per call
# of that kind, so the call's traffic is the sum of theirs.
KERNEL_NAME = {
    "mixtral": {
        "gmm_nn": ["gmm_mfma_kernel<true, 256, 256, unsigned short, true, false, false>"],
        "gmm_nt": ["gmm_mfma_kernel<false, 256, 256, unsigned short, true, false, false>"],
        "tgmm": ["tgmm_mfma_kernel<256, 256, unsigned short>"],
        "gmm_nt_swiglu_bwd": ["gmm_mfma_kernel<false, 256, 256, unsigned short, true, false, true>"],
    },
    "deepseek_v3": {
        "tgmm": ["tgmm_short_kernel<unsigned short>", "tgmm_strip_kernel<2, unsigned short>",
                 "tgmm_strip_kernel<4, unsigned short>", "tgmm_mfma_kernel<128, 256, unsigned short>",
                 "tgmm_mfma_kernel<256, 256, unsigned short>"],
        "gmm_nn": ["gmm_mfma_kernel<true, 256, 256, unsigned short, true, false, false>",
                   "gmm_mfma_kernel<true, 128, 256, unsigned short, false, false, false>"],
        "gmm_nt": ["gmm_mfma_kernel<false, 128, 256, unsigned short, false, false, false>"],
        "gmm_nt_swiglu_bwd": ["gmm_mfma_kernel<false, 256, 256, unsigned short, true, false, true>",
                              "gmm_mfma_kernel<false, 128, 256, unsigned short, false, false, true>"],
    },
}
# Memory-bound kinds: the symbol prefix of the kernel that moves their data.
MEM_KERNEL_PREFIX = {
    "permute": "permute_scatter_kernel",
    "combine": "gather_sum_kernel<unsigned short, true",
    "permute_bwd": "gather_sum_kernel<unsigned short, false",
    "combine_bwd": "combine_bwd_kernel<unsigned short",
    "swiglu": "swiglu_kernel<unsigned short",
    "swiglu_bwd": "swiglu_bwd_kernel<unsigned short",
}


def kernel_source_digest() -> str:
    """Digest of every HIP source and header of the library, with comments
    and blank lines removed, so that counters stay tied to the code they
    were taken on."""
    import re
    csrc = os.path.join(ROOT, "mixture_experts_grouped_top_amd", "csrc")
    text = ""
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name)) as f:
                text += f.read()
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_json(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{workload}_traffic.json")


def traffic_for(workload: str, kind: str):
    """Calibrated HBM bytes per call of `kind` (the sum over the kernels it
    launches) from the committed PMC summary, or None (absent, taken on
    other sources, or a kernel missing from it)."""
    try:
        with open(traffic_json(workload)) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256_16") != kernel_source_digest():
        return None
    ks = d.get("kernels", {})

    def find(sym):
        hits = [k for k in ks if sym in k]
        return ks[hits[0]]["hbm_bytes_per_dispatch"] if len(hits) == 1 else None
    names = KERNEL_NAME.get(workload, {}).get(kind)
    if names is None and kind in MEM_KERNEL_PREFIX:
        names = [MEM_KERNEL_PREFIX[kind]]
    if not names:
        return None
    vals = [find(n) for n in names]
    return None if any(v is None for v in vals) else int(sum(vals))


COPY_ROWS, COPY_COLS = 32768, 16384      # bf16 rows copied by the calibration run (1 GiB)
COPY_KERNEL = "permute_scatter_kernel"


def copy_calibration():
    """A plain copy of known size: moe_permute with one expert and top-1 is
    the identity permutation, so its row-scatter kernel reads and writes
    COPY_ROWS x COPY_COLS bf16 once each (1 GiB each way)."""
    import torch
    import mixture_experts_grouped_top_amd as moe
    moe.load()
    x = torch.ones((COPY_ROWS, COPY_COLS), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((COPY_ROWS, 1), dtype=torch.int32, device="cuda")
    for _ in range(3):
        moe.moe_permute(x, ids, 1)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {COPY_ROWS}x{COPY_COLS} bf16, 3 copies")


def _pmc_per_dispatch(path, counter):
    """{kernel symbol: [counter value summed over its dimensions, per dispatch]}"""
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def traffic_summary(workload, bench_fetch, bench_write, copy_fetch, copy_write):
    """Average FETCH_SIZE / WRITE_SIZE (KiB) per dispatch of every kernel of a
    bench run, scaled by known_bytes / measured_bytes of the copy kernel."""
    known = COPY_ROWS * COPY_COLS * 2

    def copy_avg(path, counter):
        v = [x for k, xs in _pmc_per_dispatch(path, counter).items() if COPY_KERNEL in k for x in xs]
        return sum(v) / len(v)
    f_fetch = known / (1024.0 * copy_avg(copy_fetch, "FETCH_SIZE"))
    f_write = known / (1024.0 * copy_avg(copy_write, "WRITE_SIZE"))
    bench_cmd = (f"python bench.py --workload {workload} --extra-workloads '' --steps 2 "
                 "--warmup 1 --no-cpu-baseline --no-kernel-events")
    out = {"workload": workload, "source_sha256_16": kernel_source_digest(),
           "calibration": {"copy_bytes_each_way": known, "fetch_scale": round(f_fetch, 4),
                           "write_scale": round(f_write, 4), "kernel": COPY_KERNEL},
           "commands": [
               f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/pmc_fetch -o p -- {bench_cmd}",
               f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/pmc_write -o p -- {bench_cmd}",
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/pmc_copy_fetch -o p "
               "-- python bench.py --copy-calibration",
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/pmc_copy_write -o p "
               "-- python bench.py --copy-calibration"],
           "kernels": {}}
    fetch = _pmc_per_dispatch(bench_fetch, "FETCH_SIZE")
    write = _pmc_per_dispatch(bench_write, "WRITE_SIZE")
    for name in sorted(set(fetch) & set(write)):
        if name.startswith(("at::", "void at::", "__amd")):
            continue
        f, wv = fetch[name], write[name]
        fk, wk = sum(f) / len(f), sum(wv) / len(wv)
        out["kernels"][name] = {
            "dispatches": len(f), "fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
            "hbm_bytes_per_dispatch": round(1024.0 * (fk * f_fetch + wk * f_write))}
    with open(traffic_json(workload), "w") as fh:
        json.dump(out, fh, indent=1)
    log(f"[bench] wrote {traffic_json(workload)}")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w, host, tokens: int):
    """The float64 oracle, as it stands, on the first `tokens` tokens (all
    if 0) of the workload, with the expert weights regenerated on the host."""
    import numpy as np
    import moe_synth as ms
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    T = w.T if tokens <= 0 else min(tokens, w.T)
    sl = slice(0, T)
    wi0, wi1, wo = (ms.gen_expert_weights(w, k) for k in ("wi_0", "wi_1", "wo"))
    kw = dict(score=w.score, renorm=w.renorm, bias=host["bias"])
    t0 = time.perf_counter()
    f = oracle.moe_forward(host["x"][sl], wi0, wi1, wo, w.K, Wg=host["Wg"],
                           logits=None if host["logits"] is None else host["logits"][sl],
                           align=w.align, capacity=w.capacity, n_chunks=w.n_chunks, **kw)
    oracle.moe_backward(f, host["dy"][sl], host["x"][sl], wi0, wi1, wo, w.K, Wg=host["Wg"], **kw)
    dt = time.perf_counter() - t0
    R = int((f["perm"]["row_of_slot"] >= 0).sum())
    flops = 18.0 * R * w.D * w.F
    what = "all" if T == w.T else f"the first {T} of"
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"float64 oracle forward+backward on {what} {w.T} tokens ({R} routed "
                      f"rows, all {w.E} experts) of the same workload; {dt:.1f} s wall"}


def gen_device_inputs(name: str, args):
    import torch
    import moe_synth as ms
    w = ms.get_workload(name)
    t0 = time.time()
    g = ms.device_inputs(w, threads=min(16, len(os.sched_getaffinity(0))))
    host = g.pop("host")
    log(f"[bench] {name}: generated inputs in {time.time() - t0:.1f}s")
    g["wi"] = None
    if args.fused_wi:
        g["wi"] = torch.cat([g.pop("wi_0"), g.pop("wi_1")], dim=2).contiguous()
        g["wi_0"] = g["wi_1"] = None
        torch.cuda.empty_cache()
    return w, g, host


def vendor_batched_forward(w, g, plan, reps: int = 10) -> dict:
    """The forward's three expert GEMMs as a dense per-expert batched GEMM
    from the vendor library (torch.bmm) over the capacity-padded buffers the
    plan just filled ([E, C, D] x [E, D, F], all operands contiguous), timed
    like the library's own calls, for context beside them."""
    import torch
    E, C, D, F = w.E, w.capacity, w.D, w.F
    xs = plan.x_sorted[:E * C].view(E, C, D)
    act = plan.act[:E * C].view(E, C, F)
    h = torch.empty((E, C, F), dtype=xs.dtype, device=xs.device)
    y = torch.empty((E, C, D), dtype=xs.dtype, device=xs.device)

    def fwd():
        torch.bmm(xs, g["wi_0"], out=h)
        torch.bmm(xs, g["wi_1"], out=h)
        torch.bmm(act, g["wo"], out=y)
    fwd()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fwd()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    return {"ms_three_gemms": round(ms, 4), "library": "torch.bmm (hipBLASLt / rocBLAS)",
            "shape": f"{E} x [{C}, {D}] . [{D}, {F}] (twice) and [{C}, {F}] . [{F}, {D}]"}


def vendor_dense_gemm(w, g, plan, R: int, reps: int = 5) -> dict:
    """The up-projection's product (rows x D . D x F per expert) through the
    vendor library on an even split of the routed rows (C = R / E rows per
    expert, from x_sorted): a batched NN GEMM (torch.bmm over [E, C, D] x
    [E, D, F], the layout the library's gmm_nn call reads) and, per expert,
    the NT form (torch.mm against a [F, D] copy of the weight, both operands
    contraction-contiguous, as nn.Linear multiplies).  Each call follows the same cache-evicting
    scratch write as the library's bracketed calls; for context beside the
    library's gmm_nn."""
    import torch
    E, D, F = w.E, w.D, w.F
    C = R // E
    xs = plan.x_sorted[:E * C].view(E, C, D)
    wi = g["wi_0"]
    wt = wi.transpose(1, 2).contiguous()
    h = torch.empty((E, C, F), dtype=xs.dtype, device=xs.device)
    scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        tot = 0.0
        for i in range(reps):
            scratch.fill_(float(i))
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            tot += s.elapsed_time(e)
        return tot / reps

    def nt():
        for e_ in range(E):
            torch.mm(xs[e_], wt[e_].t(), out=h[e_])
    ms_nn = timed(lambda: torch.bmm(xs, wi, out=h))
    ms_nt = timed(nt)
    flops = 2.0 * E * C * D * F
    del wt, h, scratch
    torch.cuda.empty_cache()
    return {"shape": f"{E} x [{C}, {D}] . [{D}, {F}]", "library": "torch (hipBLASLt / rocBLAS)",
            "bmm_nn_ms": round(ms_nn, 4), "bmm_nn_tflops": round(flops / ms_nn / 1e9, 1),
            "linear_nt_ms": round(ms_nt, 4), "linear_nt_tflops": round(flops / ms_nt / 1e9, 1)}


def measure(name: str, args, headline: bool, inputs=None, capacity_layout: bool = False) -> dict:
    """Time a workload's step on the GPU, then time each call."""
    import torch
    import mixture_experts_grouped_top_amd as moe

    w, g, host = inputs if inputs is not None else gen_device_inputs(name, args)
    dtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
    shape = moe.MoEShape(T=w.T, D=w.D, F=w.F, E=w.E, K=w.K, dtype=dtype, score=w.score,
                         renorm=w.renorm, align=w.align, capacity=w.capacity,
                         capacity_layout=capacity_layout,
                         n_chunks=w.n_chunks, pad_rows_to=w.pad_rows_to,
                         fused_wi=args.fused_wi, fp8=args.fp8)
    plan = moe.MoEPlan(shape)
    peak = PEAK_FP8_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS

    def step():
        plan.forward(g["x"], g["wi_0"], g["wi_1"], g["wo"], Wg=g["Wg"], logits=g["logits"],
                     bias=g["bias"], wi=g["wi"])
        plan.backward(g["dy"], g["x"], g["wi_0"], g["wi_1"], g["wo"], Wg=g["Wg"],
                      bias=g["bias"], wi=g["wi"])

    # one untimed step to read back the routed counts (flops and bytes labels)
    step()
    torch.cuda.synchronize()
    counts = plan.idx["counts"]
    R = int(counts.sum().item())
    plan.kept_rows_override = R
    plan.padded_rows_override = int(plan.idx["group_offsets"][-1].item())
    plan.nonempty_groups_override = int((counts > 0).sum().item())
    for _ in range(max(0, args.warmup - 1)):
        step()
    torch.cuda.synchronize()
    run = step
    if args.graph:
        # the step's launches captured once (the plan owns every buffer, so
        # the capture allocates nothing) and replayed as one graph
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
        run()
        torch.cuda.synchronize()

    # pass 1: the step time, nothing but the path's own launches in the stream
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    gc.collect()
    gc.disable()   # a collection pass stalls the launching thread (as timeit does)
    try:
        start.record()
        for _ in range(args.steps):
            run()
        end.record()
        torch.cuda.synchronize()
    finally:
        gc.enable()
    ms_step = start.elapsed_time(end) / args.steps
    err = int(plan.err.item())
    flops = 18.0 * R * w.D * w.F
    tflops = flops / (ms_step * 1e-3) / 1e12
    if capacity_layout:
        name = f"{name} (capacity layout)"
    log(f"[bench] {name}: {ms_step:.3f} ms/step, {tflops:.1f} TFLOP/s, R={R}, "
        f"padded rows={plan.padded_rows}, non-empty experts={plan.nonempty_groups}, err={err}")

    # pass 2: every expert GEMM and memory-bound call bracketed by events,
    # each after a cache-evicting scratch write
    kernels = {}
    if not args.no_kernel_events and args.kernel_steps > 0:
        scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        rec = LaunchRecorder(flush=scratch)
        plan.recorder = rec
        gc.collect()
        gc.disable()
        try:
            rec.active = True
            for _ in range(args.kernel_steps):
                step()
            torch.cuda.synchronize()
            rec.active = False
        finally:
            gc.enable()
        plan.recorder = None
        kernels = rec.summary(peak)
        del scratch
    roofline = None
    step_roofline = None
    if kernels:
        # the step's floor: each recorded call at its own roofline (the larger
        # of its flops at the MFMA peak and its algorithmic bytes at 8 TB/s)
        floor_ms = 1e3 * sum(max(v["flops"] / (peak * 1e12), v["bytes"] / (PEAK_HBM_GBS * 1e9))
                             for v in kernels.values()) / args.kernel_steps
        step_roofline = {
            "floor_ms": round(floor_ms, 4), "frac": round(floor_ms / ms_step, 4),
            "calls": "expert GEMMs, permute, SwiGLU, combine and their backward (the router "
                     "GEMM and routing, a few tens of microseconds, are not recorded)"}
        log(f"[bench]   step floor {floor_ms:.3f} ms at each call's roofline: "
            f"{100 * floor_ms / ms_step:.1f}% of the measured step")
        kind = max(kernels, key=lambda k: kernels[k]["ms"])
        k = kernels[kind]
        if k["bound"] == "mfma":
            ach, pk, unit = k["tflops"], peak, "TFLOP/s"
        else:
            ach, pk, unit = k["gbs"], PEAK_HBM_GBS, "GB/s"
        plain = not (args.fused_wi or args.fp8)
        roofline = {"bound": k["bound"], "kind": kind,
                    "kernels": KERNEL_NAME.get(w.name, {}).get(kind, [kind]) if plain else [kind],
                    "achieved": round(ach, 2), "peak": pk, "unit": unit,
                    "frac": round(ach / pk, 4),
                    "traffic": traffic_for(w.name, kind) if plain and not capacity_layout else None,
                    "avg_launch_ms": round(k["avg_ms"], 4),
                    "flops_per_launch": k["flops"] / k["launches"],
                    "algorithmic_bytes_per_launch": round(k["bytes"] / k["launches"])}
    for kk, v in kernels.items():
        log(f"[bench]   {kk:18s} {v['launches']:3d} launches  avg {v['avg_ms']:.3f} ms  "
            f"{v['tflops']:7.1f} TFLOP/s  {v['gbs']:6.0f} GB/s  bound {v['bound']} "
            f"({100 * v['frac']:.0f}% of it)")
    rec_out = {
        "ms_per_step": round(ms_step, 4), "tflops": round(tflops, 3),
        "mfma_peak_frac": round(tflops / peak, 4), "device_error_flags": err, "dtype": w.dtype,
        "config": {"workload": w.name, "tokens": w.T, "d_model": w.D, "d_ff": w.F,
                   "experts": w.E, "top_k": w.K, "score": w.score, "renorm": w.renorm,
                   "align_size": w.align, "capacity": w.capacity, "chunks": w.n_chunks,
                   "fused_wi": bool(args.fused_wi), "fp8": bool(args.fp8),
                   "capacity_layout": bool(capacity_layout), "graph": bool(args.graph),
                   "routed_rows": R,
                   "padded_rows": plan.padded_rows, "nonempty_experts": plan.nonempty_groups},
        "roofline": roofline,
        "step_roofline": step_roofline,
        "kernels": {kk: {"launches": v["launches"], "avg_ms": round(v["avg_ms"], 4),
                         "tflops": round(v["tflops"], 2),
                         "algorithmic_bytes": int(v["bytes"] / v["launches"]),
                         "gbs": round(v["gbs"], 1), "bound": v["bound"],
                         "roofline_frac": round(v["frac"], 4),
                         "traffic": None if capacity_layout else traffic_for(w.name, kk)}
                    for kk, v in kernels.items()},
    }
    if capacity_layout:
        rec_out["vendor_batched_fwd"] = vendor_batched_forward(w, g, plan)
    if (headline and not capacity_layout and w.dtype == "bf16" and not args.fp8
            and not args.fused_wi and w.E <= 16):
        v = vendor_dense_gemm(w, g, plan, R)
        if "gmm_nn" in kernels:
            v["library_gmm_nn_ms"] = round(kernels["gmm_nn"]["avg_ms"], 4)
            v["library_gmm_nn_tflops"] = round(kernels["gmm_nn"]["tflops"], 1)
        rec_out["vendor_dense_gemm"] = v
        log(f"[bench] vendor dense GEMM context: {v}")
    del plan
    if inputs is None:
        del g
    gc.collect()
    torch.cuda.empty_cache()
    if headline and not args.no_cpu_baseline:
        t1 = time.time()
        rec_out["cpu_baseline"] = cpu_baseline(w, host, args.cpu_tokens)
        log(f"[bench] cpu baseline: {rec_out['cpu_baseline']} ({time.time() - t1:.1f}s)")
    return rec_out


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import mixture_experts_grouped_top_amd as moe
    moe.load()
    head = measure(args.workload, args, headline=True)
    extras = {}
    for name in [n for n in args.extra_workloads.split(",") if n and n != args.workload]:
        import moe_synth as ms
        inputs = gen_device_inputs(name, args)
        extras[name] = measure(name, args, headline=False, inputs=inputs)
        extras[name]["cpu_baseline"] = None
        extras[name]["cpu_baseline_note"] = (
            "not run: the oracle's per-expert float64 weights alone (256 experts x 3 x "
            "7168 x 2048) take minutes to form on the host; the headline workload's "
            "baseline is the one reported")
        if ms.get_workload(name).capacity > 0 and not args.fp8 and not args.fused_wi:
            # the same step in the capacity-padded batched layout (every expert
            # C rows), against the compact grouped layout
            cap = measure(name, args, headline=False, inputs=inputs, capacity_layout=True)
            g_ms, b_ms = extras[name]["ms_per_step"], cap["ms_per_step"]
            fw = {k: v for k, v in cap["kernels"].items() if k == "gmm_nn"}
            extras[name]["capacity_layout"] = cap
            extras[name]["grouped_vs_batched"] = {
                "grouped_ms_per_step": g_ms, "batched_ms_per_step": b_ms,
                "batched_over_grouped": round(b_ms / g_ms, 3),
                "forward_gemms_ms": {
                    "grouped": round(3 * extras[name]["kernels"]["gmm_nn"]["avg_ms"], 4)
                    if "gmm_nn" in extras[name]["kernels"] else None,
                    "batched_library_kernels": round(3 * fw["gmm_nn"]["avg_ms"], 4)
                    if fw else None,
                    "batched_vendor_bmm": cap["vendor_batched_fwd"]["ms_three_gemms"]},
                "context": "the MaxText grouped-GEMM pull request reports grouped GEMM about "
                           "1.2x faster than batch GEMM on its hardware (context only)"}
        del inputs
    out = {
        "metric": METRIC, "value": head["tflops"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("fp8 e4m3/e5m2 GEMM operands, bf16 activations" if args.fp8 else
                  head["dtype"]),
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights; no dataset)",
        "config": head["config"],
        "mfma_peak_frac": head["mfma_peak_frac"],
        "roofline": head["roofline"],
        "step_roofline": head.get("step_roofline"),
        "cpu_baseline": head.get("cpu_baseline"),
        "device_error_flags": head["device_error_flags"],
        "kernels": head["kernels"],
        "vendor_dense_gemm": head.get("vendor_dense_gemm"),
        "workloads": extras,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
