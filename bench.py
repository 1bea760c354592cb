#!/usr/bin/env python3
"""MoE expert-FFN forward+backward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral]

A step is one pass of the whole path over one batch of synthetic input:
router GEMM, top-k routing, permute, the up-projection grouped GEMMs,
SwiGLU, the down-projection grouped GEMM and the weighted combine, then the
hand-derived backward (combine backward, grouped GEMMs with the rhs
transposed, transposed grouped GEMMs for the expert weight gradients,
SwiGLU backward, permute backward, routing backward and the router GEMM
backward).  Inputs are resident in HBM before the timed region starts.

`value` is expert-FFN TFLOP/s: 18 * R * d_model * d_ff algorithmic flops per
step (R = kept routed rows; padding rows and the router GEMM excluded)
divided by the step time.  Prints ONE JSON line on stdout; everything else
goes to stderr.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE FFN fwd+bwd grouped-GEMM TFLOP/s and % of bf16 MFMA peak, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="mixtral")
    p.add_argument("--cpu-tokens", type=int, default=2048,
                   help="tokens of the workload the CPU oracle baseline runs on")
    p.add_argument("--fused-wi", action="store_true",
                   help="one [E, D, 2F] up-projection weight [wi_0 | wi_1]")
    p.add_argument("--fp8", action="store_true",
                   help="FP8 expert GEMMs (e4m3 forward, e5m2 backward, current scaling)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-kernel-events", action="store_true",
                   help="do not bracket the expert GEMM launches with events")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain row copy of known size (for scaling HBM counters)")
    p.add_argument("--traffic-summary", nargs=4, metavar=("BENCH_FETCH", "BENCH_WRITE",
                                                           "COPY_FETCH", "COPY_WRITE"),
                   help="turn four rocprofv3 --pmc counter_collection.csv files into "
                        "profiles/gmm_mixtral_traffic.json and exit")
    return p.parse_args()


def gen_inputs(w, threads: int):
    """Seeded inputs (CPU), generated per expert in parallel."""
    import numpy as np
    import moe_synth as ms
    t0 = time.time()
    with cf.ThreadPoolExecutor(threads) as ex:
        futs = {name: [ex.submit(ms.gen_expert_weight, w, name, e) for e in range(w.E)]
                for name in ("wi_0", "wi_1", "wo")}
        x = ms.gen_x(w)
        dy = ms.gen_dy(w)
        Wg = ms.gen_gate(w) if w.logits == "gemm" else None
        logits = ms.gen_uniform_logits(w) if w.logits == "uniform" else None
        bias = ms.gen_logit_bias(w)
        weights = {k: [f.result() for f in v] for k, v in futs.items()}
    log(f"[bench] generated inputs in {time.time() - t0:.1f}s")
    return dict(x=x, dy=dy, Wg=Wg, logits=logits, bias=bias, **weights)


def to_gpu(inp, dtype):
    import numpy as np
    import torch

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
        return t.to(dtype) if dtype != torch.float32 else t

    out = {k: up(inp[k]) if inp[k] is not None else None for k in ("x", "dy", "Wg")}
    for k in ("wi_0", "wi_1", "wo"):
        out[k] = torch.stack([up(a) for a in inp[k]])
    for k in ("logits", "bias"):   # float32 router inputs
        out[k] = torch.from_numpy(inp[k]).cuda() if inp[k] is not None else None
    return out


class _Bracket:
    """Context manager recording a start and an end event around launches."""

    __slots__ = ("rec", "kind", "flops", "nbytes", "s")

    def __init__(self, rec, kind, flops, nbytes):
        self.rec, self.kind, self.flops, self.nbytes = rec, kind, flops, nbytes

    def __enter__(self):
        rec = self.rec
        if rec.active:
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

    def __init__(self):
        import torch
        self.torch = torch
        self.items = []
        self.active = False

    def __call__(self, kind, flops=0.0, nbytes=0.0):
        return _Bracket(self, kind, flops, nbytes)

    def summary(self):
        agg = {}
        for kind, flops, nbytes, s, e in self.items:
            ms = s.elapsed_time(e)
            a = agg.setdefault(kind, dict(launches=0, ms=0.0, flops=0.0, bytes=0.0))
            a["launches"] += 1
            a["ms"] += ms
            a["flops"] += flops
            a["bytes"] += nbytes
        for a in agg.values():
            a["avg_ms"] = a["ms"] / a["launches"]
            a["tflops"] = a["flops"] / (a["ms"] * 1e-3) / 1e12
            a["gbs"] = a["bytes"] / (a["ms"] * 1e-3) / 1e9
        return agg


# Kernel symbol behind each recorded launch kind for the bf16 workloads
# (the rocprofv3 summary is matched on this name).
# These are the 256 x 256 tile variants the Mixtral-8x7B shape runs on.
KERNEL_NAME = {
    "gmm_nn": "gmm_mfma_kernel<true, 256, 256, unsigned short, true, false, false>",
    "gmm_nt": "gmm_mfma_kernel<false, 256, 256, unsigned short, true, false, false>",
    "tgmm": "tgmm_mfma_kernel<256, 256, unsigned short>",
    "gmm_nt_swiglu_bwd": "gmm_mfma_kernel<false, 256, 256, unsigned short, true, false, true>",
    "gmm_up_chunk": "gmm_mfma_kernel<true, 128, 256, float, false, false, false>",
}


def kernel_source_digest() -> str:
    """Digest of the grouped-GEMM source and the helpers it includes, with
    comments and blank lines removed, so that counters stay tied to the code
    they were taken on."""
    import re
    csrc = os.path.join(ROOT, "mixture_experts_grouped_top_amd", "csrc")
    text = ""
    for name in ("gmm.hip", "common.h"):
        with open(os.path.join(csrc, name)) as f:
            text += f.read()
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_from_profiles(kind: str, workload: str):
    """HBM bytes per launch of the dominant kernel from the committed PMC
    summary (taken on the Mixtral-8x7B shape), or None if absent, taken on a
    different kernel source or for another workload."""
    if workload != "mixtral":
        return None
    path = os.path.join(ROOT, "profiles", "gmm_mixtral_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    k = d.get("kernels", {}).get(kind)
    if not k or d.get("gmm_source_sha256_16") != kernel_source_digest():
        return None
    return k.get("hbm_bytes_per_launch")


COPY_ROWS, COPY_COLS = 32768, 16384      # bf16 rows copied by the calibration run (1 GiB)
COPY_KERNEL = "permute_scatter_kernel"
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "gmm_mixtral_traffic.json")


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


def _pmc_per_dispatch(path, counter, name_part):
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter or name_part not in r["Kernel_Name"]:
            continue
        d = int(r["Dispatch_Id"])
        per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
    return list(per.values())


def traffic_summary(bench_fetch, bench_write, copy_fetch, copy_write):
    """Average FETCH_SIZE / WRITE_SIZE (KiB) per dispatch of each GEMM kernel,
    scaled by known_bytes / measured_bytes of the copy kernel."""
    known = COPY_ROWS * COPY_COLS * 2
    cf = _pmc_per_dispatch(copy_fetch, "FETCH_SIZE", COPY_KERNEL)
    cw = _pmc_per_dispatch(copy_write, "WRITE_SIZE", COPY_KERNEL)
    f_fetch = known / (1024.0 * sum(cf) / len(cf))
    f_write = known / (1024.0 * sum(cw) / len(cw))
    out = {"gmm_source_sha256_16": kernel_source_digest(),
           "calibration": {"copy_bytes_each_way": known, "fetch_scale": round(f_fetch, 4),
                           "write_scale": round(f_write, 4), "kernel": COPY_KERNEL},
           "commands": [
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/pmc_bench_fetch -o p "
               "-- python bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-kernel-events",
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/pmc_bench_write -o p "
               "-- python bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-kernel-events",
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/pmc_copy_fetch -o p "
               "-- python bench.py --copy-calibration",
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/pmc_copy_write -o p "
               "-- python bench.py --copy-calibration"],
           "kernels": {}}
    for kind, name in KERNEL_NAME.items():
        f = _pmc_per_dispatch(bench_fetch, "FETCH_SIZE", name)
        wv = _pmc_per_dispatch(bench_write, "WRITE_SIZE", name)
        if not f or not wv:
            continue
        fk, wk = sum(f) / len(f), sum(wv) / len(wv)
        out["kernels"][kind] = {
            "dispatches": len(f), "fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
            "hbm_bytes_per_launch": round(1024.0 * (fk * f_fetch + wk * f_write))}
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(out, fh, indent=1)
    log(f"[bench] wrote {TRAFFIC_JSON}")


def cpu_baseline(w, inp, tokens: int):
    """The float64 oracle, as it stands, on the first `tokens` tokens."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    T = min(tokens, w.T)
    sl = slice(0, T)
    wi0, wi1, wo = (np.stack(inp[k]) for k in ("wi_0", "wi_1", "wo"))
    kw = dict(score=w.score, renorm=w.renorm, bias=inp["bias"])
    t0 = time.perf_counter()
    f = oracle.moe_forward(inp["x"][sl], wi0, wi1, wo, w.K, Wg=inp["Wg"],
                           logits=None if inp["logits"] is None else inp["logits"][sl],
                           align=w.align, capacity=w.capacity, n_chunks=w.n_chunks, **kw)
    oracle.moe_backward(f, inp["dy"][sl], inp["x"][sl], wi0, wi1, wo, w.K, Wg=inp["Wg"], **kw)
    dt = time.perf_counter() - t0
    R = int((f["perm"]["row_of_slot"] >= 0).sum())
    flops = 18.0 * R * w.D * w.F
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 oracle forward+backward on the first {T} of {w.T} tokens "
                      f"({R} routed rows, all {w.E} experts) of the same workload; "
                      f"{dt:.1f} s wall"}


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
    import numpy as np
    import torch
    import moe_synth as ms
    import mixture_experts_grouped_top_amd as moe

    moe.load()
    w = ms.get_workload(args.workload)
    dtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
    threads = min(16, len(os.sched_getaffinity(0)))
    inp = gen_inputs(w, threads)
    g = to_gpu(inp, dtype)
    g["wi"] = None
    if args.fused_wi:
        g["wi"] = torch.cat([g.pop("wi_0"), g.pop("wi_1")], dim=2).contiguous()
        g["wi_0"] = g["wi_1"] = None
        torch.cuda.empty_cache()
    shape = moe.MoEShape(T=w.T, D=w.D, F=w.F, E=w.E, K=w.K, dtype=dtype, score=w.score,
                         renorm=w.renorm, align=w.align, capacity=w.capacity,
                         n_chunks=w.n_chunks, pad_rows_to=w.pad_rows_to,
                         fused_wi=args.fused_wi, fp8=args.fp8)
    plan = moe.MoEPlan(shape)
    peak = PEAK_FP8_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS

    def step():
        plan.forward(g["x"], g["wi_0"], g["wi_1"], g["wo"], Wg=g["Wg"], logits=g["logits"],
                     bias=g["bias"], wi=g["wi"])
        plan.backward(g["dy"], g["x"], g["wi_0"], g["wi_1"], g["wo"], Wg=g["Wg"], bias=g["bias"],
                      wi=g["wi"])

    # one untimed step to learn the kept row count (dropping) for the flop count
    step()
    torch.cuda.synchronize()
    R = int(plan.idx["counts"].sum().item())
    plan.kept_rows_override = R
    plan.padded_rows_override = int(plan.idx["group_offsets"][-1].item())
    for _ in range(max(0, args.warmup - 1)):
        step()
    rec = LaunchRecorder()
    if not args.no_kernel_events:
        plan.recorder = rec
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    # no cyclic garbage collection inside the timed region (as timeit does):
    # a collection pass stalls the launching thread for tens of milliseconds
    gc.collect()
    gc.disable()
    try:
        rec.active = True
        start.record()
        for _ in range(args.steps):
            step()
        end.record()
        torch.cuda.synchronize()
        rec.active = False
    finally:
        gc.enable()
    ms_step = start.elapsed_time(end) / args.steps
    err = int(plan.err.item())
    flops = 18.0 * R * w.D * w.F
    tflops = flops / (ms_step * 1e-3) / 1e12
    log(f"[bench] {args.workload}: {ms_step:.3f} ms/step, {tflops:.1f} TFLOP/s, R={R}, err={err}")

    kernels = rec.summary()
    roofline = None
    gemm = {k: v for k, v in kernels.items() if v["flops"] > 0}
    if gemm:
        kind = max(gemm, key=lambda k: gemm[k]["ms"])
        k = gemm[kind]
        ach = k["tflops"]
        plain = not (args.fused_wi or args.fp8)
        traffic = traffic_from_profiles(kind, args.workload) if plain else None
        label = KERNEL_NAME.get(kind, kind) if args.workload == "mixtral" and plain else kind
        roofline = {"bound": "mfma", "kernel": label,
                    "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(ach / peak, 4), "traffic": traffic,
                    "avg_launch_ms": round(k["avg_ms"], 4),
                    "flops_per_launch": k["flops"] / k["launches"]}
    for kk, v in kernels.items():
        rate = (f"{v['tflops']:.1f} TFLOP/s" if v["flops"] else
                f"{v['gbs']:.0f} GB/s ({100 * v['gbs'] / PEAK_HBM_GBS:.0f}% of HBM)")
        log(f"[bench]   {kk:12s} {v['launches']:4d} launches  avg {v['avg_ms']:.3f} ms  {rate}")
    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(w, inp, args.cpu_tokens)
        log(f"[bench] cpu baseline: {cpu} ({time.time() - t0:.1f}s)")

    out = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("fp8 e4m3/e5m2 GEMM operands, bf16 activations" if args.fp8 else
                  "bf16" if dtype == torch.bfloat16 else "f32"),
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights; no dataset)",
        "config": {"workload": w.name, "tokens": w.T, "d_model": w.D, "d_ff": w.F,
                   "experts": w.E, "top_k": w.K, "score": w.score, "renorm": w.renorm,
                   "align_size": w.align, "capacity": w.capacity, "chunks": w.n_chunks,
                   "fused_wi": bool(args.fused_wi), "fp8": bool(args.fp8), "routed_rows": R},
        "mfma_peak_frac": round(tflops / peak, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "device_error_flags": err,
        "kernels": {k: ({"launches": v["launches"], "avg_ms": round(v["avg_ms"], 4),
                         "tflops": round(v["tflops"], 2)} if v["flops"] else
                        {"launches": v["launches"], "avg_ms": round(v["avg_ms"], 4),
                         "algorithmic_bytes": int(v["bytes"] / v["launches"]),
                         "gbs": round(v["gbs"], 1),
                         "hbm_frac": round(v["gbs"] / PEAK_HBM_GBS, 4)})
                    for k, v in kernels.items()},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
