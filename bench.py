"""Benchmark of the MoE layer forward on one MI355X.

One step = one full layer forward (route -> permute -> FC1+SwiGLU -> FC2
(-> shared expert) -> combine) over one synthetic batch already resident in
HBM.  Prints ONE JSON line.  The default workload is the DeepSeek-V3-shaped
layer, the largest of the five layer shapes (T=8192, h=7168, E=256, top-8
sigmoid with a selection-only expert bias, ffn 2048, one shared expert of
ffn 2048, bf16 with an fp32 router); --config picks another layer shape.

Per-stage durations come from HIP events recorded at every stage boundary
on the stream the kernels run on, in a pass of K steps of their own
(median, p10, p90 are reported).  The timed region then runs K plain
forwards whose only events are the two around the dominant single-kernel
stage: its average launch duration there gives the roofline object.
`traffic` (HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE
counters) is read from profiles/ and reported only while the kernel source
is unchanged since the counters were taken.  After the timed region, a second pass times each step with the
last-level caches flushed first (a 512 MiB write before every step; the
flush is outside the events) and reports it as "cold".

Layer options (on by default, --no-gather / --no-overlap /
--no-fuse-route-permute to turn off): the permute writes no row copies and
FC1 gathers token rows through sorted_token; the shared expert (when the
layer has one) runs on a second stream, joined before the combine; route and
permute run as one library call (moe_route_permute), which reuses the
router's counting pass for the permute; top-1 layers without a shared expert
run FC2 with the combine as its epilogue (moe_grouped_fc2_combine, or its
MXFP8 twin; --no-fuse-combine to turn off).  With the overlap on, main-stream stage
times include contention with the shared expert.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/sec + grouped-GEMM TFLOPS (% of MI355X bf16 MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 (used for fp32 layers)
KERNEL_SOURCES = {  # stage -> source file that holds its kernel
    "route": "route.hip", "permute": "permute.hip", "route_permute": "route.hip",
    "fc1": "gmm.hip", "fc2": "gmm.hip", "fc2_combine": "gmm.hip",
    "shared": "gmm.hip", "combine": "combine.hip", "quantize": "mx.hip",
}
MX_SOURCES = {"fc1": "gmm_mx.hip", "fc2": "gmm_mx.hip", "fc2_combine": "gmm_mx.hip",
              "shared": "gmm_mx.hip"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="dsv3")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-sample-tokens", type=int, default=None,
                   help="tokens the oracle runs for the cpu_baseline leg (default: per layer)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="run one plain device copy of this size first (counter calibration)")
    p.add_argument("--no-gather", action="store_true", help="materialise permuted_x")
    p.add_argument("--no-overlap", action="store_true", help="shared expert on the main stream")
    p.add_argument("--no-fuse-route-permute", action="store_true",
                   help="route and permute as two library calls")
    p.add_argument("--no-fuse-combine", action="store_true",
                   help="top-1 layers: FC2 and the combine as two library calls")
    p.add_argument("--no-tile-queue", action="store_true",
                   help="grouped GEMMs with one workgroup per tile instead of the per-XCD tile queue")
    p.add_argument("--no-fold-shared", action="store_true",
                   help="shared expert in launches of its own (on a second stream unless "
                        "--no-overlap) instead of the routed launches' last tiles")
    p.add_argument("--no-cold", action="store_true", help="skip the cache-flushed pass")
    p.add_argument("--no-clock", action="store_true",
                   help="skip the clock pass (extra forwards with clock probes on a second stream)")
    p.add_argument("--precision", default="bf16", choices=("bf16", "mxfp8"),
                   help="expert GEMM operands (mxfp8: OCP MX blocks of 32, E4M3)")
    return p.parse_args()


def _code_only(text: str) -> str:
    """C++ source without its comments and blank lines, so that a counter
    summary stays current across comment edits but not across code edits.
    (The sources hold no string literal with // or /* in it.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_hash(stage: str, mx: bool = False) -> str:
    """Hash of the code a stage's kernel is built from: its source file and
    the shared headers (comments and blank lines dropped), and the build
    flags."""
    src = MX_SOURCES[stage] if mx and stage in MX_SOURCES else KERNEL_SOURCES[stage]
    path = os.path.join(ROOT, "combine_router_gating_amd", "csrc", src)
    csrc = os.path.join(ROOT, "combine_router_gating_amd", "csrc")
    headers = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".h"))
    h = hashlib.sha256()
    for f in [path] + headers:
        h.update(_code_only(open(f, encoding="utf-8").read()).encode())
    h.update(open(os.path.join(ROOT, "combine_router_gating_amd", "build.py"), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(stage: str, workload: str, mx: bool = False):
    """HBM bytes per launch from a committed counter summary, if current."""
    path = os.path.join(ROOT, "profiles", f"pmc_{stage}_{workload}{'_mxfp8' if mx else ''}.md")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            kv[k.strip()] = v.strip().strip("`")
    if kv.get("source_sha256") != source_hash(stage, mx):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def stage_work(cfg, n, T, fs, gather=False, mx=False, fold=False):
    """Algorithmic bytes and flops of each stage (kept rows only, no padding,
    each tensor moved once).  With `gather` the permute moves no rows; with
    `mx` the GEMM operands are MXFP8 (1 byte per value + 1 scale byte per 32)
    and the expert outputs bf16; with `fold` the fc1 and fc2 stages also run
    the shared expert's FC1 and FC2 (one launch each)."""
    b = 4 if cfg.dtype == "f32" else 2
    h, f, E, K = cfg.h, cfg.f, cfg.E, cfg.K
    N = int(sum(n))
    active = int(sum(1 for v in n if v > 0))
    w = {
        "route": (T * h * b + E * h * 4 + T * E * (4 + 4 + 1) + E * 4, 2.0 * T * h * E),
        "permute": ((0 if gather else T * h * b + N * h * b) + T * E * (1 + 4) + N * 8 + T * K * 4
                    + E * 4, 0.0),
        "fc1": (active * 2 * h * f * b + N * h * b + N * f * b, 4.0 * N * h * f),
        "fc2": (active * h * f * b + N * f * b + N * h * b, 2.0 * N * h * f),
        "combine": (N * h * b + T * K * 4 + N * 4 + T * h * b + (T * h * b if fs else 0), 0.0),
    }
    if fs:
        w["shared"] = (3 * h * fs * b + 2 * T * h * b + 2 * T * fs * b, 6.0 * T * h * fs)
        if fold:
            f1, f2 = w["fc1"], w["fc2"]
            w["fc1"] = (f1[0] + 2 * h * fs * b + T * h * b + T * fs * b, f1[1] + 4.0 * T * h * fs)
            w["fc2"] = (f2[0] + h * fs * b + T * fs * b + T * h * b, f2[1] + 2.0 * T * h * fs)
    # route and permute as one call: the map and probs are written once and
    # read back by the scatter
    w["route_permute"] = (w["route"][0] + w["permute"][0], w["route"][1])
    # FC2 with the top-1 combine as its epilogue: act and W_down read, out
    # written (kept rows scaled, dropped rows zero), no expert_out round trip
    w["fc2_combine"] = (active * h * f * b + N * f * b + T * h * b + N * 8 + T * K * 4,
                        2.0 * N * h * f)
    if mx:
        q = 1.0 + 1.0 / 32
        w["quantize"] = (T * h * b + T * h * q, 0.0)
        w["fc1"] = (active * 2 * h * f * q + N * h * q + N * f * q, 4.0 * N * h * f)
        w["fc2"] = (active * h * f * q + N * f * q + N * h * b, 2.0 * N * h * f)
        w["fc2_combine"] = (active * h * f * q + N * f * q + T * h * b + N * 8 + T * K * 4,
                            2.0 * N * h * f)
        if fs:
            w["shared"] = (3 * h * fs * q + T * h * q + 2 * T * fs * q + T * h * b, 6.0 * T * h * fs)
    return w


def copy_bandwidth(dev, mib=512, reps=10):
    """GB/s (bytes read + written) of torch's device-to-device copy of a
    `mib` MiB buffer: the plain streaming rate the HBM-bound kernels are
    compared with."""
    import torch

    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        b.copy_(a)
    t1.record()
    torch.cuda.synchronize()
    sec = t0.elapsed_time(t1) * 1e-3 / reps
    del a, b
    return 2 * n * 4 / sec / 1e9


def cpu_baseline(cfg, inp, sample_tokens, min_seconds=10.0):
    """The oracle, as it stands, on the first `sample_tokens` tokens of the
    batch run as a batch of their own (same weights and routing options)."""
    import numpy as np

    import datagen
    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    affinity = len(os.sched_getaffinity(0))
    S = min(sample_tokens, cfg.T)
    f64 = datagen.to_f64
    x = f64(inp["x"][:S])
    wr = f64(inp["w_router"])
    br = f64(inp["b_router"]) if "b_router" in inp else None
    eb = inp["expert_bias"].cpu().numpy() if "expert_bias" in inp else None
    # host copies of the weights in their stored values (fp32 holds bf16 exactly)
    host = {k: inp[k].to("cpu", torch_float32()).numpy() for k in ("w_gate", "w_up", "w_down")}
    shared = None
    if "shared_gate" in inp:
        shared = tuple(f64(inp[k]) for k in ("shared_gate", "shared_up", "shared_down"))

    def weights(e):
        return (host["w_gate"][e].astype(np.float64), host["w_up"][e].astype(np.float64),
                host["w_down"][e].astype(np.float64))

    # repeat the sample until about 10 s of CPU work have been timed
    runs, total = 0, 0.0
    while runs == 0 or (total < min_seconds and runs < 20):
        t0 = time.perf_counter()
        oracle.moe_forward(x, wr, br, weights, K=cfg.K, dtype=cfg.dtype, score=cfg.score,
                           pre_softmax=cfg.pre_softmax, expert_bias=eb,
                           capacity_factor=cfg.capacity_factor, min_capacity=cfg.min_capacity,
                           shared=shared)
        total += time.perf_counter() - t0
        runs += 1
    dt = total / runs
    # the oracle's only multi-threaded part is NumPy's BLAS (the float64
    # matmuls); everything else runs on one thread
    return {"value": S / dt, "unit": "tokens/s", "cores": int(min(blas_threads, affinity)),
            "kind": "oracle",
            "sample": f"first {S} of {cfg.T} tokens run as one batch (same weights and routing "
                      f"options; capacity recomputed for that batch), float64 NumPy, "
                      f"{runs} run(s), {total:.1f} s in total",
            "affinity_cores": affinity, "blas_threads": int(blas_threads),
            "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def clock_pass(layer, dev, step_ms: float, steps: int):
    """Shader clock while the layer runs: one-wave probes (moe_clock_probe:
    s_memtime cycles over s_memrealtime ticks) queued back to back on a
    second stream during extra forwards whose times are not used.  A probe
    wave holds registers on one CU, which keeps one GEMM workgroup off that
    CU while it runs, so this pass is separate from the timed ones."""
    import torch
    import combine_router_gating_amd as moe_lib
    total_us = max(1000.0, min(steps * step_ms * 1e3, 300e3))
    window = int(max(200.0, min(5000.0, total_us / 8)))
    n = max(1, int(total_us // window))
    buf = torch.zeros((n, 2), dtype=torch.int64, device=dev)
    side = torch.cuda.Stream(device=dev)
    nsteps = int(total_us / (step_ms * 1e3)) + 2
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for k in range(n):
            moe_lib.moe_clock_probe(buf[k], window)
    for _ in range(nsteps):
        layer.forward()
    torch.cuda.synchronize()
    mhz = sorted(100.0 * c / t for c, t in buf.cpu().tolist() if t > 0)
    if not mhz:
        return None
    return {"unit": "MHz", "min": round(mhz[0]), "median": round(mhz[len(mhz) // 2]),
            "max": round(mhz[-1]), "windows": len(mhz), "window_us": window,
            "source": "s_memtime cycles / s_memrealtime ticks of one-wave probes "
                      "(moe_clock_probe) on a second stream, back to back during "
                      f"{nsteps} extra forwards"}


def torch_float32():
    import torch
    return torch.float32


DEFAULT_CPU_SAMPLE = {"tiny": 256, "switch": 8192, "mixtral": 256, "qwen3": 512, "dsv3": 128}


def load_stats(n):
    """tokens_per_expert spread: min, max, mean, coefficient of variation."""
    import numpy as np
    a = np.asarray(n, np.float64)
    mean = float(a.mean()) if a.size else 0.0
    return {"min": int(a.min()) if a.size else 0, "max": int(a.max()) if a.size else 0,
            "mean": mean, "cv": float(a.std() / mean) if mean else 0.0,
            "empty_experts": int((a == 0).sum())}


def pct(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v), q))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this layer runs on one GPU's share of experts)", file=sys.stderr)
        sys.exit(2)
    import torch

    import datagen
    from combine_router_gating_amd.layer import MoELayerForward

    cfg = datagen.CONFIGS[args.config]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        bb = torch.empty_like(a)
        bb.copy_(a)
        torch.cuda.synchronize()
        del a, bb
    inp = datagen.make_inputs(cfg, seed=args.seed, device=dev)
    gather = not args.no_gather
    mx = args.precision == "mxfp8"
    layer = MoELayerForward(inp, K=cfg.K, score=cfg.score, pre_softmax=cfg.pre_softmax,
                            capacity_factor=cfg.capacity_factor, min_capacity=cfg.min_capacity,
                            gather=gather, overlap_shared=not args.no_overlap,
                            precision=args.precision,
                            fuse_route_permute=not args.no_fuse_route_permute,
                            fuse_combine=not args.no_fuse_combine,
                            fold_shared=not args.no_fold_shared,
                            tile_queue=not args.no_tile_queue)
    for _ in range(args.warmup):
        layer.forward()
    torch.cuda.synchronize()

    # Stage breakdown: K steps with events at every stage boundary on the
    # main stream (the events themselves cost ~10-20 us a step, so this pass
    # is kept out of the timed region).
    stages = layer.stages()
    events = []

    def mark(name):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        events[-1].append((name, ev))

    torch.cuda.synchronize()
    for _ in range(args.steps):
        events.append([])
        layer.forward(mark)
    torch.cuda.synchronize()

    per_step = {s: [] for s in stages}
    fwd = []
    for evs in events:
        for (name, a), (_, b) in zip(evs[:-1], evs[1:]):
            per_step[name].append(a.elapsed_time(b))
        fwd.append(evs[0][1].elapsed_time(evs[-1][1]))
    stage_ms = {s: sum(v) / len(v) for s, v in per_step.items()}
    single_kernel = ("fc1", "fc2", "fc2_combine", "shared", "combine")
    dom = max((s for s in stage_ms if s in single_kernel), key=lambda s: stage_ms[s])
    after_dom = stages[stages.index(dom) + 1] if stages.index(dom) + 1 < len(stages) else "end"

    # Timed region: K plain forwards; the only events are the two around the
    # dominant kernel (its average launch duration for the roofline).
    dom_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]

    def dom_mark(i):
        def m(name):
            if name == dom:
                dom_ev[i][0].record()
            elif name == after_dom:
                dom_ev[i][1].record()
        return m

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        layer.forward(dom_mark(i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    dom_ms = [a.elapsed_time(b) for a, b in dom_ev]

    n = layer.tokens_per_expert.cpu().tolist()
    N = int(sum(n))
    work = stage_work(cfg, n, cfg.T, layer.fs if layer.shared else 0, gather, mx,
                      layer.fold_shared)
    gemm_stages = [s for s in ("fc1", "fc2", "fc2_combine", "shared") if s in stage_ms]
    gemm_flops = sum(work[s][1] for s in gemm_stages)
    gemm_bytes = sum(work[s][0] for s in gemm_stages)
    gemm_ms = sum(stage_ms[s] for s in gemm_stages)
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    peak_tf = (MFMA_FP8_PEAK_TFLOPS if mx else
               MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else FP32_PEAK_TFLOPS)
    attainable_tf = min(peak_tf, gemm_flops / gemm_bytes * HBM_PEAK_GBS * 1e9 / 1e12)

    nbytes, flops = work[dom]
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
    dom_avg = sum(dom_ms) / len(dom_ms)
    sec = dom_avg * 1e-3
    if flops and flops / nbytes >= ridge:
        roof = {"bound": "mfma", "achieved": flops / sec / 1e12, "peak": peak_tf,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": nbytes / sec / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = read_traffic(dom, cfg.name, mx)
    roof["kernel"] = dom
    # context for HBM fractions: what a plain device copy reaches on this GPU now
    copy_gbs = copy_bandwidth(dev)
    if roof["bound"] == "hbm":
        roof["copy_GBs"] = copy_gbs
        roof["frac_of_copy"] = roof["achieved"] / copy_gbs
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_flops"] = flops
    roof["avg_launch_ms"] = dom_avg

    stage_report = {}
    for s in stages:
        nb, fl = work[s]
        sec_s = stage_ms[s] * 1e-3
        stage_report[s] = {"ms": round(stage_ms[s], 4), "p10": round(pct(per_step[s], 10), 4),
                           "p50": round(pct(per_step[s], 50), 4),
                           "p90": round(pct(per_step[s], 90), 4),
                           "GB/s": round(nb / sec_s / 1e9, 1),
                           "TFLOP/s": round(fl / sec_s / 1e12, 1) if fl else 0.0}
        if s in ("permute", "combine", "quantize"):  # HBM-bound stages
            stage_report[s]["frac_of_hbm_peak"] = round(nb / sec_s / 1e9 / HBM_PEAK_GBS, 4)
            stage_report[s]["frac_of_copy"] = round(nb / sec_s / 1e9 / copy_gbs, 4)

    clock = None if args.no_clock else clock_pass(layer, dev, ms_per_step, args.steps)

    cold = None
    if not args.no_cold:
        flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)
        cold_ms = []
        for i in range(max(5, min(args.steps, 20))):
            flush.fill_(float(i))
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            layer.forward()
            b.record()
            torch.cuda.synchronize()
            cold_ms.append(a.elapsed_time(b))
        del flush
        cold = {"tokens_per_s_median": cfg.T / (pct(cold_ms, 50) * 1e-3),
                "ms_p10": round(pct(cold_ms, 10), 4), "ms_p50": round(pct(cold_ms, 50), 4),
                "ms_p90": round(pct(cold_ms, 90), 4), "steps": len(cold_ms),
                "flush": "512 MiB device write before each step, outside the events"}

    value = cfg.T / (ms_per_step * 1e-3)
    rec = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8-e4m3 expert GEMMs (OCP MX blocks of 32), bf16 elsewhere" if mx else cfg.dtype,
        "data": "synthetic (seeded; random-init weights)",
        "config": {"workload": f"{cfg.name}: T={cfg.T} h={cfg.h} E={cfg.E} K={cfg.K} f={cfg.f}"
                               f" {cfg.score}{'' if cfg.pre_softmax else '-renorm'}"
                               f" cap={cfg.capacity_factor} shared_f={cfg.shared_f}",
                   "tokens": cfg.T, "routed_rows": N, "dropped": cfg.T * cfg.K - N,
                   "parallelism": "single GPU, EP=1",
                   "gather_fc1": layer.gather, "shared_overlap": layer.overlap_shared,
                   "route_permute_fused": layer.fused, "fc2_combine_fused": layer.fused_combine,
                   "shared_folded": layer.fold_shared, "tile_queue": layer.queue is not None,
                   "expert_precision": args.precision,
                   "tokens_per_expert": load_stats(n)},
        "forward_ms": {"mean": sum(fwd) / len(fwd), "p10": pct(fwd, 10), "p50": pct(fwd, 50),
                       "p90": pct(fwd, 90)},
        "gemm_tflops": gemm_tflops,
        "gemm_frac_of_mfma_peak": gemm_tflops / peak_tf,
        "gemm_attainable_tflops": attainable_tf,
        "gemm_frac_of_attainable": gemm_tflops / attainable_tf,
        "stages": stage_report,
        "roofline": roof,
        "copy_GBs": copy_gbs,
        "clock": clock,
    }
    if cold:
        rec["cold"] = cold
    if not args.no_cpu_baseline:
        S = args.cpu_sample_tokens or DEFAULT_CPU_SAMPLE.get(cfg.name, 256)
        rec["cpu_baseline"] = cpu_baseline(cfg, inp, S)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
