"""Benchmark of the MI355X MoE layer: one JSON line on stdout.

A step is one moe_forward call (routing, expert sort, activation quant,
GEMM1 + SwiGLU + requant, GEMM2 + weighted FP32 combine, BF16 finalize) on
a batch of T synthetic tokens already resident in HBM (--combine picks the
transport of the weighted GEMM2 rows: fp32 by default, or bf16 / fp8).

The headline (`value`, `ms_per_step`, `roofline`, `cpu_baseline`) is the
largest configuration that one GPU holds: the DeepSeek-V4-Pro-shaped expert
layer (H=7168, I=3072, E=384, top_k=6, all experts resident) with MXFP4
activations (A4W4) at T=16384 tokens.  `sweep` then times every
configuration point of the five workloads -- V4-Pro decode T=1..64 and prefill
T=512..8192 (A8W4, uniform and skewed routing), A4W4 T=1..16384, and the four
V4.1-Flash TP-shard shapes at 16 token counts (A8W4) -- each with its GEMM1
roofline entry (--sweep workload: only the headline workload's points;
--sweep none: none).

Between steps the router logits rotate over 8 pre-drawn sets, so successive
calls touch different experts.  Each token count is timed in passes over the
same calls: eager launches (this is `value` and `ms_per_step`), HIP-graph
replay (one graph captured per logits set; decode sizes only in the sweep),
eager launches with HIP events the library records around every kernel on
the launch stream (per-kernel times; an event record costs a few
microseconds, so this pass is not used for the step time), and each call on
its own after a 512 MiB device read that evicts the last-level cache
(`us_per_call_flushed`: p10, median, p90).  The roofline entry is for the
dominant kernel (GEMM1), against whichever ceiling needs the longer time: HBM
bandwidth with its algorithmic bytes per launch (touched experts x gate/up
weight bytes, codes + E8M0 scales, + the quantised token rows read + the
requantised rows written), or the dense MFMA peak of its operand formats
with its algorithmic FLOPs (4 T top_k H I).  layer_mfma_frac is the whole
layer's 6 T top_k H I FLOPs per step against that peak.

combine_transports: the headline workload again with the weighted GEMM2 rows carried to the
FP32 top-k sum as BF16 or MXFP8 rows (one more rounding per term; not the value).

cpu_baseline: the CPU oracle (test infrastructure, single-threaded C) timed
on a bounded sample of the headline workload: routing, sort and quantisation
of all T tokens plus the expert FFN of as many sampled tokens as fit about
15 s; cpu_baseline_all_cores: the same oracle over token partitions, one
thread per host core (up to 16), on 2 sampled tokens per thread.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--T T]
                  [--sweep all|workload|none] [--no-transports] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
# the headline: the largest configuration one GPU holds (7168 x 3072, 384 x 6, A4W4)
HEADLINE = ("v4pro_a4w4", 16384)
# the sweep's workloads, grouped so that workloads sharing an expert set follow each other
SWEEP = ("v4pro_decode", "v4pro_prefill", "v4pro_prefill_skewed", "v4pro_a4w4",
         "v41flash_i640_e384", "v41flash_i1152_e384", "v41flash_i640_e128", "v41flash_i1152_e128")
# MI355X dense matrix peaks, TFLOP/s: MXFP8 x MXFP4 runs at the FP8 rate, MXFP4 x MXFP4 at FP4's
MFMA_PEAK_TFLOPS = {0: 5000.0, 1: 10100.0}
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "quantized_moe_expert_softmax_amd", "csrc")
# sources that decide GEMM1's memory traffic, by plan variant: its kernel, the shared GEMM code
# and the weight layout (the traffic lines in profiles/ are keyed by the hash of these)
GEMM_SOURCES = {
    0: ("gemm_common.h", "gemm_stream.hip", "prepack.hip", "mx_device.h", "internal.h"),
    1: ("gemm_common.h", "gemm_tiled.hip", "prepack.hip", "mx_device.h", "internal.h"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=HEADLINE[0])
    p.add_argument("--T", type=int, default=None,
                   help="headline token count (default: %d for the default workload, else the "
                        "workload's largest)" % HEADLINE[1])
    p.add_argument("--act", type=int, default=None, help="0 = MXFP8 (A8W4), 1 = MXFP4 (A4W4)")
    p.add_argument("--sweep", default="all", choices=("all", "workload", "none"),
                   help="configuration points timed after the headline")
    p.add_argument("--no-sweep", action="store_true", help="same as --sweep none")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-transports", action="store_true",
                   help="skip timing the headline with the BF16 and MXFP8 row transports")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="about how long the single-thread oracle FFN sample runs")
    p.add_argument("--prequant", action="store_true",
                   help="feed MX-quantised activations (moe_forward_prequant)")
    p.add_argument("--combine", default="fp32", choices=("fp32", "bf16", "fp8"),
                   help="transport of the weighted GEMM2 rows into the FP32 top-k sum")
    p.add_argument("--plans", default=None, metavar="JSON",
                   help="install a plan table written by quantized_moe_expert_softmax_amd.tune")
    p.add_argument("--copy-calibrate", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB three times (the "
                        "known-size kernel that scales the HBM byte counters)")
    return p.parse_args()


def copy_calibration(torch, mib, reps=3):
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "reps": reps}), flush=True)


def gemm_source_hash(variant=1):
    """Hash of the sources of GEMM1's plan variant (1 tiled; 0 stream, 2 fused and 3 decode run
    the stream GEMM1)."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES[1 if variant == 1 else 0]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def build_info(torch):
    """What produced the numbers: a hash of the library's HIP sources (the GPU
    box's copy of the tree has no git metadata), the GEMM-source hash the
    traffic figures are keyed by, and the torch / HIP runtime and device."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + fh.read())
    return {"csrc_sha256": h.hexdigest()[:16],
            "gemm_source_hash": {"stream": gemm_source_hash(0), "tiled": gemm_source_hash(1)},
            "torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
            "device": torch.cuda.get_device_name(0)}


def measured_traffic(workload, T, act, plan):
    """HBM bytes per GEMM1 launch from the committed rocprofv3 --pmc summary
    (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, each scaled by what the
    same counter reads for a plain copy of known size), or (None, None) when
    there is none for this workload and plan or the sources of that plan's
    GEMM1 changed since the counters were taken."""
    import glob
    src = gemm_source_hash(plan[0])
    want_plan = "%d:%d" % (plan[0], plan[1])
    for path in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        with open(path) as fh:
            for line in fh:
                line = line.strip()
                if not line.startswith("traffic:"):
                    continue
                kv = dict(t.split("=", 1) for t in line[len("traffic:"):].split())
                if (kv.get("kernel") == "gemm1" and kv.get("workload") == workload
                        and int(kv.get("T", -1)) == T and int(kv.get("act", -1)) == act
                        and kv.get("plan") == want_plan and kv.get("source") == src):
                    b = (float(kv["fetch_kib"]) * float(kv["fetch_scale"]) +
                         float(kv["write_kib"]) * float(kv["write_scale"])) * 1024.0
                    return b, os.path.relpath(path, ROOT)
    return None, None


def touched_experts(moe, layer, ws, T, top_k, act):
    import numpy as np
    offs = moe.moe_workspace_offsets(layer, T, top_k, act)
    o = offs[moe.MOE_WS_COUNTS]
    counts = ws[o:o + 4 * layer.E].cpu().numpy().view(np.int32)
    return int((counts > 0).sum())


def gemm1_bytes(layer, U, T, top_k, act):
    H, I = layer.H, layer.I
    a1 = (H if act == 0 else H // 2) + H // 32
    a2 = (I if act == 0 else I // 2) + I // 32
    return U * (I * H + 2 * I * H // 32) + T * a1 + T * top_k * a2


def gemm1_flops(layer, T, top_k):
    # every assignment row times the expert's 2I gate/up rows over K = H
    return 2.0 * T * top_k * layer.H * 2 * layer.I


def roofline_entry(layer, U, T, top_k, act, g1_ms):
    """Roofline of GEMM1 (the dominant kernel): its algorithmic bytes against
    HBM and its algorithmic FLOPs against the dense MFMA peak of its operand
    formats; `bound` is the ceiling that needs the longer time, `achieved` the
    launch's rate against it (the other ceiling's fraction is kept beside)."""
    b = gemm1_bytes(layer, U, T, top_k, act)
    f = gemm1_flops(layer, T, top_k)
    t = g1_ms * 1e-3
    gbs, tfs = b / t / 1e9, f / t / 1e12
    pk = MFMA_PEAK_TFLOPS[act]
    hbm_bound = b / (HBM_PEAK_GBS * 1e9) >= f / (pk * 1e12)
    e = {"bound": "hbm" if hbm_bound else "mfma", "kernel": "gemm1",
         "achieved": round(gbs if hbm_bound else tfs, 1),
         "peak": HBM_PEAK_GBS if hbm_bound else pk,
         "unit": "GB/s" if hbm_bound else "TFLOP/s",
         "frac": round((gbs / HBM_PEAK_GBS) if hbm_bound else (tfs / pk), 4)}
    if hbm_bound:
        e["mfma_frac"] = round(tfs / pk, 4)
    else:
        e["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    return e, b


def layer_weight_bytes(layer, U):
    H, I = layer.H, layer.I
    return U * (I * H + 2 * I * H // 32 + H * I // 2 + H * I // 32)


COMBINES = {"fp32": 0, "bf16": 1, "fp8": 2}


def time_T(moe, torch, layer, wl, T, act, steps, warmup, combine=0, prequant=False,
           graphs=True):
    """Passes over the same `steps` calls (logits rotating over 8 sets): eager
    launches and (graphs) HIP-graph replays (one graph captured per logits
    set), both with no events; an eager pass with per-kernel HIP events; and
    the calls one by one after a cache-evicting read.  prequant: the calls
    take x already MX-quantised (moe_forward_prequant; the codes are made
    once, outside the timed region)."""
    x = torch.from_numpy(wl.x(T).view("int16")).cuda().view(torch.bfloat16)
    lgs = [torch.from_numpy(wl.logits(T, r)).cuda() for r in range(8)]
    ws = moe.alloc_workspace(layer, T, wl.top_k, act)
    y = torch.empty((T, wl.H), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    if prequant:
        xc, xs = moe.moe_quant_act(x, act)

    def call(lg, s=None):
        if prequant:
            moe.moe_forward_prequant(layer, xc, xs, lg, wl.top_k, act, y=y, ws=ws, stream=s,
                                     combine=combine)
        else:
            moe.moe_forward(layer, x, lg, wl.top_k, act, y=y, ws=ws, stream=s, combine=combine)

    Us = []
    for r in range(8):
        call(lgs[r])
        torch.cuda.synchronize()
        Us.append(touched_experts(moe, layer, ws, T, wl.top_k, act))
    for i in range(warmup):
        call(lgs[i % 8], stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(lgs[i % 8], stream)
    torch.cuda.synchronize()
    dt_eager = time.perf_counter() - t0

    dt_graph = None
    if graphs:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        gl = []
        for r in range(8):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                call(lgs[r], cap)
            gl.append(g)
        torch.cuda.synchronize()
        for i in range(warmup):
            gl[i % 8].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            gl[i % 8].replay()
        torch.cuda.synchronize()
        dt_graph = time.perf_counter() - t0
        del gl

    moe.moe_profile_enable(layer, True, steps)
    for i in range(steps):
        call(lgs[i % 8], stream)
    torch.cuda.synchronize()
    kern, ncalls = moe.moe_profile_read(layer)
    moe.moe_profile_enable(layer, False)
    U = sum(Us[i % 8] for i in range(ncalls)) / max(ncalls, 1)

    # per-call times with a cold last-level cache: before each call (outside its
    # events) a 512 MiB device read evicts the 256 MB MALL (a read leaves no dirty
    # lines to be written back during the call); HIP events on the launch stream
    # bracket the call alone
    flush = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        flush.sum()
        ev[i][0].record(stream)
        call(lgs[i % 8], stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_call = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    del flush

    def pct(q):
        return round(per_call[min(len(per_call) - 1, int(q * len(per_call)))], 2)
    flushed = {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9)}
    plan = moe.moe_get_plan(layer, T, wl.top_k, act)
    return {"dt_eager": dt_eager, "dt_graph": dt_graph, "kern": kern, "ncalls": ncalls, "U": U,
            "flushed": flushed, "plan": [plan["variant"], plan["rows"]], "steps": steps}


def point_entry(layer, wl, T, act, r):
    """The sweep entry of one configuration point."""
    nc = max(r["ncalls"], 1)
    g1 = r["kern"]["gemm1"] / nc
    d = r["dt_eager"] / r["steps"]
    roof, _ = roofline_entry(layer, r["U"], T, wl.top_k, act, g1)
    e = {
        "us_per_call": round(d * 1e6, 2),
        "us_per_call_flushed": r["flushed"],
        "tokens_per_s": round(T / d, 1),
        "touched_experts": round(r["U"], 1),
        "layer_weight_GBps": round(layer_weight_bytes(layer, r["U"]) / d / 1e9, 1),
        "layer_mfma_frac": round(6.0 * T * wl.top_k * wl.H * wl.I / d / 1e12 /
                                 MFMA_PEAK_TFLOPS[act], 4),
        "gemm1_us": round(g1 * 1e3, 2),
        "roofline_gemm1": {k: roof[k] for k in ("bound", "achieved", "unit", "frac")},
        "plan": r["plan"],
        "kernels_us": {k: round(v / nc * 1e3, 2) for k, v in r["kern"].items()},
    }
    if r["dt_graph"] is not None:
        e["us_per_call_graph"] = round(r["dt_graph"] * 1e6 / r["steps"], 2)
    return e


def cpu_baseline(moe, torch, layer_dev_weights, wl, T, act, seconds):
    """Oracle on a bounded sample: route/sort/quant of all T tokens + the FFN of
    as many evenly spaced tokens as fit about `seconds` (at least 2)."""
    import numpy as np
    import oracle
    w13, w13s, w2, w2s = layer_dev_weights
    x = wl.x(T)
    lg = wl.logits(T, 0)
    t0 = time.perf_counter()
    ids, _ = oracle.route(lg, wl.top_k)
    oracle.sort(ids, wl.E)
    oracle.mx_quantize_bf16(x, act)
    t_front = time.perf_counter() - t0
    cache = {}

    def wfor(e):
        if e not in cache:
            cache[e] = tuple(a[e].cpu().numpy() for a in (w13, w13s, w2, w2s))
        return cache[e]

    def fetch(rows):  # the sampled tokens' experts, outside the timed part
        sel, _ = oracle.route(lg[rows], wl.top_k)
        for e in set(int(v) for v in sel.reshape(-1)):
            wfor(e)
    # one token first, to size the sample
    first = np.array([T // 2], np.int64)
    fetch(first)
    t0 = time.perf_counter()
    oracle.forward_rows(x, lg, first, wfor, wl.top_k, act)
    t_one = time.perf_counter() - t0
    n = int(max(2, min(T, 64, seconds / max(t_one, 1e-6))))
    sample = np.unique(np.linspace(0, T - 1, num=n).astype(np.int64))
    fetch(sample)
    t0 = time.perf_counter()
    oracle.forward_rows(x, lg, sample, wfor, wl.top_k, act)
    t_ffn = time.perf_counter() - t0
    per_token = t_front / T + t_ffn / len(sample)
    return {
        "value": 1.0 / per_token,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "front_s_per_token": t_front / T,
        "sample": ("route+sort+quant of all %d tokens (%.2f s) + expert FFN of %d evenly spaced "
                   "tokens (%.2f s); value = 1 / (front time per token + FFN time per sampled "
                   "token)" % (T, t_front, len(sample), t_ffn)),
    }


def cpu_baseline_all_cores(torch, layer_dev_weights, wl, T, act, single):
    """The same oracle over token partitions, one thread per host core (its C
    entry points keep no state between calls; ctypes releases the GIL), on a
    bounded sample of 2 tokens per thread.  `single` is the single-thread
    result, whose routing/sort/quant time per token is reused."""
    import concurrent.futures
    import platform
    import numpy as np
    import oracle
    w13, w13s, w2, w2s = layer_dev_weights
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    x = wl.x(T)
    lg = wl.logits(T, 0)
    n = min(T, 2 * cores)
    sample = np.unique(np.linspace(0, T - 1, num=n).astype(np.int64))
    cache = {}
    sel, _ = oracle.route(lg[sample], wl.top_k)
    for e in sorted(set(int(v) for v in sel.reshape(-1))):
        cache[e] = tuple(a[e].cpu().numpy() for a in (w13, w13s, w2, w2s))
    parts = [p for p in np.array_split(sample, cores) if len(p)]
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(parts)) as ex:
        list(ex.map(lambda part: oracle.forward_rows(x, lg, part, cache.__getitem__, wl.top_k, act),
                    parts))
    t_ffn = time.perf_counter() - t0
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    per_token = single["front_s_per_token"] + t_ffn / len(sample)
    return {
        "value": 1.0 / per_token,
        "unit": "tokens/s",
        "cores": len(parts),
        "kind": "oracle",
        "sample": ("expert FFN of %d sampled tokens in %d threads (%.2f s wall) + the single-thread "
                   "route+sort+quant time per token; host %s" % (len(sample), len(parts), t_ffn,
                                                                 model)),
    }


def sweep_points(args, wl_head, T_head, act_override):
    """(workload, T) of every configuration point to time after the headline."""
    from quantized_moe_expert_softmax_amd import synth
    mode = "none" if args.no_sweep else args.sweep
    if mode == "none":
        return []
    names = SWEEP if mode == "all" else (wl_head.name,)
    pts = []
    for n in names:
        for t in synth.WORKLOADS[n].Ts:
            if (n, t) != (wl_head.name, T_head):
                pts.append((n, t))
    return pts


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (a layer's "
              "experts all fit one MI355X); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibrate:
        copy_calibration(torch, args.copy_calibrate)
        return
    import quantized_moe_expert_softmax_amd as moe
    from quantized_moe_expert_softmax_amd import synth

    wl = synth.WORKLOADS[args.workload]
    act = wl.act if args.act is None else args.act
    T = args.T or (HEADLINE[1] if wl.name == HEADLINE[0] else max(wl.Ts))
    torch.cuda.set_device(0)
    plans = None
    if args.plans:
        with open(args.plans) as fh:
            plans = json.load(fh)["plans"]
    layers = {}

    def layer_for(w):
        """The layer of workload w (one expert set resident at a time)."""
        key = (w.H, w.I, w.E, w.seed)
        if key not in layers:
            for k in list(layers):
                layers.pop(k)[1].close()
            torch.cuda.empty_cache()
            log("building %s weights on the device (H=%d I=%d E=%d)" % (w.name, w.H, w.I, w.E))
            t0 = time.perf_counter()
            wd = synth.device_weights(w.H, w.I, w.E, w.seed)
            lay = moe.moe_prepare_weights(w.E, w.H, w.I, *wd)
            if plans:
                moe.moe_set_plans(lay, plans)
            torch.cuda.synchronize()
            log("weights ready in %.1f s" % (time.perf_counter() - t0))
            layers[key] = (wd, lay)
        return layers[key]

    combine = COMBINES[args.combine]
    w, layer = layer_for(wl)
    layers.clear()  # the headline's expert set is released once the sweep moves on
    layers[(wl.H, wl.I, wl.E, wl.seed)] = (None, layer)
    r = time_T(moe, torch, layer, wl, T, act, args.steps, args.warmup, combine, args.prequant)
    ms_step = r["dt_eager"] * 1e3 / args.steps
    value = T * args.steps / r["dt_eager"]
    ncalls = max(r["ncalls"], 1)
    g1_ms = r["kern"]["gemm1"] / ncalls
    roof, g1_bytes = roofline_entry(layer, r["U"], T, wl.top_k, act, g1_ms)
    kernels_us = {k: round(v / ncalls * 1e3, 2) for k, v in r["kern"].items()}
    log("T=%d: %.1f us/step (eager), %.1f graph, %.0f tokens/s, gemm1 %.1f us, roofline %s, "
        "kernels %s" % (T, ms_step * 1e3, r["dt_graph"] * 1e6 / args.steps, value, g1_ms * 1e3,
                        roof, kernels_us))

    head_entry = point_entry(layer, wl, T, act, r)

    # the headline workload with the other transports of the weighted GEMM2 rows into
    # the FP32 top-k sum (one more rounding per term: an alternative, not the value)
    transports = {}
    if combine == 0 and not args.no_transports:
        for name, c in (("bf16", 1), ("fp8", 2)):
            rt = time_T(moe, torch, layer, wl, T, act, max(5, args.steps // 2), args.warmup, c,
                        args.prequant, graphs=False)
            d = rt["dt_eager"] / rt["steps"]
            nc = max(rt["ncalls"], 1)
            transports[name] = {"us_per_call": round(d * 1e6, 2), "tokens_per_s": round(T / d, 1),
                                "gemm2_us": round(rt["kern"]["gemm2"] / nc * 1e3, 2),
                                "combine_us": round(rt["kern"]["combine"] / nc * 1e3, 2)}
            log("transport %s: %s" % (name, transports[name]))

    cpu = cpu_all = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        cpu = cpu_baseline(moe, torch, w, wl, T, act, args.cpu_seconds)
        cpu_all = cpu_baseline_all_cores(torch, w, wl, T, act, cpu)
        cpu.pop("front_s_per_token")
    del w  # the layer keeps its packed copy
    traffic, traffic_src = measured_traffic(wl.name, T, act, r["plan"])

    sweep = {}
    for name, t in sweep_points(args, wl, T, args.act):
        sw = synth.WORKLOADS[name]
        sact = sw.act if args.act is None or name != wl.name else act
        _, lay = layer_for(sw)
        decode = t <= 64
        rr = time_T(moe, torch, lay, sw, t, sact, args.steps if decode else max(5, args.steps // 2),
                    args.warmup, combine, args.prequant, graphs=decode)
        sweep.setdefault(name, {})[str(t)] = point_entry(lay, sw, t, sact, rr)
        log("%s T=%d: %s" % (name, t, sweep[name][str(t)]))
    sweep.setdefault(wl.name, {})[str(T)] = head_entry

    dtype = "mxfp8xmxfp4" if act == 0 else "mxfp4xmxfp4"
    line = {
        "metric": "MoE layer tokens/s at T=%d (%s) on one MI355X; us/call vs T in sweep"
                  % (T, "A8W4" if act == 0 else "A4W4"),
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_graph": round(r["dt_graph"] * 1e3 / args.steps, 4),
        # per-call HIP-event times after a 512 MiB cache-evicting read (microseconds)
        "us_per_call_flushed": r["flushed"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": "%s H=%d I=%d E=%d top_k=%d T=%d %s%s" % (
            wl.name, wl.H, wl.I, wl.E, wl.top_k, T, "A8W4" if act == 0 else "A4W4",
            ("" if combine == 0 else " combine=" + args.combine) +
            (" prequant" if args.prequant else "")),
            "global_batch": T, "parallelism": "single-gpu"},
        "roofline": dict(roof, **{
            "traffic": None if traffic is None else int(traffic),
            "traffic_source": traffic_src, "bytes_per_launch": int(g1_bytes),
            "flops_per_launch": gemm1_flops(layer, T, wl.top_k),
            "avg_launch_us": round(g1_ms * 1e3, 2)}),
        # the whole layer's 6 T k H I algorithmic FLOPs per step against the dense MFMA peak
        "layer_mfma_frac": head_entry["layer_mfma_frac"],
        "plan": r["plan"],
        "kernels_us": kernels_us,
        # the same workload with the weighted GEMM2 rows carried to the FP32 sum as BF16 or
        # MXFP8 (the pages' combine payloads) instead of FP32
        "combine_transports": transports or None,
        "sweep": sweep,
        "cpu_baseline": cpu,
        # the same oracle over token partitions on all host cores (a baseline, not the target)
        "cpu_baseline_all_cores": cpu_all,
        "build": build_info(torch),
    }
    print(json.dumps(line), flush=True)
    for _, lay in layers.values():
        lay.close()


if __name__ == "__main__":
    main()
