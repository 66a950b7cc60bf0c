"""Plan-table tuner for one layer.

For each token count it times every GEMM plan the library builds (the stream
variant and each tiled tile height) on the production moe_forward, and keeps
the fastest one when it beats the built-in choice by a margin; otherwise the
built-in choice stays.  The result is installed with moe_set_plans and
returned as a list of plan dicts (t_max = the tuned token count: a call uses
the entry of the smallest tuned count >= its T).  This is the per-token-bucket
configuration tuning the pages describe ("[HIP] gfx950 A8W4 fused_moe configs
for DSv4.1 TP-sharded experts", Changes), measured on the call that serves.

  python -m quantized_moe_expert_softmax_amd.tune --workload v4pro_prefill --T 512 1024 4096
"""
from __future__ import annotations

import argparse
import json
import sys
import time

from . import (MOE_PLAN_DECODE, MOE_PLAN_FUSED, MOE_PLAN_STREAM, MOE_PLAN_TILED,
               alloc_workspace, moe_forward, moe_get_plan, moe_set_plans)


_NAMES = {MOE_PLAN_STREAM: "stream", MOE_PLAN_TILED: "tiled", MOE_PLAN_FUSED: "fused",
          MOE_PLAN_DECODE: "decode"}


def candidates(act: int, include_fused: bool = False):
    """Plans to time: the stream plan, the decode plan (token-major GEMM2 with
    the combine folded in) and every tiled tile height (both activation
    formats); the fused single launch only when the caller opts in (its
    bounded waits rely on having the device to itself)."""
    rows = (32, 64, 96, 128, 160, 192)
    fused = [(MOE_PLAN_FUSED, 16)] if include_fused else []
    return ([(MOE_PLAN_STREAM, 16), (MOE_PLAN_DECODE, 16)] + fused +
            [(MOE_PLAN_TILED, r) for r in rows])


def _time(layer, x, lgs, top_k, act, y, ws, steps, warmup):
    import torch
    for i in range(warmup):
        moe_forward(layer, x, lgs[i % len(lgs)], top_k, act, y=y, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moe_forward(layer, x, lgs[i % len(lgs)], top_k, act, y=y, ws=ws)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def tune(layer, inputs, top_k: int, act: int, steps: int = 10, warmup: int = 3,
         margin: float = 0.03, log=None, include_fused: bool = False):
    """inputs: {T: (x [T, H] bf16 device tensor, [logits [T, E] fp32 device tensors])}.
    Returns (table, report); the table is also installed on the layer.
    include_fused: also time MOE_PLAN_FUSED (opt-in; see moe.h)."""
    import torch
    table, report = [], {}
    for T in sorted(inputs):
        x, lgs = inputs[T]
        ws = alloc_workspace(layer, T, top_k, act)
        y = torch.empty((T, layer.H), dtype=torch.bfloat16, device=x.device)
        moe_set_plans(layer, [])
        builtin = moe_get_plan(layer, T, top_k, act)
        times = {}
        for variant, rows in candidates(act, include_fused):
            moe_set_plans(layer, [dict(act=act, top_k=top_k, t_max=T, variant=variant, rows=rows)])
            times[(variant, rows)] = _time(layer, x, lgs, top_k, act, y, ws, steps, warmup)
        best = min(times, key=times.get)
        base = times[(builtin["variant"], builtin["rows"])]
        pick = best if times[best] < (1.0 - margin) * base else (builtin["variant"], builtin["rows"])
        table.append(dict(act=act, top_k=top_k, t_max=T, variant=pick[0], rows=pick[1]))
        report[T] = {"builtin": [builtin["variant"], builtin["rows"]], "pick": list(pick),
                     "us": {"%s/%d" % (_NAMES[v], r): round(t * 1e6, 1)
                            for (v, r), t in times.items()}}
        if log:
            log("T=%d builtin=%s pick=%s %s" % (T, report[T]["builtin"], report[T]["pick"],
                                                report[T]["us"]))
    moe_set_plans(layer, table)
    return table, report


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--workload", default="v4pro_prefill")
    p.add_argument("--T", type=int, nargs="+", required=True)
    p.add_argument("--act", type=int, default=None)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--out", default=None, help="write the table as JSON")
    p.add_argument("--include-fused", action="store_true",
                   help="also time the fused single launch (needs the device to itself)")
    a = p.parse_args()
    import torch
    from . import moe_prepare_weights, synth
    wl = synth.WORKLOADS[a.workload]
    act = wl.act if a.act is None else a.act
    w = synth.device_weights(wl.H, wl.I, wl.E, wl.seed)
    layer = moe_prepare_weights(wl.E, wl.H, wl.I, *w)
    del w
    inputs = {}
    for T in a.T:
        x = torch.from_numpy(wl.x(T).view("int16")).cuda().view(torch.bfloat16)
        inputs[T] = (x, [torch.from_numpy(wl.logits(T, r)).cuda() for r in range(4)])
    table, report = tune(layer, inputs, wl.top_k, act, a.steps, a.warmup,
                         log=lambda s: print(s, file=sys.stderr, flush=True),
                         include_fused=a.include_fused)
    out = {"workload": a.workload, "act": act, "plans": table, "report": report}
    if a.out:
        with open(a.out, "w") as fh:
            json.dump(out, fh, indent=1)
    print(json.dumps(out))
    layer.close()


if __name__ == "__main__":
    main()
