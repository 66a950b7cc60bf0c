"""GPU parity at every configuration point of the benchmarked workloads, at
full size, in the launch configuration the benchmark times (one moe_forward
call over the whole batch, the built-in plan).

On every row: routing ids and weights, counts / offsets, the expert
permutation and the first-stage codes and scales against the oracle
(bit-exact; weights within 4 ulp).  Then the staged checks of
tests/layer_check.py (A2 a valid neighbour of the oracle's, GEMM2 of the
device A2 and the combine exact, y within tolerance) on

* sampled tokens: the first and last token, the first and last token routed
  to the most loaded expert, a token of the least loaded non-empty expert and
  a few random ones (every one of their top_k assignments);
* sorted rows of the most loaded expert: the first and last row of each of
  its m-blocks (work items) and every row of its last, partial m-block.

The oracle runs on the host's cores (about a second per token at 7168 x 3072
single-threaded).
"""
import numpy as np
import pytest

import quantized_moe_expert_softmax_amd as moe
from quantized_moe_expert_softmax_amd import synth
from tests.gpu_util import bf16_dev, bf16_host_bits, dev
from tests.layer_check import check_front, check_sorted_rows, check_tokens

pytestmark = pytest.mark.gpu

_cache = {}


def _shape(wl):
    key = (wl.H, wl.I, wl.E, wl.seed)
    if key not in _cache:
        import torch
        for k in list(_cache):  # keep one expert set resident at a time
            _cache.pop(k)[1].close()
        torch.cuda.empty_cache()
        w = synth.device_weights(wl.H, wl.I, wl.E, wl.seed)
        layer = moe.moe_prepare_weights(wl.E, wl.H, wl.I, *w)
        _cache[key] = (w, layer)
    return _cache[key]


def sample_rows(ids, E, n_random=2, seed=0):
    T = ids.shape[0]
    counts = np.bincount(ids.reshape(-1), minlength=E)
    hot = int(np.argmax(counts))
    nz = np.where(counts > 0)[0]
    cold = int(nz[np.argmin(counts[nz])])
    hot_tokens = np.where((ids == hot).any(axis=1))[0]
    cold_tokens = np.where((ids == cold).any(axis=1))[0]
    rows = [0, T - 1, hot_tokens[0], hot_tokens[-1], cold_tokens[0]]
    rows += list(np.random.default_rng(seed).integers(0, T, n_random))
    return sorted(set(int(r) for r in rows))


def mblock_rows(offsets, e, bm):
    """Sorted rows of expert e to check: first and last of each bm-row m-block,
    and all rows of the last m-block when it is partial."""
    lo, hi = int(offsets[e]), int(offsets[e + 1])
    rows = set()
    for b0 in range(lo, hi, bm):
        b1 = min(b0 + bm, hi)
        rows.update((b0, b1 - 1))
        if b1 - b0 < bm:
            rows.update(range(b0, b1))
    return np.array(sorted(rows), np.int64)


def run_case(name, T, act=None, n_random=2, combine=moe.MOE_COMBINE_FP32):
    import torch
    wl = synth.WORKLOADS[name]
    act = wl.act if act is None else act
    w, layer = _shape(wl)
    x = wl.x(T)
    lg = wl.logits(T)
    ws = moe.alloc_workspace(layer, T, wl.top_k, act)
    y = moe.moe_forward(layer, bf16_dev(x), dev(lg), wl.top_k, act, ws=ws, combine=combine)
    torch.cuda.synchronize()
    yb = bf16_host_bits(y)
    what = "%s T=%d act=%d combine=%d" % (name, T, act, combine)
    front = check_front(layer, ws, x, lg, wl.top_k, act)
    wcache = {}

    def wfor(e):
        if e not in wcache:
            wcache[e] = tuple(a[e].cpu().numpy() for a in w)
        return wcache[e]
    tokens = sample_rows(front[0], wl.E, n_random=n_random, seed=T)
    st = check_tokens(layer, ws, yb, x, lg, wl.top_k, act, wfor, tokens, combine, front, what)
    counts = np.bincount(front[0].reshape(-1), minlength=wl.E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    plan = moe.moe_get_plan(layer, T, wl.top_k, act)
    rows = mblock_rows(offsets, int(np.argmax(counts)), plan["rows"])
    sr = check_sorted_rows(layer, ws, x, wl.top_k, act, wfor, rows, front, combine,
                           what + " hot expert m-blocks")
    print("%s plan=%s tokens=%d rel=%.2e max_row=%.2e a2_mism=%.1e | hot-expert rows=%d "
          "a2_mism=%.1e" % (what, (plan["variant"], plan["rows"]), st["tokens"], st["rel"],
                            st["max_row"], st["a2_mism"], sr["rows"], sr["a2_mism"]))


def _points(name):
    return [(name, T) for T in synth.WORKLOADS[name].Ts]


# every configuration point: V4-Pro-shaped A8W4 decode and prefill (uniform and
# skewed routing), A4W4, and the V4.1-Flash TP-sharded shapes
POINTS = (_points("v4pro_decode") + _points("v4pro_prefill") + _points("v4pro_prefill_skewed") +
          _points("v4pro_a4w4") + _points("v41flash_i640_e384") + _points("v41flash_i1152_e384") +
          _points("v41flash_i640_e128") + _points("v41flash_i1152_e128"))


@pytest.mark.parametrize("name,T", POINTS)
def test_config_point(name, T):
    run_case(name, T)


@pytest.mark.parametrize("combine", [moe.MOE_COMBINE_BF16, moe.MOE_COMBINE_FP8])
@pytest.mark.parametrize("name,T", [("v4pro_decode", 8), ("v4pro_prefill", 8192),
                                    ("v41flash_i640_e384", 32768)])
def test_combine_transports(name, T, combine):
    run_case(name, T, n_random=1, combine=combine)
