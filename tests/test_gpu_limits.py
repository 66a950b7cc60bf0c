"""GPU parity at the largest sizes the interface takes: T = 2^20 tokens,
E = 1024 experts, top_k = 8 (8M assignments), with skewed router logits so
that a few experts hold far more rows than the mean.  H and I are kept small
(256, 128) so that the 2^20 x 1024 logits and the 8M staged rows fit easily.

The oracle routes 2^20 x 1024 logits in about a minute, so the exact
comparisons run on sampled tokens (routing ids and weights, the first-stage
codes and scales, the BF16 output); the grouping step is checked on every
assignment through properties that determine it uniquely: counts equal the
histogram of the ids, offsets their exclusive prefix sum, and perm lists
every assignment once, ordered by (expert, assignment index).
"""
import sys

import numpy as np
import pytest

import oracle
import quantized_moe_expert_softmax_amd as moe
from quantized_moe_expert_softmax_amd import synth
from tests.gpu_util import (ROUTE_ULP_TOL, assert_output_close, bf16_dev, bf16_host_bits, dev,
                            ulp_diff, ws_view)

pytestmark = pytest.mark.gpu

T, H, I, E, K = 1 << 20, 256, 128, 1024, 8
_inputs = {}


def _say(msg):
    print(msg)
    sys.stdout.flush()


def _data():
    if not _inputs:
        _say("limits: drawing T=%d H=%d E=%d inputs" % (T, H, E))
        _inputs["w"] = synth.all_weights(H, I, E, seed=29)
        _inputs["x"] = synth.tokens_bf16(T, H, seed=30)
        _inputs["lg"] = synth.router_logits(T, E, seed=31, skewed=True)
    return _inputs["w"], _inputs["x"], _inputs["lg"]


@pytest.mark.parametrize("act", [0, 1])
def test_max_sizes(act):
    import torch
    w, x, lg = _data()
    N = T * K
    layer = moe.moe_prepare_weights(E, H, I, *(dev(a) for a in w))
    try:
        ws = moe.alloc_workspace(layer, T, K, act)
        _say("limits: act=%d forward, workspace %.2f GB" % (act, ws.numel() / 1e9))
        y = moe.moe_forward(layer, bf16_dev(x), dev(lg), K, act, ws=ws)
        torch.cuda.synchronize()
        yb = bf16_host_bits(y)
        del y
        offs = moe.moe_workspace_offsets(layer, T, K, act)
        ids = ws_view(ws, offs, moe.MOE_WS_IDS, N * 4, np.int32)
        wts = ws_view(ws, offs, moe.MOE_WS_WEIGHTS, N * 4, np.float32).reshape(T, K)
        counts = ws_view(ws, offs, moe.MOE_WS_COUNTS, E * 4, np.int32)
        offsets = ws_view(ws, offs, moe.MOE_WS_OFFSETS, (E + 1) * 4, np.int32)
        perm = ws_view(ws, offs, moe.MOE_WS_PERM, N * 4, np.int32)
        slot = ws_view(ws, offs, moe.MOE_WS_SLOT, N * 4, np.int32)
        a1row = H if act == 0 else H // 2
        a1c = ws_view(ws, offs, moe.MOE_WS_A1_CODES, T * a1row).reshape(T, a1row)
        a1s = ws_view(ws, offs, moe.MOE_WS_A1_SCALES, T * (H // 32)).reshape(T, H // 32)
    finally:
        del ws
        layer.close()
        torch.cuda.empty_cache()

    # every routing result valid: k distinct experts per token, weights a distribution
    ids2 = ids.reshape(T, K)
    assert ids.min() >= 0 and ids.max() < E
    assert (np.diff(np.sort(ids2, axis=1), axis=1) > 0).all()
    assert (wts > 0).all() and np.abs(wts.sum(axis=1, dtype=np.float64) - 1).max() < 1e-5
    # the grouping, on all 8M assignments
    assert np.array_equal(counts, np.bincount(ids, minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(perm), np.arange(N, dtype=np.int32))
    key = ids[perm].astype(np.int64) * N + perm
    assert (np.diff(key) > 0).all()
    assert np.array_equal(slot[perm], np.arange(N, dtype=np.int32))
    _say("limits: act=%d largest expert %d rows (mean %.0f)" % (act, counts.max(), N / E))

    # sampled tokens: the ends, the first and last rows of the largest and the
    # smallest non-empty expert groups, and random ones
    hot = int(np.argmax(counts))
    nz = np.where(counts > 0)[0]
    cold = int(nz[np.argmin(counts[nz])])
    ends = [perm[offsets[e]] // K for e in (hot, cold)] + [perm[offsets[e + 1] - 1] // K
                                                           for e in (hot, cold)]
    rows = [0, T - 1] + [int(t) for t in ends]
    rows += list(np.random.default_rng(act).integers(0, T, 250))
    rows = np.array(sorted(set(rows)))

    rid, rw = oracle.route(lg[rows], K)
    assert np.array_equal(ids2[rows], rid)
    assert ulp_diff(wts[rows], rw).max() <= ROUTE_ULP_TOL
    xc, xs = oracle.mx_quantize_bf16(x[rows], act)
    assert np.array_equal(a1c[rows], xc)
    assert np.array_equal(a1s[rows], xs)
    ref = oracle.forward(x[rows], lg[rows], *w, K, act)
    rel, row = assert_output_close(yb[rows], ref, "limits act=%d rows=%d" % (act, len(rows)))
    _say("limits: act=%d rows=%d rel=%.2e max_row=%.2e" % (act, len(rows), rel, row))
