"""The layer-level parity check of one device forward call against the oracle
(the steps are listed in tests/gpu_util.py).

Used by every GPU forward test: small shapes check every token, the full-size
configurations a sample of tokens and, through `check_sorted_rows`, whole
m-blocks of sorted rows.  The oracle's reference for the checked tokens is
composed from its per-step entry points (GEMM1 rows -> GEMM2 rows -> combine),
which reproduce its whole-layer evaluation bit for bit (pinned on the CPU), so
the GEMM1 work is shared with the A2 check; the oracle runs in a thread pool
(its C entry points keep no state and release the GIL)."""
import concurrent.futures
import os

import numpy as np

import oracle
import quantized_moe_expert_softmax_amd as moe
from tests.gpu_util import (A2_MISMATCH_TOL, ROUTE_ULP_TOL, a2_compare, a2_mismatch_ok, sum_bound, assert_output_close,
                            assert_rows_match, bf16_host_bits, ulp_diff, ws_a2_rows, ws_rows, ws_view)


def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return 4


def _parallel(fn, n, *arrays):
    """fn(*slices) over row chunks of the arrays, results concatenated per output."""
    if n == 0:
        return fn(*(a[:0] for a in arrays))
    nt = min(_threads(), n)
    bounds = np.linspace(0, n, nt + 1).astype(int)
    parts = [tuple(a[bounds[i]:bounds[i + 1]] for a in arrays) for i in range(nt)
             if bounds[i + 1] > bounds[i]]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(parts)) as ex:
        outs = list(ex.map(lambda p: fn(*p), parts))
    if isinstance(outs[0], tuple):
        return tuple(np.concatenate([o[i] for o in outs]) for i in range(len(outs[0])))
    return np.concatenate(outs)


class Experts:
    """Host copies of the experts a check needs, stacked into a compact set."""

    def __init__(self, weights_for):
        self.weights_for = weights_for
        self.slot = {}
        self.parts = []

    def slabs(self, experts):
        for e in np.unique(experts):
            e = int(e)
            if e not in self.slot:
                self.slot[e] = len(self.parts)
                self.parts.append(self.weights_for(e))
        self._stack = None
        return np.array([self.slot[int(e)] for e in experts], np.int32)

    def stacked(self):
        if getattr(self, "_stack", None) is None:
            self._stack = tuple(np.stack([p[i] for p in self.parts]) for i in range(4))
        return self._stack


def check_front(layer, ws, x, lg, k, act):
    """Step 1 checks on every token: ids, weights, counts, offsets, perm, slot,
    A1 codes and scales.  Returns (ids [T,k], weights [T,k], perm, slot)."""
    T, H = x.shape
    E = layer.E
    N = T * k
    offs = moe.moe_workspace_offsets(layer, T, k, act)
    rid, rw = oracle.route(lg, k)
    gid = ws_view(ws, offs, moe.MOE_WS_IDS, N * 4, np.int32)
    assert np.array_equal(gid, rid.reshape(-1)), "routing ids differ"
    gw = ws_view(ws, offs, moe.MOE_WS_WEIGHTS, N * 4, np.float32)
    assert ulp_diff(gw, rw.reshape(-1)).max() <= ROUTE_ULP_TOL, "routing weights differ"
    rc, ro, rp = oracle.sort(rid, E)
    assert np.array_equal(ws_view(ws, offs, moe.MOE_WS_COUNTS, E * 4, np.int32), rc)
    assert np.array_equal(ws_view(ws, offs, moe.MOE_WS_OFFSETS, (E + 1) * 4, np.int32), ro)
    perm = ws_view(ws, offs, moe.MOE_WS_PERM, N * 4, np.int32)
    assert np.array_equal(perm, rp), "expert permutation differs"
    slot = ws_view(ws, offs, moe.MOE_WS_SLOT, N * 4, np.int32)
    assert np.array_equal(slot[rp], np.arange(N)), "inverse permutation differs"
    a1row = H if act == 0 else H // 2
    xc, xs = _parallel(lambda xx: oracle.mx_quantize_bf16(xx, act), T, x)
    assert np.array_equal(ws_view(ws, offs, moe.MOE_WS_A1_CODES, T * a1row).reshape(T, a1row),
                          xc), "A1 codes differ"
    assert np.array_equal(ws_view(ws, offs, moe.MOE_WS_A1_SCALES, T * (H // 32)).reshape(T, -1),
                          xs), "A1 scales differ"
    return rid, gw.reshape(T, k), perm, slot, xc, xs


def _a2_rows(ws, offs, N, I, act, p):
    return ws_a2_rows(ws, offs, N, I, act, p)


def _staged_rows(ws, offs, T, k, H, combine, p):
    """The device's weighted rows at sorted positions p, decoded to FP32 (the
    values its combine sums), plus the raw transport bytes."""
    o = offs[moe.MOE_WS_ROWS]
    if combine == moe.MOE_COMBINE_FP32:
        raw = ws_rows(ws, o, 4 * H, p)
        return raw.view(np.float32), raw, None
    if combine == moe.MOE_COMBINE_BF16:
        raw = ws_rows(ws, o, 2 * H, p)
        return (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32), raw, None
    N = T * k
    codes = ws_rows(ws, o, H, p)
    scales = ws_rows(ws, o + N * H, H // 32, p)
    return oracle.mx_dequantize(codes, scales, H, 0), codes, scales


def swiglu_delta(gu, gu_abs, H, I, act):
    """Bound on |h_device - h_oracle| per A2 element, from the two GEMM1
    evaluations: each gate and up sum may differ by d = sum_bound(H, act) *
    sum|terms|; h = silu(g) * u then differs by at most |silu(g)| d_u +
    max|silu'| (|u| + d_u) d_g (|silu'| <= 1.1), plus a few FP32 roundings of
    the SwiGLU itself (the exponential, the division, the product)."""
    g, u = gu[:, :I].astype(np.float64), gu[:, I:].astype(np.float64)
    dg = sum_bound(H, act) * gu_abs[:, :I].astype(np.float64)
    du = sum_bound(H, act) * gu_abs[:, I:].astype(np.float64)
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    h = silu * u
    return np.abs(silu) * du + 1.1 * (np.abs(u) + du) * dg + 8 * 2.0 ** -24 * np.abs(h)


def _check_rows(layer, ws, offs, T, k, act, a, front, ex, combine, what):
    """Steps 2 and 3 on the assignments a (flat ids t*k + j): the device A2
    rows against the oracle's, and the device's staging rows against the
    oracle's GEMM2 of the device A2.  Returns the oracle's weighted rows (from
    its own A2), the device's decoded staging rows and the per-assignment
    flag of an A2 difference."""
    H, I = layer.H, layer.I
    ids, wts, perm, slot, xc, xs = front
    p = slot[a]
    sl = ex.slabs(ids.reshape(-1)[a])
    w13, w13s, w2, w2s = ex.stacked()
    tok = a // k
    amask = 0x7F if act == 0 else 0x77  # codes without their sign bits
    # oracle A2 from the exact A1 rows, with the gate / up sums the SwiGLU read
    r_c, r_s, gu = _parallel(
        lambda c, s, q: oracle.gemm1_rows(c, s, q, w13, w13s, act, want_gu=True), a.size,
        xc[tok], xs[tok], sl)
    # sum |a_k w_k| of each gate / up column: the same step on sign-stripped codes
    _, _, gu_abs = _parallel(
        lambda c, s, q: oracle.gemm1_rows(c & amask, s, q, w13 & 0x77, w13s, act, want_gu=True),
        a.size, xc[tok], xs[tok], sl)
    delta = swiglu_delta(gu, gu_abs, H, I, act)
    g_c, g_s = _a2_rows(ws, offs, T * k, I, act, p)
    mism, row_diff = a2_compare(g_c, g_s, r_c, r_s, act, what, delta)
    assert a2_mismatch_ok(mism, a.size * I), "%s: A2 mismatch fraction %.3g > %.0e" % (
        what, mism, A2_MISMATCH_TOL)
    wa = wts.reshape(-1)[a].astype(np.float32)
    gemm2 = lambda c, s, q, w: oracle.gemm2_rows(c, s, q, w, w2, w2s, act)
    r_rows = _parallel(gemm2, a.size, r_c, r_s, sl, wa)
    # GEMM2 of the device's A2: rows whose A2 equals the oracle's share r_rows
    dev_ref = r_rows.astype(np.float64)
    d = np.where(row_diff)[0]
    if d.size:
        dev_ref[d] = _parallel(gemm2, d.size, g_c[d], g_s[d], sl[d], wa[d])
    a_abs = _parallel(lambda c, s, q, w: oracle.gemm2_rows(c & amask, s, q, w, w2 & 0x77, w2s, act),
                      a.size, g_c, g_s, sl, np.abs(wa)).astype(np.float64)
    g_vals, g_raw, g_sc = _staged_rows(ws, offs, T, k, H, combine, p)
    if combine == moe.MOE_COMBINE_FP32:
        assert_rows_match(g_vals, dev_ref, a_abs, I, act, what)
    elif combine == moe.MOE_COMBINE_BF16:
        # one BF16 rounding of an FP32 row within the summation bound
        tol = sum_bound(I, act) * a_abs + 2.0 ** -8 * np.abs(dev_ref) + 1e-37
        bad = ~(np.abs(g_vals.astype(np.float64) - dev_ref) <= tol)
        assert not bad.any(), "%s: BF16 staging rows off at %d elements" % (what, int(bad.sum()))
    else:
        # the MXFP8 row of an FP32 row within the summation bound: a valid neighbour
        c8, s8 = oracle.mx_quantize(dev_ref.astype(np.float32), 0)
        a2_compare(g_raw, g_sc, c8, s8, 0, what + " FP8 staging", sum_bound(I, act) * a_abs)
    return r_rows, g_vals, row_diff, mism


def check_sorted_rows(layer, ws, x, k, act, weights_for, p, front, combine=moe.MOE_COMBINE_FP32,
                      what=""):
    """Steps 2 and 3 on the sorted rows p (e.g. whole m-blocks of one expert):
    every A2 and staging row a work item wrote there."""
    T = x.shape[0]
    offs = moe.moe_workspace_offsets(layer, T, k, act)
    perm = front[2]
    a = perm[np.asarray(p, np.int64)].astype(np.int64)
    _, _, row_diff, mism = _check_rows(layer, ws, offs, T, k, act, a, front, Experts(weights_for),
                                       combine, what)
    return {"rows": int(a.size), "a2_mism": mism, "rows_a2_differs": int(row_diff.sum())}


def check_tokens(layer, ws, y_bits, x, lg, k, act, weights_for, tokens=None,
                 combine=moe.MOE_COMBINE_FP32, front=None, what=""):
    """Steps 2-5 for the given tokens (all when None).  front: check_front's
    result (computed here when None).  Returns a dict of statistics."""
    T, H = x.shape
    if front is None:
        front = check_front(layer, ws, x, lg, k, act)
    tokens = np.arange(T) if tokens is None else np.unique(np.asarray(tokens, np.int64))
    offs = moe.moe_workspace_offsets(layer, T, k, act)
    a = (tokens[:, None] * k + np.arange(k)[None, :]).reshape(-1)   # assignments, slot order
    r_rows, g_vals, row_diff, mism = _check_rows(layer, ws, offs, T, k, act, a, front,
                                                 Experts(weights_for), combine, what)
    y_ref = oracle.combine(r_rows, k, combine)
    # the combine of the device's rows, exactly
    yb = np.asarray(y_bits)[tokens]
    y_dev = oracle.combine(g_vals.reshape(-1, H), k, moe.MOE_COMBINE_FP32)
    bad = np.where((y_dev != yb).any(axis=1))[0]
    if bad.size:
        r0 = bad[0]
        cols = np.where(y_dev[r0] != yb[r0])[0]
        rows_t = g_vals.reshape(-1, k, H)[r0]
        raise AssertionError(
            "%s: y is not the FP32 slot-order sum of the staging rows at tokens %s; token %d "
            "columns %s: device y %s, sum of its staging rows %s, the rows there %s" % (
                what, tokens[bad][:8].tolist(), tokens[r0], cols[:4].tolist(),
                [hex(v) for v in yb[r0][cols[:4]]], [hex(v) for v in y_dev[r0][cols[:4]]],
                rows_t[:, cols[:2]].T.tolist()))
    explained = row_diff.reshape(-1, k).any(axis=1)
    rel, row = assert_output_close(yb, y_ref, what, explained)
    return {"tokens": int(tokens.size), "rel": rel, "max_row": row, "a2_mism": mism,
            "rows_a2_differs": int(row_diff.sum())}


def forward_and_check(layer, x, lg, k, act, weights_for, combine=moe.MOE_COMBINE_FP32,
                      tokens=None, what=""):
    """One forward on a poisoned workspace, then the whole check."""
    import torch
    from tests.gpu_util import bf16_dev, dev
    T = x.shape[0]
    ws = moe.alloc_workspace(layer, T, k, act)
    ws.fill_(0xA5)  # any read of an unwritten byte shows up
    y = moe.moe_forward(layer, bf16_dev(x), dev(lg), k, act, ws=ws, combine=combine)
    torch.cuda.synchronize()
    yb = bf16_host_bits(y)
    st = check_tokens(layer, ws, yb, x, lg, k, act, weights_for, tokens, combine, what=what)
    return yb, ws, st
