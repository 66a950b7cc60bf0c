"""Shared helpers of the GPU parity tests (device transfer, comparisons).

The layer's parity check, in the order the layer computes:

1. routing ids, counts / offsets, the expert permutation and the first-stage
   codes and scales: bit-exact against the oracle;
2. the requantised SwiGLU activations (A2): where floating point decides a
   code (the device's FP32 GEMM1 accumulation order and SwiGLU differ from
   the oracle's by a few ulps, which can move h across a rounding boundary
   or a block maximum across a power of two), several codes are correct.
   Every device block must be a valid neighbour of the oracle's: scale
   exponents at most one apart, every element within one grid step (at the
   larger of the two scales) of the oracle's value; and at most 1e-3 of the
   elements (or one block's 32, in a smaller comparison) may differ at all;
3. GEMM2 from the device's own A2: each weighted FP32 staging row equals
   the oracle's GEMM2 of that A2 row times its routing weight, element by
   element, within the FP32 summation bound 2 K 2^-24 sum|a_i w_i|;
4. the combine: y[t] is exactly the oracle's FP32 slot-order sum of the
   device's staging rows of token t, rounded to BF16;
5. y against the oracle's whole layer: relative L2 <= 1e-2 over the compared
   rows, and every row within 3e-2 unless its assignments' A2 differ from the
   oracle's (then 2-4 have shown that the row is the layer evaluated on a
   valid A2).
"""
import numpy as np

from tests import mxref

# Final-output criteria (relative L2 norm over the compared rows and the
# largest per-row relative L2 error).
REL_L2_TOL = 1e-2
ROW_REL_TOL = 3e-2
# Routing weights: the device evaluates exp(l_j - l_0) / sum over the picks in
# double and rounds once to FP32, the oracle the full softmax over the picks;
# the two roundings may land a few ulps apart.
ROUTE_ULP_TOL = 4
# Largest fraction of A2 elements whose value may differ from the oracle's (a
# comparison of fewer than 32 / 1e-3 elements may hold one differing block).
A2_MISMATCH_TOL = 1e-3


def a2_mismatch_ok(frac, n_elements):
    return frac * n_elements <= max(A2_MISMATCH_TOL * n_elements, 32)


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits):
    import torch
    return dev(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)


def host(t):
    return t.detach().cpu().numpy()


def bf16_host_bits(t):
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def row_errors(y_bits, ref_bits):
    """Relative L2 over all rows and the relative L2 error of each row."""
    y = bf16_to_f64(y_bits)
    r = bf16_to_f64(ref_bits)
    rel = np.linalg.norm(y - r) / max(np.linalg.norm(r), 1e-30)
    rown = np.linalg.norm(r, axis=1)
    rowe = np.linalg.norm(y - r, axis=1)
    row_rel = np.where(rown > 0, rowe / np.maximum(rown, 1e-30), rowe)
    return rel, row_rel


def output_errors(y_bits, ref_bits):
    rel, row_rel = row_errors(y_bits, ref_bits)
    return rel, float(row_rel.max()) if row_rel.size else 0.0


def assert_output_close(y_bits, ref_bits, what="", explained=None):
    """rel L2 <= REL_L2_TOL; every row within ROW_REL_TOL unless explained[row]
    (its A2 differs from the oracle's and the stage checks passed)."""
    rel, row_rel = row_errors(y_bits, ref_bits)
    bad = row_rel > ROW_REL_TOL
    if explained is not None:
        bad &= ~np.asarray(explained, bool)
    row = float(row_rel.max()) if row_rel.size else 0.0
    assert rel <= REL_L2_TOL and not bad.any(), \
        "%s: rel L2 %.3g (tol %.0e), max row rel %.3g (tol %.0e, unexplained rows %s)" % (
            what, rel, REL_L2_TOL, row, ROW_REL_TOL, np.where(bad)[0][:8].tolist())
    return rel, row


def ws_view(ws, offs, region, nbytes, dtype=np.uint8):
    """Host copy of a workspace region."""
    o = offs[region]
    return ws[o:o + nbytes].cpu().numpy().view(dtype)


def ws_rows(ws, offset, row_bytes, rows):
    """Host copy of the given rows of a [n][row_bytes] array at byte offset
    `offset` of the workspace (gathered on the device)."""
    import torch
    rows = np.asarray(rows, np.int64)
    if rows.size == 0:
        return np.zeros((0, row_bytes), np.uint8)
    n = int(rows.max()) + 1
    view = ws[offset:offset + n * row_bytes].view(n, row_bytes)
    return view.index_select(0, torch.from_numpy(rows).to(ws.device)).cpu().numpy()


def unpack_fp4(packed):
    packed = np.asarray(packed)
    out = np.zeros(packed.shape[:-1] + (packed.shape[-1] * 2,), np.int64)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


# ---- A2 validity -------------------------------------------------------------

_MBITS = {0: 3, 1: 1}
_EMIN = {0: -6, 1: 0}


def _grid_step(q, fmt):
    """Spacing of the element grid at magnitude q (in units of the block scale)."""
    q = np.maximum(np.abs(q), 1e-300)
    e = np.maximum(np.floor(np.log2(q)), _EMIN[fmt])
    return np.exp2(e - _MBITS[fmt])


def a2_compare(g_codes, g_scales, r_codes, r_scales, fmt, what=""):
    """Device A2 rows against the oracle's (same rows, codes as stored: bytes
    for E4M3, packed pairs for E2M1).  Asserts every block is a valid
    neighbour (scale exponents at most one apart, each element within one
    grid step at the larger scale of the oracle's value) and returns (fraction
    of elements whose value differs, per-row flag of any difference)."""
    gc = np.asarray(g_codes)
    rc = np.asarray(r_codes)
    if fmt == 1:
        gc, rc = unpack_fp4(gc), unpack_fp4(rc)
    gc = gc.astype(np.int64)
    rc = rc.astype(np.int64)
    gX = np.asarray(g_scales, np.int64) - 127
    rX = np.asarray(r_scales, np.int64) - 127
    n, K = gc.shape
    if n == 0:
        return 0.0, np.zeros(0, bool)
    assert np.all(np.abs(gX - rX) <= 1), "%s: A2 scales more than one apart" % what
    tab = mxref.code_table(fmt)
    gq = tab[gc].reshape(n, K // 32, 32)
    rq = tab[rc].reshape(n, K // 32, 32)
    assert not np.isnan(gq).any(), "%s: device A2 holds a NaN code" % what
    gv = gq * np.exp2(gX)[:, :, None]
    rv = rq * np.exp2(rX)[:, :, None]
    Xm = np.maximum(gX, rX)[:, :, None]
    q = np.maximum(np.abs(gv), np.abs(rv)) * np.exp2(-Xm)
    tol = _grid_step(q, fmt) * np.exp2(Xm) * (1 + 1e-6)
    diff = np.abs(gv - rv)
    bad = diff > tol
    assert not bad.any(), "%s: A2 element off by more than one grid step at rows %s" % (
        what, np.unique(np.where(bad)[0])[:8].tolist())
    differs = (gv != rv).reshape(n, K)
    return float(differs.mean()), differs.any(axis=1)


# ---- GEMM2 and combine from the device's A2 -------------------------------------

def assert_rows_match(g_rows, ref, absref, K, what=""):
    """Device FP32 rows against the oracle's within 2 K 2^-24 sum|terms| (both
    sides sum K products in FP32 in their own order)."""
    g = np.asarray(g_rows, np.float64)
    r = np.asarray(ref, np.float64)
    tol = (2.0 * K + 8.0) * 2.0 ** -24 * np.asarray(absref, np.float64) + 1e-37
    bad = ~(np.abs(g - r) <= tol)
    assert not bad.any(), "%s: %d staging elements differ from the oracle's GEMM2 of the " \
        "device A2 (first rows %s; max |d| %.3g, tol there %.3g)" % (
            what, int(bad.sum()), np.unique(np.where(bad)[0])[:8].tolist(),
            float(np.abs(g - r)[bad].max()), float(tol[bad][np.argmax(np.abs(g - r)[bad])]))
