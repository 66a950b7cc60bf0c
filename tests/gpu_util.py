"""Shared helpers of the GPU parity tests (device transfer, comparisons).

The layer's parity check, in the order the layer computes:

1. routing ids, counts / offsets, the expert permutation and the first-stage
   codes and scales: bit-exact against the oracle;
2. the requantised SwiGLU activations (A2): where floating point decides a
   code (the device's GEMM1 sums in another order, and with the scaled
   FP8 x FP4 matrix instruction at less than FP32 precision, see MFMA_EPS),
   several codes are correct.  Every device block must be a valid neighbour
   of the oracle's: scale exponents at most one apart, and every element
   within one grid step (at the larger of the two scales) plus the bound on
   |h_device - h_oracle| that the two GEMM1 evaluations allow; and at most
   1e-3 of the elements (or one block's 32, in a smaller comparison) may
   differ at all;
3. GEMM2 from the device's own A2: each weighted FP32 staging row equals
   the oracle's GEMM2 of that A2 row times its routing weight, element by
   element, within the summation bound (MFMA_EPS + (2K + 8) 2^-24)
   sum|a_i w_i|;
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
# Error of one scaled MFMA (16x16x128) against the exact dot product, relative
# to the sum of the magnitudes of its terms, by activation format (the weights
# are E2M1).  Measured on the device (random operands in both formats' full
# code ranges and Gaussian-like blocks, 1.5M results each, compared with exact
# double sums): E4M3 x E2M1 is off by up to 2^-12.5 (2^-10.8 of the largest
# term), so it does not sum at FP32 precision; E2M1 x E2M1 is exact.  The
# bound doubles the worst measured error.
MFMA_EPS = {0: 2.0 ** -11, 1: 0.0}


def sum_bound(K, act):
    """Bound on |device - oracle| of a K-term sum, per unit of sum|terms|: the
    device's MFMA error plus the FP32 rounding of both evaluation orders."""
    return MFMA_EPS[act] + (2.0 * K + 8.0) * 2.0 ** -24


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


def a2_step_bytes(act):
    """Code bytes of one A2 row per K step of 128 (E4M3: 128, packed E2M1: 64)."""
    return 128 if act == 0 else 64


def a2_to_ws(codes, scales, act):
    """The workspace's K-step-major A2 bytes ([I/128][N][step bytes] codes,
    [I/128][N][4] scales) from row-major sorted rows [N][...]."""
    n, sb = codes.shape[0], a2_step_bytes(act)
    S = codes.shape[1] // sb
    c = np.ascontiguousarray(codes.reshape(n, S, sb).transpose(1, 0, 2))
    s = np.ascontiguousarray(scales.reshape(n, S, 4).transpose(1, 0, 2))
    return c, s


def ws_a2_rows(ws, offs, N, I, act, rows):
    """Host copies of sorted rows `rows` of A2 (codes [n][I or I/2], scales
    [n][I/32]), gathered on the device from the workspace's K-step-major
    layout over N = T * top_k rows."""
    import torch
    from quantized_moe_expert_softmax_amd import MOE_WS_A2_CODES, MOE_WS_A2_SCALES
    rows = np.asarray(rows, np.int64)
    S, sb = I // 128, a2_step_bytes(act)
    idx = torch.from_numpy(rows).to(ws.device)
    oc, os_ = offs[MOE_WS_A2_CODES], offs[MOE_WS_A2_SCALES]
    c = ws[oc:oc + S * N * sb].view(S, N, sb).index_select(1, idx)
    s = ws[os_:os_ + S * N * 4].view(S, N, 4).index_select(1, idx)
    c = c.permute(1, 0, 2).reshape(rows.size, S * sb).cpu().numpy()
    s = s.permute(1, 0, 2).reshape(rows.size, S * 4).cpu().numpy()
    return c, s


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


def a2_compare(g_codes, g_scales, r_codes, r_scales, fmt, what="", delta=None):
    """Device MX rows (A2) against the oracle's (same rows, codes as stored:
    bytes for E4M3, packed pairs for E2M1).  delta [n, K]: a bound on the
    difference of the values the two sides quantised (None: 0).  Asserts every
    block is a valid neighbour (scale exponents at most one apart, each element
    within delta plus one grid step at the larger scale of the oracle's value)
    and returns (fraction of elements whose value differs, per-row flag of any
    difference)."""
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
    if delta is not None:
        tol = tol + np.asarray(delta, np.float64).reshape(n, K // 32, 32)
    diff = np.abs(gv - rv)
    bad = diff > tol
    if bad.any():
        r_, b_, e_ = (int(v[0]) for v in np.where(bad))
        raise AssertionError(
            "%s: %d elements off by more than one grid step plus the GEMM1 bound (rows %s); "
            "first: row %d block %d elem %d device %.6g (scale 2^%d) oracle %.6g (2^%d) tol %.3g "
            "block max %.6g" % (what, int(bad.sum()), np.unique(np.where(bad)[0])[:8].tolist(),
                                r_, b_, e_, gv[r_, b_, e_], gX[r_, b_], rv[r_, b_, e_], rX[r_, b_],
                                tol[r_, b_, e_], np.abs(rv[r_, b_]).max()))
    differs = (gv != rv).reshape(n, K)
    return float(differs.mean()), differs.any(axis=1)


# ---- GEMM2 and combine from the device's A2 -------------------------------------

def assert_rows_match(g_rows, ref, absref, K, act, what=""):
    """Device FP32 rows against the oracle's within sum_bound(K, act) times
    sum|terms| (both sides sum K products in their own order)."""
    g = np.asarray(g_rows, np.float64)
    r = np.asarray(ref, np.float64)
    tol = sum_bound(K, act) * np.asarray(absref, np.float64) + 1e-37
    bad = ~(np.abs(g - r) <= tol)
    assert not bad.any(), "%s: %d staging elements differ from the oracle's GEMM2 of the " \
        "device A2 (first rows %s; max |d| %.3g, tol there %.3g)" % (
            what, int(bad.sum()), np.unique(np.where(bad)[0])[:8].tolist(),
            float(np.abs(g - r)[bad].max()), float(tol[bad][np.argmax(np.abs(g - r)[bad])]))
