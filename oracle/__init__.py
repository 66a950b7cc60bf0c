"""CPU oracle of the routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``moe_oracle.c`` (plain,
single-threaded C99, no code shared with the GPU library) through ctypes and
builds that library with gcc on first use when it is missing.

Every function states the step of the layer it evaluates; the C source cites
the pages it follows.  Activation formats: ``0`` = MXFP8 E4M3 (A8W4),
``1`` = MXFP4 E2M1 (A4W4).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

FMT_E4M3 = 0
FMT_E2M1 = 1

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c99",
             "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile moe_oracle.c into liboracle.so (gcc, no FMA contraction)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_long
        lib.oracle_mx_quantize.argtypes = [P, i64, i32, i32, P, P]
        lib.oracle_mx_quantize_bf16.argtypes = [P, i64, i32, i32, P, P]
        lib.oracle_mx_dequantize.argtypes = [P, P, i64, i32, i32, P]
        lib.oracle_code_value.argtypes = [i32, ctypes.c_uint]
        lib.oracle_code_value.restype = ctypes.c_double
        lib.oracle_float_to_bf16.argtypes = [P, i64, P]
        lib.oracle_route.argtypes = [P, i32, i32, i32, P, P]
        lib.oracle_sort.argtypes = [P, i32, i32, i32, P, P, P]
        lib.oracle_forward.argtypes = [P, P, i32, i32, i32, i32, i32, i32, P, P, P, P, i32,
                                       i32, P, P, P, P, P]
        lib.oracle_gemm1_rows.argtypes = [P, P, i64, i32, i32, i32, P, P, P, P, P, P]
        lib.oracle_gemm2_rows.argtypes = [P, P, i64, i32, i32, i32, P, P, P, P, P]
        lib.oracle_combine.argtypes = [P, i64, i32, i32, i32, P, P]
        for f in (lib.oracle_mx_quantize, lib.oracle_mx_quantize_bf16, lib.oracle_mx_dequantize,
                  lib.oracle_float_to_bf16, lib.oracle_route, lib.oracle_sort,
                  lib.oracle_forward, lib.oracle_gemm1_rows, lib.oracle_gemm2_rows,
                  lib.oracle_combine):
            f.restype = None
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def code_bytes_per_row(K: int, fmt: int) -> int:
    return K if fmt == FMT_E4M3 else K // 2


def mx_quantize(v, fmt: int):
    """MX-quantise float32 rows [rows, K] along K in 1x32 blocks.

    Returns (codes, scales): codes [rows, K] (E4M3) or [rows, K/2] (E2M1
    pairs, even element in the low nibble); scales [rows, K/32] E8M0 bytes.
    """
    v = _c(v, np.float32)
    rows, K = v.shape
    codes = np.zeros((rows, code_bytes_per_row(K, fmt)), np.uint8)
    scales = np.zeros((rows, K // 32), np.uint8)
    _load().oracle_mx_quantize(_ptr(v), rows, K, fmt, _ptr(codes), _ptr(scales))
    return codes, scales


def mx_quantize_bf16(x_bits, fmt: int):
    """Same as mx_quantize for bf16 rows given as uint16 bit patterns."""
    x = _c(x_bits, np.uint16)
    rows, K = x.shape
    codes = np.zeros((rows, code_bytes_per_row(K, fmt)), np.uint8)
    scales = np.zeros((rows, K // 32), np.uint8)
    _load().oracle_mx_quantize_bf16(_ptr(x), rows, K, fmt, _ptr(codes), _ptr(scales))
    return codes, scales


def mx_dequantize(codes, scales, K: int, fmt: int):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows = scales.shape[0]
    out = np.zeros((rows, K), np.float32)
    _load().oracle_mx_dequantize(_ptr(codes), _ptr(scales), rows, K, fmt, _ptr(out))
    return out


def code_value(fmt: int, code: int) -> float:
    return _load().oracle_code_value(fmt, code)


def float_to_bf16(f):
    f = _c(f, np.float32)
    out = np.zeros(f.shape, np.uint16)
    _load().oracle_float_to_bf16(_ptr(f), f.size, _ptr(out))
    return out


def route(logits, top_k: int):
    """Top-k softmax routing: ids [T, k] int32 and renormalised weights [T, k] fp32."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.zeros((T, top_k), np.int32)
    w = np.zeros((T, top_k), np.float32)
    _load().oracle_route(_ptr(logits), T, E, top_k, _ptr(ids), _ptr(w))
    return ids, w


def sort(ids, E: int):
    """Expert grouping of the flat assignments: counts [E], offsets [E+1], perm [N]."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    perm = np.zeros(T * k, np.int32)
    _load().oracle_sort(_ptr(ids), T, E, k, _ptr(counts), _ptr(offsets), _ptr(perm))
    return counts, offsets, perm


COMBINE_FP32, COMBINE_BF16, COMBINE_FP8 = 0, 1, 2


def forward(x_bits, logits, w13, w13s, w2, w2s, top_k: int, fmt: int,
            acc_double: bool = False, want_f32: bool = False, want_a2: bool = False,
            expert_map=None, combine: int = COMBINE_FP32):
    """The whole layer for every token of x.

    x_bits [T, H] uint16 (bf16), logits [T, E] fp32, w13 [E, 2I, H/2] (gate rows
    first, then up rows), w13s [E, 2I, H/32], w2 [E, H, I/2], w2s [E, H, I/32].
    Returns y [T, H] as bf16 bit patterns (uint16), plus optionally the fp32
    combine and the requantised SwiGLU activations (indexed by assignment).
    combine: how each weighted GEMM2 row enters the FP32 top-k sum -- as it is
    (COMBINE_FP32), rounded to bf16 (COMBINE_BF16), or MXFP8-quantised along H
    and dequantised (COMBINE_FP8); the last two need acc_double False.
    """
    assert combine in (COMBINE_FP32, COMBINE_BF16, COMBINE_FP8)
    assert combine == COMBINE_FP32 or not acc_double
    x = _c(x_bits, np.uint16)
    logits = _c(logits, np.float32)
    w13 = _c(w13, np.uint8)
    w13s = _c(w13s, np.uint8)
    w2 = _c(w2, np.uint8)
    w2s = _c(w2s, np.uint8)
    T, H = x.shape
    E = logits.shape[1]
    I = w2.shape[2] * 2
    nslab = w13.shape[0]
    assert w13.shape == (nslab, 2 * I, H // 2) and w13s.shape == (nslab, 2 * I, H // 32)
    assert w2.shape == (nslab, H, I // 2) and w2s.shape == (nslab, H, I // 32)
    assert logits.shape[0] == T
    if expert_map is None:
        assert nslab == E
        emap = None
    else:
        emap = _c(expert_map, np.int32)
        assert emap.shape == (E,)
    y = np.zeros((T, H), np.uint16)
    yf = np.zeros((T, H), np.float32) if want_f32 else None
    a2c = np.zeros((T * top_k, code_bytes_per_row(I, fmt)), np.uint8) if want_a2 else None
    a2s = np.zeros((T * top_k, I // 32), np.uint8) if want_a2 else None
    _load().oracle_forward(_ptr(x), _ptr(logits), T, H, I, E, top_k, fmt,
                           _ptr(w13), _ptr(w13s), _ptr(w2), _ptr(w2s), int(bool(acc_double)),
                           int(combine), _ptr(y), _ptr(yf), _ptr(a2c), _ptr(a2s), _ptr(emap))
    out = [y]
    if want_f32:
        out.append(yf)
    if want_a2:
        out.extend([a2c, a2s])
    return out[0] if len(out) == 1 else tuple(out)


def forward_rows(x_bits, logits, rows, weights_for, top_k: int, fmt: int,
                 acc_double: bool = False, combine: int = COMBINE_FP32):
    """The layer on a subset of tokens, fetching only the experts they use.

    Every step of the layer is per token, so the output rows of a subset equal
    the same rows of the whole-batch evaluation.  ``weights_for(e)`` returns
    expert ``e``'s four canonical arrays (w13 [2I, H/2], w13s [2I, H/32],
    w2 [H, I/2], w2s [H, I/32]); they are stacked into a compact set and
    addressed through an expert map, which leaves the arithmetic unchanged.
    Returns y [len(rows), H] as bf16 bit patterns.
    """
    rows = np.asarray(rows, np.int64)
    lg = _c(np.asarray(logits)[rows], np.float32)
    E = lg.shape[1]
    ids, _ = route(lg, top_k)
    used = sorted(set(int(e) for e in ids.reshape(-1)))
    emap = np.full(E, 0, np.int32)
    parts = [weights_for(e) for e in used]
    for i, e in enumerate(used):
        emap[e] = i
    w13 = np.stack([p[0] for p in parts])
    w13s = np.stack([p[1] for p in parts])
    w2 = np.stack([p[2] for p in parts])
    w2s = np.stack([p[3] for p in parts])
    return forward(np.asarray(x_bits)[rows], lg, w13, w13s, w2, w2s, top_k, fmt,
                   acc_double=acc_double, expert_map=emap, combine=combine)


# ---- the layer's steps on their own (FP32 evaluation, as oracle_forward runs
# them), for checking a device's intermediate results row by row ----

def gemm1_rows(a1_codes, a1_scales, slab, w13, w13s, fmt: int, want_gu: bool = False):
    """Steps 3-5 (GEMM1, SwiGLU, requantisation) on n given rows.

    a1_codes [n, H or H/2], a1_scales [n, H/32]: the quantised token row of
    each assignment; slab [n]: its expert's index into w13 [S, 2I, H/2] /
    w13s [S, 2I, H/32].  Returns the A2 rows (codes [n, I or I/2], scales
    [n, I/32]) and, when want_gu, the FP32 GEMM1 results [n, 2I] (gate
    columns, then up columns) the SwiGLU read.
    """
    a1c = _c(a1_codes, np.uint8)
    a1s = _c(a1_scales, np.uint8)
    sl = _c(slab, np.int32).reshape(-1)
    w13 = _c(w13, np.uint8)
    w13s = _c(w13s, np.uint8)
    n = sl.size
    I = w13.shape[1] // 2
    H = w13.shape[2] * 2
    assert a1c.shape == (n, code_bytes_per_row(H, fmt)) and a1s.shape == (n, H // 32)
    assert sl.size == 0 or (sl.min() >= 0 and sl.max() < w13.shape[0])
    a2c = np.zeros((n, code_bytes_per_row(I, fmt)), np.uint8)
    a2s = np.zeros((n, I // 32), np.uint8)
    gu = np.zeros((n, 2 * I), np.float32) if want_gu else None
    _load().oracle_gemm1_rows(_ptr(a1c), _ptr(a1s), n, H, I, fmt, _ptr(sl), _ptr(w13), _ptr(w13s),
                              _ptr(a2c), _ptr(a2s), _ptr(gu))
    return (a2c, a2s, gu) if want_gu else (a2c, a2s)


def gemm2_rows(a2_codes, a2_scales, slab, wts, w2, w2s, fmt: int):
    """Step 6 before the transport on n given rows: the weighted FP32 GEMM2 row
    wts[r] * (A2 row r times every down row of expert slab[r]).

    a2_codes [n, I or I/2], a2_scales [n, I/32], slab [n], wts [n] fp32,
    w2 [S, H, I/2], w2s [S, H, I/32].  Returns rows [n, H] fp32.
    """
    a2c = _c(a2_codes, np.uint8)
    a2s = _c(a2_scales, np.uint8)
    sl = _c(slab, np.int32).reshape(-1)
    wt = _c(wts, np.float32).reshape(-1)
    w2 = _c(w2, np.uint8)
    w2s = _c(w2s, np.uint8)
    n = sl.size
    H = w2.shape[1]
    I = w2.shape[2] * 2
    assert a2c.shape == (n, code_bytes_per_row(I, fmt)) and a2s.shape == (n, I // 32)
    assert wt.size == n and (n == 0 or (sl.min() >= 0 and sl.max() < w2.shape[0]))
    rows = np.zeros((n, H), np.float32)
    _load().oracle_gemm2_rows(_ptr(a2c), _ptr(a2s), n, H, I, fmt, _ptr(sl), _ptr(wt), _ptr(w2),
                              _ptr(w2s), _ptr(rows))
    return rows


def combine(rows, top_k: int, mode: int = COMBINE_FP32, want_f32: bool = False):
    """The transport and FP32 slot-order sum of the weighted rows, then BF16.

    rows [T*top_k, H] fp32 by assignment a = t*top_k + j.  Returns y [T, H]
    as bf16 bit patterns (and the FP32 sums when want_f32).
    """
    r = _c(rows, np.float32)
    n, H = r.shape
    assert n % top_k == 0 and mode in (COMBINE_FP32, COMBINE_BF16, COMBINE_FP8)
    T = n // top_k
    y = np.zeros((T, H), np.uint16)
    yf = np.zeros((T, H), np.float32) if want_f32 else None
    _load().oracle_combine(_ptr(r), T, top_k, H, mode, _ptr(y), _ptr(yf))
    return (y, yf) if want_f32 else y
