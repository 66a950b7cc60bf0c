"""Brute-force MX helpers for the tests, written independently of the oracle.

Element rounding is a nearest-code search over every finite code (ties to the
even code, saturating); values come from the codes' bit fields.  These serve
as an independent check of the oracle and to build expected values of
constructed cases; nothing here is used by the GPU library.
"""
import math

import numpy as np

E4M3, E2M1 = 0, 1
EMAX = {E4M3: 8, E2M1: 2}


def grid(fmt):
    """(codes, values) of every finite code, from the bit fields."""
    if fmt == E2M1:
        mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
        codes = np.arange(16)
        vals = np.array([(-1.0 if c & 8 else 1.0) * mags[c & 7] for c in codes])
        return codes, vals
    codes, vals = [], []
    for c in range(256):
        mag = c & 0x7F
        if mag == 0x7F:
            continue
        e, m = mag >> 3, mag & 7
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        codes.append(c)
        vals.append(-v if c & 0x80 else v)
    return np.array(codes), np.array(vals)


def code_table(fmt):
    codes, vals = grid(fmt)
    t = np.full(256 if fmt == E4M3 else 16, np.nan)
    t[codes] = vals
    return t


def nearest_codes(q, fmt):
    q = np.asarray(q, np.float64).reshape(-1)
    codes, vals = grid(fmt)
    pos = codes < (0x80 if fmt == E4M3 else 8)
    pc, pv = codes[pos], vals[pos]
    a = np.abs(q)
    out = np.empty(q.size, np.int64)
    step = 1 << 16
    for s in range(0, q.size, step):
        aa = a[s:s + step]
        dist = np.abs(aa[:, None] - pv[None, :])
        best = dist.min(axis=1, keepdims=True)
        cand = dist == best
        even = cand & ((pc[None, :] & 1) == 0)
        pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
        mag = pc[pick]
        mag = np.where(aa >= pv.max(), pc[np.argmax(pv)], mag)
        out[s:s + step] = mag
    signbit = 0x80 if fmt == E4M3 else 0x8
    return np.where(np.signbit(q), out | signbit, out)


def quantize(v, fmt):
    """Rows of float64 values [R, K] -> (codes [R, K] unpacked ints, exps [R, K/32])."""
    v = np.asarray(v, np.float64)
    R, K = v.shape
    blk = v.reshape(R, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    X = np.full(amax.shape, -127, np.int64)
    nz = amax > 0
    X[nz] = np.clip(np.floor(np.log2(amax[nz])).astype(np.int64) - EMAX[fmt], -127, 127)
    q = blk * np.exp2(-X.astype(np.float64))[:, :, None]
    codes = nearest_codes(q, fmt).reshape(R, K)
    return codes, X


def dequantize(codes, X, fmt):
    R, K = codes.shape
    vals = code_table(fmt)[codes].reshape(R, K // 32, 32)
    return (vals * np.exp2(X.astype(np.float64))[:, :, None]).reshape(R, K)


def unpack_fp4(packed):
    packed = np.asarray(packed)
    out = np.zeros(packed.shape[:-1] + (packed.shape[-1] * 2,), np.int64)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def pack_fp4(codes):
    codes = np.asarray(codes, np.int64)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def dequant_weights(w, ws):
    """Canonical MXFP4 [.., R, K/2] + E8M0 [.., R, K/32] -> float64 [.., R, K]."""
    codes = unpack_fp4(w)
    vals = code_table(E2M1)[codes]
    sh = vals.shape
    vals = vals.reshape(sh[:-1] + (sh[-1] // 32, 32))
    scale = np.exp2(np.asarray(ws, np.float64) - 127.0)
    return (vals * scale[..., None]).reshape(sh)


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def silu(g):
    return g / (1.0 + np.exp(-g))
