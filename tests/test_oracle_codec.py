"""Pins of the oracle's MX codec and BF16 rounding (CPU only).

The oracle's element rounding (double arithmetic + nearbyint on the binade
spacing) is checked against an independent brute-force nearest-code search
over every finite code, against hand-derived worked examples
(tests/golden/mx_worked_examples.txt), against exact round trips of every
representable code, and against torch's bf16 cast.
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_worked_examples.txt")
E4M3, E2M1 = oracle.FMT_E4M3, oracle.FMT_E2M1
EMAX = {E4M3: 8, E2M1: 2}


def _grid(fmt):
    """Every finite code and its value, enumerated from the bit fields.

    E4M3 (OCP E4M3FN): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
    field 0 is subnormal with step 2^-9; the all-ones magnitude 0x7F is NaN.
    E2M1: the eight magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 and a sign bit.
    """
    if fmt == E2M1:
        mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
        codes = list(range(16))
        vals = [(-1.0 if c & 8 else 1.0) * mags[c & 7] for c in codes]
        return np.array(codes), np.array(vals)
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


def test_grid_anchors():
    codes, vals = _grid(E4M3)
    d = dict(zip(codes.tolist(), vals.tolist()))
    assert d[0x7E] == 448.0 and d[0x01] == 2.0 ** -9 and d[0x08] == 2.0 ** -6 and d[0x38] == 1.0
    pos = vals[codes < 0x80]
    assert np.all(np.diff(pos) > 0) and pos.size == 127
    codes4, vals4 = _grid(E2M1)
    assert vals4[:8].tolist() == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


@pytest.mark.parametrize("fmt", [E4M3, E2M1])
def test_code_value_matches_grid(fmt):
    codes, vals = _grid(fmt)
    for c, v in zip(codes.tolist(), vals.tolist()):
        got = oracle.code_value(fmt, c)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), (c, got, v)


def brute_codes(q, fmt):
    """Nearest code to each scaled value q (ties -> even code, saturating)."""
    codes, vals = _grid(fmt)
    q = np.asarray(q, np.float64)
    sign = np.signbit(q)
    a = np.abs(q)
    pos = codes < (0x80 if fmt == E4M3 else 8)
    pc, pv = codes[pos], vals[pos]
    maxv = pv.max()
    dist = np.abs(a[:, None] - pv[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among equal distances prefer the even code; a single candidate wins outright
    even = cand & ((pc[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    mag = pc[pick]
    mag = np.where(a >= maxv, pc[np.argmax(pv)], mag)
    signbit = 0x80 if fmt == E4M3 else 0x8
    return np.where(sign, mag | signbit, mag).astype(np.int64)


def brute_exponent(block_amax, fmt):
    if block_amax == 0:
        return -127
    return int(min(127, max(-127, math.floor(math.log2(block_amax)) - EMAX[fmt])))


def _unpack(codes, fmt, K):
    codes = np.asarray(codes)
    if fmt == E4M3:
        return codes.astype(np.int64)
    out = np.zeros(codes.shape[:-1] + (K,), np.int64)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


@pytest.mark.parametrize("fmt", [E4M3, E2M1])
@pytest.mark.parametrize("X", [-100, -8, 0, 5, 60])
def test_every_code_round_trips(fmt, X):
    codes, vals = _grid(fmt)
    maxcode = 0x7E if fmt == E4M3 else 0x7
    # element 0 of every block is the largest code, so the block exponent is X
    others = codes[codes != maxcode]
    nblk = -(-others.size // 31)
    blk = np.full((nblk, 32), maxcode, np.int64)
    flat = np.concatenate([others, np.full(nblk * 31 - others.size, maxcode)])
    blk[:, 1:] = flat.reshape(nblk, 31)
    lut = dict(zip(codes.tolist(), vals.tolist()))
    v = np.vectorize(lambda c: lut[int(c)])(blk) * 2.0 ** X
    v32 = v.astype(np.float32)
    assert np.array_equal(v32.astype(np.float64), v)  # exactly representable
    q, s = oracle.mx_quantize(v32, fmt)
    assert np.all(s == X + 127)
    assert np.array_equal(_unpack(q, fmt, 32), blk)
    back = oracle.mx_dequantize(q, s, 32, fmt)
    assert np.array_equal(back.view(np.uint32), v32.view(np.uint32))  # -0 included


def _finite_bf16():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


@pytest.mark.parametrize("fmt", [E4M3, E2M1])
def test_every_bf16_as_block_amax(fmt):
    """Each finite bf16 value alone in a block: scale from its own exponent."""
    v = _finite_bf16()
    blocks = np.zeros((v.size, 32), np.float32)
    blocks[:, 0] = v
    q, s = oracle.mx_quantize(blocks, fmt)
    codes = _unpack(q, fmt, 32)[:, 0]
    exp_s = np.array([brute_exponent(abs(float(x)), fmt) for x in v])
    assert np.array_equal(s[:, 0].astype(np.int64), exp_s + 127)
    scaled = v.astype(np.float64) * np.exp2(-exp_s.astype(np.float64))
    assert np.array_equal(codes, brute_codes(scaled, fmt))


@pytest.mark.parametrize("fmt", [E4M3, E2M1])
@pytest.mark.parametrize("X", [-120, -3, 0, 40])
def test_every_bf16_under_fixed_anchor(fmt, X):
    """Element rounding (incl. subnormals and ties) with the scale pinned by an anchor."""
    v = _finite_bf16().astype(np.float64)
    anchor = 2.0 ** (EMAX[fmt] + X)
    v = v[np.abs(v) <= anchor]
    blocks = np.zeros((v.size, 32), np.float32)
    blocks[:, 0] = anchor
    blocks[:, 1] = v
    q, s = oracle.mx_quantize(blocks, fmt)
    assert np.all(s[:, 0] == X + 127)
    codes = _unpack(q, fmt, 32)[:, 1]
    assert np.array_equal(codes, brute_codes(v * 2.0 ** -X, fmt))


def _parse_value(tok):
    return float.fromhex(tok) if tok.lstrip("-").startswith("0x") else float(tok)


def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        fmt_s, vals_s, scale_s, codes_s = [p.strip() for p in line.split(";")]
        vals = {int(a): _parse_value(b) for a, b in (t.split("=") for t in vals_s.split())}
        codes = {int(a): int(b, 16) for a, b in (t.split("=") for t in codes_s.split())}
        rows.append((fmt_s, vals, int(scale_s), codes))
    return rows


def test_golden_has_examples():
    assert len(_golden_rows()) >= 12


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: "%s-%s" % (r[0], r[2]))
def test_worked_examples(row):
    fmt_s, vals, scale, codes = row
    fmt = E4M3 if fmt_s == "e4m3" else E2M1
    blk = np.zeros((1, 32), np.float32)
    for i, v in vals.items():
        blk[0, i] = np.float32(v)
        assert float(blk[0, i]) == v or fmt_s == "e4m3" and i == 1  # 0.1 is not exact; others are
    q, s = oracle.mx_quantize(blk, fmt)
    assert int(s[0, 0]) == scale
    got = _unpack(q, fmt, 32)[0]
    want = np.zeros(32, np.int64)
    for i, c in codes.items():
        want[i] = c
    assert got.tolist() == want.tolist()


def test_bf16_path_equals_float_path():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 256)).astype(np.float32)
    import torch
    xb = torch.from_numpy(x).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    for fmt in (E4M3, E2M1):
        a = oracle.mx_quantize_bf16(bits, fmt)
        b = oracle.mx_quantize(xb.to(torch.float32).numpy(), fmt)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_float_to_bf16_matches_torch():
    import torch
    rng = np.random.default_rng(5)
    f = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
        # exact ties: low half exactly 0x8000 with even and odd upper halves
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)[10:],
        np.array([0.0, -0.0, 1e-45, -1e-45, 3.3e38], np.float32),
    ]).astype(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.float_to_bf16(f), want)
