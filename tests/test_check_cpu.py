"""The GPU parity check itself, exercised on the CPU with a workspace filled
from the oracle (no device): it accepts the oracle's own intermediate
results, accepts a valid neighbouring A2 block when the staging rows and the
output follow from it, and rejects a planted mistake at every step (a staging
element, an A2 code, an output element, a swapped assignment)."""
import numpy as np
import pytest

import oracle
import quantized_moe_expert_softmax_amd as moe
from quantized_moe_expert_softmax_amd import synth
from tests import layer_check as lc
from tests.gpu_util import a2_step_bytes, a2_to_ws

T, H, I, E, K = 12, 256, 256, 8, 3
REGIONS = moe.MOE_WS_NUM


class FakeLayer:
    E, H, I = E, H, I


def _layout(act):
    N = T * K
    a1row = H if act == 0 else H // 2
    a2row = I if act == 0 else I // 2
    sizes = {moe.MOE_WS_IDS: 4 * N, moe.MOE_WS_WEIGHTS: 4 * N, moe.MOE_WS_COUNTS: 4 * E,
             moe.MOE_WS_OFFSETS: 4 * (E + 1), moe.MOE_WS_PERM: 4 * N,
             moe.MOE_WS_A1_CODES: T * a1row, moe.MOE_WS_A1_SCALES: T * H // 32,
             moe.MOE_WS_A2_CODES: N * a2row, moe.MOE_WS_A2_SCALES: N * I // 32,
             moe.MOE_WS_ROWS: 4 * N * H, moe.MOE_WS_SLOT: 4 * N}
    offs, o = [0] * REGIONS, 0
    for r in range(REGIONS):
        offs[r] = o
        o += (sizes[r] + 255) // 256 * 256
    return offs, o


def _fake_device(act, seed=3):
    """A workspace and output holding exactly what the oracle computes."""
    import torch
    w = synth.all_weights(H, I, E, seed)
    x = synth.tokens_bf16(T, H, seed + 1)
    lg = synth.router_logits(T, E, seed + 2)
    ids, wts = oracle.route(lg, K)
    counts, offsets, perm = oracle.sort(ids, E)
    slot = np.empty_like(perm)
    slot[perm] = np.arange(perm.size, dtype=np.int32)
    xc, xs = oracle.mx_quantize_bf16(x, act)
    y, _, a2c, a2s = oracle.forward(x, lg, *w, K, act, want_f32=True, want_a2=True)
    rows = oracle.gemm2_rows(a2c, a2s, ids.reshape(-1), wts.reshape(-1), w[2], w[3], act)
    offs, total = _layout(act)
    ws = np.zeros(total, np.uint8)

    def put(region, arr):
        b = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        ws[offs[region]:offs[region] + b.size] = b
    put(moe.MOE_WS_IDS, ids.astype(np.int32))
    put(moe.MOE_WS_WEIGHTS, wts.astype(np.float32))
    put(moe.MOE_WS_COUNTS, counts)
    put(moe.MOE_WS_OFFSETS, offsets)
    put(moe.MOE_WS_PERM, perm)
    put(moe.MOE_WS_SLOT, slot)
    put(moe.MOE_WS_A1_CODES, xc)
    put(moe.MOE_WS_A1_SCALES, xs)
    # sorted row p holds assignment perm[p]; stored K-step-major
    c2, s2 = a2_to_ws(a2c[perm], a2s[perm], act)
    put(moe.MOE_WS_A2_CODES, c2)
    put(moe.MOE_WS_A2_SCALES, s2)
    put(moe.MOE_WS_ROWS, rows[perm])
    return torch.from_numpy(ws), y, x, lg, w, offs


@pytest.fixture
def patched(monkeypatch):
    state = {}
    monkeypatch.setattr(moe, "moe_workspace_offsets", lambda layer, t, k, act: state["offs"])
    return state


def _check(state, ws, y, x, lg, w, act):
    wf = lambda e: tuple(a[e] for a in w)
    return lc.check_tokens(FakeLayer(), ws, y, x, lg, K, act, wf, what="fake")


@pytest.mark.parametrize("act", [0, 1])
def test_accepts_the_oracle_itself(patched, act):
    ws, y, x, lg, w, offs = _fake_device(act)
    patched["offs"] = offs
    st = _check(patched, ws, y, x, lg, w, act)
    assert st["a2_mism"] == 0 and st["rows_a2_differs"] == 0 and st["rel"] == 0


def _a2_region(ws, offs, act):
    """The workspace's A2 codes and scales as [I/128][N][step bytes] and
    [I/128][N][4] views (K-step-major)."""
    N, S, sb = T * K, I // 128, a2_step_bytes(act)
    c = ws[offs[moe.MOE_WS_A2_CODES]:offs[moe.MOE_WS_A2_CODES] + S * N * sb].view(S, N, sb)
    s = ws[offs[moe.MOE_WS_A2_SCALES]:offs[moe.MOE_WS_A2_SCALES] + S * N * 4].view(S, N, 4)
    return c, s


def _row(v, p):
    """Sorted row p of a K-step-major [S][N][b] view, as one row-major row."""
    return v[:, p, :].reshape(-1).numpy().copy()


def _set_row(v, p, row):
    import torch
    v[:, p, :] = torch.from_numpy(np.ascontiguousarray(row).reshape(v.shape[0], v.shape[2]))


def test_rejects_a_staging_element(patched):
    import torch
    ws, y, x, lg, w, offs = _fake_device(0)
    patched["offs"] = offs
    r = ws[offs[moe.MOE_WS_ROWS]:offs[moe.MOE_WS_ROWS] + 4 * T * K * H].view(torch.float32)
    r[5 * H + 17] *= 1.01
    with pytest.raises(AssertionError, match="staging elements differ"):
        _check(patched, ws, y, x, lg, w, 0)


def test_rejects_an_a2_code_two_steps_off(patched):
    ws, y, x, lg, w, offs = _fake_device(0)
    patched["offs"] = offs
    c, _ = _a2_region(ws, offs, 0)
    row = _row(c, 4)
    i = int(np.argmax((row & 0x7F) > 0x10))
    row[i] = int(row[i]) + 2 if (row[i] & 0x7F) < 0x7C else int(row[i]) - 2
    _set_row(c, 4, row)
    with pytest.raises(AssertionError, match="grid step"):
        _check(patched, ws, y, x, lg, w, 0)


def test_rejects_an_output_element(patched):
    ws, y, x, lg, w, offs = _fake_device(1)
    patched["offs"] = offs
    y = y.copy()
    y[3, 100] ^= 0x0040
    with pytest.raises(AssertionError, match="slot-order sum"):
        _check(patched, ws, y, x, lg, w, 1)


def test_rejects_swapped_staging_rows(patched):
    import torch
    ws, y, x, lg, w, offs = _fake_device(0)
    patched["offs"] = offs
    r = ws[offs[moe.MOE_WS_ROWS]:offs[moe.MOE_WS_ROWS] + 4 * T * K * H].view(torch.float32)
    r = r.view(T * K, H)
    tmp = r[0].clone()
    r[0] = r[1]
    r[1] = tmp
    with pytest.raises(AssertionError):
        _check(patched, ws, y, x, lg, w, 0)


def test_accepts_a_valid_neighbouring_a2_block(patched):
    """A block whose largest element is exactly 256 units of its scale (h's
    block maximum on a power of two): a device whose FP32 h lands a hair below
    it picks the next lower scale, where that element saturates at 448 half-
    units.  Fake that block, recompute the row's staging and the output from
    it: the check passes and reports the row as differing."""
    import torch
    from tests import mxref
    act = 0
    ws, y, x, lg, w, offs = _fake_device(act)
    patched["offs"] = offs
    c, s = _a2_region(ws, offs, act)
    cn = np.stack([_row(c, q) for q in range(T * K)])
    # a block whose largest magnitude code is 0x78 (256 units)
    blkmax = (cn.reshape(T * K, I // 32, 32) & 0x7F).max(axis=2)
    p, b = map(int, np.argwhere(blkmax == 0x78)[0])
    codes = cn[p].copy()
    sc = _row(s, p)
    vals = oracle.mx_dequantize(codes[None], sc[None], I, act)[0].astype(np.float64)
    X = int(sc[b]) - 127
    codes[32 * b:32 * b + 32] = mxref.nearest_codes(vals[32 * b:32 * b + 32] * 2.0 ** -(X - 1), 0)
    sc[b] -= 1
    _set_row(c, p, codes)
    _set_row(s, p, sc)
    perm = ws[offs[moe.MOE_WS_PERM]:offs[moe.MOE_WS_PERM] + 4 * T * K].view(torch.int32).numpy()
    ids = ws[offs[moe.MOE_WS_IDS]:offs[moe.MOE_WS_IDS] + 4 * T * K].view(torch.int32).numpy()
    wts = ws[offs[moe.MOE_WS_WEIGHTS]:offs[moe.MOE_WS_WEIGHTS] + 4 * T * K].view(torch.float32).numpy()
    a = int(perm[p])
    row = oracle.gemm2_rows(codes[None], sc[None], ids[a:a + 1], wts[a:a + 1], w[2], w[3], act)
    r = ws[offs[moe.MOE_WS_ROWS]:offs[moe.MOE_WS_ROWS] + 4 * T * K * H].view(torch.float32)
    r.view(T * K, H)[p] = torch.from_numpy(row[0])
    rows = r.view(T * K, H).numpy()
    slot = np.empty_like(perm)
    slot[perm] = np.arange(perm.size, dtype=np.int32)
    y2 = oracle.combine(rows[slot], K, oracle.COMBINE_FP32)
    st = _check(patched, ws, y2, x, lg, w, act)
    assert st["rows_a2_differs"] == 1 and 0 < st["a2_mism"] <= 32 / (T * K * I) + 1e-12
    # two scales apart is not a neighbour
    sc[b] -= 1
    _set_row(s, p, sc)
    with pytest.raises(AssertionError, match="more than one apart"):
        _check(patched, ws, y2, x, lg, w, act)
