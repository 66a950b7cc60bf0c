"""GPU parity of the whole layer at sizes the oracle finishes in seconds.

Every row is compared: bit-exact for routing ids, the expert permutation and
the first-stage codes/scales (read from the forward workspace), within the
stated tolerances for the BF16 output.  The identity-expert construction is
compared bit-exact.  Shapes span several MFMA tiles and ragged tails."""
import numpy as np
import pytest

import oracle
import quantized_moe_expert_softmax_amd as moe
from quantized_moe_expert_softmax_amd import synth
from tests import test_oracle_layer as ol
from tests.gpu_util import assert_output_close, bf16_dev, bf16_host_bits, dev
from tests.layer_check import check_front, check_tokens, forward_and_check

pytestmark = pytest.mark.gpu


def _layer(w13, w13s, w2, w2s):
    E, I2, Hh = w13.shape
    return moe.moe_prepare_weights(E, Hh * 2, I2 // 2, dev(w13), dev(w13s), dev(w2), dev(w2s))


def _run(layer, x, lg, k, act, combine=moe.MOE_COMBINE_FP32):
    import torch
    T = x.shape[0]
    ws = moe.alloc_workspace(layer, T, k, act)
    ws.fill_(0xA5)  # poison: any read of an unwritten byte shows up
    y = moe.moe_forward(layer, bf16_dev(x), dev(lg), k, act, ws=ws, combine=combine)
    torch.cuda.synchronize()
    return bf16_host_bits(y), ws


def host_weights(w):
    """weights_for(e) of a host expert set (w13, w13s, w2, w2s stacked by expert)."""
    return lambda e: tuple(a[e] for a in w)


def _check_workspace(layer, ws, x, lg, k, act):
    """Bit-exact first-stage checks on every token (see tests/layer_check.py)."""
    return check_front(layer, ws, x, lg, k, act)


def _small(T, H, I, E, k, seed):
    w = synth.all_weights(H, I, E, seed)
    x = synth.tokens_bf16(T, H, seed + 1)
    lg = synth.router_logits(T, E, seed + 2)
    return w, x, lg


CASES = [
    # (T, H, I, E, k) -- the tiny workload, ragged m-tiles, K not a multiple of 512
    (16, 256, 128, 8, 2),
    (37, 384, 256, 5, 3),
    (64, 640, 384, 16, 4),
    (3, 128, 128, 1, 1),
    (130, 512, 640, 32, 8),
    (1, 1024, 1152, 64, 6),
    # more than one 256-token sort block: the separate route/sort/quant kernels
    (300, 256, 256, 16, 4),
    # the largest expert count and top_k: fused front kernel (T <= 16) and not
    (1, 256, 128, 1024, 8),
    (16, 256, 128, 1024, 8),
    (17, 256, 128, 1024, 8),
]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("T,H,I,E,k", CASES)
def test_forward_small(T, H, I, E, k, act):
    """Every token: ids / perm / A1 bit-exact, A2 a valid neighbour of the
    oracle's, GEMM2 of the device A2 and the combine exact, y within the
    layer's tolerances of the oracle."""
    w, x, lg = _small(T, H, I, E, k, seed=T + H + I + E + k)
    layer = _layer(*w)
    what = "T=%d H=%d I=%d E=%d k=%d act=%d" % (T, H, I, E, k, act)
    _, _, st = forward_and_check(layer, x, lg, k, act, host_weights(w), what=what)
    print(what, st)


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("T,H,I,E,k", [(37, 384, 256, 5, 3), (300, 512, 640, 16, 4)])
def test_forward_wide_weight_scales(T, H, I, E, k, act):
    """Weight scale bytes drawn over 2^-19 .. 2^13 independently per 1x32
    block (the generated weights span two adjacent bytes per K): every block
    of the scaled MFMA's B operand carries its own exponent, so a scale
    applied to the wrong block or row shows up; the same check as above."""
    w13, w13s, w2, w2s = synth.all_weights(H, I, E, seed=T + 7)
    rng = np.random.default_rng(T + 11)
    w13s = rng.integers(108, 141, size=w13s.shape, dtype=np.uint8)
    w2s = rng.integers(108, 141, size=w2s.shape, dtype=np.uint8)
    w = (w13, w13s, w2, w2s)
    x = synth.tokens_bf16(T, H, T + 8)
    lg = synth.router_logits(T, E, T + 9)
    layer = _layer(*w)
    what = "wide scales T=%d H=%d I=%d E=%d k=%d act=%d" % (T, H, I, E, k, act)
    _, _, st = forward_and_check(layer, x, lg, k, act, host_weights(w), what=what)
    print(what, st)


@pytest.mark.parametrize("act", [0, 1])
def test_identity_experts_exact(act):
    H, I, E, T = 256, 128, 8, 16
    w13, w13s, w2, w2s, cmap, tau = ol.identity_experts(H, I, E, 5)
    x, lg = ol.identity_inputs(T, H, E, 6)
    layer = _layer(w13, w13s, w2, w2s)
    y, _ = _run(layer, x, lg, 1, act)
    ids, _ = oracle.route(lg, 1)
    want = ol.identity_expected(x, ids, cmap, tau, act, H, I)
    assert np.array_equal(ol.mxref.bf16_to_f64(y), want)
    ref = oracle.forward(x, lg, w13, w13s, w2, w2s, 1, act)
    assert np.array_equal(ol.mxref.bf16_to_f64(y), ol.mxref.bf16_to_f64(ref))


def test_identity_experts_larger():
    """Identity construction at a multi-tile shape (I spans 10 units, 5 K-steps)."""
    H, I, E, T = 1024, 640, 12, 200
    w13, w13s, w2, w2s, cmap, tau = ol.identity_experts(H, I, E, 7)
    x, lg = ol.identity_inputs(T, H, E, 8)
    layer = _layer(w13, w13s, w2, w2s)
    for act in (0, 1):
        y, _ = _run(layer, x, lg, 1, act)
        ids, _ = oracle.route(lg, 1)
        want = ol.identity_expected(x, ids, cmap, tau, act, H, I)
        assert np.array_equal(ol.mxref.bf16_to_f64(y), want)


def test_mispaired_gate_up_fails_parity():
    """Negative control: feeding the layer gate/up rows swapped must break parity."""
    T, H, I, E, k = 16, 256, 128, 8, 2
    w, x, lg = _small(T, H, I, E, k, seed=3)
    w13, w13s, w2, w2s = w
    sw = np.ascontiguousarray(np.concatenate([w13[:, I:], w13[:, :I]], axis=1))
    sws = np.ascontiguousarray(np.concatenate([w13s[:, I:], w13s[:, :I]], axis=1))
    layer = _layer(sw, sws, w2, w2s)
    y, _ = _run(layer, x, lg, k, 0)
    ref = oracle.forward(x, lg, w13, w13s, w2, w2s, k, 0)
    from tests.gpu_util import output_errors
    rel, _ = output_errors(y, ref)
    assert rel > 0.5


def test_zero_tokens_is_noop():
    import torch
    w, x, lg = _small(4, 256, 128, 8, 2, seed=4)
    layer = _layer(*w)
    y = torch.full((0, 256), 7, dtype=torch.bfloat16, device="cuda")
    x0 = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    l0 = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    out = moe.moe_forward(layer, x0, l0, 2, 0, y=y, ws=ws)
    assert out.shape == (0, 256)


def test_workspace_too_small_is_rejected():
    import torch
    w, x, lg = _small(8, 256, 128, 8, 2, seed=5)
    layer = _layer(*w)
    need = moe.moe_workspace_bytes(layer, 8, 2, 0)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward(layer, bf16_dev(x), dev(lg), 2, 0, ws=ws)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE


def test_repeat_calls_agree():
    """Same inputs twice: ids/perm/codes and the output are identical (the top-k
    sum runs in slot order, so the layer is deterministic)."""
    w, x, lg = _small(64, 512, 256, 16, 4, seed=6)
    layer = _layer(*w)
    y1, ws1 = _run(layer, x, lg, 4, 0)
    y2, ws2 = _run(layer, x, lg, 4, 0)
    offs = moe.moe_workspace_offsets(layer, 64, 4, 0)
    end = offs[moe.MOE_WS_A2_CODES]
    assert np.array_equal(ws1[:end].cpu().numpy(), ws2[:end].cpu().numpy())
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("T,H,I,E,k,combine", [(16, 256, 128, 8, 2, 0), (37, 384, 256, 5, 3, 0),
                                               (300, 256, 256, 16, 4, 0),
                                               (130, 512, 640, 32, 8, 1)])
def test_prequant_entry(T, H, I, E, k, combine, act):
    """The layer fed the oracle's MX codes and scales of x gives the BF16
    entry's output bit for bit (the quantiser is exact), which passes the
    whole check against the oracle."""
    w, x, lg = _small(T, H, I, E, k, seed=T + 11 * k)
    layer = _layer(*w)
    y, _, _ = forward_and_check(layer, x, lg, k, act, host_weights(w), combine,
                                what="prequant T=%d act=%d" % (T, act))
    xc, xs = oracle.mx_quantize_bf16(x, act)
    ws = moe.alloc_workspace(layer, T, k, act)
    ws.fill_(0xA5)
    yq = moe.moe_forward_prequant(layer, dev(xc), dev(xs), dev(lg), k, act, ws=ws,
                                  combine=combine)
    import torch
    torch.cuda.synchronize()
    yq = bf16_host_bits(yq)
    assert np.array_equal(yq, y)


@pytest.mark.parametrize("act", [0, 1])
def test_prequant_scales_4_byte_aligned(act):
    """Token scales at a 4-byte but not 16-byte aligned address (allowed by the
    prequant entry) take the tiled GEMM1's per-step scale copies instead of the
    16-byte ones of four K steps (H = 512 would allow those): same output as
    the BF16 entry, bit for bit."""
    import torch
    T, H, I, E, k = 130, 512, 640, 32, 8
    w, x, lg = _small(T, H, I, E, k, seed=21 + act)
    layer = _layer(*w)
    assert moe.moe_get_plan(layer, T, k, act)["variant"] == moe.MOE_PLAN_TILED
    y, _, _ = forward_and_check(layer, x, lg, k, act, host_weights(w),
                                what="prequant-4-aligned act=%d" % act)
    xc, xs = oracle.mx_quantize_bf16(x, act)
    buf = torch.zeros(xs.size + 64, dtype=torch.uint8, device="cuda")
    xs_dev = buf[4:4 + xs.size].view(xs.shape)
    xs_dev.copy_(torch.from_numpy(np.ascontiguousarray(xs)))
    assert xs_dev.data_ptr() % 16 == 4
    yq = moe.moe_forward_prequant(layer, dev(xc), xs_dev, dev(lg), k, act)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host_bits(yq), y)


def test_graph_capture_replays():
    """moe_forward captured into a HIP graph replays to the eager result, repeatedly."""
    import torch
    w, x, lg = _small(32, 512, 256, 16, 4, seed=7)
    layer = _layer(*w)
    xd, ld = bf16_dev(x), dev(lg)
    ws = moe.alloc_workspace(layer, 32, 4, 0)
    y = torch.empty((32, 512), dtype=torch.bfloat16, device="cuda")
    moe.moe_forward(layer, xd, ld, 4, 0, y=y, ws=ws)
    torch.cuda.synchronize()
    eager = bf16_host_bits(y).copy()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_forward(layer, xd, ld, 4, 0, y=y, ws=ws, stream=s)
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_output_close(bf16_host_bits(y), eager, "graph replay")


@pytest.mark.parametrize("combine", [moe.MOE_COMBINE_BF16, moe.MOE_COMBINE_FP8])
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("T,H,I,E,k", [CASES[0], CASES[4], CASES[5], CASES[6]])
def test_forward_combine_transports(T, H, I, E, k, act, combine):
    """The compressed combine transports: staging rows are one BF16 rounding
    (or a valid MXFP8 quantisation) of the oracle's GEMM2 of the device A2,
    y is exactly their FP32 slot-order sum, and y is within the tolerances of
    the oracle's same transport; the FP8 one must differ from the FP32
    transport (it quantises)."""
    w, x, lg = _small(T, H, I, E, k, seed=T + H + I + E + k)
    layer = _layer(*w)
    what = "T=%d act=%d combine=%d" % (T, act, combine)
    y, _, st = forward_and_check(layer, x, lg, k, act, host_weights(w), combine, what=what)
    if combine == moe.MOE_COMBINE_FP8:
        y32, _ = _run(layer, x, lg, k, act)
        assert not np.array_equal(y, y32)
    print(what, st)


def test_forward_rejects_unknown_flags():
    import torch
    w, x, lg = _small(8, 256, 128, 8, 2, seed=16)
    layer = _layer(*w)
    ws = moe.alloc_workspace(layer, 8, 2, 0)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward(layer, bf16_dev(x), dev(lg), 2, 0, ws=ws, combine=3)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    torch.cuda.synchronize()
