"""Bit-exact GPU checks with the identity-expert construction at the full
contraction lengths of the benchmarked layers (K = 7168 / 3072 and 5120 /
640), under every GEMM plan the library builds, in both activation formats.

With top_k = 1 the layer's output is y[t, h] = xq[t, c_e(tau_e(h))] exactly
(tests/test_oracle_layer.py: identity_experts), so any wrong expert, gate/up
mispairing, row or column mapping, K-step, scale byte or store in any plan
shows up as a changed bit; the closed form is computed with the brute-force
quantiser, independently of both the oracle and the library."""
import numpy as np
import pytest

import quantized_moe_expert_softmax_amd as moe
from quantized_moe_expert_softmax_amd import tune
from tests import mxref
from tests import test_oracle_layer as ol
from tests.gpu_util import bf16_dev, bf16_host_bits, dev

pytestmark = pytest.mark.gpu

SHAPES = [(7168, 3072, 4, 200), (5120, 640, 6, 300)]  # (H, I, E, T): ~50 rows per expert
_layers = {}


def _setup(H, I, E, T):
    key = (H, I, E, T)
    if key not in _layers:
        for k in list(_layers):
            _layers.pop(k)[0].close()
        w13, w13s, w2, w2s, cmap, tau = ol.identity_experts_packed(H, I, E, 17)
        layer = moe.moe_prepare_weights(E, H, I, dev(w13), dev(w13s), dev(w2), dev(w2s))
        x, lg = ol.identity_inputs(T, H, E, 18)
        want = {}
        ids = np.argmax(lg, axis=1)[:, None]  # top-1 of distinct Gaussian logits
        for act in (0, 1):
            want[act] = ol.identity_expected(x, ids, cmap, tau, act, H, I)
        _layers[key] = (layer, x, lg, want)
    return _layers[key]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("H,I,E,T", SHAPES)
def test_identity_every_plan_full_k(H, I, E, T, act):
    import torch
    layer, x, lg, want = _setup(H, I, E, T)
    xd, ld = bf16_dev(x), dev(lg)
    for variant, rows in tune.candidates(act, include_fused=True):
        moe.moe_set_plans(layer, [dict(act=act, top_k=1, t_max=T, variant=variant, rows=rows)])
        ws = moe.alloc_workspace(layer, T, 1, act)
        ws.fill_(0xA5)
        y = moe.moe_forward(layer, xd, ld, 1, act, ws=ws)
        torch.cuda.synchronize()
        got = mxref.bf16_to_f64(bf16_host_bits(y))
        bad = np.where((got != want[act]).any(axis=1))[0]
        assert bad.size == 0, "H=%d I=%d act=%d plan (%d, %d): tokens %s differ" % (
            H, I, act, variant, rows, bad[:8].tolist())
        if variant == moe.MOE_PLAN_FUSED:
            assert moe.moe_fused_status(layer, ws, T, 1, act) == 0
    moe.moe_set_plans(layer, [])
