"""Weight sets owned by the caller and swapped per layer: one handle serves
several layers' packed weights (moe_pack_weights + moe_bind_weights), each
call giving the output of a handle that owns the same weights (bit-equal) and
the oracle's; captured graphs keep the weights bound at capture."""
import numpy as np
import pytest

import oracle
import quantized_moe_expert_softmax_amd as moe
from quantized_moe_expert_softmax_amd import synth
from tests.gpu_util import assert_output_close, bf16_dev, bf16_host_bits, dev

pytestmark = pytest.mark.gpu

T, H, I, E, K = 37, 384, 256, 12, 3


def _layers(n):
    return [synth.all_weights(H, I, E, seed=40 + i) for i in range(n)]


def _call(layer, xd, ld, act, ws):
    import torch
    y = moe.moe_forward(layer, xd, ld, K, act, ws=ws)
    torch.cuda.synchronize()
    return bf16_host_bits(y)


@pytest.mark.parametrize("act", [0, 1])
def test_one_handle_many_layers(act):
    import torch
    ws_all = _layers(3)
    x = synth.tokens_bf16(T, H, 50)
    lg = synth.router_logits(T, E, 51)
    xd, ld = bf16_dev(x), dev(lg)
    packed = [moe.moe_pack_weights(E, H, I, *(dev(a) for a in w)) for w in ws_all]
    torch.cuda.synchronize()
    shared = moe.moe_create_layer(E, H, I)
    ws = moe.alloc_workspace(shared, T, K, act)
    with pytest.raises(moe.MoeError):  # no weights bound yet
        moe.moe_forward(shared, xd, ld, K, act, ws=ws)
    first = []
    for w, pk in zip(ws_all, packed):
        moe.moe_bind_weights(shared, pk)
        y = _call(shared, xd, ld, act, ws)
        own = moe.moe_prepare_weights(E, H, I, *(dev(a) for a in w))
        assert np.array_equal(y, _call(own, xd, ld, act, moe.alloc_workspace(own, T, K, act)))
        own.close()
        assert_output_close(y, oracle.forward(x, lg, *w, K, act), "layer act=%d" % act)
        first.append(y)
    # back to the first layer: the same bytes again
    moe.moe_bind_weights(shared, packed[0])
    assert np.array_equal(_call(shared, xd, ld, act, ws), first[0])
    assert not np.array_equal(first[0], first[1])


def test_own_weights_restored_and_graphs_keep_their_binding():
    import torch
    w0, w1 = _layers(2)
    x = synth.tokens_bf16(T, H, 52)
    lg = synth.router_logits(T, E, 53)
    xd, ld = bf16_dev(x), dev(lg)
    layer = moe.moe_prepare_weights(E, H, I, *(dev(a) for a in w0))
    pk1 = moe.moe_pack_weights(E, H, I, *(dev(a) for a in w1))
    ws = moe.alloc_workspace(layer, T, K, 0)
    y0 = _call(layer, xd, ld, 0, ws)
    moe.moe_bind_weights(layer, pk1)
    y1 = _call(layer, xd, ld, 0, ws)
    moe.moe_bind_weights(layer, None)
    assert np.array_equal(_call(layer, xd, ld, 0, ws), y0)
    # one graph per binding, replayed alternately with eager work in between
    s = torch.cuda.Stream()
    outs = [torch.empty((T, H), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    graphs = []
    for i, pk in enumerate((None, pk1)):
        moe.moe_bind_weights(layer, pk)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            moe.moe_forward(layer, xd, ld, K, 0, y=outs[i], ws=ws, stream=s)
        graphs.append(g)
    moe.moe_bind_weights(layer, None)
    for _ in range(3):
        for i, want in enumerate((y0, y1)):
            outs[i].zero_()
            graphs[i].replay()
            torch.cuda.synchronize()
            assert np.array_equal(bf16_host_bits(outs[i]), want)
        assert np.array_equal(_call(layer, xd, ld, 0, ws), y0)
