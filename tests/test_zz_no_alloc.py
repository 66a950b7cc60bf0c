"""moe_forward_noalloc (the forward on the library's static device workspace)
against moe_forward_ex on the same inputs: bit-equal outputs on two calls in a
row, the second with fewer tokens (the array keeps the first call's contents),
in both activation formats and two combine transports; a call whose workspace
exceeds the array is rejected before anything is enqueued."""
import numpy as np
import pytest

import quantized_moe_expert_softmax_amd as moe
from quantized_moe_expert_softmax_amd import synth
from tests.gpu_util import bf16_dev, bf16_host_bits, dev

pytestmark = pytest.mark.gpu

SHAPES = [
    # (H, I, E, top_k, T first, T second)
    (512, 256, 16, 4, 200, 37),     # separate route/sort kernels, then the fused front path
    (2048, 1024, 16, 6, 64, 5),     # router kernel + front, then the fused front path
    (7168, 3072, 8, 6, 16, 1),      # the 7168 x 3072 expert shape at decode sizes
]


def _layer(H, I, E):
    w = synth.all_weights(H, I, E, 77)
    return moe.moe_prepare_weights(E, H, I, *(dev(a) for a in w))


@pytest.mark.parametrize("combine", [moe.MOE_COMBINE_FP32, moe.MOE_COMBINE_BF16])
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("H,I,E,k,T1,T2", SHAPES)
def test_noalloc_matches_forward(H, I, E, k, T1, T2, act, combine):
    import torch
    layer = _layer(H, I, E)
    for T in (T1, T2):
        x = bf16_dev(synth.tokens_bf16(T, H, T + act))
        lg = dev(synth.router_logits(T, E, T + 3 * act))
        ws = moe.alloc_workspace(layer, T, k, act)
        want = moe.moe_forward(layer, x, lg, k, act, ws=ws, combine=combine)
        y = torch.full((T, H), 7.0, dtype=torch.bfloat16, device="cuda")
        got = moe.moe_forward_noalloc(layer, x, lg, k, act, y, combine=combine)
        torch.cuda.synchronize()
        assert got is y
        assert np.array_equal(bf16_host_bits(y), bf16_host_bits(want)), (H, I, E, k, T, act)
    layer.close()


def test_noalloc_rejects_calls_beyond_the_array():
    import torch
    H, I, E, k = 512, 256, 16, 4
    layer = _layer(H, I, E)
    T = 10000  # N * H * 4 bytes of FP32 staging rows alone: 82 MB > 64 MiB
    assert moe.moe_workspace_bytes(layer, T, k, 0) > moe.MOE_NOALLOC_SCRATCH_BYTES
    x = bf16_dev(synth.tokens_bf16(T, H, 5))
    lg = dev(synth.router_logits(T, E, 6))
    y = torch.full((T, H), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_noalloc(layer, x, lg, k, 0, y)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    assert "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())  # nothing was enqueued
    # the largest T that fits still runs and matches moe_forward
    Tmax = T
    while moe.moe_workspace_bytes(layer, Tmax, k, 0) > moe.MOE_NOALLOC_SCRATCH_BYTES:
        Tmax -= 16
    xs, ls = x[:Tmax].contiguous(), lg[:Tmax].contiguous()
    want = moe.moe_forward(layer, xs, ls, k, 0)
    got = moe.moe_forward_noalloc(layer, xs, ls, k, 0, y[:Tmax])
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host_bits(got), bf16_host_bits(want))
    layer.close()
