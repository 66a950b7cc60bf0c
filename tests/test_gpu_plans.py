"""The per-layer plan table: every GEMM plan the library builds gives the
oracle's result (bit-exact ids / perm / A1 bytes, the output within the
stated tolerances), the table is looked up in order, invalid entries are
rejected, and the tuner produces a valid table."""
import numpy as np
import pytest

import oracle
import quantized_moe_expert_softmax_amd as moe
from quantized_moe_expert_softmax_amd import tune
from tests.gpu_util import assert_output_close, bf16_dev, dev
from tests.layer_check import forward_and_check
from tests.test_gpu_forward import _layer, _run, _small, host_weights

pytestmark = pytest.mark.gpu

# ragged: 300 tokens x 4 slots over 16 experts (~75 rows each): every tile
# height leaves a partial m-block, and the stream plan many partial m-tiles
SHAPE = (300, 256, 256, 16, 4)


@pytest.mark.parametrize("act", [0, 1])
def test_every_plan_matches_oracle(act):
    T, H, I, E, k = SHAPE
    w, x, lg = _small(T, H, I, E, k, seed=11)
    layer = _layer(*w)
    for variant, rows in tune.candidates(act, include_fused=True):
        plan = dict(act=act, top_k=k, t_max=T, variant=variant, rows=rows)
        moe.moe_set_plans(layer, [plan])
        got = moe.moe_get_plan(layer, T, k, act)
        assert (got["variant"], got["rows"]) == (variant, rows)
        forward_and_check(layer, x, lg, k, act, host_weights(w), what="plan %s" % plan)


def test_table_lookup_order_and_fallback():
    T, H, I, E, k = 64, 256, 128, 8, 2
    w, _, _ = _small(T, H, I, E, k, seed=12)
    layer = _layer(*w)
    builtin_100 = moe.moe_get_plan(layer, 100, k, 0)
    builtin_4 = moe.moe_get_plan(layer, 4, k, 0)
    builtin_k1 = moe.moe_get_plan(layer, 100, 1, 1)
    moe.moe_set_plans(layer, [
        dict(act=0, top_k=k, t_max=8, variant=moe.MOE_PLAN_TILED, rows=160),
        dict(act=0, top_k=k, t_max=64, variant=moe.MOE_PLAN_STREAM, rows=16),
        dict(act=1, top_k=k, t_max=1000, variant=moe.MOE_PLAN_TILED, rows=128),
    ])
    assert moe.moe_get_plan(layer, 4, k, 0)["rows"] == 160
    assert moe.moe_get_plan(layer, 8, k, 0)["rows"] == 160
    assert moe.moe_get_plan(layer, 9, k, 0)["variant"] == moe.MOE_PLAN_STREAM
    assert moe.moe_get_plan(layer, 100, k, 0) == builtin_100  # no entry: built-in choice
    assert moe.moe_get_plan(layer, 100, k, 1)["rows"] == 128
    assert moe.moe_get_plan(layer, 100, 1, 1) == builtin_k1  # top_k must match too
    moe.moe_set_plans(layer, [])
    assert moe.moe_get_plan(layer, 4, k, 0) == builtin_4


# The built-in choice on the layer shapes it was measured on (7168 x 3072 with
# E = 384, top_k = 6; the 5120 x {640, 1152} shards with E = 384 x 6 and
# 128 x 3): weight streaming up to 4 rows per expert (with the token-major
# GEMM2 at T <= 2), tiled at least 64 rows,
# BM covering the mean plus 1.5 sigma up to 160 rows, and above that the tile
# with the fewest expected padded rows.  It depends on T, top_k and E only.
BUILTIN = [
    # (E, top_k, T, variant, rows)
    (384, 6, 1, moe.MOE_PLAN_DECODE, 16),      # T <= 2: token-major GEMM2, combine folded in
    (384, 6, 2, moe.MOE_PLAN_DECODE, 16),
    (384, 6, 3, moe.MOE_PLAN_STREAM, 16),
    (384, 6, 128, moe.MOE_PLAN_STREAM, 16),    # 2 rows per expert
    (384, 6, 256, moe.MOE_PLAN_STREAM, 16),    # 4 rows: the last streamed
    (384, 6, 257, moe.MOE_PLAN_TILED, 64),     # 4.02 rows: tiled, at the 64-row minimum
    (384, 6, 1024, moe.MOE_PLAN_TILED, 64),
    (384, 6, 2048, moe.MOE_PLAN_TILED, 64),    # mean 32 + 1.5 sigma -> 48 -> even MT
    (384, 6, 4096, moe.MOE_PLAN_TILED, 96),    # mean 64 -> 76 rows
    (384, 6, 8192, moe.MOE_PLAN_TILED, 160),   # mean 128 -> 145 rows
    (384, 6, 16384, moe.MOE_PLAN_TILED, 160),  # mean 256: fewest padded rows at 160
    (384, 6, 24576, moe.MOE_PLAN_TILED, 128),  # mean 384: at 128
    (384, 6, 32768, moe.MOE_PLAN_TILED, 192),  # mean 512: at 192
    (128, 3, 170, moe.MOE_PLAN_STREAM, 16),    # 3.98 rows
    (128, 3, 171, moe.MOE_PLAN_TILED, 64),     # 4.01 rows
    (128, 3, 16384, moe.MOE_PLAN_TILED, 128),  # mean 384
    (128, 3, 32768, moe.MOE_PLAN_TILED, 160),  # mean 768
]


@pytest.mark.parametrize("E,k", sorted({(c[0], c[1]) for c in BUILTIN}))
def test_builtin_plan_choices(E, k):
    w, _, _ = _small(1, 128, 128, E, k, seed=13)
    layer = _layer(*w)
    for e_, k_, T, variant, rows in BUILTIN:
        if (e_, k_) != (E, k):
            continue
        for act in (0, 1):  # both activation formats take the same rule
            got = moe.moe_get_plan(layer, T, k, act)
            assert (got["variant"], got["rows"]) == (variant, rows), (E, k, T, act, got)


@pytest.mark.parametrize("bad", [
    dict(rows=48), dict(rows=224, act=1), dict(variant=4), dict(act=5), dict(top_k=0),
    dict(top_k=9), dict(t_max=0), dict(variant=moe.MOE_PLAN_STREAM, rows=32),
    dict(variant=moe.MOE_PLAN_FUSED, rows=32), dict(variant=moe.MOE_PLAN_DECODE, rows=32),
])
def test_invalid_plans_rejected(bad):
    w, _, _ = _small(16, 256, 128, 8, 2, seed=13)
    layer = _layer(*w)
    good = dict(act=0, top_k=2, t_max=16, variant=moe.MOE_PLAN_TILED, rows=64)
    moe.moe_set_plans(layer, [good])
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_set_plans(layer, [good, dict(good, **bad)])
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    assert moe.moe_get_plan(layer, 16, 2, 0)["rows"] == 64  # table unchanged


def test_tuner_installs_a_valid_table():
    import torch
    T1, T2, H, I, E, k = 24, 200, 256, 256, 16, 4
    w, _, _ = _small(T2, H, I, E, k, seed=14)
    layer = _layer(*w)
    inputs = {}
    for T in (T1, T2):
        _, x, lg = _small(T, H, I, E, k, seed=15 + T)
        inputs[T] = (bf16_dev(x), [dev(lg)])
    table, report = tune.tune(layer, inputs, k, 0, steps=2, warmup=1)
    assert [e["t_max"] for e in table] == [T1, T2]
    for e in table:
        assert (e["variant"], e["rows"]) in tune.candidates(0)
        assert moe.moe_get_plan(layer, e["t_max"], k, 0)["rows"] == e["rows"]
    # the tuned layer still matches the oracle
    _, x, lg = _small(T2, H, I, E, k, seed=15 + T2)
    y, _ = _run(layer, x, lg, k, 0)
    assert_output_close(y, oracle.forward(x, lg, *w, k, 0), "tuned")
    torch.cuda.synchronize()


# the fused launch over both front paths (T <= 16 fused front kernel, else the
# separate route/sort kernels), ragged m-tiles, one expert, E > 256 items
FUSED_CASES = [(1, 256, 128, 8, 2), (16, 256, 128, 8, 2), (37, 384, 256, 5, 3),
               (3, 128, 128, 1, 1), (130, 512, 640, 32, 8), (1, 1024, 1152, 64, 6),
               (300, 256, 256, 16, 4), (17, 256, 128, 1024, 8)]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("T,H,I,E,k", FUSED_CASES)
def test_fused_plan(T, H, I, E, k, act):
    """The fused launch passes the layer check, none of its bounded waits gave
    up (moe_fused_status), and repeated calls on one workspace agree bit for
    bit (its counters are cleared by every call's routing launch)."""
    w, x, lg = _small(T, H, I, E, k, seed=T + H + E)
    layer = _layer(*w)
    moe.moe_set_plans(layer, [dict(act=act, top_k=k, t_max=T, variant=moe.MOE_PLAN_FUSED,
                                   rows=16)])
    y, ws, _ = forward_and_check(layer, x, lg, k, act, host_weights(w),
                                 what="fused T=%d H=%d I=%d E=%d k=%d act=%d" % (T, H, I, E, k, act))
    assert moe.moe_fused_status(layer, ws, T, k, act) == 0
    import torch
    xd, ld = bf16_dev(x), dev(lg)
    for _ in range(3):
        y2 = moe.moe_forward(layer, xd, ld, k, act, ws=ws)
    torch.cuda.synchronize()
    assert moe.moe_fused_status(layer, ws, T, k, act) == 0
    from tests.gpu_util import bf16_host_bits
    assert np.array_equal(bf16_host_bits(y2), y)


# Tiled plans where K / 128 is a multiple of four, so that the activation
# scales are copied four K steps at a time (H = 512, I = 512: one such group
# in each GEMM; H = 1024, I = 1536: two and three), every tile height in both
# formats, with partial m-blocks at every height.
SCALE_GROUP_SHAPES = [(700, 512, 512, 16, 4), (300, 1024, 1536, 8, 2)]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("T,H,I,E,k", SCALE_GROUP_SHAPES)
def test_tiled_scale_groups(T, H, I, E, k, act):
    w, x, lg = _small(T, H, I, E, k, seed=T + H + act)
    layer = _layer(*w)
    for variant, rows in tune.candidates(act):
        if variant != moe.MOE_PLAN_TILED:
            continue
        moe.moe_set_plans(layer, [dict(act=act, top_k=k, t_max=T, variant=variant, rows=rows)])
        forward_and_check(layer, x, lg, k, act, host_weights(w),
                          what="tiled rows=%d T=%d H=%d I=%d act=%d" % (rows, T, H, I, act))


# Tiled plans with more items than workgroups (one per CU, 256) and K of 1 or 2
# steps of 128: a consumer wave's weight copies run NB - 1 = 3 steps ahead,
# so they reach into the next item and the one after it (MT <= 8), or
# re-read the last step until the next item issues its own (MT = 10).
MANY_ITEMS = [
    (0, 32, 4096, 256, 128, 64, 4),    # MT 2: ~512 GEMM1 items, S = 2 / 1
    (0, 96, 4096, 128, 512, 64, 4),    # MT 6: ~768 GEMM1 items, S = 1 / 4
    (0, 96, 8192, 128, 256, 64, 4),    # MT 6, I = 256: 8 A2 blocks a row
    (0, 160, 16384, 128, 128, 64, 4),  # MT 10: ~450 items
    (0, 192, 16384, 128, 128, 64, 4),  # MT 12: ~380 items, per-item prologue
    (1, 64, 8192, 256, 128, 64, 4),    # MXFP4 MT 4: ~512 items
    (1, 128, 16384, 128, 128, 64, 4),  # MXFP4 MT 8: ~512 items, S = 1 / 1
    (1, 96, 8192, 128, 256, 64, 4),    # MXFP4 MT 6, I = 256
]


@pytest.mark.parametrize("act,rows,T,H,I,E,k", MANY_ITEMS)
def test_tiled_many_items_per_workgroup(act, rows, T, H, I, E, k):
    w, x, lg = _small(T, H, I, E, k, seed=rows + T)
    layer = _layer(*w)
    moe.moe_set_plans(layer, [dict(act=act, top_k=k, t_max=T, variant=moe.MOE_PLAN_TILED,
                                   rows=rows)])
    what = "tiled rows=%d T=%d H=%d I=%d act=%d" % (rows, T, H, I, act)
    _, _, st = forward_and_check(layer, x, lg, k, act, host_weights(w), what=what)
    print(what, st)


# Plan DECODE (token-major GEMM2 with the combine folded in) at its limits:
# eight waves per item when the items outnumber the CUs (T * H / 32 > CUs)
# with top_k = 8 (one epilogue wave per slot, all eight busy), and sixteen
# waves at one token with top_k = 8; both formats; ragged: experts shared by
# the two tokens.
DECODE_TM_CASES = [(2, 5120, 256, 16, 8), (1, 2048, 384, 8, 8), (2, 7168, 128, 12, 5)]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("T,H,I,E,k", DECODE_TM_CASES)
def test_decode_plan_limits(T, H, I, E, k, act):
    w, x, lg = _small(T, H, I, E, k, seed=T * 13 + H + k)
    layer = _layer(*w)
    moe.moe_set_plans(layer, [dict(act=act, top_k=k, t_max=T, variant=moe.MOE_PLAN_DECODE,
                                   rows=16)])
    forward_and_check(layer, x, lg, k, act, host_weights(w),
                      what="decode limits T=%d H=%d I=%d E=%d k=%d act=%d" % (T, H, I, E, k, act))
    layer.close()
