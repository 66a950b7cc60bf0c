"""GPU parity of the integer-exact stages against the oracle (bit-exact):
routing ids (weights within a few ulp), the expert sort and the 1x32 MX
activation quantisation, through the C-ABI stage entry points."""
import numpy as np
import pytest

import oracle
from quantized_moe_expert_softmax_amd import synth
from tests.gpu_util import ROUTE_ULP_TOL, bf16_dev, dev, host, ulp_diff

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import quantized_moe_expert_softmax_amd as m
    m.load_library()
    return m


ROUTE_CASES = [(16, 8, 2, False), (64, 384, 6, False), (1000, 128, 3, False), (33, 1024, 8, False),
               (4096, 384, 6, True), (7, 5, 5, False), (1, 384, 1, False), (300, 65, 4, False)]


@pytest.mark.parametrize("T,E,k,skew", ROUTE_CASES)
def test_route(moe, T, E, k, skew):
    lg = synth.router_logits(T, E, T + E, skewed=skew)
    ids, w = moe.moe_route(dev(lg), k)
    rid, rw = oracle.route(lg, k)
    assert np.array_equal(host(ids), rid)
    assert ulp_diff(host(w), rw).max() <= ROUTE_ULP_TOL


def test_route_ties(moe):
    lg = np.zeros((3, 200), np.float32)
    lg[0, [150, 3, 77]] = 2.0
    lg[1, :] = -1.0
    lg[2, 64:130] = 5.0
    ids, w = moe.moe_route(dev(lg), 4)
    rid, rw = oracle.route(lg, 4)
    assert np.array_equal(host(ids), rid)
    assert ulp_diff(host(w), rw).max() <= ROUTE_ULP_TOL


def test_route_signed_zero_ties(moe):
    # -0 and +0 compare equal: equal logits go by the lower expert index
    lg = np.full((2, 130), -1.0, np.float32)
    lg[0, [5, 3, 1]] = [-0.0, 0.0, -0.0]
    lg[1, [129, 64, 0]] = [0.0, -0.0, 0.0]
    ids, w = moe.moe_route(dev(lg), 3)
    rid, rw = oracle.route(lg, 3)
    assert np.array_equal(host(ids), rid)
    assert host(ids)[0].tolist() == [1, 3, 5] and host(ids)[1].tolist() == [0, 64, 129]
    assert ulp_diff(host(w), rw).max() <= ROUTE_ULP_TOL


def test_route_nan_rows_pick_valid_experts(moe):
    # NaN logits are outside the contract (the picks of such a row are
    # unspecified), but the ids stay distinct experts below E
    E, k = 200, 8
    lg = np.random.default_rng(11).standard_normal((6, E)).astype(np.float32)
    bits = lg.view(np.uint32)
    bits[0, :] = 0xFFFFFFFF
    bits[1, ::3] = 0x7FC00000
    bits[2, 190:] = 0xFFFFFFFF
    bits[3, :8] = 0xFFC00001
    bits[4, 100] = 0x7F800001
    ids = host(moe.moe_route(dev(lg), k)[0])
    assert ids.min() >= 0 and ids.max() < E
    assert all(len(set(r.tolist())) == k for r in ids)
    # the rows without NaN still match the oracle
    rid, _ = oracle.route(lg[5:], k)
    assert np.array_equal(ids[5:], rid)


SORT_CASES = [(1, 8, 2), (16, 8, 2), (255, 384, 6), (256, 384, 6), (257, 384, 6), (4096, 384, 6),
              (8192, 128, 3), (32768, 384, 6), (100, 1024, 8), (3, 1, 1)]


@pytest.mark.parametrize("T,E,k", SORT_CASES)
def test_sort(moe, T, E, k):
    lg = synth.router_logits(T, E, 7 * T + E, skewed=(T % 2 == 0 and E >= 8))
    rid, _ = oracle.route(lg, k)
    counts, offsets, perm = moe.moe_sort(dev(rid), E)
    rc, ro, rp = oracle.sort(rid, E)
    assert np.array_equal(host(counts), rc)
    assert np.array_equal(host(offsets), ro)
    assert np.array_equal(host(perm), rp)


# The largest sizes the interface takes (T = 2^20 tokens, E = 1024 experts,
# top_k = 8): a uniform spread, one expert holding about a third of the 8M
# assignments, every token on every expert, one expert only.
SORT_LIMIT_CASES = [(1 << 20, 1024, 8, 0.0), (1 << 20, 1024, 8, 0.3), (1 << 20, 8, 8, 0.0),
                    (1 << 16, 1, 1, 0.0)]


@pytest.mark.parametrize("T,E,k,hot", SORT_LIMIT_CASES)
def test_sort_limits(moe, T, E, k, hot):
    rid = synth.expert_ids(T, E, k, seed=E + k, hot=hot)
    counts, offsets, perm = moe.moe_sort(dev(rid), E)
    rc, ro, rp = oracle.sort(rid, E)
    assert np.array_equal(host(counts), rc)
    assert np.array_equal(host(offsets), ro)
    assert np.array_equal(host(perm), rp)


def _special_bf16_rows(H):
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    finite = (bits[np.isfinite(f)]).astype(np.uint16)
    n = -(-finite.size // H) * H
    rows = np.zeros(n, np.uint16)
    rows[:finite.size] = finite
    return rows.reshape(-1, H)


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("T,H", [(1, 128), (16, 256), (64, 7168), (513, 5120), (8192, 7168)])
def test_quant_random(moe, act, T, H):
    x = synth.tokens_bf16(T, H, T + H)
    codes, scales = moe.moe_quant_act(bf16_dev(x), act)
    rc, rs = oracle.mx_quantize_bf16(x, act)
    assert np.array_equal(host(scales), rs)
    assert np.array_equal(host(codes), rc)


@pytest.mark.parametrize("act", [0, 1])
def test_quant_every_bf16(moe, act):
    """Every finite bf16 pattern, in blocks mixing magnitudes, zeros, -0 and subnormals."""
    x = _special_bf16_rows(1024)
    rng = np.random.default_rng(0)
    shuffled = x.reshape(-1)[rng.permutation(x.size)].reshape(x.shape)
    for arr in (x, shuffled):
        codes, scales = moe.moe_quant_act(bf16_dev(arr), act)
        rc, rs = oracle.mx_quantize_bf16(arr, act)
        assert np.array_equal(host(scales), rs)
        assert np.array_equal(host(codes), rc)


@pytest.mark.parametrize("act", [0, 1])
def test_quant_scaled_blocks(moe, act):
    """Blocks whose amax sits at every binade, so every element binade and tie occurs."""
    rng = np.random.default_rng(1)
    H = 1024
    x = rng.standard_normal((64, H)).astype(np.float32)
    x *= np.exp2(rng.integers(-130, 120, size=(64, H // 32)))[:, :, None].repeat(32, 2).reshape(64, H)
    import torch
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, scales = moe.moe_quant_act(bf16_dev(xb), act)
    rc, rs = oracle.mx_quantize_bf16(xb, act)
    assert np.array_equal(host(scales), rs)
    assert np.array_equal(host(codes), rc)


def test_stage_determinism(moe):
    T, E, k, H = 4096, 384, 6, 7168
    lg = dev(synth.router_logits(T, E, 3, skewed=True))
    x = bf16_dev(synth.tokens_bf16(T, H, 3))
    a = moe.moe_route(lg, k)
    b = moe.moe_route(lg, k)
    assert all(np.array_equal(host(p), host(q)) for p, q in zip(a, b))
    s1 = moe.moe_sort(a[0], E)
    s2 = moe.moe_sort(a[0], E)
    assert all(np.array_equal(host(p), host(q)) for p, q in zip(s1, s2))
    q1 = moe.moe_quant_act(x, 0)
    q2 = moe.moe_quant_act(x, 0)
    assert all(np.array_equal(host(p), host(q)) for p, q in zip(q1, q2))
