"""The seeded input generators: the same seed gives the same inputs (every
test and benchmark depends on it), different seeds give different ones, and
the draws have the shapes and distributions the workloads state."""
import numpy as np

from quantized_moe_expert_softmax_amd import synth


def test_same_seed_same_inputs():
    for f in (lambda s: synth.tokens_bf16(37, 256, s), lambda s: synth.router_logits(37, 16, s),
              lambda s: synth.router_logits(37, 16, s, skewed=True),
              lambda s: synth.expert_ids(37, 16, 4, s)):
        assert np.array_equal(f(5), f(5))
        assert not np.array_equal(f(5), f(6))
    a, b = synth.all_weights(256, 128, 4, seed=3), synth.all_weights(256, 128, 4, seed=3)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
    c = synth.all_weights(256, 128, 4, seed=4)
    assert not np.array_equal(a[0], c[0])


def test_expert_weights_do_not_depend_on_the_set_size_drawn():
    # expert e's weights are drawn from its own stream: the stacked set and the
    # per-expert draw agree
    w = synth.all_weights(256, 128, 4, seed=7)
    for e in range(4):
        one = synth.expert_weights(256, 128, 4, e, seed=7)
        assert all(np.array_equal(s[e], o) for s, o in zip(w, one))


def test_shapes_and_distributions():
    T, H, I, E = 512, 256, 128, 8
    x = synth.tokens_bf16(T, H, 1)
    assert x.shape == (T, H) and x.dtype == np.uint16
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    assert abs(xf.mean()) < 0.02 and abs(xf.std() - 1.0) < 0.02  # N(0, 1) in bf16
    lg = synth.router_logits(T, E, 2)
    assert lg.shape == (T, E) and lg.dtype == np.float32 and abs(lg.std() - 1.0) < 0.05
    w13, w13s, w2, w2s = synth.all_weights(H, I, E, seed=0)
    assert w13.shape == (E, 2 * I, H // 2) and w13s.shape == (E, 2 * I, H // 32)
    assert w2.shape == (E, H, I // 2) and w2s.shape == (E, H, I // 32)
    assert all(a.dtype == np.uint8 for a in (w13, w13s, w2, w2s))
    ids = synth.expert_ids(T, E, 4, 3)
    assert ids.shape == (T, 4)
    assert all(len(set(r)) == 4 for r in ids)  # k distinct experts per token


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with a message before any
    device work."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
