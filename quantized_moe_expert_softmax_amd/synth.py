"""Seeded synthetic inputs for the routed-expert MoE layer.

This module is shared by the tests, the benchmark and the oracle checks.  It
holds no step of the layer's arithmetic: it draws random numbers and random
MX code bytes from fixed distributions.

Workloads (the shapes the pages measure; there are no checkpoints, prompts or
datasets here, so these stand in for them):

* ``tiny``      T=16, H=256, I=128, E=8, top_k=2, A8W4.
* ``v4pro``     H=7168, I=3072, E=384, top_k=6 (the DeepSeek-V4-Pro expert
                shape of the Test Result of FlyDSL #972), decode T in {1,2,8,32,64}, prefill
                T in {512,1024,4096,8192} with uniform or skewed routing, A4W4
                at T in {1,64,512,1024,8192,16384}.
* ``v41flash``  H=5120, I in {640, 1152}, (E, top_k) in {(384, 6), (128, 3)}
                (the DSv4.1 TP-sharded shapes of aiter #6125 Changes), 16 token
                counts 1..32768, A8W4.

Value distributions:

* x ~ N(0, 1) in fp32, rounded to bf16 (torch's round-to-nearest-even cast).
* router logits ~ N(0, 1) fp32; "skewed" adds a fixed per-expert bias drawn
  from N(0, 1.5) (standard deviation 1.5), which gives a heavy-tailed expert
  load with some experts left empty.
* expert weights are drawn directly as MXFP4: each E2M1 code gets a uniform
  sign and a magnitude code with the frequencies that 1x32-block MXFP4
  quantisation of Gaussian weights produces (codes 0..7 = 0, 0.5, 1, 1.5, 2,
  3, 4, 6 in units of the block scale); each E8M0 byte is
  127 + floor(log2(1/sqrt(K)) - 1.3 + u) with u ~ U[0, 1), so the dequantised
  weights have a standard deviation near 1/sqrt(K) (K = H for the gate/up
  weights, K = I for the down weights).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterator

import numpy as np

# Magnitude-code frequencies in 1/128 units (codes 0..7).
_MAG_FREQ_128 = (11, 21, 19, 17, 20, 18, 14, 8)


def _nibble_table() -> np.ndarray:
    mag = np.repeat(np.arange(8, dtype=np.uint8), _MAG_FREQ_128)  # 128 entries
    assert mag.size == 128
    b = np.arange(256)
    return (mag[b & 127] | ((b >> 7) << 3)).astype(np.uint8)      # 8 random bits -> code


_NIB = _nibble_table()
# Two random bytes -> one packed byte (low nibble from the first byte).
_PAIR = (_NIB[np.arange(65536) & 255] | (_NIB[np.arange(65536) >> 8] << 4)).astype(np.uint8)


def _scale_table(K: int) -> np.ndarray:
    """Random byte b -> E8M0 byte 127 + floor(c + (b + 0.5) / 256)."""
    c = math.log2(1.0 / math.sqrt(K)) - 1.3
    u = (np.arange(256) + 0.5) / 256.0
    return (127 + np.floor(c + u)).astype(np.uint8)


def _fp4_codes(rng: np.random.Generator, nbytes: int) -> np.ndarray:
    raw = np.frombuffer(rng.bytes(2 * nbytes), dtype=np.uint16)
    return _PAIR[raw]


def _scales(rng: np.random.Generator, n: int, K: int) -> np.ndarray:
    raw = np.frombuffer(rng.bytes(n), dtype=np.uint8)
    return _scale_table(K)[raw]


def expert_weights(H: int, I: int, E: int, e: int, seed: int = 0):
    """Canonical MXFP4 weights of expert e of an (H, I, E) expert set.

    Returns w13 [2I, H/2] (rows [0, I) gate, [I, 2I) up; E2M1 pairs, even
    element in the low nibble), w13s [2I, H/32], w2 [H, I/2], w2s [H, I/32].
    Depends only on (H, I, E, e, seed), so every token count and activation
    format of a shape shares the same experts.
    """
    rng = np.random.default_rng([0x3E7, H, I, E, e, seed])
    w13 = _fp4_codes(rng, 2 * I * H // 2).reshape(2 * I, H // 2)
    w13s = _scales(rng, 2 * I * H // 32, H).reshape(2 * I, H // 32)
    w2 = _fp4_codes(rng, H * I // 2).reshape(H, I // 2)
    w2s = _scales(rng, H * I // 32, I).reshape(H, I // 32)
    return w13, w13s, w2, w2s


def all_weights(H: int, I: int, E: int, seed: int = 0):
    """Stacked canonical weights of every expert (small shapes only)."""
    parts = [expert_weights(H, I, E, e, seed) for e in range(E)]
    return tuple(np.stack([p[i] for p in parts]) for i in range(4))


def iter_weights(H: int, I: int, E: int, seed: int = 0) -> Iterator[tuple]:
    for e in range(E):
        yield expert_weights(H, I, E, e, seed)


def tokens_bf16(T: int, H: int, seed: int) -> np.ndarray:
    """x ~ N(0,1) rounded to bf16; returned as uint16 bit patterns [T, H]."""
    import torch
    rng = np.random.default_rng([0x51, T, H, seed])
    x = rng.standard_normal((T, H), dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def expert_bias(E: int, seed: int = 1234) -> np.ndarray:
    rng = np.random.default_rng([seed, E])
    return (rng.standard_normal(E) * 1.5).astype(np.float32)


def router_logits(T: int, E: int, seed: int, skewed: bool = False) -> np.ndarray:
    """Router logits [T, E] fp32 ~ N(0,1), plus the fixed expert bias when skewed."""
    rng = np.random.default_rng([0x10, T, E, seed])
    lg = rng.standard_normal((T, E), dtype=np.float32)
    if skewed:
        lg = (lg + expert_bias(E)[None, :]).astype(np.float32)
    return lg


def expert_ids(T: int, E: int, k: int, seed: int, hot: float = 0.0) -> np.ndarray:
    """Expert ids [T, k] int32: k distinct experts per token drawn uniformly
    from [0, E) (k <= E); with probability hot a token's first id becomes
    expert 0 (an overloaded expert), its ids staying distinct."""
    rng = np.random.default_rng([0x1D, T, E, k, seed])
    ids = np.zeros((T, k), np.int64)
    taken = np.zeros((T, 0), np.int64)
    for j in range(k):
        # a uniform pick among the E - j experts not yet taken: draw a rank and
        # step it past every taken id at or below it, in ascending order
        v = rng.integers(0, E - j, T)
        for c in range(j):
            v += v >= taken[:, c]
        ids[:, j] = v
        taken = np.sort(np.concatenate([taken, v[:, None]], axis=1), axis=1)
    if hot > 0:
        m = rng.random(T) < hot
        first = ids[:, 0].copy()
        for j in range(1, k):
            clash = m & (ids[:, j] == 0)
            ids[clash, j] = first[clash]
        ids[m, 0] = 0
    return ids.astype(np.int32)


# Activation formats (the library's act dtype values).
MXFP8 = 0  # A8W4
MXFP4 = 1  # A4W4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    I: int
    E: int
    top_k: int
    act: int
    Ts: tuple
    skewed: bool = False
    seed: int = 0

    def x(self, T: int) -> np.ndarray:
        return tokens_bf16(T, self.H, self.seed * 1000 + 1)

    def logits(self, T: int, rotation: int = 0) -> np.ndarray:
        return router_logits(T, self.E, self.seed * 1000 + 17 + rotation, self.skewed)


WORKLOADS = {
    "tiny": Workload("tiny", 256, 128, 8, 2, MXFP8, (16,), seed=1),
    "v4pro_decode": Workload("v4pro_decode", 7168, 3072, 384, 6, MXFP8, (1, 2, 8, 32, 64), seed=2),
    "v4pro_prefill": Workload("v4pro_prefill", 7168, 3072, 384, 6, MXFP8,
                              (512, 1024, 4096, 8192), seed=3),
    "v4pro_prefill_skewed": Workload("v4pro_prefill_skewed", 7168, 3072, 384, 6, MXFP8,
                                     (512, 1024, 4096, 8192), skewed=True, seed=3),
    "v4pro_a4w4": Workload("v4pro_a4w4", 7168, 3072, 384, 6, MXFP4,
                           (1, 64, 512, 1024, 8192, 16384), seed=4),
}
_FLASH_TS = tuple(2 ** i for i in range(16))
for _I in (640, 1152):
    for _E, _k in ((384, 6), (128, 3)):
        _n = "v41flash_i%d_e%d" % (_I, _E)
        WORKLOADS[_n] = Workload(_n, 5120, _I, _E, _k, MXFP8, _FLASH_TS, seed=5)


def device_weights(H: int, I: int, E: int, seed: int = 0, device="cuda", chunk: int = 8):
    """Canonical MXFP4 weights of a whole (H, I, E) expert set, drawn on the GPU.

    Same code and scale distributions as expert_weights(), drawn with torch's
    seeded device generator (much faster for the 13.5 GB expert sets; the
    values differ from the numpy path).  Returns uint8 device tensors
    w13 [E, 2I, H/2], w13s [E, 2I, H/32], w2 [E, H, I/2], w2s [E, H, I/32].
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((0x3E7 * 1000003 + H * 7919 + I * 104729 + E * 1299709 + seed) % (2 ** 62))
    pair = torch.from_numpy(_PAIR).to(device)
    s13 = torch.from_numpy(_scale_table(H)).to(device)
    s2 = torch.from_numpy(_scale_table(I)).to(device)
    w13 = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=device)
    w13s = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=device)
    w2 = torch.empty((E, H, I // 2), dtype=torch.uint8, device=device)
    w2s = torch.empty((E, H, I // 32), dtype=torch.uint8, device=device)

    def fill(dst, table, hi):
        flat = dst.view(-1)
        per = dst[0].numel()
        for e0 in range(0, E, chunk):
            n = min(chunk, E - e0) * per
            raw = torch.randint(0, hi, (n,), generator=g, device=device, dtype=torch.int64)
            flat[e0 * per:e0 * per + n] = table[raw]

    fill(w13, pair, 65536)
    fill(w13s, s13, 256)
    fill(w2, pair, 65536)
    fill(w2s, s2, 256)
    return w13, w13s, w2, w2s
