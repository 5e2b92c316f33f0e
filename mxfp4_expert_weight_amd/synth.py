"""Seeded synthetic inputs for the MXFP4 expert-weight MoE decode layer.

This module only draws random inputs. It holds none of the layer's arithmetic
(no dequantisation, no routing, no expert MLP), so both the float64 oracle and
the HIP path can consume what it produces without sharing any of the method.

Workloads (shapes from the pages: 512 routed experts, top-8, one shared
expert, hidden 2560, moe_intermediate 768 -- "3 Ways to Improve MoE Inference
on NVIDIA DGX Spark" digest, sections 2 and 3; the 4-token verify window of
the MTP section 5):

  tiny            M=1   H=256  I=128 E=16  k=2  plain router, 1 set, seed 0
  ling_m1         M=1   H=2560 I=768 E=512 k=8  plain router
  ling_m4_mtp     M=4   same shapes, per-token logit bias steering the four
                        top-8 sets to overlap slot-by-slot with probability 0.3
  ling_m32_zipf   M=32  same shapes, per-expert Zipf(1.1) popularity bias
  ling_m512_prefill M=512 same shapes, plain router

Value recipe (all configs):
  x         bf16 bits of N(0,1) float32 samples, round-to-nearest-even
  w_router  float32 N(0, 0.02^2)
  codes     uniform random bytes (each nibble uniform over the 16 E2M1 codes)
  scales    E8M0 bytes uniform over [120, 127]
  The shared expert is stored at expert index E with the same format.

Every layer set l of a workload draws from
numpy PCG64(SeedSequence(seed).spawn(sets)[l]) in a fixed order:
x, w_router, logit bias, then the four expert-bank arrays
(w13 codes, w13 scales, w2 codes, w2 scales), each for all E+1 experts.
Drawing the banks last means ``banks=False`` reproduces x/router/bias exactly.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int          # tokens in the batch
    H: int          # hidden size (K of gate/up, N of down)
    I: int          # expert intermediate size
    E: int          # routed experts
    k: int          # experts kept per token
    shared: bool    # one always-on shared expert at index E
    routing: str    # "plain" | "overlap" | "zipf"
    sets: int       # distinct layer weight sets rotated per call
    seed: int


WORKLOADS = {
    "tiny": Workload("tiny", 1, 256, 128, 16, 2, True, "plain", 1, 0),
    "ling_m1": Workload("ling_m1", 1, 2560, 768, 512, 8, True, "plain", 40, 1),
    "ling_m4_mtp": Workload("ling_m4_mtp", 4, 2560, 768, 512, 8, True, "overlap", 40, 2),
    "ling_m32_zipf": Workload("ling_m32_zipf", 32, 2560, 768, 512, 8, True, "zipf", 40, 3),
    "ling_m512_prefill": Workload("ling_m512_prefill", 512, 2560, 768, 512, 8, True, "plain", 40, 4),
}

# Steering constants for the constructed router workloads.
OVERLAP_PROB = 0.3      # slot reuses an expert already chosen by an earlier token
OVERLAP_BIAS = 8.0      # additive logit bias on each token's chosen 8 experts
ZIPF_S = 1.1            # popularity exponent over expert ranks 1..E
ZIPF_BETA = 0.5         # bias_e = beta * ln p_e - max


@dataclass
class LayerSet:
    """One layer's inputs, canonical layouts (row-major, C-contiguous)."""
    wl: Workload
    x_bits: np.ndarray          # uint16 [M][H]      bf16 bit patterns
    w_router: np.ndarray        # float32 [E][H]
    bias: Optional[np.ndarray]  # None | float32 [E] | float32 [M][E]
    w13_q: Optional[np.ndarray] = None  # uint8 [E+1][2I][H/2]  (gate rows, then up rows)
    w13_s: Optional[np.ndarray] = None  # uint8 [E+1][2I][H/32]
    w2_q: Optional[np.ndarray] = None   # uint8 [E+1][H][I/2]
    w2_s: Optional[np.ndarray] = None   # uint8 [E+1][H][I/32]

    @property
    def bias_row_stride(self) -> int:
        if self.bias is None or self.bias.ndim == 1:
            return 0
        return self.bias.shape[1]


def rng_for(wl: Workload, set_idx: int) -> np.random.Generator:
    if not 0 <= set_idx < wl.sets:
        raise ValueError(f"set {set_idx} out of range for {wl.name} ({wl.sets} sets)")
    ss = np.random.SeedSequence(wl.seed).spawn(wl.sets)[set_idx]
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def random_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    words = (n + 7) // 8
    b = rng.integers(0, np.iinfo(np.uint64).max, size=words, dtype=np.uint64,
                     endpoint=True).view(np.uint8)[:n]
    return b.reshape(shape)


def random_scales(rng: np.random.Generator, shape) -> np.ndarray:
    """E8M0 exponent bytes uniform over [120, 127]."""
    return (random_bytes(rng, shape) & 7) + np.uint8(120)


def _overlap_bias(rng: np.random.Generator, M: int, E: int, k: int) -> np.ndarray:
    """Per-token bias steering each token's top-k set.

    Token 0 takes k distinct uniform experts.  For each later token, each of
    its k slots, with probability OVERLAP_PROB, reuses a uniformly chosen
    expert from the union of earlier tokens' sets that this token does not hold
    yet; otherwise it takes a fresh expert outside that union.
    """
    bias = np.zeros((M, E), dtype=np.float32)
    union: list[int] = []
    for t in range(M):
        mine: list[int] = []
        for _ in range(k):
            reuse_pool = [e for e in union if e not in mine]
            fresh = np.setdiff1d(np.arange(E), np.array(union + mine, dtype=np.int64))
            if t > 0 and reuse_pool and (rng.random() < OVERLAP_PROB or fresh.size == 0):
                mine.append(reuse_pool[rng.integers(len(reuse_pool))])
            else:
                mine.append(int(fresh[rng.integers(len(fresh))]))
        bias[t, mine] = OVERLAP_BIAS
        for e in mine:
            if e not in union:
                union.append(e)
    return bias


def _zipf_bias(rng: np.random.Generator, E: int) -> np.ndarray:
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-ZIPF_S)
    p /= p.sum()
    perm = rng.permutation(E)           # expert perm[r] has popularity rank r+1
    pe = np.empty(E)
    pe[perm] = p
    b = ZIPF_BETA * np.log(pe)
    return (b - b.max()).astype(np.float32)


def layer_set(wl: Workload | str, set_idx: int = 0, banks: bool = True) -> LayerSet:
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    rng = rng_for(wl, set_idx)
    x_bits = f32_to_bf16_bits(rng.standard_normal((wl.M, wl.H), dtype=np.float32))
    w_router = (rng.standard_normal((wl.E, wl.H), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    if wl.routing == "plain":
        bias = None
    elif wl.routing == "overlap":
        bias = _overlap_bias(rng, wl.M, wl.E, wl.k)
    elif wl.routing == "zipf":
        bias = _zipf_bias(rng, wl.E)
    else:
        raise ValueError(wl.routing)
    ls = LayerSet(wl, x_bits, w_router, bias)
    if banks:
        n = wl.E + 1
        ls.w13_q = random_bytes(rng, (n, 2 * wl.I, wl.H // 2))
        ls.w13_s = random_scales(rng, (n, 2 * wl.I, wl.H // 32))
        ls.w2_q = random_bytes(rng, (n, wl.H, wl.I // 2))
        ls.w2_s = random_scales(rng, (n, wl.H, wl.I // 32))
    return ls


def custom(name: str, M: int, H: int, I: int, E: int, k: int, shared: bool = True,
           routing: str = "plain", seed: int = 0, sets: int = 1) -> Workload:
    """A workload of arbitrary shape (edge-case tests: ragged tails, tiny E)."""
    if H % 32 or I % 32:
        raise ValueError("H and I must be multiples of the 32-element scale block")
    return Workload(name, M, H, I, E, k, shared, routing, sets, seed)


# --------------------------------------------------------------- LM head --
# The Ling LM head: 2,560 -> 157,184 (digest, section 2).
LMHEAD_VOCAB, LMHEAD_HIDDEN = 157184, 2560


@dataclass
class LmHeadSet:
    x_bits: np.ndarray       # bf16 [M][H]
    w_bits: np.ndarray       # bf16 [V][H] head weights (input of the quantiser)
    codes: np.ndarray        # uint8 [V][H] E4M3 codes, uniform over the 254 finite codes
    scales: np.ndarray       # fp32 [V], log-uniform in [2^-13, 2^-12) (near the quantiser's s = amax/448 of N(0, 0.02) rows)


def lmhead_set(M: int, V: int, H: int, seed: int) -> LmHeadSet:
    """x ~ N(0, 1) and head weights ~ N(0, 0.02), rounded to bf16; random
    finite E4M3 codes and row scales for the projection alone (independent of
    the weights, so the projection can be checked at any size)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    x = f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    w = f32_to_bf16_bits((rng.standard_normal((V, H)) * 0.02).astype(np.float32))
    codes = random_bytes(rng, (V, H))
    codes = np.where((codes & 0x7F) == 0x7F, codes ^ 0x01, codes).astype(np.uint8)   # no NaN codes
    scales = (2.0 ** rng.uniform(-13, -12, V)).astype(np.float32)
    return LmHeadSet(x, w, codes, scales)


def draft_ids(true_ids: np.ndarray, E: int, accuracy: float, rng: np.random.Generator) -> np.ndarray:
    """A synthetic draft pass's routing for a layer (int32 [T][k]), standing in
    for the draft model of speculative decoding (MoE-SpeQ article, 4.1): each
    (token, slot) keeps the layer's true expert with probability `accuracy`,
    else takes a uniformly random expert outside that token's true set and not
    yet in its draft set.  `true_ids` [T][k] are the layer's own routed ids."""
    true_ids = np.asarray(true_ids).reshape(-1, np.asarray(true_ids).shape[-1])
    out = np.empty_like(true_ids, dtype=np.int32)
    for t, row in enumerate(true_ids):
        taken = set(int(e) for e in row)
        for s, e in enumerate(row):
            if rng.random() < accuracy:
                out[t, s] = e
                continue
            while True:
                c = int(rng.integers(0, E))
                if c not in taken:
                    break
            taken.add(c)
            out[t, s] = c
    return out
