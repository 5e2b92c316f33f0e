"""Plain float64 definition of the W4A8 variant of the MoE layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): slow, obviously
correct, written step by step from the definitions.

What it computes, and where it is stated:
  * The baseline deployment of the Ling model runs its MXFP4 experts with
    8-bit activations, "W4A8" ("3 Ways to Improve MoE Inference on NVIDIA DGX
    Spark" digest, section 2).  The layer is otherwise the W4A16 layer of
    moe_oracle (router, top-k, renormalised softmax, SwiGLU experts, shared
    expert, weighted combine).

Readings taken where the pages are silent:
  * The 8-bit activations are MXFP8 in the OCP microscaling sense: blocks of
    32 consecutive elements along the reduction axis share one E8M0 scale
    X = 2^(floor(log2 amax) - 8), where 8 is the exponent of E4M3's largest
    power of two; the exponent is clamped to the E8M0 range [-127, 127]; an
    all-zero block takes X = 2^-127.  Each element is the E4M3 code nearest to
    v / X (ties to the even mantissa), the quotient first clamped to +-448.
  * Quantised are the experts' inputs: x for the routed and shared experts
    (the router keeps the bf16 x, as the gate stays at high precision), and
    h = SiLU(g) * u for the down projection, quantised straight from its
    value (the pages say only "W4A8": no other rounding of h is implied).
  * Products and sums are then exact float64 arithmetic on the dequantised
    values.
"""
from __future__ import annotations

import numpy as np

from .lmhead_oracle import E4M3_MAX, e4m3_decode, e4m3_round
from .moe_oracle import (bf16_bits_to_f64, dequant_mxfp4, router_logits, silu, sort_by_expert,
                         topk_softmax)

MX_BLOCK = 32
E4M3_EMAX = 8            # E4M3's largest power of two is 2^8 (256 <= 448 < 512)
E8M0_MIN, E8M0_MAX = -127, 127


def bf16_round(v: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (8 significant bits, ties to even), as
    float64.  Normal binades keep 8 bits; below 2^-126 the quantum is fixed at
    the bf16 subnormal step 2^-133."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, fe = np.frexp(np.where(a > 0, a, 1.0))       # a = m * 2^fe, m in [0.5, 1): floor(log2 a) = fe - 1
    quantum = np.ldexp(1.0, np.maximum(fe - 1 - 7, -133).astype(np.int64))
    r = np.round(v / quantum) * quantum             # np.round: half to even; v / quantum is exact
    return np.where(a > 0, r, v)


def mxfp8_scale_exponent(block_amax: np.ndarray) -> np.ndarray:
    """E8M0 exponent of a block from its largest magnitude (see the header)."""
    a = np.asarray(block_amax, dtype=np.float64)
    _, fe = np.frexp(np.where(a > 0, a, 1.0))       # a = m * 2^fe, m in [0.5, 1): floor(log2 a) = fe - 1
    e = (fe - 1) - E4M3_EMAX
    e = np.clip(e, E8M0_MIN, E8M0_MAX)
    return np.where(a > 0, e, E8M0_MIN).astype(np.int64)


def mxfp8_quantize(v: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Rows of float64 values [..., K] (K % 32 == 0) -> (E4M3 codes uint8
    [..., K], E8M0 scale bytes uint8 [..., K/32]); block b of a row is
    elements [32b, 32b + 32)."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % MX_BLOCK == 0
    blocks = v.reshape(v.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    e = mxfp8_scale_exponent(np.max(np.abs(blocks), axis=-1))
    q = blocks / np.ldexp(1.0, e)[..., None]        # exact: a power-of-two division
    codes = e4m3_round(np.clip(q, -E4M3_MAX, E4M3_MAX))
    return codes.reshape(v.shape), (e + 127).astype(np.uint8)


def mxfp8_dequantize(codes: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """value = e4m3(code) * 2^(scale byte - 127), per 32-element block."""
    c = np.asarray(codes)
    K = c.shape[-1]
    vals = e4m3_decode(c).reshape(c.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    sc = np.ldexp(1.0, np.asarray(scale_bytes).astype(np.int64) - 127)
    return (vals * sc[..., None]).reshape(c.shape)


def mxfp8_fake_quant(v: np.ndarray) -> np.ndarray:
    """The value an MXFP8 round trip gives each element."""
    return mxfp8_dequantize(*mxfp8_quantize(v))


def expert_hidden(xq: np.ndarray, w13_q, w13_s) -> np.ndarray:
    """h = SiLU(g) * u of one expert for quantised input rows xq [n][H], before
    any rounding: g, u from the MXFP4 gate (rows 0..I-1) and up (I..2I-1)
    weights."""
    W13 = dequant_mxfp4(w13_q, w13_s)
    I = W13.shape[0] // 2
    return silu(xq @ W13[:I].T) * (xq @ W13[I:].T)


def expert_mlp_w4a8(xq: np.ndarray, w13_q, w13_s, w2_q, w2_s) -> np.ndarray:
    """One expert over already quantised input rows xq [n][H] (float64):
    h quantised to MXFP8 along I from its float64 value, then the down
    projection."""
    h = mxfp8_fake_quant(expert_hidden(xq, w13_q, w13_s))
    W2 = dequant_mxfp4(w2_q, w2_s)
    return h @ W2.T


def moe_layer_w4a8(x_bits, w_router, bias, w13_q, w13_s, w2_q, w2_s, k: int, shared: bool = True):
    """The W4A8 layer for all M tokens: routing on the bf16 x, experts on the
    MXFP8 x.  Returns dict(y float64 [M][H], ids, weights, logits, offsets,
    sorted_pairs, active, num_active, xq) with xq the quantised expert input."""
    xf = bf16_bits_to_f64(x_bits)
    E = np.asarray(w_router).shape[0]
    logits = router_logits(xf, w_router, bias)
    ids, w = topk_softmax(logits, k)
    offsets, pairs, active, D = sort_by_expert(ids, E)
    xq = mxfp8_fake_quant(xf)
    y = np.zeros_like(xf)
    wflat = w.ravel()
    for e in active:
        seg = pairs[offsets[e]:offsets[e + 1]]
        toks = seg // k
        out = expert_mlp_w4a8(xq[toks], w13_q[e], w13_s[e], w2_q[e], w2_s[e])
        np.add.at(y, toks, wflat[seg][:, None] * out)
    if shared:
        y += expert_mlp_w4a8(xq, w13_q[E], w13_s[E], w2_q[E], w2_s[E])
    return dict(y=y, ids=ids, weights=w, logits=logits, offsets=offsets,
                sorted_pairs=pairs, active=active, num_active=D, xq=xq)


def moe_layer_w4a8_tokens(tokens, x_bits, w_router, bias, w13_q, w13_s, w2_q, w2_s,
                          k: int, shared: bool = True):
    """moe_layer_w4a8 for a subset of token rows, one token at a time (tokens
    do not interact; the MXFP8 blocks of x run along a token's own row).
    bias may be None, [E] or [M][E] (indexed by the original row)."""
    xf_all = bf16_bits_to_f64(x_bits)
    E = np.asarray(w_router).shape[0]
    ys, ids_l, w_l, lg_l = [], [], [], []
    for t in tokens:
        b = None
        if bias is not None:
            b = bias if np.ndim(bias) == 1 else np.asarray(bias)[t]
        xf = xf_all[t:t + 1]
        logits = router_logits(xf, w_router, b)
        ids, w = topk_softmax(logits, k)
        xq = mxfp8_fake_quant(xf)
        y = np.zeros_like(xf)
        for s in range(k):
            e = int(ids[0, s])
            y += w[0, s] * expert_mlp_w4a8(xq, w13_q[e], w13_s[e], w2_q[e], w2_s[e])
        if shared:
            y += expert_mlp_w4a8(xq, w13_q[E], w13_s[E], w2_q[E], w2_s[E])
        ys.append(y[0]); ids_l.append(ids[0]); w_l.append(w[0]); lg_l.append(logits[0])
    return dict(y=np.array(ys), ids=np.array(ids_l), weights=np.array(w_l), logits=np.array(lg_l))
