"""Plain float64 definition of the MXFP4 expert-weight MoE decode layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): slow, obviously
correct, written step by step from the definitions, with no blocking, fusion
or reordering beyond what a definition states.

What the layer computes, and where it is stated:
  * The decode MoE layer routes each token to 8 of 512 routed experts plus one
    shared expert ("3 Ways to Improve MoE Inference on NVIDIA DGX Spark"
    digest, section 2; the Vietnamese rewrite, "Mo hinh va dieu kien thu
    nghiem").
  * A gate network scores every expert and only the top-k are activated
    ("NVIDIA three-layer optimisation ... 42.5%" news rewrite, paragraph
    "sparse activation and expert routing"); the gate is kept at high precision
    because the softmax is sensitive to quantisation error (MoE-SpeQ article,
    section 2.1 table).
  * Expert weights are MXFP4 (digest, sections 2 and 3).  The pages name the
    format but do not define it; the encoding used here is the OCP
    Microscaling (MX) v1.0 one: E2M1 elements (sign bit, 2 exponent bits with
    bias 1, 1 mantissa bit) sharing one E8M0 scale 2^(s-127) per 32
    consecutive elements along the reduction axis.
  * All (token, expert) pairs are collected, sorted by expert id, and each
    expert runs once over its tokens (MoE-SpeQ article, section 4.2); the
    expert results are reduced across experts (section 3.2).
  * Each expert is a SwiGLU MLP: h = SiLU(x W_gate^T) * (x W_up^T),
    out = h W_down^T, combined with the renormalised routing weights; the
    shared expert is added with weight 1.  (The pages do not spell out the
    expert MLP; this is the plainest reading for a gate/up/down expert.)

Readings taken where the pages are silent:
  element 2j of a code byte is its low nibble; scale blocks run along K of a
  row-major [N][K] weight; gate rows are stacked before up rows in w13;
  top-k is chosen on logits (softmax is monotone) with ties to the lower
  expert index and slots ordered by descending logit; routed scaling factor
  1, shared-expert weight 1, no shared gate; activations are bf16 (W4A16)
  and are not quantised.
"""
from __future__ import annotations

import numpy as np

# E2M1 magnitudes for the 3-bit magnitude field (exponent:mantissa) 0..7.
E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
BLOCK = 32


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """A bf16 value is the upper 16 bits of an IEEE binary32; exact in float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit E2M1 code -> float64: bit 3 is the sign, bits 2..0 index the magnitude."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDE[c & 7]
    return np.where((c >> 3) & 1, -mag, mag)


def e8m0_decode(s: np.ndarray) -> np.ndarray:
    """E8M0 scale byte -> 2^(s-127); 255 encodes NaN."""
    s = np.asarray(s).astype(np.int64)
    v = np.ldexp(1.0, s - 127)
    return np.where(s == 255, np.nan, v)


def dequant_mxfp4(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """MXFP4 tensor [..., N, K/2] codes + [..., N, K/32] scales -> float64 [..., N, K].

    Element 2j of a row is the low nibble of code byte j, element 2j+1 the
    high nibble; element k uses scale byte k // 32 of its row.
    """
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.uint8)
    K = q.shape[-1] * 2
    if s.shape[-1] * BLOCK != K or s.shape[:-1] != q.shape[:-1]:
        raise ValueError(f"codes {q.shape} and scales {s.shape} do not describe one MXFP4 tensor")
    codes = np.empty(q.shape[:-1] + (K,), dtype=np.uint8)
    codes[..., 0::2] = q & 0x0F
    codes[..., 1::2] = q >> 4
    scale = np.repeat(e8m0_decode(s), BLOCK, axis=-1)
    return e2m1_decode(codes) * scale


def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """logits[t][e] = x_t . W_r[e] + bias (bias: None, [E] or [M][E]); float64."""
    logits = np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)
    return logits


def topk_softmax(logits: np.ndarray, k: int):
    """Top-k experts per token and their renormalised softmax weights.

    Selection is on logits: descending, ties to the lower expert index.  The
    weights are softmax restricted to the kept experts,
    w_i = exp(l_i - l_max) / sum_{j in top-k} exp(l_j - l_max),
    which equals the full softmax renormalised over the kept set.
    Returns (ids int32 [M][k], weights float64 [M][k]).
    """
    logits = np.asarray(logits, dtype=np.float64)
    if not np.all(np.isfinite(logits)):
        raise ValueError("non-finite logits")
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    top = np.take_along_axis(logits, order, axis=1)
    ex = np.exp(top - top[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w


def sort_by_expert(ids: np.ndarray, E: int):
    """Stable counting sort of the flattened (token, slot) pairs p = t*k + s by expert.

    Returns (expert_offsets int32 [E+1], sorted_pairs int32 [M*k],
    active_experts int32 [D] ascending, D).
    """
    flat = np.asarray(ids).ravel().astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    sorted_pairs = np.argsort(flat, kind="stable").astype(np.int32)
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    active = np.nonzero(counts)[0].astype(np.int32)
    return offsets, sorted_pairs, active, int(active.size)


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g), evaluated without overflow for large |g|."""
    g = np.asarray(g, dtype=np.float64)
    e = np.exp(-np.abs(g))                       # in (0, 1]
    sig = np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return g * sig


def expert_mlp(xf: np.ndarray, w13_q, w13_s, w2_q, w2_s) -> np.ndarray:
    """One expert over token rows xf [n][H] (float64) -> [n][H].

    w13 holds W_gate (rows 0..I-1) then W_up (rows I..2I-1), each [I][H];
    w2 is W_down [H][I].  Linear maps use out = in W^T: out[j] = sum_k W[j][k] in[k].
    """
    W13 = dequant_mxfp4(w13_q, w13_s)
    I = W13.shape[0] // 2
    g = xf @ W13[:I].T
    u = xf @ W13[I:].T
    h = silu(g) * u
    W2 = dequant_mxfp4(w2_q, w2_s)
    return h @ W2.T


def moe_layer(x_bits, w_router, bias, w13_q, w13_s, w2_q, w2_s, k: int, shared: bool = True):
    """The whole layer for all M tokens.

    Returns dict(y float64 [M][H], ids, weights, logits, offsets, sorted_pairs,
    active, num_active).
    """
    xf = bf16_bits_to_f64(x_bits)
    M = xf.shape[0]
    E = np.asarray(w_router).shape[0]
    logits = router_logits(xf, w_router, bias)
    ids, w = topk_softmax(logits, k)
    offsets, pairs, active, D = sort_by_expert(ids, E)
    y = np.zeros_like(xf)
    wflat = w.ravel()
    for e in active:
        seg = pairs[offsets[e]:offsets[e + 1]]
        toks = seg // k
        out = expert_mlp(xf[toks], w13_q[e], w13_s[e], w2_q[e], w2_s[e])
        np.add.at(y, toks, wflat[seg][:, None] * out)
    if shared:
        y += expert_mlp(xf, w13_q[E], w13_s[E], w2_q[E], w2_s[E])
    return dict(y=y, ids=ids, weights=w, logits=logits, offsets=offsets,
                sorted_pairs=pairs, active=active, num_active=D)


def moe_layer_tokens(tokens, x_bits, w_router, bias, w13_q, w13_s, w2_q, w2_s,
                     k: int, shared: bool = True):
    """The layer output for a subset of token rows, one token at a time.

    Tokens do not interact in the layer, so y_t depends on row t only; this is
    the same definition as moe_layer evaluated per token (used to sample large
    batches).  bias may be None, [E] or [M][E] (indexed by the original row).
    Returns dict(y [len(tokens)][H], ids, weights, logits).
    """
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
        y = np.zeros_like(xf)
        for s in range(k):
            e = int(ids[0, s])
            y += w[0, s] * expert_mlp(xf, w13_q[e], w13_s[e], w2_q[e], w2_s[e])
        if shared:
            y += expert_mlp(xf, w13_q[E], w13_s[E], w2_q[E], w2_s[E])
        ys.append(y[0]); ids_l.append(ids[0]); w_l.append(w[0]); lg_l.append(logits[0])
    return dict(y=np.array(ys), ids=np.array(ids_l), weights=np.array(w_l), logits=np.array(lg_l))
