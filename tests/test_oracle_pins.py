"""Pins for the float64 oracle: every check compares it with something other
than itself -- bit-field decoding written independently of the oracle's table,
hand-worked fixtures under tests/golden/, brute force in plain Python loops on
tiny inputs, closed forms and exact power-of-two metamorphics."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from mxfp4_expert_weight_amd import synth


# ---------------------------------------------------------------- dequant --

def e2m1_bitfield(c: int) -> float:
    """E2M1 from its bit fields: sign | 2-bit exponent (bias 1) | 1-bit mantissa."""
    sign = -1.0 if (c >> 3) & 1 else 1.0
    e = (c >> 1) & 3
    m = c & 1
    if e == 0:
        return sign * 0.5 * m                      # subnormal: 0 or 0.5
    return sign * math.ldexp(1.0 + 0.5 * m, e - 1)


def test_e2m1_value_set_is_the_mxfp4_table():
    vals = {oracle.e2m1_decode(np.array([c]))[0] for c in range(16)}
    assert vals == {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0}


def test_dequant_exhaustive_codes_and_scales():
    # every code in both nibble positions, every finite scale byte
    for s in range(0, 255):
        q = np.zeros((16, 16), dtype=np.uint8)        # 16 rows x 32 elements
        for c in range(16):
            q[c, :] = c | (((c + 5) & 15) << 4)
        sc = np.full((16, 1), s, dtype=np.uint8)
        got = oracle.dequant_mxfp4(q, sc)
        for c in range(16):
            lo = e2m1_bitfield(c) * math.ldexp(1.0, s - 127)
            hi = e2m1_bitfield((c + 5) & 15) * math.ldexp(1.0, s - 127)
            assert np.all(got[c, 0::2] == lo) and np.all(got[c, 1::2] == hi), (c, s)


def test_dequant_scale_255_is_nan():
    got = oracle.dequant_mxfp4(np.array([[0x72] * 16], np.uint8), np.array([[255]], np.uint8))
    assert np.all(np.isnan(got))


def test_dequant_handworked_bytes(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "dequant_handworked.json")))
    for case in d["cases"]:
        b = int(case["byte"], 16)
        q = np.full((1, 16), b, dtype=np.uint8)
        sc = np.array([[case["scale"]]], dtype=np.uint8)
        got = oracle.dequant_mxfp4(q, sc)[0]
        assert got[0] == case["values"][0] and got[1] == case["values"][1], case
        assert np.all(got[0::2] == got[0]) and np.all(got[1::2] == got[1])


def test_dequant_scale_block_runs_along_k():
    # scale byte j of a row applies to elements 32j .. 32j+31 of that row only
    q = np.full((2, 64), 0x22, dtype=np.uint8)       # every element 1.0, K = 128
    sc = np.array([[127, 128, 129, 130], [120, 121, 122, 123]], dtype=np.uint8)
    got = oracle.dequant_mxfp4(q, sc)
    for r in range(2):
        for j in range(4):
            assert np.all(got[r, 32 * j:32 * (j + 1)] == 2.0 ** (int(sc[r, j]) - 127))


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3E80, 0x7F7F, 0x0001], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 0.25, 3.3895313892515355e38, 2.0 ** -133]
    assert list(oracle.bf16_bits_to_f64(bits)) == want


# ---------------------------------------------------------------- routing --

def test_routing_handworked(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "routing_handworked.json")))
    for case in d["cases"]:
        ids, w = oracle.topk_softmax(np.array([case["logits"]]), case["k"])
        assert list(ids[0]) == case["ids"], case
        np.testing.assert_allclose(w[0], case["weights"], rtol=0, atol=1e-15)


def brute_topk(l, k):
    """Enumerate every k-subset; keep the max-sum one, lowest indices among ties."""
    best = None
    for S in itertools.combinations(range(len(l)), k):      # lexicographic order
        sc = sum(l[e] for e in S)
        if best is None or sc > best[0]:
            best = (sc, S)
    chosen = sorted(best[1], key=lambda e: (-l[e], e))
    z = sum(math.exp(l[e] - l[chosen[0]]) for e in chosen)
    return chosen, [math.exp(l[e] - l[chosen[0]]) / z for e in chosen]


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    for E, k in [(4, 1), (6, 2), (8, 3), (12, 4), (16, 2)]:
        # integer-valued logits force plenty of exact ties
        logits = rng.integers(-3, 4, size=(5, E)).astype(np.float64)
        ids, w = oracle.topk_softmax(logits, k)
        for t in range(5):
            bids, bw = brute_topk(list(logits[t]), k)
            assert list(ids[t]) == bids
            np.testing.assert_allclose(w[t], bw, rtol=0, atol=1e-14)


def test_topk_invariants():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((50, 512)) * 1.01
    ids, w = oracle.topk_softmax(logits, 8)
    assert np.all(np.abs(w.sum(1) - 1) < 1e-12)
    assert np.all(np.diff(np.take_along_axis(logits, ids.astype(np.int64), 1), axis=1) <= 0)
    assert all(len(set(r)) == 8 for r in ids)
    # equals the full softmax renormalised over the kept experts
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    pk = np.take_along_axis(p, ids.astype(np.int64), 1)
    np.testing.assert_allclose(w, pk / pk.sum(1, keepdims=True), rtol=1e-12)
    # adding a constant to all logits of a token changes nothing
    ids2, w2 = oracle.topk_softmax(logits + 3.25, 8)
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=1e-12)


def test_router_logits_bias_forms():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 64))
    wr = rng.standard_normal((10, 64)).astype(np.float32)
    b1 = rng.standard_normal(10).astype(np.float32)
    l0 = oracle.router_logits(x, wr)
    np.testing.assert_array_equal(oracle.router_logits(x, wr, b1), l0 + b1.astype(np.float64))
    np.testing.assert_array_equal(oracle.router_logits(x, wr, np.tile(b1, (3, 1))), l0 + b1.astype(np.float64))
    # dot products written out by hand
    for t in range(3):
        for e in range(10):
            assert abs(l0[t, e] - sum(x[t, i] * float(wr[e, i]) for i in range(64))) < 1e-12


# ---------------------------------------------------------------- sort --

def test_sort_matches_brute_force():
    rng = np.random.default_rng(11)
    for M, k, E in [(1, 2, 16), (4, 8, 512), (32, 8, 64), (7, 3, 5), (1, 1, 1)]:
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(M)]).astype(np.int32)
        off, pairs, active, D = oracle.sort_by_expert(ids, E)
        flat = list(ids.ravel())
        want = sorted(range(M * k), key=lambda p: (flat[p], p))
        assert list(pairs) == want
        assert off[0] == 0 and off[-1] == M * k and np.all(np.diff(off) >= 0)
        for e in range(E):
            assert off[e + 1] - off[e] == flat.count(e)
        assert list(active) == sorted(set(flat)) and D == len(set(flat))


# ---------------------------------------------------------------- expert MLP --

def test_silu_closed_forms():
    g = np.array([0.0, 2.0, -1.0, 800.0, -800.0, 40.0])
    got = oracle.silu(g)
    assert got[0] == 0.0
    assert abs(got[1] - 1.761594155955764888) < 1e-15     # 2e^2/(1+e^2)
    assert abs(got[2] + 0.268941421369995120) < 1e-16     # -1/(1+e)
    assert got[3] == 800.0 and got[4] == -0.0 and np.isfinite(got).all()
    assert abs(got[5] - 40.0) < 1e-15


def _mxfp4_from_entries(N, K, entries):
    q = np.zeros((N, K // 2), dtype=np.uint8)
    s = np.full((N, K // 32), 127, dtype=np.uint8)
    for r, c, code, sc in entries:
        if c % 2 == 0:
            q[r, c // 2] |= code
        else:
            q[r, c // 2] |= code << 4
        s[r, c // 32] = sc
    return q, s


def test_expert_mlp_handworked(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "mlp_handworked.json")))
    H, I = d["H"], d["I"]
    x = np.zeros((1, H))
    for i, v in d["x_nonzero"]:
        x[0, i] = v
    gate_q, gate_s = _mxfp4_from_entries(I, H, d["gate"])
    up_q, up_s = _mxfp4_from_entries(I, H, d["up"])
    w13_q = np.concatenate([gate_q, up_q]); w13_s = np.concatenate([gate_s, up_s])
    w2_q, w2_s = _mxfp4_from_entries(H, I, d["down"])
    y = oracle.expert_mlp(x, w13_q, w13_s, w2_q, w2_s)[0]
    want = np.zeros(H)
    for j, v in d["y_nonzero"]:
        want[j] = float(v)
    np.testing.assert_allclose(y, want, rtol=1e-15, atol=0)


# ------------------------------------------------- whole layer, brute force --

def _brute_layer(ls, k):
    """Plain-Python-loop evaluation of the layer on a tiny LayerSet."""
    M, H = ls.x_bits.shape
    E = ls.w_router.shape[0]
    I = ls.w13_q.shape[1] // 2

    def xval(b):
        return float(np.frombuffer(np.uint32(int(b) << 16).tobytes(), np.float32)[0])

    def wval(q, s, r, c):
        byte = int(q[r, c // 2])
        code = byte & 15 if c % 2 == 0 else byte >> 4
        return e2m1_bitfield(code) * math.ldexp(1.0, int(s[r, c // 32]) - 127)

    def mlp(e, xv):
        h = []
        for j in range(I):
            g = sum(wval(ls.w13_q[e], ls.w13_s[e], j, c) * xv[c] for c in range(H))
            u = sum(wval(ls.w13_q[e], ls.w13_s[e], I + j, c) * xv[c] for c in range(H))
            h.append(g / (1.0 + math.exp(-g)) * u)
        return [sum(wval(ls.w2_q[e], ls.w2_s[e], r, j) * h[j] for j in range(I)) for r in range(H)]

    ys = []
    for t in range(M):
        xv = [xval(b) for b in ls.x_bits[t]]
        logits = []
        for e in range(E):
            b = 0.0
            if ls.bias is not None:
                b = float(ls.bias[e] if ls.bias.ndim == 1 else ls.bias[t, e])
            logits.append(sum(xv[c] * float(ls.w_router[e, c]) for c in range(H)) + b)
        chosen, w = brute_topk(logits, k)
        y = [0.0] * H
        for e, we in zip(chosen, w):
            out = mlp(e, xv)
            y = [a + we * o for a, o in zip(y, out)]
        if ls.wl.shared:
            out = mlp(E, xv)
            y = [a + o for a, o in zip(y, out)]
        ys.append(y)
    return np.array(ys)


@pytest.mark.parametrize("routing", ["plain", "zipf", "overlap"])
def test_layer_matches_brute_force_loops(routing):
    wl = synth.custom("brute", M=3, H=32, I=32, E=5, k=2, routing=routing, seed=21)
    ls = synth.layer_set(wl)
    got = oracle.moe_layer(ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s,
                           ls.w2_q, ls.w2_s, wl.k, wl.shared)["y"]
    want = _brute_layer(ls, wl.k)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11 * np.abs(want).max())


def test_layer_dense_equals_sparse_tiny():
    """Run every expert and combine with a dense weight vector that is zero off
    the top-k: equals the sparse (sorted, deduplicated) evaluation."""
    ls = synth.layer_set("tiny")
    wl = ls.wl
    r = oracle.moe_layer(ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s,
                         ls.w2_q, ls.w2_s, wl.k, wl.shared)
    xf = oracle.bf16_bits_to_f64(ls.x_bits)
    dense_w = np.zeros((wl.M, wl.E))
    np.put_along_axis(dense_w, r["ids"].astype(np.int64), r["weights"], 1)
    y = np.zeros_like(xf)
    for e in range(wl.E):
        y += dense_w[:, e:e + 1] * oracle.expert_mlp(xf, ls.w13_q[e], ls.w13_s[e], ls.w2_q[e], ls.w2_s[e])
    y += oracle.expert_mlp(xf, ls.w13_q[wl.E], ls.w13_s[wl.E], ls.w2_q[wl.E], ls.w2_s[wl.E])
    np.testing.assert_allclose(r["y"], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_layer_single_expert_reduces_to_dense_swiglu():
    wl = synth.custom("dense1", M=6, H=64, I=96, E=1, k=1, shared=False, seed=5)
    ls = synth.layer_set(wl)
    r = oracle.moe_layer(ls.x_bits, ls.w_router, None, ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s, 1, False)
    assert np.all(r["weights"] == 1.0) and np.all(r["ids"] == 0)
    xf = oracle.bf16_bits_to_f64(ls.x_bits)
    Wg = oracle.dequant_mxfp4(ls.w13_q[0, :96], ls.w13_s[0, :96])
    Wu = oracle.dequant_mxfp4(ls.w13_q[0, 96:], ls.w13_s[0, 96:])
    Wd = oracle.dequant_mxfp4(ls.w2_q[0], ls.w2_s[0])
    g = np.einsum("mk,nk->mn", xf, Wg)
    want = np.einsum("mn,hn->mh", g * (1 / (1 + np.exp(-g))) * np.einsum("mk,nk->mn", xf, Wu), Wd)
    np.testing.assert_allclose(r["y"], want, rtol=1e-11, atol=1e-11 * np.abs(want).max())


def _layer(ls, **over):
    a = dict(x_bits=ls.x_bits, w_router=ls.w_router, bias=ls.bias, w13_q=ls.w13_q,
             w13_s=ls.w13_s, w2_q=ls.w2_q, w2_s=ls.w2_s)
    a.update(over)
    return oracle.moe_layer(a["x_bits"], a["w_router"], a["bias"], a["w13_q"], a["w13_s"],
                            a["w2_q"], a["w2_s"], ls.wl.k, ls.wl.shared)["y"]


def test_metamorphic_power_of_two_scales():
    wl = synth.custom("meta", M=4, H=64, I=64, E=6, k=2, routing="plain", seed=9)
    ls = synth.layer_set(wl)
    y = _layer(ls)
    # doubling every down-projection scale doubles y exactly
    assert np.array_equal(_layer(ls, w2_s=ls.w2_s + 1), 2 * y)
    # doubling every up-row scale doubles u, hence h and y, exactly
    s_up = ls.w13_s.copy(); s_up[:, wl.I:] += 1
    assert np.array_equal(_layer(ls, w13_s=s_up), 2 * y)
    # the gate goes through SiLU, so doubling gate scales does not double y
    s_g = ls.w13_s.copy(); s_g[:, :wl.I] += 1
    assert not np.allclose(_layer(ls, w13_s=s_g), 2 * y, rtol=1e-3)


def test_metamorphic_expert_permutation():
    wl = synth.custom("perm", M=4, H=64, I=32, E=7, k=3, routing="plain", seed=13)
    ls = synth.layer_set(wl)
    perm = np.random.default_rng(1).permutation(wl.E)
    full = np.concatenate([perm, [wl.E]])              # shared stays last
    y2 = _layer(ls, w_router=ls.w_router[perm], w13_q=ls.w13_q[full], w13_s=ls.w13_s[full],
                w2_q=ls.w2_q[full], w2_s=ls.w2_s[full])
    np.testing.assert_allclose(y2, _layer(ls), rtol=1e-13, atol=1e-13 * np.abs(y2).max())


def test_token_independence_and_sampled_tokens():
    wl = synth.custom("tok", M=5, H=64, I=32, E=8, k=2, routing="overlap", seed=17)
    ls = synth.layer_set(wl)
    full = oracle.moe_layer(ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s,
                            ls.w2_q, ls.w2_s, wl.k, wl.shared)
    sub = oracle.moe_layer_tokens([3, 0], ls.x_bits, ls.w_router, ls.bias, ls.w13_q,
                                  ls.w13_s, ls.w2_q, ls.w2_s, wl.k, wl.shared)
    np.testing.assert_allclose(sub["y"], full["y"][[3, 0]], rtol=1e-12, atol=1e-12 * np.abs(sub["y"]).max())
    assert np.array_equal(sub["ids"], full["ids"][[3, 0]])
    one = oracle.moe_layer(ls.x_bits[2:3], ls.w_router, ls.bias[2:3], ls.w13_q, ls.w13_s,
                           ls.w2_q, ls.w2_s, wl.k, wl.shared)
    np.testing.assert_allclose(one["y"][0], full["y"][2], rtol=1e-12, atol=1e-12 * np.abs(one["y"]).max())
