"""Pins of the W4A8 oracle (CPU).

The MXFP8 quantiser against hand-worked blocks and against brute-force nearest
search over the 254 finite E4M3 values; the bf16 rounding against hand-worked
ties and a brute-force search over every finite bf16 value; exact power-of-two
equivariance; and the layer against a hand-built expert whose output exposes
where the two quantisations sit, the routing of the bf16 layer, and scale
metamorphics."""
import json
import math
import os

import numpy as np

import oracle
from mxfp4_expert_weight_amd import synth


def _f(s):
    return float.fromhex(s) if "x" in s else float(s)


def _finite_e4m3():
    v = oracle.e4m3_decode(np.arange(256))
    codes = np.arange(256)[np.isfinite(v)]
    return codes, v[np.isfinite(v)]


def test_mxfp8_handworked(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "mxfp8_handworked.json")))
    for b in d["blocks"]:
        v = np.zeros((1, 32))
        v[0, :len(b["values"])] = [_f(s) for s in b["values"]]
        codes, sb = oracle.mxfp8_quantize(v)
        want = [int(c, 16) for c in b["codes"]]
        assert list(codes[0, :len(want)]) == want, b["why"]
        assert np.all(codes[0, len(want):] == 0) and sb[0, 0] == b["scale_byte"], b["why"]


def test_bf16_round_handworked(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "mxfp8_handworked.json")))
    for r in d["bf16_round"]:
        assert oracle.bf16_round(np.array([_f(r["value"])]))[0] == _f(r["rounded"]), r["why"]


def test_bf16_round_brute_force():
    """Nearest of all finite bf16 values (from their bit patterns), ties to
    the pattern with an even last bit."""
    bits = np.arange(0x7F80, dtype=np.uint32)                      # non-negative finite patterns
    vals = (bits << 16).view(np.float32).astype(np.float64)
    rng = np.random.default_rng(3)
    picks = rng.integers(0, len(vals) - 1, 4000)
    frac = rng.choice([0.5, 0.25, 0.75, rng.random()], 4000)
    tests = vals[picks] + frac * (vals[picks + 1] - vals[picks])
    tests = np.concatenate([tests, vals[rng.integers(0, len(vals), 200)]])
    for t in tests:
        d = np.abs(vals - t)
        best = np.flatnonzero(d == d.min())
        want = vals[best[0]] if len(best) == 1 else vals[best[(bits[best] & 1) == 0][0]]
        assert oracle.bf16_round(np.array([t]))[0] == want, t
        assert oracle.bf16_round(np.array([-t]))[0] == -want, t


def test_mxfp8_brute_force_nearest():
    """Per block: the scale puts the largest magnitude in [256, 512) (or is
    clamped to 2^-127), and every code is the nearest finite E4M3 value to
    clamp(v / X, -448, 448), ties to an even code."""
    codes_all, vals_all = _finite_e4m3()
    rng = np.random.default_rng(7)
    for trial in range(300):
        mag = 2.0 ** rng.integers(-140, 40)
        v = rng.standard_normal(32) * mag
        v[rng.random(32) < 0.2] = 0.0
        if trial % 7 == 0:
            v = np.round(v / mag * 4) / 4 * mag                  # many ties
        codes, sb = oracle.mxfp8_quantize(v[None])
        e = int(sb[0, 0]) - 127
        amax = np.max(np.abs(v))
        if amax > 0 and e > -127:
            assert 256 <= amax / 2.0 ** e < 512, (amax, e)
        elif amax > 0:
            assert amax / 2.0 ** -127 < 512
        else:
            assert e == -127
        for i in range(32):
            q = min(max(v[i] / 2.0 ** e, -448.0), 448.0)
            d = np.abs(vals_all - q)
            best = np.flatnonzero(d == d.min())
            if len(best) > 1:
                best = best[(codes_all[best] & 1) == 0]
            want = codes_all[best[0]]
            if want == 0x00 and math.copysign(1.0, q) < 0:
                want = 0x80                                   # zero keeps its sign
            if want == 0x80 and math.copysign(1.0, q) > 0:
                want = 0x00
            assert codes[0, i] == want, (trial, i, v[i], q, hex(codes[0, i]), hex(want))


def test_mxfp8_properties():
    rng = np.random.default_rng(11)
    v = rng.standard_normal((6, 128)) * 2.0 ** rng.integers(-20, 20, (6, 1))
    fq = oracle.mxfp8_fake_quant(v)
    assert np.array_equal(oracle.mxfp8_fake_quant(fq), fq)                 # idempotent
    for j in (-5, 1, 9):                                                  # power-of-two equivariance
        assert np.array_equal(oracle.mxfp8_fake_quant(v * 2.0 ** j), fq * 2.0 ** j)
    w = v.copy()
    w[:, 32:64] *= 1000.0                                                 # blocks are independent
    fw = oracle.mxfp8_fake_quant(w)
    assert np.array_equal(fw[:, :32], fq[:, :32]) and np.array_equal(fw[:, 64:], fq[:, 64:])
    # error: at most half a quantum of the element's binade, except clamped maxima
    codes, sb = oracle.mxfp8_quantize(v)
    X = np.repeat(2.0 ** (sb.astype(np.int64) - 127), 32, axis=1)
    q = np.abs(v) / X
    binade = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    half_quantum = 2.0 ** (binade - 4) * X
    ok = (np.abs(fq - v) <= half_quantum * (1 + 1e-12)) | (q > 448)
    assert ok.all()


# ------------------------------------------------------------------ layer --
def _mxfp4_rows(rows, exp):
    """Float rows [R][K] whose entries are E2M1 values times 2^exp -> MXFP4
    codes [R][K/2] (low nibble first) and scale bytes [R][K/32] (127 + exp)."""
    table = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
    rows = np.asarray(rows, dtype=np.float64)
    R, K = rows.shape
    q = np.zeros((R, K // 2), np.uint8)
    for r in range(R):
        for k in range(K):
            val = rows[r, k] / 2.0 ** exp
            q[r, k // 2] |= (table[abs(val)] | (8 if val < 0 else 0)) << (4 * (k % 2))
    return q, np.full((R, K // 32), 127 + exp, np.uint8)


def test_layer_quantisation_points_handbuilt():
    """One expert, k = 1, no shared expert, H = I = 32.  Gate rows read
    x[0] = 1 with weight 48, so g = 48 and SiLU(g) = 48 exactly in float64;
    up row i = 6 x[i] + 0.5 x[i+1]; down = identity.  Then
    y = q(48 * (6 q(x)_i + 0.5 q(x)_{i+1})) where q is the MXFP8 round trip:
    x quantised before the experts, h quantised from its exact value.  The
    input is chosen so that h has more significant bits than bf16 keeps and
    rounding h to bf16 first would move three of its codes: the pin tells the
    two readings apart."""
    H = I = 32
    rng = np.random.default_rng(13)
    x = np.round(rng.standard_normal(H) * 64) / 64 * 2.0 ** rng.integers(-3, 3, H)
    x[0] = 1.0
    x_bits = synth.f32_to_bf16_bits(x.astype(np.float32))[None]
    xb = oracle.bf16_bits_to_f64(x_bits)[0]
    gate = np.zeros((I, H)); gate[:, 0] = 48.0
    up = np.zeros((I, H))
    for i in range(I):
        up[i, i] = 6.0
        up[i, (i + 1) % I] = 0.5
    down = np.eye(H)
    qg, sg = _mxfp4_rows(gate, 3)                    # 48 = 6 * 2^3
    qu, su = _mxfp4_rows(up, 0)
    q13, s13 = np.vstack([qg, qu]), np.vstack([sg, su])
    q2, s2 = _mxfp4_rows(down, 0)
    assert np.array_equal(oracle.dequant_mxfp4(q13, s13), np.vstack([gate, up]))
    assert np.array_equal(oracle.dequant_mxfp4(q2, s2), down)
    out = oracle.moe_layer_w4a8(x_bits, np.ones((1, H)), None, q13[None], s13[None], q2[None], s2[None],
                                k=1, shared=False)
    xq = oracle.mxfp8_fake_quant(xb[None])[0]
    assert xq[0] == 1.0
    h = 48.0 * (6.0 * xq + 0.5 * np.roll(xq, -1))
    want = oracle.mxfp8_fake_quant(h[None])[0]
    assert np.array_equal(out["y"][0], want)
    # and the quantisations are visible: neither x nor h is left unquantised
    assert not np.array_equal(want, 48.0 * (6.0 * xb + 0.5 * np.roll(xb, -1)))
    assert not np.array_equal(want, h)
    # h quantised from bf16(h) instead would differ in three elements
    via_bf16 = oracle.mxfp8_fake_quant(oracle.bf16_round(h)[None])[0]
    assert int(np.sum(via_bf16 != want)) == 3


def test_mxfp8_of_h_is_not_mxfp8_of_bf16_h():
    """A value one part in 2^12 above an E4M3 midpoint rounds up directly, but
    to the midpoint (then down, to the even code) through bf16's 8 bits: in a
    block whose largest element is 256 (X = 1), 136 + 1/32 -> code 144 direct,
    136 -> 128 through bf16."""
    v = np.zeros((1, 32))
    v[0, 0] = 256.0
    v[0, 1] = 136.0 + 1.0 / 32
    assert oracle.bf16_round(v[0, 1:2])[0] == 136.0
    assert oracle.mxfp8_fake_quant(v)[0, 1] == 144.0
    assert oracle.mxfp8_fake_quant(oracle.bf16_round(v))[0, 1] == 128.0


def _tiny():
    wl = synth.WORKLOADS["tiny"]
    return wl, synth.layer_set(wl, 0)


def test_layer_routing_is_the_bf16_layers():
    wl, ls = _tiny()
    a = oracle.moe_layer(ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s, wl.k)
    b = oracle.moe_layer_w4a8(ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s, wl.k)
    assert np.array_equal(a["ids"], b["ids"]) and np.array_equal(a["weights"], b["weights"])
    rel = np.sqrt(np.mean((a["y"] - b["y"]) ** 2) / np.mean(a["y"] ** 2))
    assert 1e-4 < rel < 0.1, rel                          # 8-bit activations: close, not equal


def test_layer_scale_metamorphics():
    """+1 on every down scale doubles y; +1 on every up scale doubles u, so h
    and its MXFP8 round trip double, and so does y."""
    wl, ls = _tiny()
    args = (ls.x_bits, ls.w_router, ls.bias)
    base = oracle.moe_layer_w4a8(*args, ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s, wl.k)["y"]
    y2 = oracle.moe_layer_w4a8(*args, ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s + 1, wl.k)["y"]
    assert np.array_equal(y2, 2 * base)
    I = ls.w13_s.shape[1] // 2
    s13 = ls.w13_s.copy()
    s13[:, I:] += 1
    y3 = oracle.moe_layer_w4a8(*args, ls.w13_q, s13, ls.w2_q, ls.w2_s, wl.k)["y"]
    assert np.array_equal(y3, 2 * base)


def test_layer_tokens_matches_layer():
    small = synth.custom("m4_small", M=4, H=256, I=128, E=16, k=2)
    ls = synth.layer_set(small, 0)
    full = oracle.moe_layer_w4a8(ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s, small.k)
    part = oracle.moe_layer_w4a8_tokens([3, 1], ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s, ls.w2_q,
                                        ls.w2_s, small.k)
    np.testing.assert_allclose(part["y"], full["y"][[3, 1]], rtol=1e-12, atol=1e-12)
