"""Pins of the FP8 LM-head oracle (CPU): the E4M3 decode against its bit-field
closed form on all 256 codes, rounding against brute-force nearest search and
hand-worked ties, the quantiser's scale rule, and a hand-worked projection."""
import json
import math
import os

import numpy as np

import oracle


def e4m3_bitfield(c):
    sign = -1.0 if (c >> 7) & 1 else 1.0
    e, m = (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sign * math.ldexp(m / 8.0, -6)
    return sign * math.ldexp(1.0 + m / 8.0, e - 7)


def test_e4m3_decode_all_codes():
    got = oracle.e4m3_decode(np.arange(256))
    for c in range(256):
        want = e4m3_bitfield(c)
        assert (math.isnan(want) and math.isnan(got[c])) or got[c] == want, (hex(c), got[c], want)
    finite = got[np.isfinite(got)]
    assert finite.max() == 448.0 and finite.min() == -448.0 and len(finite) == 254


def test_e4m3_handworked(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "lmhead_handworked.json")))
    for case in d["decode"]:
        assert oracle.e4m3_decode(np.array([int(case["code"], 16)]))[0] == case["value"], case
    for case in d["round"]:
        assert oracle.e4m3_round(np.array([case["value"]]))[0] == int(case["code"], 16), case


def test_e4m3_round_is_identity_on_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(oracle.e4m3_round(oracle.e4m3_decode(codes)), codes)


def test_e4m3_round_brute_force_nearest():
    rng = np.random.default_rng(11)
    q = np.concatenate([rng.uniform(-500, 500, 20000), rng.standard_normal(20000) * 1e-2,
                        rng.standard_normal(20000) * 2.0 ** -8])
    got = oracle.e4m3_round(q)
    table = [(c, e4m3_bitfield(c)) for c in range(256) if not math.isnan(e4m3_bitfield(c))]
    for v, code in zip(q[:3000], got[:3000]):          # exhaustive search on a sample
        qc = min(max(v, -448.0), 448.0)
        best = min(abs(qc - t) for _, t in table)
        cands = [c for c, t in table if abs(qc - t) == best and (math.copysign(1, t) == math.copysign(1, qc) or t != 0)]
        if len(cands) > 1:                               # a tie: the even mantissa
            cands = [c for c in cands if (c & 1) == 0]
        vals = {e4m3_bitfield(c) for c in cands}
        assert e4m3_bitfield(int(code)) in vals, (v, hex(code), [hex(c) for c in cands])
    # the decoded value is never farther than half a step of its binade
    dec = oracle.e4m3_decode(got)
    qc = np.clip(q, -448, 448)
    step = np.where(np.abs(qc) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(qc), 2.0 ** -6))) - 3))
    assert np.all(np.abs(dec - qc) <= step / 2 + 1e-300)


def test_quantize_scale_rule_and_range():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((64, 2560)) * 0.02).astype(np.float32)
    w[7] = 0.0                                          # an all-zero row
    bits = (w.view(np.uint32) >> 16).astype(np.uint16)  # truncate to bf16 for the test input
    codes, scales = oracle.lmhead_quantize(bits)
    wf = (bits.astype(np.uint32) << 16).view(np.float32)
    amax = np.abs(wf).max(axis=1)
    for r in range(64):
        if r == 7:
            assert scales[r] == 1.0 and np.all(codes[r] == 0)
            continue
        assert scales[r] == np.float32(amax[r] / np.float32(448.0))
        dec = oracle.e4m3_decode(codes[r])
        assert np.abs(dec).max() == 448.0                # the row's largest element lands on 448
        # dequantised within half an E4M3 step (relative 2^-4) or the subnormal step
        err = np.abs(dec * scales[r] - wf[r])
        tol = np.maximum(np.abs(wf[r]) * 2.0 ** -4, 2.0 ** -10 * scales[r]) * 1.0001
        assert np.all(err <= tol)


def test_logits_handworked(golden_dir):
    d = json.load(open(os.path.join(golden_dir, "lmhead_handworked.json")))["logits"]
    x = np.array([[int(b, 16) for b in d["x_bits"]]], dtype=np.uint16)
    codes = np.array([[int(c, 16) for c in row] for row in d["codes"]], dtype=np.uint8)
    got = oracle.lmhead_logits(x, codes, np.array(d["scales"], dtype=np.float32))
    assert list(got[0]) == d["logits"]


def test_logits_scale_linearity():
    """Doubling a row's scale doubles exactly that row's logits (power of two)."""
    rng = np.random.default_rng(2)
    x = rng.integers(0x3C00, 0x4200, size=(3, 96)).astype(np.uint16)
    codes = rng.integers(0, 256, size=(5, 96)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10
    s = rng.uniform(0.5, 2.0, 5).astype(np.float32)
    a = oracle.lmhead_logits(x, codes, s)
    s2 = s.copy(); s2[3] *= 2
    b = oracle.lmhead_logits(x, codes, s2)
    assert np.array_equal(b[:, 3], 2 * a[:, 3]) and np.array_equal(np.delete(b, 3, 1), np.delete(a, 3, 1))
