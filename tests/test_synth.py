"""The seeded input generator: determinism, value ranges and the routing
structure of each workload (distinct experts at M=4, Zipf skew at M=32,
>=16-token experts at M=512), measured with the oracle's routing."""
import numpy as np
import pytest

import oracle
from mxfp4_expert_weight_amd import synth


def test_deterministic_and_banks_drawn_last():
    a = synth.layer_set("tiny")
    b = synth.layer_set("tiny")
    for f in ["x_bits", "w_router", "w13_q", "w13_s", "w2_q", "w2_s"]:
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = synth.layer_set("tiny", banks=False)
    assert np.array_equal(a.x_bits, c.x_bits) and np.array_equal(a.w_router, c.w_router)
    assert c.w13_q is None


def test_shapes_dtypes_ranges():
    ls = synth.layer_set("tiny")
    wl = ls.wl
    assert ls.x_bits.shape == (1, 256) and ls.x_bits.dtype == np.uint16
    assert ls.w_router.shape == (16, 256) and ls.w_router.dtype == np.float32
    assert ls.w13_q.shape == (17, 256, 128) and ls.w13_s.shape == (17, 256, 8)
    assert ls.w2_q.shape == (17, 256, 64) and ls.w2_s.shape == (17, 256, 4)
    assert ls.w13_s.min() >= 120 and ls.w13_s.max() <= 127 and ls.w2_s.min() >= 120
    assert set(np.unique(ls.w13_s)) == set(range(120, 128))
    nib = np.concatenate([ls.w13_q.ravel() & 15, ls.w13_q.ravel() >> 4])
    cnt = np.bincount(nib, minlength=16)
    assert cnt.min() > 0.9 * nib.size / 16 and cnt.max() < 1.1 * nib.size / 16
    assert abs(np.std(ls.w_router) - 0.02) < 0.002
    xf = oracle.bf16_bits_to_f64(ls.x_bits)
    assert abs(xf.std() - 1.0) < 0.15
    assert wl.H % 32 == 0 and wl.I % 32 == 0


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 1.0 + 2 ** -8 + 2 ** -20],
                 dtype=np.float32)
    # 1+2^-8 is halfway between 1 and 1+2^-7: ties to even -> 1.0
    # 1+3*2^-8 is halfway between 1+2^-7 and 1+2^-6: ties to even -> 1+2^-6
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 1.0 + 2 ** -7])
    got = oracle.bf16_bits_to_f64(synth.f32_to_bf16_bits(f))
    assert np.array_equal(got, want)


def _routing_counts(wl, set_idx):
    ls = synth.layer_set(wl, set_idx, banks=False)
    logits = oracle.router_logits(oracle.bf16_bits_to_f64(ls.x_bits), ls.w_router, ls.bias)
    ids, _ = oracle.topk_softmax(logits, wl.k)
    return ids, np.bincount(ids.ravel(), minlength=wl.E)


def test_m1_plain_routes_eight_distinct():
    for l in range(5):
        ids, cnt = _routing_counts(synth.WORKLOADS["ling_m1"], l)
        assert (cnt > 0).sum() == 8


def test_m4_overlap_distinct_experts_in_range():
    wl = synth.WORKLOADS["ling_m4_mtp"]
    Ds = []
    for l in range(wl.sets):
        ids, cnt = _routing_counts(wl, l)
        D = int((cnt > 0).sum())
        assert 8 <= D <= 32
        Ds.append(D)
        # the steered sets are exactly the top-8 (bias +8 dominates the logit spread)
        ls = synth.layer_set(wl, l, banks=False)
        for t in range(wl.M):
            assert set(ids[t]) == set(np.nonzero(ls.bias[t])[0])
    # per-slot overlap probability 0.3: E[D] ~ 8 + 3*8*0.7 ~ 24.8
    assert 22.0 < np.mean(Ds) < 27.5


def test_m32_zipf_is_skewed():
    wl = synth.WORKLOADS["ling_m32_zipf"]
    mx, act = [], []
    for l in range(10):
        _, cnt = _routing_counts(wl, l)
        mx.append(cnt.max()); act.append((cnt > 0).sum())
    assert 12 <= np.mean(mx) <= 26          # heaviest expert takes ~20 of 32 tokens
    assert 80 <= np.mean(act) <= 135        # ~106 distinct experts of 512


def test_m512_has_mfma_sized_experts():
    wl = synth.WORKLOADS["ling_m512_prefill"]
    ge16 = []
    for l in range(4):
        _, cnt = _routing_counts(wl, l)
        assert (cnt > 0).sum() >= 505
        ge16.append((cnt >= 16).sum())
    assert sum(ge16) >= 4                   # ~4.5 experts per set take >= 16 tokens


def test_set_index_checked():
    with pytest.raises(ValueError):
        synth.layer_set("tiny", 1)


def test_draft_ids():
    """The synthetic draft routing: accuracy 1 keeps every true expert,
    accuracy 0 keeps none, and a token's drafted experts are distinct."""
    rng = np.random.default_rng(0)
    true = np.stack([rng.choice(512, size=8, replace=False) for _ in range(4)]).astype(np.int32)
    assert np.array_equal(synth.draft_ids(true, 512, 1.0, np.random.default_rng(1)), true)
    d0 = synth.draft_ids(true, 512, 0.0, np.random.default_rng(2))
    for t in range(4):
        assert len(set(d0[t])) == 8
        assert not set(d0[t]) & set(true[t])
        assert d0[t].min() >= 0 and d0[t].max() < 512
    # about half kept at accuracy 0.5 (4,000 slots: 5 sigma is 160)
    big = np.stack([rng.choice(512, size=8, replace=False) for _ in range(500)]).astype(np.int32)
    dh = synth.draft_ids(big, 512, 0.5, np.random.default_rng(3))
    kept = int((dh == big).sum())
    assert abs(kept - 2000) < 160
    for t in range(500):
        assert len(set(dh[t])) == 8
