"""Pins of the expert prefetch oracle (CPU): hand-worked lists, priorities and
line checksums (tests/golden/prefetch_handworked.json), a byte-by-byte brute force
of the checksum, a pairwise-rank brute force of the selection, and the
invariants the definition fixes (MoE-SpeQ article, 4.1 and 4.3)."""
import json
import os

import numpy as np
import pytest

from oracle import prefetch_oracle as P


@pytest.fixture(scope="module")
def golden(golden_dir):
    return json.load(open(os.path.join(golden_dir, "prefetch_handworked.json")))


def test_select_handworked(golden):
    for c in golden["select"]:
        got = P.select_experts(np.array(c["draft_ids"], dtype=np.int64).reshape(-1), c["E"], c["has_shared"],
                               c["max_experts"])
        assert got.tolist() == c["list"], c["why"]


def test_priority_handworked(golden):
    c = golden["priority"]
    got = P.prefetch_priority(c["heat"], c["sizes"], c["times"])
    np.testing.assert_allclose(got, c["priority"], rtol=0, atol=1e-15)


def _hand_bank():
    H = I = 32
    w13_q = np.zeros((2, 2 * I, H // 2), np.uint8)
    w13_s = np.zeros((2, 2 * I, H // 32), np.uint8)
    w2_q = np.zeros((2, H, I // 2), np.uint8)
    w2_s = np.zeros((2, H, I // 32), np.uint8)
    w13_q[0] = 0x01
    w13_s[0] = 0x7F
    w2_q[0] = np.tile(np.array([1, 2, 3, 4], np.uint8), H * I // 2 // 4).reshape(H, I // 2)
    w2_s[0] = 0xFF
    return w13_q, w13_s, w2_q, w2_s


def test_checksum_handworked(golden):
    c = golden["checksum"]
    bank = _hand_bank()
    for parts, key in ((1, "entry0_parts1"), (2, "entry0_parts2"), (3, "entry0_parts3")):
        got = P.prefetch_checksums(*bank, [0, 1], 2, parts)
        assert got.tolist() == [c[key], 0], (parts, got)


def _brute_checksum(arrays, e):
    """Byte loop: byte i of a region adds b * 256^(i mod 64) when i mod 64 < 4
    (the first word of each 64-byte line)."""
    total = 0
    for a in arrays:
        flat = a[e].reshape(-1).tolist()
        for i, b in enumerate(flat):
            if i % 64 < 4:
                total += int(b) << (8 * (i % 64))
    return total % (1 << 32)


@pytest.mark.parametrize("seed,H,I", [(0, 64, 32), (1, 32, 32), (2, 96, 160)])
def test_checksum_brute_force(seed, H, I):
    """Random banks; (32, 32) and (96, 160) give down scales of 32 and 480
    bytes per expert, whose last line is short."""
    rng = np.random.default_rng(seed)
    E = 3
    bank = (rng.integers(0, 256, (E + 1, 2 * I, H // 2), dtype=np.uint8),
            rng.integers(0, 256, (E + 1, 2 * I, H // 32), dtype=np.uint8),
            rng.integers(0, 256, (E + 1, H, I // 2), dtype=np.uint8),
            rng.integers(0, 256, (E + 1, H, I // 32), dtype=np.uint8))
    ids = [3, 0, 2, 1]
    for parts in (1, 2, 3):
        arrays = ([bank[0], bank[1]] if parts & 1 else []) + ([bank[2], bank[3]] if parts & 2 else [])
        want = [_brute_checksum(arrays, e) for e in ids]
        assert P.prefetch_checksums(*bank, ids, len(ids), parts).tolist() == want


def test_checksum_skips_and_duplicates():
    bank = _hand_bank()
    c0 = int(P.prefetch_checksums(*bank, [0], 1, 3)[0])
    assert P.prefetch_checksums(*bank, [0, -1, 5, 0], 3, 3).tolist() == [c0, 0, 0, 0]   # past num_live
    assert P.prefetch_checksums(*bank, [0, -1, 5, 0], 4, 3).tolist() == [c0, 0, 0, c0]  # a duplicate reads again
    assert P.prefetch_checksums(*bank, [0, 0], 0, 3).tolist() == [0, 0]
    # the two parts add up (mod 2^32) to both
    s1 = int(P.prefetch_checksums(*bank, [0], 1, 1)[0])
    s2 = int(P.prefetch_checksums(*bank, [0], 1, 2)[0])
    assert (s1 + s2) % (1 << 32) == c0


def _rank_brute(heat):
    """Position of each picked expert by pairwise comparison."""
    E = len(heat)
    out = [None] * E
    for e in range(E):
        if heat[e] > 0:
            r = sum(1 for j in range(E) if heat[j] > heat[e] or (heat[j] == heat[e] and j < e))
            out[r] = e
    return [e for e in out if e is not None]


@pytest.mark.parametrize("seed", range(6))
def test_select_brute_force_and_invariants(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(4, 40))
    T, k = int(rng.integers(1, 9)), int(rng.integers(1, 4))
    k = min(k, E)
    # draft routing: k distinct experts per token from a small pool, so heats tie often
    pool = rng.choice(E, size=min(E, 2 * k + 1), replace=False)
    ids = np.stack([rng.choice(pool, size=k, replace=False) for _ in range(T)])
    heat = P.expert_heat(ids, E)
    assert heat.sum() == T * k
    for has_shared in (False, True):
        for max_n in (0, 1, 3, E + 1):
            got = P.select_experts(ids, E, has_shared, max_n).tolist()
            want = (([E] if has_shared else []) + _rank_brute(heat.tolist()))[:max_n]
            assert got == want
            assert len(set(got)) == len(got)
            assert all(e == E or heat[e] > 0 for e in got)
    # the draft's picks, whatever their order, give the same list
    perm = rng.permutation(ids.reshape(-1))
    assert P.select_experts(perm, E, True, E + 1).tolist() == P.select_experts(ids, E, True, E + 1).tolist()


def test_uniform_bank_priority_is_heat_order():
    heat = np.array([0, 5, 2, 5, 1, 0, 2])
    pr = P.prefetch_priority(heat, np.full(7, 3.13e6), np.full(7, 3.13e6 / 8e12))
    order = [e for e in np.argsort(-pr, kind="stable") if heat[e] > 0]
    assert order == [1, 3, 2, 6, 4]


def test_unequal_sizes_change_order():
    """Size and transfer time do enter the priority where they differ."""
    pr = P.prefetch_priority([1, 1], [1.0, 2.0], [1.0, 1.0])
    assert pr[1] > pr[0]
