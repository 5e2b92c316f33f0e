"""GPU parity of the expert prefetch calls against the oracle (MoE-SpeQ
article, 4.1 and 4.3), through the C ABI.

moe_prefetch_select: the list and its length equal the oracle's exactly
(integer work).  moe_prefetch_experts: every entry's checksum equals the
oracle's word sum exactly, for every part choice, live count, skipped and
repeated entries, from the smallest shapes to the largest the bank allows.
A layer run after a prefetch (on its own stream, joined by an event) matches
the float64 oracle to the layer tolerance and routes exactly as without it."""
import numpy as np
import pytest

import oracle
from gpu_common import assert_layer_close, need_gpu, say
from mxfp4_expert_weight_amd import binding as B
from mxfp4_expert_weight_amd import synth

pytestmark = pytest.mark.gpu


def _i32(torch, a):
    return torch.tensor(np.asarray(a, dtype=np.int32).reshape(-1), dtype=torch.int32, device="cuda")


def _select(torch, ids, E, has_shared, max_n):
    ids = np.asarray(ids, dtype=np.int32).reshape(-1)
    d_ids = _i32(torch, ids) if ids.size else None
    out = torch.full((max(max_n, 1),), 12345, dtype=torch.int32, device="cuda")
    num = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    B.moe_prefetch_select(d_ids, ids.size, E, has_shared, max_n, out, num)
    torch.cuda.synchronize()
    return out.cpu().numpy()[:max_n], int(num.item())


def _check_select(torch, ids, E, has_shared, max_n, what):
    say(f"prefetch select {what}: n_ids={np.asarray(ids).size} E={E} shared={has_shared} max={max_n}")
    got, n = _select(torch, ids, E, has_shared, max_n)
    want = oracle.select_experts(np.asarray(ids).reshape(-1), E, bool(has_shared), max_n)
    assert n == want.size, (what, n, want.size)
    assert got[:n].tolist() == want.tolist(), what
    assert np.all(got[n:] == -1), what


def test_select_handworked_cases(golden_dir):
    torch = need_gpu()
    import json
    import os
    for c in json.load(open(os.path.join(golden_dir, "prefetch_handworked.json")))["select"]:
        _check_select(torch, np.array(c["draft_ids"], dtype=np.int32), c["E"], int(c["has_shared"]),
                      c["max_experts"], c["why"])


@pytest.mark.parametrize("E,T,k,pool,max_n,shared,seed", [
    (512, 1, 8, 512, 9, 1, 0),           # decode: one draft token
    (512, 5, 8, 512, 41, 1, 1),          # five draft steps (the article's k = 5), all picks listed
    (512, 5, 8, 20, 12, 1, 2),           # heats from a small pool: many ties, cut short
    (512, 4, 8, 512, 33, 0, 3),          # no shared expert
    (16, 3, 2, 16, 17, 1, 4),            # the tiny bank
    (1024, 400, 32, 1024, 1025, 1, 5),   # largest bank, every expert listed
    (1024, 30000, 32, 1024, 100, 1, 6),  # 960,000 ids: heats in the hundreds
    (77, 9, 5, 30, 0, 1, 7),             # an empty list
])
def test_select_random(E, T, k, pool, max_n, shared, seed):
    torch = need_gpu()
    rng = np.random.default_rng(seed)
    cand = rng.choice(E, size=pool, replace=False)
    ids = np.stack([rng.choice(cand, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    # a few ids outside [0, E), which count for nothing
    flat = ids.reshape(-1)
    bad = rng.choice(flat.size, size=min(3, flat.size), replace=False)
    flat[bad[:1]] = -1
    flat[bad[1:2]] = E
    _check_select(torch, flat, E, shared, max_n, f"E={E} T={T} k={k} pool={pool}")


def _bank(torch, n, H, I, gen):
    u8 = dict(dtype=torch.uint8, device="cuda")
    return (torch.randint(0, 256, (n, 2 * I, H // 2), generator=gen, **u8),
            torch.randint(0, 256, (n, 2 * I, H // 32), generator=gen, **u8),
            torch.randint(0, 256, (n, H, I // 2), generator=gen, **u8),
            torch.randint(0, 256, (n, H, I // 32), generator=gen, **u8))


def _host_rows(bank, ids):
    """The listed experts' arrays on the host (a bank of just those entries),
    with each list entry mapped to its row there (-1 when outside the bank)."""
    n = bank[0].shape[0]
    uniq = sorted({int(e) for e in ids if 0 <= int(e) < n})
    rows = {e: i for i, e in enumerate(uniq)}
    sub = [a[uniq].cpu().numpy() if uniq else a[:0].cpu().numpy() for a in bank]
    return sub, [rows.get(int(e), -1) for e in ids]


def _check_prefetch(torch, bank, E, has_shared, H, I, ids, num_live, parts, what):
    say(f"prefetch experts {what}: H={H} I={I} E={E} shared={has_shared} ids={list(ids)[:12]} "
        f"live={num_live} parts={parts}")
    w = B.make_weights(*bank, E, H, I, has_shared)
    d_ids = _i32(torch, ids)
    d_live = _i32(torch, [num_live]) if num_live is not None else None
    cs = torch.zeros(len(ids), dtype=torch.int32, device="cuda")
    B.moe_prefetch_experts(w, d_ids, d_live, len(ids), parts, cs)
    torch.cuda.synchronize()
    got = cs.cpu().numpy().view(np.uint32)
    sub, rows = _host_rows(bank[:], [e if e < E + has_shared else -1 for e in ids])
    live = len(ids) if num_live is None else num_live
    want = oracle.prefetch_checksums(*sub, rows, live, parts)
    assert got.tolist() == want.tolist(), what


@pytest.mark.parametrize("H,I,E,shared", [
    (32, 32, 3, 1),          # smallest shapes: one 64 KB workgroup covers an expert
    (256, 128, 16, 1),       # the tiny bank
    (96, 160, 5, 0),         # ragged sizes, no shared expert
    (2560, 768, 12, 1),      # Ling expert shapes: 48 workgroups per expert
    (8192, 4096, 2, 1),      # the largest expert: 51 MB, 816 workgroups
])
def test_prefetch_checksums(H, I, E, shared):
    torch = need_gpu()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(H * 7 + I + E)
    bank = _bank(torch, E + shared, H, I, gen)
    n = E + shared
    ids = [n - 1, 0, -1, n, min(1, n - 1), 0, 1 << 30]       # shared (or last), skips, a repeat
    for parts in (1, 2, 3):
        _check_prefetch(torch, bank, E, shared, H, I, ids, None, parts, f"parts={parts}")
    _check_prefetch(torch, bank, E, shared, H, I, ids, 2, 3, "live=2")
    _check_prefetch(torch, bank, E, shared, H, I, ids, 0, 3, "live=0")
    _check_prefetch(torch, bank, E, shared, H, I, ids, 1 << 20, 3, "live above the list")


def test_prefetch_full_ling_bank():
    """A 513-entry Ling bank (1.6 GB), the decode list: shared + 8 experts."""
    torch = need_gpu()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    bank = _bank(torch, 513, 2560, 768, gen)
    ids = [512, 511, 0, 255, 256, 17, 400, 3, 499]
    _check_prefetch(torch, bank, 512, 1, 2560, 768, ids, None, 3, "ling decode list")
    _check_prefetch(torch, bank, 512, 1, 2560, 768, ids + [-1] * 24, 9, 1, "ling list, 33 rows, 9 live")


def test_select_then_prefetch_then_layer():
    """The verify-shaped flow: the draft's routing -> list -> prefetch on a
    stream of its own, the layer waits on an event after it; its output and
    routing are those of the float64 oracle (the prefetch changes nothing)."""
    torch = need_gpu()
    from mxfp4_expert_weight_amd.layer import DeviceLayerSet, LayerBuffers, run_layer
    for name in ("tiny", "ling_m4_mtp"):
        ls = synth.layer_set(name)
        wl = ls.wl
        say(f"select -> prefetch -> layer: {name}")
        d = DeviceLayerSet.from_host(ls)
        b = LayerBuffers(wl.M, wl.k, wl.E, wl.H, wl.I)
        run_layer(d, b)
        torch.cuda.synchronize()
        ids_plain = b.ids.cpu().numpy()
        draft = synth.draft_ids(ids_plain, wl.E, 0.5, np.random.default_rng(5))
        max_n = wl.M * wl.k + 1
        lst = torch.zeros(max_n, dtype=torch.int32, device="cuda")
        num = torch.zeros(1, dtype=torch.int32, device="cuda")
        cs = torch.zeros(max_n, dtype=torch.int32, device="cuda")
        d_draft = _i32(torch, draft)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            B.moe_prefetch_select(d_draft, draft.size, wl.E, 1, max_n, lst, num)
            B.moe_prefetch_experts(d.weights(), lst, num, max_n, 3, cs)
        done = torch.cuda.Event()
        done.record(side)
        torch.cuda.current_stream().wait_event(done)
        b.y.fill_(float("nan"))
        run_layer(d, b)
        torch.cuda.synchronize()
        want_list = oracle.select_experts(draft, wl.E, True, max_n)
        assert int(num.item()) == want_list.size
        assert lst.cpu().numpy()[:want_list.size].tolist() == want_list.tolist()
        want_cs = oracle.prefetch_checksums(ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s, want_list, want_list.size, 3)
        assert cs.cpu().numpy().view(np.uint32)[:want_list.size].tolist() == want_cs.tolist()
        assert np.array_equal(b.ids.cpu().numpy(), ids_plain)
        r = oracle.moe_layer(ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s,
                             wl.k, wl.shared)
        assert np.array_equal(ids_plain, r["ids"])
        assert_layer_close(b.y.cpu().numpy(), r["y"], what=f"{name} after prefetch")


def test_prefetch_in_graph_replays():
    """Select + prefetch on a side stream, captured with the layer into one HIP
    graph (fork and join by events, as the bench runs them): each replay adds
    the oracle's checksums once more and leaves the layer output the oracle's.
    Eager work (refilling y) runs between the replays."""
    torch = need_gpu()
    from mxfp4_expert_weight_amd.layer import DeviceLayerSet, LayerBuffers, run_layer
    ls = synth.layer_set("tiny")
    wl = ls.wl
    say("prefetch captured in a graph with the tiny layer")
    d = DeviceLayerSet.from_host(ls)
    b = LayerBuffers(wl.M, wl.k, wl.E, wl.H, wl.I)
    run_layer(d, b)
    torch.cuda.synchronize()
    draft = synth.draft_ids(b.ids.cpu().numpy(), wl.E, 0.5, np.random.default_rng(9))
    max_n = wl.M * wl.k + 1
    lst = torch.zeros(max_n, dtype=torch.int32, device="cuda")
    num = torch.zeros(1, dtype=torch.int32, device="cuda")
    cs = torch.zeros(max_n, dtype=torch.int32, device="cuda")
    d_draft = _i32(torch, draft)
    w = d.weights()
    side = torch.cuda.Stream()
    done = torch.cuda.Event()

    def step():
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            B.moe_prefetch_select(d_draft, draft.size, wl.E, 1, max_n, lst, num)
            B.moe_prefetch_experts(w, lst, num, max_n, 3, cs)
        done.record(side)
        cur.wait_event(done)
        run_layer(d, b)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    cs.zero_()
    torch.cuda.synchronize()
    want_list = oracle.select_experts(draft, wl.E, True, max_n)
    want_cs = oracle.prefetch_checksums(ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s, want_list, want_list.size, 3)
    r = oracle.moe_layer(ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s, wl.k, wl.shared)
    n = want_list.size
    for rep in range(1, 4):
        b.y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(num.item()) == n
        assert lst.cpu().numpy()[:n].tolist() == want_list.tolist()
        got = cs.cpu().numpy().view(np.uint32)[:n].astype(np.uint64)
        assert got.tolist() == ((want_cs.astype(np.uint64) * rep) % (1 << 32)).tolist(), rep
        assert_layer_close(b.y.cpu().numpy(), r["y"], what=f"graph replay {rep}")


# Banks above 512 experts take the 16-experts-per-lane top-k and its own
# hinting kernel: 1,024 experts with k = 8 at M = 1, and a ragged 600 at M = 3
# (one idle wave per workgroup), without a shared expert.
HINT_CUSTOM = {
    "e1024_m1": (1, 256, 128, 1024, 8, True),
    "e600_m3": (3, 512, 96, 600, 8, False),
}


@pytest.mark.parametrize("name", ["tiny", "ling_m1", "ling_m4_mtp", *HINT_CUSTOM])
def test_hinted_layer_equals_plain(name):
    """moe_layer_hinted with right, half-right, invalid and empty hints gives
    moe_layer's routing bit for bit and its output (fp32 atomics may reorder
    the sum); the M = 1 layers also against the float64 oracle."""
    torch = need_gpu()
    from mxfp4_expert_weight_amd.layer import DeviceLayerSet, LayerBuffers, run_layer
    if name in HINT_CUSTOM:
        M, H, I, E, k, shared = HINT_CUSTOM[name]
        ls = synth.layer_set(synth.custom(name, M, H, I, E, k, shared, "plain", seed=M + E))
    else:
        ls = synth.layer_set(name)
    wl = ls.wl
    d = DeviceLayerSet.from_host(ls)
    b = LayerBuffers(wl.M, wl.k, wl.E, wl.H, wl.I)
    run_layer(d, b)
    torch.cuda.synchronize()
    ref = dict(ids=b.ids.cpu().numpy(), w=b.weights.cpu().numpy(), y=b.y.cpu().numpy().astype(np.float64))
    true_active = np.unique(ref["ids"])
    draft = synth.draft_ids(ref["ids"], wl.E, 0.5, np.random.default_rng(3))
    cases = {
        "right": true_active,
        "half": np.unique(draft),
        "invalid": np.array([-1] + true_active.tolist()[:-1] + [wl.E, 1 << 20]),
        "empty": np.array([], dtype=np.int64),
    }
    rms = float(np.sqrt(np.mean(ref["y"] ** 2)))
    for what, hint in cases.items():
        say(f"moe_layer_hinted {name}: {what} hint {hint.tolist()[:10]}")
        h = torch.tensor(np.concatenate([hint, [0]]).astype(np.int32), device="cuda")
        nh = torch.tensor([hint.size], dtype=torch.int32, device="cuda")
        b.y.fill_(float("nan"))
        B.moe_layer_hinted(d.x, d.w_router, d.bias, d.bias_row_stride, d.weights(), d.M, d.k, b.logits, b.ids,
                           b.weights, b.offsets, b.pairs, b.active, b.num_active, b.y, b.ws, b.ws_bytes, h, nh)
        torch.cuda.synchronize()
        assert np.array_equal(b.ids.cpu().numpy(), ref["ids"]), what
        assert np.array_equal(b.weights.cpu().numpy(), ref["w"]), what
        y = b.y.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(y - ref["y"]) <= 1e-5 * (np.abs(ref["y"]) + rms)), what
    if wl.M == 1:
        r = oracle.moe_layer(ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s, wl.k, wl.shared)
        assert np.array_equal(ref["ids"], r["ids"])
        assert_layer_close(b.y.cpu().numpy(), r["y"], what=f"{name} hinted")
