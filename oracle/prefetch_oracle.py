"""Plain definition of the expert prefetch step: the experts a draft pass
predicts for a layer are ranked and read ahead of the layer, so that the
layer's own weight reads find them in the GPU's last-level cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): slow, obviously
correct, written step by step from the definitions.

What it computes, and where it is stated (MoE-SpeQ article):
  * 4.1: a quantised draft model runs k steps ahead; at every step each MoE
    layer's gate picks its top experts, and an expert heat map
    [layer][expert] counts those picks.  Experts are prefetched in the order
    of priority = 0.6 * heat + 0.3 * expert size + 0.1 * transfer time.
  * 4.3: the prefetch runs on a stream of its own; the verify computation
    waits on an event recorded after it.
  * 1.1 / 1.2: prefetching hides the cost of bringing the predicted experts
    to where the computation reads them.

Readings taken where the article is silent:
  * heat[e] is the number of (draft token, slot) pairs whose routed id is e;
    ids outside [0, E) count for nothing.
  * size and transfer time enter the priority divided by the bank's largest;
    in a bank whose experts all share one shape both terms are the same
    constant for every expert, so the order is the heat order.  Ties go to the
    lower expert index; experts with heat 0 are not predicted.
  * The shared expert is used by every token, so when the bank has one it is
    always listed, first; the list holds at most max_experts entries.
  * "Prefetch" brings every 64-byte line of the chosen arrays of each listed
    expert into the cache (parts bit 0: the gate/up codes and scales, bit 1:
    the down codes and scales); one 32-bit word per line is enough to make the
    memory system fetch the line, so that is what is read: the word at each
    offset 0, 64, 128, ... below the array's per-expert size, offsets counted
    from the start of that expert's part of the array.  The observable result
    is one checksum per list entry: the sum, modulo 2^32, of those
    little-endian words.  Entries whose id is outside the bank, and entries at
    or past the live count, read nothing.
"""
from __future__ import annotations

import numpy as np

PRIORITY_ALPHA = 0.6   # heat
PRIORITY_BETA = 0.3    # expert size
PRIORITY_GAMMA = 0.1   # transfer time


def expert_heat(draft_ids, E: int) -> np.ndarray:
    """Heat map row of one layer: how many draft (token, slot) pairs picked
    each routed expert (int64 [E])."""
    ids = np.asarray(draft_ids, dtype=np.int64).ravel()
    ids = ids[(ids >= 0) & (ids < E)]
    return np.bincount(ids, minlength=E).astype(np.int64)


def prefetch_priority(heat, sizes, times) -> np.ndarray:
    """alpha * heat + beta * size + gamma * transfer time, size and time each
    divided by their largest value in the bank (float64)."""
    heat = np.asarray(heat, dtype=np.float64)
    sizes = np.asarray(sizes, dtype=np.float64)
    times = np.asarray(times, dtype=np.float64)
    return (PRIORITY_ALPHA * heat + PRIORITY_BETA * sizes / sizes.max()
            + PRIORITY_GAMMA * times / times.max())


def select_experts(draft_ids, E: int, has_shared: bool, max_experts: int,
                   expert_bytes: float = 1.0, link_bytes_per_s: float = 1.0) -> np.ndarray:
    """The prefetch list of one layer (int64, at most max_experts entries):
    the shared expert (index E) first when the bank has one, then the routed
    experts with heat > 0 in descending priority, ties to the lower index."""
    heat = expert_heat(draft_ids, E)
    sizes = np.full(E, float(expert_bytes))
    times = sizes / float(link_bytes_per_s)
    pr = prefetch_priority(heat, sizes, times)
    order = np.argsort(-pr, kind="stable")           # equal priority keeps index order
    routed = [int(e) for e in order if heat[e] > 0]
    lst = ([E] if has_shared else []) + routed
    return np.asarray(lst[:max(max_experts, 0)], dtype=np.int64)


LINE_BYTES = 64


def _line_words_sum(a: np.ndarray) -> int:
    """Sum of the first little-endian 32-bit word of every 64-byte line of a
    byte array (len % 4 == 0; a last, shorter line counts too)."""
    b = np.ascontiguousarray(a, dtype=np.uint8).ravel()
    assert b.size % 4 == 0
    w = b.view("<u4").astype(np.uint64)
    return int(w[::LINE_BYTES // 4].sum())


def prefetch_checksums(w13_q, w13_s, w2_q, w2_s, expert_ids, num_live: int, parts: int) -> np.ndarray:
    """Checksum of each list entry (uint32 [len(expert_ids)]): for r < num_live
    with 0 <= expert_ids[r] < number of bank entries, the sum mod 2^32 of the
    first 32-bit word of every 64-byte line of that expert's chosen arrays;
    0 otherwise."""
    ids = np.asarray(expert_ids, dtype=np.int64).ravel()
    out = np.zeros(ids.size, dtype=np.uint32)
    nbank = w13_q.shape[0]
    chosen = ([w13_q, w13_s] if parts & 1 else []) + ([w2_q, w2_s] if parts & 2 else [])
    for r in range(min(int(num_live), ids.size)):
        e = int(ids[r])
        if not 0 <= e < nbank:
            continue
        total = 0
        for arr in chosen:
            total += _line_words_sum(arr[e])
        out[r] = total % (1 << 32)
    return out
