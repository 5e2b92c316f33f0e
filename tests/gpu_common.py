"""Helpers for the GPU parity tests: device buffers, the tolerance of the
layer output, and the checks of routing against the float64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle

U = 2.0 ** -24          # fp32 unit roundoff


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(msg: str):
    """Name the case before each GPU step (flushed, so a lost machine still shows it)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def assert_layer_close(y_gpu: np.ndarray, y_ref: np.ndarray, rms: float | None = None, what=""):
    """|gpu - ref| <= 1e-2 (|ref| + rms(ref)) per element, rms over the whole output."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    if rms is None:
        rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = np.abs(y_gpu - y_ref)
    tol = 1e-2 * (np.abs(y_ref) + rms)
    ratio = float((err / tol).max())
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    assert ratio <= 1.0, f"{what}: worst err/tol = {ratio:.3g}"
    return ratio


def router_rounding_chain(H, M):
    """Longest chain of fp32 roundings in a router logit.  Batches below 64
    tokens: each lane sums ceil(H/256) float4s (4 fmas each) in order, a
    6-level wave tree follows, then the bias; one more for slack:
    4 ceil(H/256) + 8.  Larger batches run on the matrix cores with the
    weights split exactly into three bf16 parts, so 3H exact products, and a
    32-product dot per leaf (counted as 32 roundings, the most any summation
    order of it can take).  Rows a multiple of 128: a leaf chains the three
    parts' dots smallest first, which keeps its error within 33 u of its sum
    of |x w|; each of four waves adds its 4 ceil(H/512) leaves in order, then
    the four waves' sums, then the bias: 33 + 4 ceil(H/512) + 3 + 1.
    Other rows: 16 leaves per group and weight part, the groups into the
    total in order, the three last partial groups, then the bias:
    32 + 16 + 3 ceil(H/512) + 3 + 1."""
    if M < 64:
        return 4 * -(-H // 256) + 8
    if H % 128 == 0:
        return 33 + 4 * -(-H // 512) + 3 + 1
    return 32 + 16 + 3 * -(-H // 512) + 3 + 1


def logit_error_bound(x_f64, w_router, bias, H, M):
    """Bound on |fp32 router logit - exact logit| for a launch over M tokens:
    the rounding chain times u on partial sums bounded by sum |x_i w_i|
    (+ |bias|)."""
    S = np.abs(x_f64) @ np.abs(np.asarray(w_router, np.float64)).T
    if bias is not None:
        S = S + np.abs(np.asarray(bias, np.float64))
    return router_rounding_chain(H, M) * U * S * 1.01


def check_routing(ids_gpu, w_gpu, logits_gpu, ref_logits, bound, k, what=""):
    """Compare GPU routing with the float64 oracle.

    Logits: within `bound`.  Ids: exactly the oracle's wherever the oracle's
    order of the top-(k+1) logits is decided by more than the error bounds;
    where two candidates are closer than that, either order is a correct fp32
    result, so the GPU's choice is checked for validity instead.  Weights: the
    oracle's renormalised softmax of the GPU's chosen experts, within the
    logit bounds' effect plus fp32 rounding.
    Returns the tokens whose routing was ambiguous.
    """
    M, E = ref_logits.shape
    assert np.all(np.abs(logits_gpu - ref_logits) <= bound), \
        f"{what}: logits off by {np.max(np.abs(logits_gpu - ref_logits) / bound):.3g} x bound"
    ref_ids, _ = oracle.topk_softmax(ref_logits, k)
    ambiguous = []
    for t in range(M):
        l, b = ref_logits[t], bound[t]
        order = np.argsort(-l, kind="stable")
        top = order[:min(k + 1, E)]
        decided = all(l[top[i]] - l[top[i + 1]] > b[top[i]] + b[top[i + 1]] for i in range(len(top) - 1))
        g = ids_gpu[t].astype(np.int64)
        if decided:
            assert np.array_equal(g, ref_ids[t]), f"{what}: token {t} ids {g} != {ref_ids[t]}"
        else:
            ambiguous.append(t)
            assert len(set(g.tolist())) == k and g.min() >= 0 and g.max() < E
            kth = l[ref_ids[t][-1]]
            bk = b[ref_ids[t][-1]]
            for i in range(k):
                assert l[g[i]] >= kth - (b[g[i]] + bk), f"{what}: token {t} picked a non-top expert"
                if i + 1 < k:
                    assert l[g[i]] >= l[g[i + 1]] - (b[g[i]] + b[g[i + 1]]), f"{what}: token {t} order"
        sel = l[g]
        ex = np.exp(sel - sel.max())
        w_ref = ex / ex.sum()
        tol = 2.0 * b[g].max() + (k + 16 + float(sel.max() - sel.min())) * U
        assert np.all(np.abs(w_gpu[t] - w_ref) <= tol), f"{what}: token {t} weights"
    return ambiguous


def expected_paths(wl, ids):
    """(GEMV, few-token matrix-core, scaled-MFMA) expert counts of a layer.
    Scaled MFMA: experts with >= 16 tokens when M >= 16 and H, I are multiples
    of 128.  Few-token matrix cores: 3..16 tokens (5..16 at H = 2560,
    I = 768, where the experts with up to 4 tokens run on the decode kernels'
    slot code, counted as GEMV) below the MFMA range when M > 4 and H, I are
    multiples of 256.  The rest: GEMV."""
    counts = np.bincount(np.asarray(ids).ravel(), minlength=wl.E)
    n = [int(c) for c in counts if c > 0] + ([wl.M] if wl.shared else [])
    mfma_on = wl.M >= 16 and wl.H % 128 == 0 and wl.I % 128 == 0
    mt_on = wl.M > 4 and wl.H % 256 == 0 and wl.I % 256 == 0
    paths = [0, 0, 0]
    for c in n:
        if mfma_on and c >= 16:
            paths[2] += 1
        elif mt_on and (5 if (wl.H, wl.I) == (2560, 768) else 3) <= c <= 16:
            paths[1] += 1
        else:
            paths[0] += 1
    return paths


def assert_paths(hdr, wl, ids, what):
    got = [hdr["gemv_experts"], hdr["mt_experts"], hdr["mfma_experts"]]
    assert got == expected_paths(wl, ids), f"{what}: expert paths (gemv, mt, mfma) {got}"
