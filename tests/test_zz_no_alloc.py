"""moe_layer_noalloc (the layer on the library's static per-GPU workspace)
against moe_layer (the caller's workspace), through the C ABI, on calls in a
row that shrink: a 32-token batch, then 4 and 1 tokens (the decode path), then
the batch again over what the smaller calls left in the static array."""
import numpy as np
import pytest

from gpu_common import need_gpu, say
from mxfp4_expert_weight_amd import binding as B
from mxfp4_expert_weight_amd import synth

pytestmark = pytest.mark.gpu


def _outputs(b, M, k, E):
    n = int(b.num_active.cpu().item())
    return dict(logits=b.logits[:M].cpu().numpy(), ids=b.ids[:M].cpu().numpy(), w=b.weights[:M].cpu().numpy(),
                offsets=b.offsets.cpu().numpy(), active=b.active.cpu().numpy()[:n], n=n,
                pairs=b.pairs[:M * k].cpu().numpy(), y=b.y[:M].cpu().numpy())


def _same_layer(got, ref, what):
    for key in ("logits", "ids", "w", "offsets", "active"):
        assert np.array_equal(got[key], ref[key]), f"{what}: {key}"
    assert got["n"] == ref["n"], what
    off = ref["offsets"]
    for e in ref["active"]:       # pairs of one expert: the same set (their order is not part of the result)
        a, z = off[e], off[e + 1]
        assert np.array_equal(np.sort(got["pairs"][a:z]), np.sort(ref["pairs"][a:z])), f"{what}: expert {e}"
    y, yr = got["y"], ref["y"]
    assert np.all(np.isfinite(y)), what
    # the same kernels on the same inputs: equal up to the order of the fp32
    # atomic adds into y
    rms = float(np.sqrt(np.mean(yr.astype(np.float64) ** 2)))
    assert np.allclose(y, yr, rtol=1e-5, atol=1e-5 * rms), f"{what}: max |dy| {np.abs(y - yr).max():.3g}"


def test_noalloc_matches_moe_layer():
    torch = need_gpu()
    from mxfp4_expert_weight_amd.layer import DeviceLayerSet, LayerBuffers, run_layer
    ls = synth.layer_set("ling_m32_zipf")
    wl = ls.wl
    d = DeviceLayerSet.from_host(ls)
    w = d.weights()
    big = LayerBuffers(wl.M, wl.k, wl.E, wl.H, wl.I)
    assert big.ws_bytes <= B.NOALLOC_WORKSPACE_BYTES
    out = LayerBuffers(wl.M, wl.k, wl.E, wl.H, wl.I)     # the no-alloc call's outputs (no workspace used)
    for M in (32, 4, 1, 32):
        say(f"moe_layer_noalloc vs moe_layer: ling_m32_zipf weights, M={M}")
        d.M = M
        xs = d.x
        d.x = xs[:M].contiguous()
        for b in (big, out):
            b.y.fill_(float("nan"))
            b.ids.fill_(-1)
        torch.cuda.synchronize()
        run_layer(d, big, w)
        B.moe_layer_noalloc(d.x, d.w_router, d.bias, d.bias_row_stride, w, M, wl.k, out.logits, out.ids,
                            out.weights, out.offsets, out.pairs, out.active, out.num_active, out.y, None)
        torch.cuda.synchronize()
        d.x = xs
        ref, got = _outputs(big, M, wl.k, wl.E), _outputs(out, M, wl.k, wl.E)
        _same_layer(got, ref, f"M={M}")
        assert np.all(np.isnan(out.y[M:].cpu().numpy())), f"M={M}: rows past M written"
