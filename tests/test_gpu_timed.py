"""moe_layer_ex through the C ABI: with timing events on the gate/up and down
kernels, with the caller's helper streams, or with neither, it gives
moe_layer's (moe_layer_w4a8's) routing exactly and its output within 1e-5 of
it (and within the layer tolerance of the float64 oracle for decode); the
events bound positive, finite kernel times.  Decode (the routed gate/up
kernel) and a batch (the GEMV gate/up kernel beside the matrix-core paths)
are both covered."""
import math

import numpy as np
import pytest

import oracle
from gpu_common import assert_layer_close, need_gpu, say
from mxfp4_expert_weight_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,w4a8", [("tiny", False), ("ling_m4_mtp", False), ("tiny", True),
                                       ("m24", False), ("m24", True)])
def test_ex_matches_plain(name, w4a8):
    torch = need_gpu()
    from mxfp4_expert_weight_amd.layer import DeviceLayerSet, HelperStreams, HipEvents, LayerBuffers, run_layer
    wl = synth.custom("m24", 24, 512, 512, 10, 3, True, "zipf", seed=7) if name == "m24" else name
    ls = synth.layer_set(wl)
    wl = ls.wl
    say(f"moe_layer_ex: {wl.name} w4a8={w4a8}")
    d = DeviceLayerSet.from_host(ls)
    b = LayerBuffers(wl.M, wl.k, wl.E, wl.H, wl.I)
    w = d.weights()
    run_layer(d, b, w, w4a8=w4a8)
    torch.cuda.synchronize()
    ref = dict(ids=b.ids.cpu().numpy(), w=b.weights.cpu().numpy(), logits=b.logits.cpu().numpy(),
               y=b.y.cpu().numpy(), hdr=b.header())
    ev = HipEvents()
    evs = [ev.create() for _ in range(4)]
    helpers = HelperStreams()
    cases = [dict(gateup_events=evs[:2], down_events=evs[2:]), dict(helpers=helpers),
             dict(helpers=helpers, gateup_events=evs[:2], down_events=evs[2:]), dict()]
    for kw in cases:
        b.y.fill_(float("nan"))
        torch.cuda.synchronize()
        run_layer(d, b, w, w4a8=w4a8, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(b.ids.cpu().numpy(), ref["ids"])
        assert np.array_equal(b.weights.cpu().numpy(), ref["w"])
        assert np.array_equal(b.logits.cpu().numpy(), ref["logits"])
        assert b.header() == ref["hdr"]
        y = b.y.cpu().numpy()
        assert np.all(np.isfinite(y))
        # the same layer as the plain call (fp32 atomics may reorder the sum)
        assert np.allclose(y, ref["y"], rtol=1e-5, atol=1e-5 * float(np.sqrt(np.mean(ref["y"] ** 2))))
        if "gateup_events" in kw:
            for a, z in ((evs[0], evs[1]), (evs[2], evs[3])):
                ms = ev.elapsed_ms(a, z)
                assert math.isfinite(ms) and 0.0 < ms < 1000.0, ms
    for e in evs:
        ev.destroy(e)
    if not w4a8 and wl.M <= 4:
        r = oracle.moe_layer(ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s, wl.k, wl.shared)
        assert np.array_equal(ref["ids"], r["ids"])
        assert_layer_close(b.y.cpu().numpy(), r["y"], what=f"{wl.name} ex")
