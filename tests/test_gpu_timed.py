"""The timed entry points (moe_layer_timed, moe_layer_w4a8_timed) through the
C ABI: with or without events they give moe_layer's (moe_layer_w4a8's)
routing exactly and its output within the layer tolerance of the float64
oracle, and the events bound a positive, finite kernel time.  Decode (the
routed gate/up kernel) and a batch (the GEMV gate/up kernel beside the
matrix-core paths) are both covered."""
import ctypes
import math

import numpy as np
import pytest

import oracle
from gpu_common import assert_layer_close, need_gpu, say
from mxfp4_expert_weight_amd import binding as B
from mxfp4_expert_weight_amd import synth

pytestmark = pytest.mark.gpu


class _Events:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ctypes.c_void_p(ev))


@pytest.mark.parametrize("name,w4a8", [("tiny", False), ("ling_m4_mtp", False), ("tiny", True),
                                       ("m24", False), ("m24", True)])
def test_timed_matches_untimed(name, w4a8):
    torch = need_gpu()
    from mxfp4_expert_weight_amd.layer import DeviceLayerSet, LayerBuffers, run_layer
    wl = synth.custom("m24", 24, 512, 512, 10, 3, True, "zipf", seed=7) if name == "m24" else name
    ls = synth.layer_set(wl)
    wl = ls.wl
    say(f"timed entry point: {wl.name} w4a8={w4a8}")
    d = DeviceLayerSet.from_host(ls)
    b = LayerBuffers(wl.M, wl.k, wl.E, wl.H, wl.I)
    run_layer(d, b, w4a8=w4a8)
    torch.cuda.synchronize()
    ref = dict(ids=b.ids.cpu().numpy(), w=b.weights.cpu().numpy(), logits=b.logits.cpu().numpy(),
               y=b.y.cpu().numpy())
    timed = B.moe_layer_w4a8_timed if w4a8 else B.moe_layer_timed
    ev = _Events()
    start, stop = ev.create(), ev.create()
    stream = torch.cuda.current_stream().cuda_stream
    for events in ((start, stop), (None, None)):
        b.y.fill_(float("nan"))
        torch.cuda.synchronize()
        timed(d.x, d.w_router, d.bias, d.bias_row_stride, d.weights(), d.M, d.k, b.logits, b.ids, b.weights,
              b.offsets, b.pairs, b.active, b.num_active, b.y, b.ws, b.ws_bytes, events[0], events[1], stream)
        torch.cuda.synchronize()
        assert np.array_equal(b.ids.cpu().numpy(), ref["ids"])
        assert np.array_equal(b.weights.cpu().numpy(), ref["w"])
        assert np.array_equal(b.logits.cpu().numpy(), ref["logits"])
        y = b.y.cpu().numpy()
        assert np.all(np.isfinite(y))
        # the same layer as the untimed call (fp32 atomics may reorder the sum)
        assert np.allclose(y, ref["y"], rtol=1e-5, atol=1e-5 * float(np.sqrt(np.mean(ref["y"] ** 2))))
        if events[0] is not None:
            ms = ev.elapsed_ms(start, stop)
            assert math.isfinite(ms) and 0.0 < ms < 1000.0, ms
    ev.destroy(start)
    ev.destroy(stop)
    if not w4a8 and wl.M <= 4:
        r = oracle.moe_layer(ls.x_bits, ls.w_router, ls.bias, ls.w13_q, ls.w13_s, ls.w2_q, ls.w2_s, wl.k, wl.shared)
        assert np.array_equal(ref["ids"], r["ids"])
        assert_layer_close(b.y.cpu().numpy(), r["y"], what=f"{wl.name} timed")
