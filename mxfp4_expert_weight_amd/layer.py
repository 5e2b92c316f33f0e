"""Device buffers for the layer, allocated with torch; compute goes through
the C ABI only (``binding``).  torch is used for device memory and streams.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import binding


def to_device(a: Optional[np.ndarray], device="cuda") -> Optional[torch.Tensor]:
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:          # bf16 bit patterns travel as int16 storage
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


@dataclass
class DeviceLayerSet:
    """One layer's inputs on the device (canonical layouts)."""
    x: torch.Tensor            # int16 [M][H] (bf16 bits)
    w_router: torch.Tensor     # float32 [E][H]
    bias: Optional[torch.Tensor]
    bias_row_stride: int
    w13_q: torch.Tensor
    w13_s: torch.Tensor
    w2_q: torch.Tensor
    w2_s: torch.Tensor
    M: int
    H: int
    I: int
    E: int
    k: int
    has_shared: bool

    @staticmethod
    def from_host(ls, device="cuda") -> "DeviceLayerSet":
        wl = ls.wl
        return DeviceLayerSet(to_device(ls.x_bits, device), to_device(ls.w_router, device),
                              to_device(ls.bias, device), ls.bias_row_stride,
                              to_device(ls.w13_q, device), to_device(ls.w13_s, device),
                              to_device(ls.w2_q, device), to_device(ls.w2_s, device),
                              wl.M, wl.H, wl.I, wl.E, wl.k, wl.shared)

    def weights(self) -> binding.moe_mxfp4_weights:
        return binding.make_weights(self.w13_q, self.w13_s, self.w2_q, self.w2_s, self.E, self.H,
                                    self.I, self.has_shared)


class LayerBuffers:
    """Routing, sort and output buffers for a (M, k, E, H, I) shape."""

    def __init__(self, M, k, E, H, I, device="cuda"):
        self.M, self.k, self.E, self.H, self.I = M, k, E, H, I
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        self.logits = torch.empty((M, E), **f32)
        self.ids = torch.empty((M, k), **i32)
        self.weights = torch.empty((M, k), **f32)
        self.offsets = torch.empty((E + 1,), **i32)
        self.pairs = torch.empty((M * k,), **i32)
        self.active = torch.empty((E,), **i32)
        self.num_active = torch.empty((1,), **i32)
        self.y = torch.empty((M, H), **f32)
        self.ws_bytes = binding.moe_workspace_bytes(M, k, E, H, I)
        if self.ws_bytes == 0:
            raise ValueError("shape outside the library's limits")
        self.ws = torch.empty((self.ws_bytes,), dtype=torch.uint8, device=device)

    def header(self) -> dict:
        h = self.ws[:16].view(torch.int32).cpu().tolist()
        return dict(gemv_experts=h[0], mfma_experts=h[1], mfma_items=h[2], mt_experts=h[3])


class HipEvents:
    """hipEvent_t handles made through the HIP runtime torch already loaded
    (torch's own events are created lazily, on their first record)."""

    DISABLE_TIMING = 0x2

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, timing=True) -> int:
        ev = ctypes.c_void_p()
        flags = 0 if timing else self.DISABLE_TIMING
        if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), flags) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return ev.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ctypes.c_void_p(ev))


class HelperStreams:
    """The caller-owned helper streams (two torch streams, default priority) and
    fork/join events (four, timing disabled) that let a batch's matrix-core
    expert kernels run beside the GEMV ones (moe_exec_opts).  One set per
    concurrently enqueued layer."""

    def __init__(self):
        self.streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        self._ev = HipEvents()
        self.events = [self._ev.create(timing=False) for _ in range(4)]

    def opts(self, **kw) -> binding.moe_exec_opts:
        return binding.make_opts(helper_streams=[s.cuda_stream for s in self.streams], helper_events=self.events,
                                 **kw)

    def __del__(self):
        for e in getattr(self, "events", []):
            try:
                self._ev.destroy(e)
            except Exception:
                pass


def run_layer(d: DeviceLayerSet, b: LayerBuffers, w: Optional[binding.moe_mxfp4_weights] = None,
              stream=None, fused: bool = True, w4a8: bool = False, helpers: Optional[HelperStreams] = None,
              gateup_events=None, down_events=None):
    """One layer: moe_layer (fused=True) or moe_route -> moe_sort_by_expert ->
    moe_mxfp4_forward (fused=False); same outputs, stream-ordered.  w4a8: the
    W4A8 variant (MXFP8 activations into the experts).  helpers: the batch's
    matrix-core kernels on helper streams; gateup_events / down_events: (begin,
    end) event handles bound to the GEMV gate/up / down kernels."""
    if w is None:
        w = d.weights()
    opts = None
    if w4a8 or helpers is not None or gateup_events is not None or down_events is not None:
        kw = dict(act8=w4a8, gateup_events=gateup_events, down_events=down_events)
        opts = helpers.opts(**kw) if helpers is not None else binding.make_opts(**kw)
    if fused:
        if opts is None:
            binding.moe_layer(d.x, d.w_router, d.bias, d.bias_row_stride, w, d.M, d.k, b.logits, b.ids,
                              b.weights, b.offsets, b.pairs, b.active, b.num_active, b.y, b.ws, b.ws_bytes,
                              stream)
        else:
            binding.moe_layer_ex(d.x, d.w_router, d.bias, d.bias_row_stride, w, d.M, d.k, b.logits, b.ids,
                                 b.weights, b.offsets, b.pairs, b.active, b.num_active, b.y, b.ws, b.ws_bytes,
                                 opts, stream)
        return
    binding.moe_route(d.x, d.w_router, d.bias, d.bias_row_stride, d.M, d.H, d.E, d.k, b.logits, b.ids,
                      b.weights, stream)
    binding.moe_sort_by_expert(b.ids, d.M, d.k, d.E, b.offsets, b.pairs, b.active, b.num_active, stream)
    if opts is None:
        binding.moe_mxfp4_forward(d.x, w, d.M, d.k, b.weights, b.offsets, b.pairs, b.active, b.num_active,
                                  b.y, b.ws, b.ws_bytes, stream)
    else:
        binding.moe_mxfp4_forward_ex(d.x, w, d.M, d.k, b.weights, b.offsets, b.pairs, b.active, b.num_active,
                                     b.y, b.ws, b.ws_bytes, opts, stream)
