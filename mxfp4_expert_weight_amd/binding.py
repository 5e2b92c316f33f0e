"""ctypes binding of libmoe_mxfp4.so -- argument marshalling only.

Every function has the name and argument order of the C call declared in
include/moe_mxfp4.h.  Pointer arguments accept a torch tensor (its
``data_ptr()``), an int address, or None (NULL).  ``stream`` is a hipStream_t
handle (int); None means the current torch stream when torch has a GPU, else
the default stream.  A non-OK status raises MoeError carrying the status.
There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import re

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mxfp4.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "include", "moe_mxfp4.h")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(6)


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class moe_mxfp4_weights(ctypes.Structure):
    _fields_ = [
        ("w13_q", ctypes.c_void_p),
        ("w13_s", ctypes.c_void_p),
        ("w2_q", ctypes.c_void_p),
        ("w2_s", ctypes.c_void_p),
        ("num_experts", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("has_shared", ctypes.c_int32),
    ]


class moe_exec_opts(ctypes.Structure):
    _fields_ = [
        ("act8", ctypes.c_int32),
        ("helper_streams", ctypes.c_void_p * 2),
        ("helper_events", ctypes.c_void_p * 4),
        ("gateup_events", ctypes.c_void_p * 2),
        ("down_events", ctypes.c_void_p * 2),
    ]


def make_opts(act8=False, helper_streams=None, helper_events=None, gateup_events=None,
              down_events=None) -> moe_exec_opts:
    """moe_exec_opts from plain handles (ints or None); unset fields are NULL."""
    o = moe_exec_opts()
    o.act8 = int(act8)
    for field, vals, n in (("helper_streams", helper_streams, 2), ("helper_events", helper_events, 4),
                           ("gateup_events", gateup_events, 2), ("down_events", down_events, 2)):
        if vals is not None:
            if len(vals) != n:
                raise ValueError(f"{field} takes {n} handles")
            arr = getattr(o, field)
            for i, v in enumerate(vals):
                arr[i] = v
    return o


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "moe_route": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P]),
    "moe_topk_softmax": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P, _P]),
    "moe_sort_by_expert": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P, _P, _P, _P]),
    "moe_mxfp4_forward": (ctypes.c_int, [_P, ctypes.POINTER(moe_mxfp4_weights), _I32, _I32, _P, _P,
                                         _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_layer": (ctypes.c_int, [_P, _P, _P, _I64, ctypes.POINTER(moe_mxfp4_weights), _I32, _I32, _P, _P,
                                 _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp4_forward_ex": (ctypes.c_int, [_P, ctypes.POINTER(moe_mxfp4_weights), _I32, _I32, _P, _P,
                                            _P, _P, _P, _P, _P, _SZ, ctypes.POINTER(moe_exec_opts), _P]),
    "moe_layer_ex": (ctypes.c_int, [_P, _P, _P, _I64, ctypes.POINTER(moe_mxfp4_weights), _I32, _I32, _P, _P,
                                    _P, _P, _P, _P, _P, _P, _P, _SZ, ctypes.POINTER(moe_exec_opts), _P]),
    "moe_read_probe": (ctypes.c_int, [_P, _P, _I32, _I64, _P, ctypes.c_size_t, _P, _P, _P]),
    "moe_layer_noalloc": (ctypes.c_int, [_P, _P, _P, _I64, ctypes.POINTER(moe_mxfp4_weights), _I32, _I32, _P,
                                         _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_layer_probe_stamps": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "moe_layer_probe": (ctypes.c_int, [_P, _P, _P, _I64, ctypes.POINTER(moe_mxfp4_weights), _I32, _I32, _P, _P,
                                       _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P]),
    "moe_layer_hinted": (ctypes.c_int, [_P, _P, _P, _I64, ctypes.POINTER(moe_mxfp4_weights), _I32, _I32,
                                        _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P, _P, _P, _P]),
    "moe_layer_w4a8": (ctypes.c_int, [_P, _P, _P, _I64, ctypes.POINTER(moe_mxfp4_weights), _I32, _I32, _P,
                                      _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_mxfp8_quantize": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _P, _P]),
    "moe_mxfp4_dequantize": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P]),
    "moe_prefetch_select": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "moe_prefetch_experts": (ctypes.c_int, [ctypes.POINTER(moe_mxfp4_weights), _P, _P, _I32, _I32, _P, _P]),
    "moe_lmhead_fp8_quantize": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P]),
    "moe_lmhead_fp8_logits": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _P, _P]),
}


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is not built; run `python -m mxfp4_expert_weight_amd.build` "
                "(there is no CPU fallback)")
        # torch ships its own libamdhip64 (soname libamdhip64.so.7).  Importing torch
        # first makes this library bind to that same runtime instead of loading a
        # second HIP runtime into the process (streams would not be shared).
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/moe_mxfp4.h declares."""
    src = open(HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", src)))


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(s):
    if s is not None:
        return s
    try:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
    except ImportError:
        pass
    return None


def _check(st: int, where: str):
    if st != MOE_OK:
        raise MoeError(st, where)


def status_string(st: int) -> str:
    return lib().moe_status_string(st).decode()


def moe_workspace_bytes(M, top_k, E, H, I) -> int:
    return lib().moe_workspace_bytes(M, top_k, E, H, I)


def moe_route(x, w_router, logit_bias, bias_row_stride, M, H, E, top_k, logits, topk_ids,
              topk_weights, stream=None):
    _check(lib().moe_route(_ptr(x), _ptr(w_router), _ptr(logit_bias), bias_row_stride, M, H, E,
                           top_k, _ptr(logits), _ptr(topk_ids), _ptr(topk_weights), _stream(stream)),
           "moe_route")


def moe_topk_softmax(logits, M, E, top_k, topk_ids, topk_weights, stream=None):
    _check(lib().moe_topk_softmax(_ptr(logits), M, E, top_k, _ptr(topk_ids), _ptr(topk_weights),
                                  _stream(stream)), "moe_topk_softmax")


def moe_sort_by_expert(topk_ids, M, top_k, E, expert_offsets, sorted_pairs, active_experts,
                       num_active, stream=None):
    _check(lib().moe_sort_by_expert(_ptr(topk_ids), M, top_k, E, _ptr(expert_offsets),
                                    _ptr(sorted_pairs), _ptr(active_experts), _ptr(num_active),
                                    _stream(stream)), "moe_sort_by_expert")


def make_weights(w13_q, w13_s, w2_q, w2_s, num_experts, hidden, inter, has_shared) -> moe_mxfp4_weights:
    return moe_mxfp4_weights(_ptr(w13_q), _ptr(w13_s), _ptr(w2_q), _ptr(w2_s),
                             num_experts, hidden, inter, int(has_shared))


def moe_mxfp4_forward(x, w: moe_mxfp4_weights, M, top_k, topk_weights, expert_offsets, sorted_pairs,
                      active_experts, num_active, y, workspace, workspace_bytes, stream=None):
    _check(lib().moe_mxfp4_forward(_ptr(x), ctypes.byref(w) if w is not None else None, M, top_k,
                                   _ptr(topk_weights), _ptr(expert_offsets), _ptr(sorted_pairs),
                                   _ptr(active_experts), _ptr(num_active), _ptr(y), _ptr(workspace),
                                   workspace_bytes, _stream(stream)), "moe_mxfp4_forward")


def moe_layer(x, w_router, logit_bias, bias_row_stride, w: moe_mxfp4_weights, M, top_k, logits,
              topk_ids, topk_weights, expert_offsets, sorted_pairs, active_experts, num_active, y,
              workspace, workspace_bytes, stream=None):
    _check(lib().moe_layer(_ptr(x), _ptr(w_router), _ptr(logit_bias), bias_row_stride,
                           ctypes.byref(w) if w is not None else None, M, top_k, _ptr(logits),
                           _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_offsets), _ptr(sorted_pairs),
                           _ptr(active_experts), _ptr(num_active), _ptr(y), _ptr(workspace),
                           workspace_bytes, _stream(stream)), "moe_layer")


def moe_layer_ex(x, w_router, logit_bias, bias_row_stride, w: moe_mxfp4_weights, M, top_k, logits,
                 topk_ids, topk_weights, expert_offsets, sorted_pairs, active_experts, num_active, y,
                 workspace, workspace_bytes, opts: moe_exec_opts | None = None, stream=None):
    _check(lib().moe_layer_ex(_ptr(x), _ptr(w_router), _ptr(logit_bias), bias_row_stride,
                              ctypes.byref(w) if w is not None else None, M, top_k, _ptr(logits),
                              _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_offsets), _ptr(sorted_pairs),
                              _ptr(active_experts), _ptr(num_active), _ptr(y), _ptr(workspace), workspace_bytes,
                              ctypes.byref(opts) if opts is not None else None, _stream(stream)), "moe_layer_ex")


def moe_mxfp4_forward_ex(x, w: moe_mxfp4_weights, M, top_k, topk_weights, expert_offsets, sorted_pairs,
                         active_experts, num_active, y, workspace, workspace_bytes,
                         opts: moe_exec_opts | None = None, stream=None):
    _check(lib().moe_mxfp4_forward_ex(_ptr(x), ctypes.byref(w) if w is not None else None, M, top_k,
                                      _ptr(topk_weights), _ptr(expert_offsets), _ptr(sorted_pairs),
                                      _ptr(active_experts), _ptr(num_active), _ptr(y), _ptr(workspace),
                                      workspace_bytes, ctypes.byref(opts) if opts is not None else None,
                                      _stream(stream)), "moe_mxfp4_forward_ex")


READ_PROBE_CHUNK = 16384                # MOE_READ_PROBE_CHUNK: bytes per moe_read_probe output word


def read_probe_words(n, max_bytes) -> int:
    return n * (-(-max_bytes // READ_PROBE_CHUNK))


def moe_read_probe(addrs, sizes, n, max_bytes, out, out_words, start_event=None, stop_event=None, stream=None):
    _check(lib().moe_read_probe(_ptr(addrs), _ptr(sizes), n, max_bytes, _ptr(out), out_words, start_event,
                                stop_event, _stream(stream)), "moe_read_probe")


NOALLOC_WORKSPACE_BYTES = 8 << 20      # MOE_NOALLOC_WORKSPACE_BYTES


def moe_layer_noalloc(x, w_router, logit_bias, bias_row_stride, w: moe_mxfp4_weights, M, top_k, logits,
                      topk_ids, topk_weights, expert_offsets, sorted_pairs, active_experts, num_active, y,
                      stream=None):
    _check(lib().moe_layer_noalloc(_ptr(x), _ptr(w_router), _ptr(logit_bias), bias_row_stride,
                                   ctypes.byref(w) if w is not None else None, M, top_k, _ptr(logits),
                                   _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_offsets), _ptr(sorted_pairs),
                                   _ptr(active_experts), _ptr(num_active), _ptr(y), _stream(stream)),
           "moe_layer_noalloc")


def moe_layer_probe_stamps(M, top_k, E, H, I) -> int:
    return lib().moe_layer_probe_stamps(M, top_k, E, H, I)


def moe_layer_probe(x, w_router, logit_bias, bias_row_stride, w: moe_mxfp4_weights, M, top_k, logits,
                    topk_ids, topk_weights, expert_offsets, sorted_pairs, active_experts, num_active, y,
                    workspace, workspace_bytes, stamps, num_stamps, stream=None):
    _check(lib().moe_layer_probe(_ptr(x), _ptr(w_router), _ptr(logit_bias), bias_row_stride,
                                 ctypes.byref(w) if w is not None else None, M, top_k, _ptr(logits),
                                 _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_offsets), _ptr(sorted_pairs),
                                 _ptr(active_experts), _ptr(num_active), _ptr(y), _ptr(workspace), workspace_bytes,
                                 _ptr(stamps), num_stamps, _stream(stream)), "moe_layer_probe")


def moe_layer_hinted(x, w_router, logit_bias, bias_row_stride, w: moe_mxfp4_weights, M, top_k, logits,
                     topk_ids, topk_weights, expert_offsets, sorted_pairs, active_experts, num_active, y,
                     workspace, workspace_bytes, hint_experts, num_hint, start_event=None, stop_event=None,
                     stream=None):
    _check(lib().moe_layer_hinted(_ptr(x), _ptr(w_router), _ptr(logit_bias), bias_row_stride,
                                  ctypes.byref(w) if w is not None else None, M, top_k, _ptr(logits),
                                  _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_offsets), _ptr(sorted_pairs),
                                  _ptr(active_experts), _ptr(num_active), _ptr(y), _ptr(workspace),
                                  workspace_bytes, _ptr(hint_experts), _ptr(num_hint), start_event, stop_event,
                                  _stream(stream)), "moe_layer_hinted")


def moe_layer_w4a8(x, w_router, logit_bias, bias_row_stride, w: moe_mxfp4_weights, M, top_k, logits,
                   topk_ids, topk_weights, expert_offsets, sorted_pairs, active_experts, num_active, y,
                   workspace, workspace_bytes, stream=None):
    _check(lib().moe_layer_w4a8(_ptr(x), _ptr(w_router), _ptr(logit_bias), bias_row_stride,
                                ctypes.byref(w) if w is not None else None, M, top_k, _ptr(logits),
                                _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_offsets), _ptr(sorted_pairs),
                                _ptr(active_experts), _ptr(num_active), _ptr(y), _ptr(workspace),
                                workspace_bytes, _stream(stream)), "moe_layer_w4a8")


def moe_mxfp8_quantize(x, rows, K, codes, scales, values, stream=None):
    _check(lib().moe_mxfp8_quantize(_ptr(x), rows, K, _ptr(codes), _ptr(scales), _ptr(values), _stream(stream)),
           "moe_mxfp8_quantize")


def moe_mxfp4_dequantize(q, s, rows, cols, out, stream=None):
    _check(lib().moe_mxfp4_dequantize(_ptr(q), _ptr(s), rows, cols, _ptr(out), _stream(stream)),
           "moe_mxfp4_dequantize")


def moe_prefetch_select(draft_ids, n_ids, E, has_shared, max_experts, expert_ids, num_selected, stream=None):
    _check(lib().moe_prefetch_select(_ptr(draft_ids), n_ids, E, int(has_shared), max_experts, _ptr(expert_ids),
                                     _ptr(num_selected), _stream(stream)), "moe_prefetch_select")


def moe_prefetch_experts(w: moe_mxfp4_weights, expert_ids, num_live, max_ids, parts, checksums, stream=None):
    _check(lib().moe_prefetch_experts(ctypes.byref(w) if w is not None else None, _ptr(expert_ids), _ptr(num_live),
                                      max_ids, parts, _ptr(checksums), _stream(stream)), "moe_prefetch_experts")


def moe_lmhead_fp8_quantize(w_bf16, V, H, codes, scales, stream=None):
    _check(lib().moe_lmhead_fp8_quantize(_ptr(w_bf16), V, H, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_lmhead_fp8_quantize")


def moe_lmhead_fp8_logits(x, codes, scales, M, V, H, logits, stream=None):
    _check(lib().moe_lmhead_fp8_logits(_ptr(x), _ptr(codes), _ptr(scales), M, V, H, _ptr(logits), _stream(stream)),
           "moe_lmhead_fp8_logits")
