// C ABI of the MXFP4 MoE layer: host-side argument checks, then launches.
// Nothing here allocates device memory, synchronises or keeps state between
// calls; streams and events other than the caller's `stream` come from the
// caller (moe_exec_opts).
#include <atomic>
#include <climits>

#include "kernels.h"

using namespace moe;

// Workspace of moe_layer_noalloc: one array per GPU, held until the process
// ends.  On the host, `scratch` names a stand-in, not a device address: host
// code only ever passes the address hipGetSymbolAddress returns for it.
constexpr size_t kNoAllocScratchBytes = size_t(MOE_NOALLOC_WORKSPACE_BYTES);
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_route_sizes(int32_t M, int32_t E, int32_t k) {
  if (M < 1 || M > MOE_MAX_TOKENS) return MOE_ERR_SHAPE;
  if (E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
  if (k < 1 || k > MOE_MAX_TOPK || k > E) return MOE_ERR_SHAPE;
  return MOE_OK;
}

moe_status check_hidden(int32_t H) {
  if (H < 32 || H > MOE_MAX_HIDDEN || H % 32) return MOE_ERR_SHAPE;
  return MOE_OK;
}

moe_status check_inter(int32_t I) {
  if (I < 32 || I > MOE_MAX_INTER || I % 32) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// Arguments of the expert stage; the slot records live in the workspace.  The
// MFMA fields are set when the path is on for these sizes.  act8 (W4A8): the
// experts read the MXFP8 x from the workspace.
ForwardArgs layer_args(const uint16_t* x, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                       const float* topk_weights, const int32_t* expert_offsets, const int32_t* sorted_pairs,
                       const int32_t* active_experts, const int32_t* num_active, float* y, void* workspace,
                       bool act8 = false) {
  const WorkspaceLayout L = workspace_layout(M, top_k, w->num_experts, w->hidden, w->inter);
  char* ws = reinterpret_cast<char*>(workspace);
  ForwardArgs a{};
  a.x = x;
  a.w13_q = w->w13_q; a.w13_s = w->w13_s; a.w2_q = w->w2_q; a.w2_s = w->w2_s;
  a.topk_weights = topk_weights;
  a.offsets = expert_offsets; a.sorted_pairs = sorted_pairs;
  a.active = active_experts; a.num_active = num_active;
  a.y = y;
  a.hdr = reinterpret_cast<WorkspaceHeader*>(workspace);
  a.rec = reinterpret_cast<const SlotRec*>(ws + L.rec);
  a.h = reinterpret_cast<uint16_t*>(ws + L.h);
  a.hlo = reinterpret_cast<uint16_t*>(ws + L.hlo);
  a.M = M; a.k = top_k; a.E = w->num_experts; a.H = w->hidden; a.I = w->inter;
  a.has_shared = w->has_shared;
  const bool mt = mt_path(M, a.H, a.I);
  a.mt_min = mt ? mt_min_tokens(a.H, a.I) : INT_MAX;
  a.mt_max = kMtMaxTokens;
  const bool on = mfma_path(M, a.H, a.I);
  a.mfma_min = on ? kMfmaMinTokens : INT_MAX;
  if (on) {
    a.xq_hi = reinterpret_cast<uint8_t*>(ws + L.xq_hi);
    a.xq_lo = reinterpret_cast<uint8_t*>(ws + L.xq_lo);
    a.xq_shi = reinterpret_cast<uint8_t*>(ws + L.xq_shi);
    a.xq_slo = reinterpret_cast<uint8_t*>(ws + L.xq_slo);
    a.hq_hi = reinterpret_cast<uint8_t*>(ws + L.hq_hi);
    a.hq_lo = reinterpret_cast<uint8_t*>(ws + L.hq_lo);
    a.hq_shi = reinterpret_cast<uint8_t*>(ws + L.hq_shi);
    a.hq_slo = reinterpret_cast<uint8_t*>(ws + L.hq_slo);
    a.items = reinterpret_cast<const int2*>(ws + L.items);
  }
  if (combine_rows(M, top_k, a.H)) {
    a.yp = reinterpret_cast<float*>(ws + L.yp);
    a.inv = reinterpret_cast<const int*>(ws + L.inv);
  }
  if (M > kRoutedMaxTokens) a.lists = reinterpret_cast<const int*>(ws + L.lists);
  if (act8) {
    a.act8 = 1;
    a.x = reinterpret_cast<const uint16_t*>(ws + L.xdq);
  }
  return a;
}

RecOut layer_recout(const ForwardArgs& a, void* workspace) {
  return RecOut{const_cast<SlotRec*>(a.rec), a.topk_weights, a.M, a.k, a.has_shared, a.mfma_min,
                const_cast<int2*>(a.items), reinterpret_cast<WorkspaceHeader*>(workspace), a.mt_min, a.mt_max,
                const_cast<int*>(a.inv), const_cast<int*>(a.lists)};
}

// The caller's helper streams and events (moe_exec_opts), if any: batches fork
// the matrix-core expert kernels onto them and join them back to `stream`.
// The library keeps none of its own.
struct Helpers {
  hipStream_t mt, mfma;
  hipEvent_t fork, zeroed, mt_done, mfma_done;
};

bool helpers_of(const moe_exec_opts* o, Helpers& h) {
  if (!o || !o->helper_streams[0]) return false;
  h.mt = (hipStream_t)o->helper_streams[0];
  h.mfma = (hipStream_t)o->helper_streams[1];
  h.fork = (hipEvent_t)o->helper_events[0];
  h.zeroed = (hipEvent_t)o->helper_events[1];
  h.mt_done = (hipEvent_t)o->helper_events[2];
  h.mfma_done = (hipEvent_t)o->helper_events[3];
  return true;
}

// Host check of the options: helper streams come as a pair with all four events.
moe_status check_opts(const moe_exec_opts* o) {
  if (!o) return MOE_OK;
  if (o->act8 != 0 && o->act8 != 1) return MOE_ERR_SHAPE;
  const bool any = o->helper_streams[0] || o->helper_streams[1];
  if (any) {
    if (!o->helper_streams[0] || !o->helper_streams[1]) return MOE_ERR_NULL;
    for (void* e : o->helper_events)
      if (!e) return MOE_ERR_NULL;
  }
  return MOE_OK;
}

// The expert stage: GEMV gate/up (zeroes y) and down for the experts with
// one or two tokens; with the few-token path on, its kernels take experts of
// kMtMinTokens..kMtMaxTokens tokens; with the MFMA path on, x is quantised
// first and the dense kernels take the experts listed in the work items.
// The three paths touch disjoint experts and h rows, so with the caller's
// helper streams the matrix-core kernels run beside the GEMV ones.  With
// atomics into y, their down kernels wait for the GEMV gate/up kernel that
// zeroes y; when combining by rows nothing waits, and the combine kernel runs
// after the join.  Without helpers every kernel goes on `s` in order.
// Batches of at least this many tokens put most experts on the few-token path.
constexpr int kMtFirstTokens = 256;

hipError_t launch_experts(const ForwardArgs& a, hipStream_t s, const moe_exec_opts* o) {
  const bool mfma = a.mfma_min == kMfmaMinTokens;
  const bool mt = a.mt_min != INT_MAX;
  const bool rows = a.yp != nullptr;
  const Timing tm = timing_of(o);
  hipError_t e = hipSuccess;
  Helpers q{};
  if (!(mt || mfma) || !helpers_of(o, q)) {
    if (mfma && !a.act8 && (e = launch_forward_mfma_front(a, s)) != hipSuccess) return e;
    if ((e = launch_forward(a, s, tm)) != hipSuccess) return e;
    if (mt) {
      if ((e = launch_gateup_mt(a, s)) != hipSuccess) return e;
      if (a.act8 && (e = launch_h_round_trip(a, 1, s)) != hipSuccess) return e;
      if ((e = launch_down_mt(a, s)) != hipSuccess) return e;
    }
    if (mfma) {
      if ((e = launch_gateup_mfma(a, s)) != hipSuccess) return e;
      if ((e = launch_down_mfma(a, s)) != hipSuccess) return e;
    }
    if (rows) e = launch_combine_rows(a, s);
    return e;
  }
  // the GEMV kernels go first (their few workgroups are then not queued
  // behind the matrix-core paths' many); the fork point is before them.
  // From kMtFirstTokens tokens the few-token gate/up kernel, then the
  // longest path, is enqueued ahead of them.
  if ((e = hipEventRecord(q.fork, s)) != hipSuccess) return e;
  const bool mt_first = mt && a.M >= kMtFirstTokens;
  if (mt_first) {
    if ((e = hipStreamWaitEvent(q.mt, q.fork, 0)) != hipSuccess) return e;
    if ((e = launch_gateup_mt(a, q.mt)) != hipSuccess) return e;
  }
  if ((e = launch_forward(a, s, tm, q.zeroed)) != hipSuccess) return e;
  if (mt && !mt_first && (e = hipStreamWaitEvent(q.mt, q.fork, 0)) != hipSuccess) return e;
  if (mfma && (e = hipStreamWaitEvent(q.mfma, q.fork, 0)) != hipSuccess) return e;
  if (mt && !mt_first && (e = launch_gateup_mt(a, q.mt)) != hipSuccess) return e;
  if (mt && a.act8 && (e = launch_h_round_trip(a, 1, q.mt)) != hipSuccess) return e;
  if (mfma) {
    if (!a.act8 && (e = launch_forward_mfma_front(a, q.mfma)) != hipSuccess) return e;
    if ((e = launch_gateup_mfma(a, q.mfma)) != hipSuccess) return e;
  }
  if (mt) {
    if (!rows && (e = hipStreamWaitEvent(q.mt, q.zeroed, 0)) != hipSuccess) return e;
    if ((e = launch_down_mt(a, q.mt)) != hipSuccess) return e;
    if ((e = hipEventRecord(q.mt_done, q.mt)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(s, q.mt_done, 0)) != hipSuccess) return e;
  }
  if (mfma) {
    if (!rows && (e = hipStreamWaitEvent(q.mfma, q.zeroed, 0)) != hipSuccess) return e;
    if ((e = launch_down_mfma(a, q.mfma)) != hipSuccess) return e;
    if ((e = hipEventRecord(q.mfma_done, q.mfma)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(s, q.mfma_done, 0)) != hipSuccess) return e;
  }
  if (rows) e = launch_combine_rows(a, s);
  return e;
}

// W4A8 (act8): the experts' x as MXFP8 values.  Decode batches with short
// rows round x as the gate/up kernel stages it; otherwise x is quantised once
// into the workspace (values for the GEMV and few-token paths, codes and
// scales for the scaled-MFMA path, which takes one term).
hipError_t prepare_act8(ForwardArgs& a, const uint16_t* x, int M, int H, hipStream_t s) {
  if (M <= kRoutedMaxTokens && routed_stages_x(H)) {
    a.x = x;
    return hipSuccess;
  }
  const bool mfma = a.mfma_min == kMfmaMinTokens;
  return launch_mxfp8_quantize(x, M, H, mfma ? a.xq_hi : nullptr, mfma ? a.xq_shi : nullptr,
                               const_cast<uint16_t*>(a.x), s);
}

moe_status check_bank(const moe_mxfp4_weights* w) {
  if (!w->w13_q || !w->w13_s || !w->w2_q || !w->w2_s) return MOE_ERR_NULL;
  moe_status st;
  if ((st = check_hidden(w->hidden)) != MOE_OK) return st;
  if ((st = check_inter(w->inter)) != MOE_OK) return st;
  if (w->has_shared != 0 && w->has_shared != 1) return MOE_ERR_SHAPE;
  if (!aligned16(w->w13_q) || !aligned16(w->w13_s) || !aligned16(w->w2_q) || !aligned16(w->w2_s))
    return MOE_ERR_ALIGN;
  return MOE_OK;
}

moe_status layer_impl(const uint16_t* x, const float* w_router, const float* logit_bias,
                      int64_t bias_row_stride, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                      float* logits, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                      int32_t* sorted_pairs, int32_t* active_experts, int32_t* num_active, float* y,
                      void* workspace, size_t workspace_bytes_, const moe_exec_opts* opts, void* stream,
                      const int32_t* hint = nullptr, const int32_t* num_hint = nullptr,
                      unsigned long long* probe = nullptr) {
  if (!x || !w_router || !w || !logits || !topk_ids || !topk_weights || !expert_offsets ||
      !sorted_pairs || !active_experts || !num_active || !y || !workspace)
    return MOE_ERR_NULL;
  moe_status st = check_bank(w);
  if (st != MOE_OK) return st;
  const int32_t E = w->num_experts, H = w->hidden;
  if ((st = check_route_sizes(M, E, top_k)) != MOE_OK) return st;
  if ((st = check_opts(opts)) != MOE_OK) return st;
  if (logit_bias && bias_row_stride != 0 && bias_row_stride != E) return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w_router) || ((uintptr_t)workspace & 255u)) return MOE_ERR_ALIGN;
  if (workspace_bytes_ < workspace_layout(M, top_k, E, H, w->inter).total) return MOE_ERR_WORKSPACE;
  const bool act8 = opts && opts->act8;
  hipStream_t s = (hipStream_t)stream;
  if (launch_router_logits(x, w_router, logit_bias, logit_bias ? bias_row_stride : 0, M, H, E, logits,
                           s) != hipSuccess)
    return MOE_ERR_HIP;
  ForwardArgs a = layer_args(x, w, M, top_k, topk_weights, expert_offsets, sorted_pairs, active_experts,
                             num_active, y, workspace, act8);
  a.hint = hint;
  a.num_hint = num_hint;
  if (act8 && prepare_act8(a, x, M, H, s) != hipSuccess) return MOE_ERR_HIP;
  SlotRec* rec = const_cast<SlotRec*>(a.rec);
  if (M <= kRoutedMaxTokens) {
    // decode: every gate/up block routes itself from the logits
    const RouteOut r{logits, topk_ids, topk_weights, expert_offsets, sorted_pairs, active_experts,
                     num_active, rec, expert_bits(E)};
    if (!hint && decode_fast_fits(M, H, w->inter)) {
      a.probe = probe;
      return hip_status(launch_decode(a, r, s, timing_of(opts), probe != nullptr));
    }
    if (probe) return MOE_ERR_SHAPE;               // the stamping instances exist for the decode path only
    return hip_status(launch_forward_routed(a, r, s, timing_of(opts)));
  }
  if (probe) return MOE_ERR_SHAPE;
  if (topk_sort_fits_one_block(M)) a.lists = nullptr;   // the one-workgroup sort writes records only
  const RecOut ro = layer_recout(a, workspace);
  hipError_t e;
  if (topk_sort_fits_one_block(M)) {
    e = launch_topk_sort_small(logits, M, E, top_k, topk_ids, topk_weights, expert_offsets,
                               sorted_pairs, active_experts, num_active, s, ro);
  } else {
    e = launch_topk_softmax(logits, M, E, top_k, topk_ids, topk_weights, s);
    if (e == hipSuccess)
      e = launch_sort_by_expert(topk_ids, M * top_k, E, expert_offsets, sorted_pairs, active_experts,
                                num_active, s, ro);
  }
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(launch_experts(a, s, opts));
}

moe_status forward_impl(const uint16_t* x, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                        const float* topk_weights, const int32_t* expert_offsets, const int32_t* sorted_pairs,
                        const int32_t* active_experts, const int32_t* num_active, float* y, void* workspace,
                        size_t workspace_bytes_, const moe_exec_opts* opts, void* stream) {
  if (!x || !w || !topk_weights || !expert_offsets || !sorted_pairs || !active_experts || !num_active || !y ||
      !workspace)
    return MOE_ERR_NULL;
  moe_status st = check_bank(w);
  if (st != MOE_OK) return st;
  if ((st = check_route_sizes(M, w->num_experts, top_k)) != MOE_OK) return st;
  if ((st = check_opts(opts)) != MOE_OK) return st;
  if (!aligned16(x) || ((uintptr_t)workspace & 255u)) return MOE_ERR_ALIGN;
  if (workspace_bytes_ < workspace_layout(M, top_k, w->num_experts, w->hidden, w->inter).total)
    return MOE_ERR_WORKSPACE;
  const bool act8 = opts && opts->act8;
  hipStream_t s = (hipStream_t)stream;
  ForwardArgs a = layer_args(x, w, M, top_k, topk_weights, expert_offsets, sorted_pairs, active_experts,
                             num_active, y, workspace, act8);
  if (act8) {   // the sort-driven kernels take x as MXFP8 values from the workspace
    const bool mfma = a.mfma_min == kMfmaMinTokens;
    if (launch_mxfp8_quantize(x, M, w->hidden, mfma ? a.xq_hi : nullptr, mfma ? a.xq_shi : nullptr,
                              const_cast<uint16_t*>(a.x), s) != hipSuccess)
      return MOE_ERR_HIP;
  }
  if (a.mfma_min == kMfmaMinTokens || a.mt_min != INT_MAX || a.yp) {
    // the path choice needs per-expert token counts, the combine the pairs'
    // sorted positions: records (slot lists, MFMA items, positions) first
    const RecOut ro = layer_recout(a, workspace);
    if (launch_records(expert_offsets, sorted_pairs, active_experts, num_active, a.E, ro, s) != hipSuccess)
      return MOE_ERR_HIP;
  } else {
    a.rec = nullptr;                 // few tokens: resolved from the sort outputs directly
    a.lists = nullptr;
  }
  return hip_status(launch_experts(a, s, opts));
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxScratchDevices];

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

moe_status moe_read_probe(const uint64_t* addrs, const int64_t* sizes, int32_t n, int64_t max_bytes, uint32_t* out,
                          size_t out_words, void* start_event, void* stop_event, void* stream) {
  if (!addrs || !sizes || !out) return MOE_ERR_NULL;
  if ((start_event == nullptr) != (stop_event == nullptr)) return MOE_ERR_NULL;
  if (n < 1 || n > 65535 || max_bytes < 16 || max_bytes % 16 != 0 ||
      read_probe_chunks(max_bytes) > INT32_MAX)
    return MOE_ERR_SHAPE;
  if (out_words < (size_t)n * (size_t)read_probe_chunks(max_bytes)) return MOE_ERR_SHAPE;
  if (((uintptr_t)addrs & 7u) || ((uintptr_t)sizes & 7u) || ((uintptr_t)out & 3u)) return MOE_ERR_ALIGN;
  return hip_status(launch_read_probe(addrs, sizes, n, max_bytes, out, (hipEvent_t)start_event,
                                      (hipEvent_t)stop_event, (hipStream_t)stream));
}

moe_status moe_layer_noalloc(const uint16_t* x, const float* w_router, const float* logit_bias,
                             int64_t bias_row_stride, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                             float* logits, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                             int32_t* sorted_pairs, int32_t* active_experts, int32_t* num_active, float* y,
                             void* stream) {
  // every host check first (nothing touches the device for a rejected call)
  if (!x || !w_router || !w || !logits || !topk_ids || !topk_weights || !expert_offsets || !sorted_pairs ||
      !active_experts || !num_active || !y)
    return MOE_ERR_NULL;
  moe_status st = check_bank(w);
  if (st != MOE_OK) return st;
  if ((st = check_route_sizes(M, w->num_experts, top_k)) != MOE_OK) return st;
  if (logit_bias && bias_row_stride != 0 && bias_row_stride != w->num_experts) return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_ALIGN;
  const size_t need = workspace_layout(M, top_k, w->num_experts, w->hidden, w->inter).total;
  if (need > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return MOE_ERR_HIP;
  return layer_impl(x, w_router, logit_bias, bias_row_stride, w, M, top_k, logits, topk_ids, topk_weights,
                    expert_offsets, sorted_pairs, active_experts, num_active, y, ws, kNoAllocScratchBytes, nullptr,
                    stream);
}

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is outside the supported limits";
    case MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace is smaller than moe_workspace_bytes()";
    case MOE_ERR_HIP: return "the HIP runtime rejected a launch";
  }
  return "unknown status";
}

size_t moe_workspace_bytes(int32_t M, int32_t top_k, int32_t E, int32_t H, int32_t I) {
  if (check_route_sizes(M, E, top_k) != MOE_OK || check_hidden(H) != MOE_OK ||
      check_inter(I) != MOE_OK)
    return 0;
  return workspace_layout(M, top_k, E, H, I).total;
}

moe_status moe_route(const uint16_t* x, const float* w_router, const float* logit_bias,
                     int64_t bias_row_stride, int32_t M, int32_t H, int32_t E, int32_t top_k,
                     float* logits, int32_t* topk_ids, float* topk_weights, void* stream) {
  if (!x || !w_router || !logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
  moe_status st = check_route_sizes(M, E, top_k);
  if (st != MOE_OK) return st;
  if ((st = check_hidden(H)) != MOE_OK) return st;
  if (logit_bias && bias_row_stride != 0 && bias_row_stride != E) return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_router_logits(x, w_router, logit_bias, logit_bias ? bias_row_stride : 0, M, H,
                                      E, logits, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(launch_topk_softmax(logits, M, E, top_k, topk_ids, topk_weights, s));
}

moe_status moe_topk_softmax(const float* logits, int32_t M, int32_t E, int32_t top_k,
                            int32_t* topk_ids, float* topk_weights, void* stream) {
  if (!logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
  moe_status st = check_route_sizes(M, E, top_k);
  if (st != MOE_OK) return st;
  return hip_status(launch_topk_softmax(logits, M, E, top_k, topk_ids, topk_weights, (hipStream_t)stream));
}

moe_status moe_sort_by_expert(const int32_t* topk_ids, int32_t M, int32_t top_k, int32_t E,
                              int32_t* expert_offsets, int32_t* sorted_pairs,
                              int32_t* active_experts, int32_t* num_active, void* stream) {
  if (!topk_ids || !expert_offsets || !sorted_pairs || !active_experts || !num_active)
    return MOE_ERR_NULL;
  moe_status st = check_route_sizes(M, E, top_k);
  if (st != MOE_OK) return st;
  return hip_status(launch_sort_by_expert(topk_ids, M * top_k, E, expert_offsets, sorted_pairs,
                                          active_experts, num_active, (hipStream_t)stream));
}

moe_status moe_mxfp4_forward(const uint16_t* x, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                             const float* topk_weights, const int32_t* expert_offsets,
                             const int32_t* sorted_pairs, const int32_t* active_experts,
                             const int32_t* num_active, float* y, void* workspace,
                             size_t workspace_bytes_, void* stream) {
  return forward_impl(x, w, M, top_k, topk_weights, expert_offsets, sorted_pairs, active_experts, num_active, y,
                      workspace, workspace_bytes_, nullptr, stream);
}

moe_status moe_mxfp4_forward_ex(const uint16_t* x, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                                const float* topk_weights, const int32_t* expert_offsets,
                                const int32_t* sorted_pairs, const int32_t* active_experts,
                                const int32_t* num_active, float* y, void* workspace, size_t workspace_bytes_,
                                const moe_exec_opts* opts, void* stream) {
  return forward_impl(x, w, M, top_k, topk_weights, expert_offsets, sorted_pairs, active_experts, num_active, y,
                      workspace, workspace_bytes_, opts, stream);
}

moe_status moe_layer_ex(const uint16_t* x, const float* w_router, const float* logit_bias, int64_t bias_row_stride,
                        const moe_mxfp4_weights* w, int32_t M, int32_t top_k, float* logits, int32_t* topk_ids,
                        float* topk_weights, int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* active_experts,
                        int32_t* num_active, float* y, void* workspace, size_t workspace_bytes_,
                        const moe_exec_opts* opts, void* stream) {
  return layer_impl(x, w_router, logit_bias, bias_row_stride, w, M, top_k, logits, topk_ids, topk_weights,
                    expert_offsets, sorted_pairs, active_experts, num_active, y, workspace, workspace_bytes_,
                    opts, stream);
}

moe_status moe_layer_hinted(const uint16_t* x, const float* w_router, const float* logit_bias,
                            int64_t bias_row_stride, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                            float* logits, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                            int32_t* sorted_pairs, int32_t* active_experts, int32_t* num_active, float* y,
                            void* workspace, size_t workspace_bytes_, const int32_t* hint_experts,
                            const int32_t* num_hint, void* start_event, void* stop_event, void* stream) {
  if ((hint_experts == nullptr) != (num_hint == nullptr)) return MOE_ERR_NULL;
  if (((uintptr_t)hint_experts & 3u) || ((uintptr_t)num_hint & 3u)) return MOE_ERR_ALIGN;
  moe_exec_opts o{};
  o.gateup_events[0] = start_event;
  o.gateup_events[1] = stop_event;
  return layer_impl(x, w_router, logit_bias, bias_row_stride, w, M, top_k, logits, topk_ids, topk_weights,
                    expert_offsets, sorted_pairs, active_experts, num_active, y, workspace, workspace_bytes_,
                    &o, stream, hint_experts, num_hint);
}

size_t moe_layer_probe_stamps(int32_t M, int32_t top_k, int32_t E, int32_t H, int32_t I) {
  if (check_route_sizes(M, E, top_k) != MOE_OK || check_hidden(H) != MOE_OK || check_inter(I) != MOE_OK ||
      M > kRoutedMaxTokens || !decode_fast_fits(M, H, I))
    return 0;
  return decode_probe_stamps(M, top_k, E, H, I, 1);
}

moe_status moe_layer_probe(const uint16_t* x, const float* w_router, const float* logit_bias,
                           int64_t bias_row_stride, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                           float* logits, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                           int32_t* sorted_pairs, int32_t* active_experts, int32_t* num_active, float* y,
                           void* workspace, size_t workspace_bytes_, unsigned long long* stamps, size_t num_stamps,
                           void* stream) {
  if (!stamps || !w) return MOE_ERR_NULL;
  if (((uintptr_t)stamps & 7u)) return MOE_ERR_ALIGN;
  const size_t need = moe_layer_probe_stamps(M, top_k, w->num_experts, w->hidden, w->inter);
  if (need == 0 || num_stamps < need) return MOE_ERR_SHAPE;
  return layer_impl(x, w_router, logit_bias, bias_row_stride, w, M, top_k, logits, topk_ids, topk_weights,
                    expert_offsets, sorted_pairs, active_experts, num_active, y, workspace, workspace_bytes_,
                    nullptr, stream, nullptr, nullptr, stamps);
}

moe_status moe_layer(const uint16_t* x, const float* w_router, const float* logit_bias,
                     int64_t bias_row_stride, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                     float* logits, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                     int32_t* sorted_pairs, int32_t* active_experts, int32_t* num_active, float* y,
                     void* workspace, size_t workspace_bytes_, void* stream) {
  return layer_impl(x, w_router, logit_bias, bias_row_stride, w, M, top_k, logits, topk_ids, topk_weights,
                    expert_offsets, sorted_pairs, active_experts, num_active, y, workspace, workspace_bytes_,
                    nullptr, stream);
}

moe_status moe_layer_w4a8(const uint16_t* x, const float* w_router, const float* logit_bias,
                          int64_t bias_row_stride, const moe_mxfp4_weights* w, int32_t M, int32_t top_k,
                          float* logits, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                          int32_t* sorted_pairs, int32_t* active_experts, int32_t* num_active, float* y,
                          void* workspace, size_t workspace_bytes_, void* stream) {
  moe_exec_opts o{};
  o.act8 = 1;
  return layer_impl(x, w_router, logit_bias, bias_row_stride, w, M, top_k, logits, topk_ids, topk_weights,
                    expert_offsets, sorted_pairs, active_experts, num_active, y, workspace, workspace_bytes_,
                    &o, stream);
}

moe_status moe_mxfp8_quantize(const uint16_t* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                              uint16_t* values, void* stream) {
  if (!x || (!codes && !scales && !values)) return MOE_ERR_NULL;
  if (rows < 1 || K < 32 || K % 32 || rows * K >= (int64_t(1) << 40)) return MOE_ERR_SHAPE;
  if ((rows * (K / 32) + 255) / 256 > 0x7FFFFFFF) return MOE_ERR_SHAPE;
  if (!aligned16(x) || (codes && !aligned16(codes)) || (values && !aligned16(values))) return MOE_ERR_ALIGN;
  return hip_status(launch_mxfp8_quantize(x, rows, K, codes, scales, values, (hipStream_t)stream));
}

moe_status moe_mxfp4_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols,
                                float* out, void* stream) {
  if (!q || !s || !out) return MOE_ERR_NULL;
  if (rows < 1 || cols < 32 || cols % 32 || rows * cols >= (int64_t(1) << 40)) return MOE_ERR_SHAPE;
  if ((rows * (cols / 8) + 255) / 256 > 0x7FFFFFFF) return MOE_ERR_SHAPE;
  if (!aligned16(q) || ((uintptr_t)out & 15u)) return MOE_ERR_ALIGN;
  return hip_status(launch_dequant(q, s, rows, cols, out, (hipStream_t)stream));
}

moe_status moe_prefetch_select(const int32_t* draft_ids, int32_t n_ids, int32_t E, int32_t has_shared,
                               int32_t max_experts, int32_t* expert_ids, int32_t* num_selected, void* stream) {
  if (!num_selected || (n_ids > 0 && !draft_ids) || (max_experts > 0 && !expert_ids)) return MOE_ERR_NULL;
  if (n_ids < 0 || n_ids > kPrefetchMaxIds || E < 1 || E > MOE_MAX_EXPERTS || (has_shared != 0 && has_shared != 1) ||
      max_experts < 0 || max_experts > kPrefetchMaxList)
    return MOE_ERR_SHAPE;
  if (((uintptr_t)draft_ids & 3u) || ((uintptr_t)expert_ids & 3u) || ((uintptr_t)num_selected & 3u))
    return MOE_ERR_ALIGN;
  return hip_status(launch_prefetch_select(draft_ids, n_ids, E, has_shared, max_experts, expert_ids, num_selected,
                                           (hipStream_t)stream));
}

moe_status moe_prefetch_experts(const moe_mxfp4_weights* w, const int32_t* expert_ids, const int32_t* num_live,
                                int32_t max_ids, int32_t parts, uint32_t* checksums, void* stream) {
  if (!w || !w->w13_q || !w->w13_s || !w->w2_q || !w->w2_s) return MOE_ERR_NULL;
  if (max_ids > 0 && (!expert_ids || !checksums)) return MOE_ERR_NULL;
  if (w->num_experts < 1 || w->num_experts > MOE_MAX_EXPERTS || (w->has_shared != 0 && w->has_shared != 1))
    return MOE_ERR_SHAPE;
  if (check_hidden(w->hidden) != MOE_OK || check_inter(w->inter) != MOE_OK) return MOE_ERR_SHAPE;
  if (max_ids < 0 || max_ids > kPrefetchMaxList || parts < 1 || parts > 3) return MOE_ERR_SHAPE;
  if (!aligned16(w->w13_q) || !aligned16(w->w13_s) || !aligned16(w->w2_q) || !aligned16(w->w2_s) ||
      ((uintptr_t)expert_ids & 3u) || ((uintptr_t)num_live & 3u) || ((uintptr_t)checksums & 3u))
    return MOE_ERR_ALIGN;
  if (max_ids == 0) return MOE_OK;
  const int64_t H = w->hidden, I = w->inter;
  // bytes per expert of each array (multiples of 32 for H, I % 32 == 0)
  const int64_t n13q = 2 * I * (H / 2), n13s = 2 * I * (H / 32);
  const int64_t n2q = H * (I / 2), n2s = H * (I / 32);
  PrefetchArgs a{};
  int q = 0;
  auto add = [&](const uint8_t* p, int64_t n) {
    a.base[q] = p;
    a.bytes[q++] = n;
  };
  if (parts & 1) { add(w->w13_q, n13q); add(w->w13_s, n13s); }
  if (parts & 2) { add(w->w2_q, n2q); add(w->w2_s, n2s); }
  a.nreg = q;
  a.nbank = w->num_experts + w->has_shared;
  a.ids = expert_ids;
  a.num_live = num_live;
  a.max_ids = max_ids;
  a.checksums = checksums;
  return hip_status(launch_prefetch(a, (hipStream_t)stream));
}

moe_status moe_lmhead_fp8_quantize(const uint16_t* w_bf16, int32_t V, int32_t H, uint8_t* codes, float* scales,
                                   void* stream) {
  if (!w_bf16 || !codes || !scales) return MOE_ERR_NULL;
  if (V < 1 || H < 32 || H % 32 || H > MOE_MAX_HIDDEN || (int64_t)V * H >= (int64_t(1) << 40)) return MOE_ERR_SHAPE;
  if (!aligned16(w_bf16) || ((uintptr_t)codes & 7u) || ((uintptr_t)scales & 3u)) return MOE_ERR_ALIGN;
  return hip_status(launch_lmhead_quantize(w_bf16, V, H, codes, scales, (hipStream_t)stream));
}

moe_status moe_lmhead_fp8_logits(const uint16_t* x, const uint8_t* codes, const float* scales, int32_t M,
                                 int32_t V, int32_t H, float* logits, void* stream) {
  if (!x || !codes || !scales || !logits) return MOE_ERR_NULL;
  if (M < 1 || M > MOE_LMHEAD_MAX_TOKENS || V < 1 || H < 32 || H % 32 || H > MOE_MAX_HIDDEN ||
      (int64_t)M * H > MOE_LMHEAD_MAX_TOKENS * 4096 || (int64_t)V * H >= (int64_t(1) << 40))
    return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || ((uintptr_t)scales & 3u) || ((uintptr_t)logits & 3u))
    return MOE_ERR_ALIGN;
  return hip_status(launch_lmhead_fp8(x, codes, scales, M, V, H, logits, (hipStream_t)stream));
}

}  // extern "C"
