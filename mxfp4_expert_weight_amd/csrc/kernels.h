// Internal launch interface between the C ABI (capi.hip) and the kernels.
#pragma once

#include "common.h"

namespace moe {

// Per-expert work record written by the sort epilogue of moe_layer: one 64-byte
// load gives an expert kernel its expert, token count and first tokens, instead
// of a chain of dependent loads through num_active, active, offsets and pairs.
constexpr int kRecTokens = 4;
// Largest batch whose routing runs inside every gate/up block: an expert then
// has at most kRecTokens tokens, all of them in its slot record.
constexpr int kRoutedMaxTokens = kRecTokens;
struct SlotRec {
  int32_t e;                  // expert index in the bank (E = shared), -1 = no work
  int32_t n;                  // tokens of this expert
  int32_t pbeg;               // first sorted position, -1 for the shared expert
  int32_t hrow0;              // h row of the first token
  int32_t tok[kRecTokens];    // first tokens
  float w[kRecTokens];        // their routing weights (1 for the shared expert)
  int32_t pad[4];
};
static_assert(sizeof(SlotRec) == 64, "record size");

struct ForwardArgs {
  const uint16_t* x;          // [M][H] bf16
  const uint8_t* w13_q;       // [E+S][2I][H/2]
  const uint8_t* w13_s;       // [E+S][2I][H/32]
  const uint8_t* w2_q;        // [E+S][H][I/2]
  const uint8_t* w2_s;        // [E+S][H][I/32]
  const float* topk_weights;  // [M][k]
  const int* offsets;         // [E+1]
  const int* sorted_pairs;    // [M*k]
  const int* active;          // [E]
  const int* num_active;      // [1]
  float* y;                   // [M][H]
  uint16_t* h;                // [M*k + M][I] bf16 (workspace)
  uint16_t* hlo;              // [M*k + M][I] bf16 residual of the GEMV path's h (h = hi + lo)
  WorkspaceHeader* hdr;       // workspace header
  const SlotRec* rec;         // slot records, or null (then resolved from the sort outputs)
  int M, k, E, H, I, has_shared;
  // few-token matrix-core path (experts with mt_min..mt_max tokens, below
  // mfma_min; mt_min = INT_MAX when off)
  int mt_min, mt_max;
  // MFMA path (experts with >= mfma_min tokens; mfma_min = INT_MAX when off)
  int mfma_min;
  uint8_t *xq_hi, *xq_lo;     // [M][H] two-term MXFP8 (E4M3) codes of x
  uint8_t *xq_shi, *xq_slo;   // [M][H/32] their E8M0 scales
  uint8_t *hq_hi, *hq_lo;     // [M*k + M][I] two-term MXFP8 codes of h (MFMA experts' rows)
  uint8_t *hq_shi, *hq_slo;   // [M*k + M][I/32]
  const int2* items;          // MFMA work items (slot, 64-token tile); count in hdr->mfma_items
  // Combine by rows (large batches): the down kernels store w * (h . Wd) of
  // every pair into its own row of yp (same row order as h) and a combine
  // kernel sums each token's rows into y; null: fp32 atomics into y.
  float* yp;                  // [M*k + M][H] (workspace)
  const int* inv;             // [M*k]: sorted position of flattened pair t*k+s, -1 if dropped
  // Slot lists (batches with records): the GEMV experts' slots at lists[0..),
  // the few-token experts' at lists[max_slots..), counts in the header; the
  // kernels of those paths loop over them instead of a grid row per slot.
  const int* lists;
  // W4A8 variant: the experts take x as MXFP8 values (bf16: a.x holds them,
  // or the decode gate/up kernel rounds x as it stages it), h goes through an
  // MXFP8 round trip in place between gate/up and down, and the MFMA path
  // carries x and h as one MXFP8 term (codes in xq_hi/hq_hi, scales in
  // xq_shi/hq_shi; the _lo terms are unused).
  int act8;
  // Decode hint (moe_layer_hinted): the routed experts a draft pass predicts,
  // ascending, hint[0 .. *num_hint); null: none.  Only read by the decode
  // gate/up kernel, whose idle waves touch the hinted rows during the routing.
  const int* hint;
  const int* num_hint;
  // Phase stamps of the decode kernels' measurement instances (null otherwise).
  unsigned long long* probe;
};

// The few-token matrix-core path (mt.hip): batches of more than
// kRoutedMaxTokens tokens whose reduction lengths are multiples of its
// 256-element chunk; experts with kMtMinTokens..kMtMaxTokens tokens.
constexpr int kMtMinTokens = 3;
// At H = 2560, I = 768 the batch experts with up to 4 tokens run on the decode
// kernels' slot code, so the few-token kernels start at 5.
inline int mt_min_tokens(int H, int I) { return (H == 2560 && I == 768) ? kRoutedMaxTokens + 1 : kMtMinTokens; }
constexpr int kMtMaxTokens = 16;
constexpr int kMtChunk = 256;

// The MFMA path: experts with at least kMfmaMinTokens tokens run as dense
// products on the scaled MXFP4 matrix cores when M reaches that many tokens
// and both reduction lengths are multiples of the instruction's K.
constexpr int kMfmaMinTokens = 16;
constexpr int kMfmaTileTokens = 64;     // tokens per work item
constexpr int kMfmaK = 128;             // K of one v_mfma_scale_f32_16x16x128_f8f6f4
inline bool mfma_path(int M, int H, int I) {
  return M >= kMfmaMinTokens && H % kMfmaK == 0 && I % kMfmaK == 0;
}
inline bool mt_path(int M, int H, int I) { return M > kRoutedMaxTokens && H % kMtChunk == 0 && I % kMtChunk == 0; }

// Work items of the MFMA kernels are (slot, tile) pairs: at most
// ceil(pairs/64) + (number of MFMA experts <= pairs/16) of them.
__host__ __device__ inline int mfma_max_items(int M, int k) {
  const int pairs = M * k + M;
  return (pairs + kMfmaTileTokens - 1) / kMfmaTileTokens + pairs / kMfmaMinTokens + 1;
}

// Workspace: header | slot records (one per possible active expert + shared) |
// h | (MFMA path only) two-term MXFP8 x, two-term MXFP8 h, MFMA work items.
__host__ __device__ inline int max_slots(int M, int k, int E) { return (E < M * k ? E : M * k) + 1; }
// Combine by rows: batches of at least kCombineRowsMinTokens tokens whose
// partial rows fit in kCombineRowsMaxBytes.
constexpr int kCombineRowsMinTokens = 16;
constexpr size_t kCombineRowsMaxBytes = size_t(1) << 30;
inline bool combine_rows(int M, int k, int H) {
  return M >= kCombineRowsMinTokens && ((size_t)M * k + M) * H * sizeof(float) <= kCombineRowsMaxBytes;
}
struct WorkspaceLayout {
  size_t rec, h, hlo, xq_hi, xq_lo, xq_shi, xq_slo, hq_hi, hq_lo, hq_shi, hq_slo, items, yp, inv, lists, xdq, total;
};
inline WorkspaceLayout workspace_layout(int M, int k, int E, int H, int I) {
  WorkspaceLayout w{};
  const size_t pairs = (size_t)M * k + M;
  size_t o = sizeof(WorkspaceHeader);
  auto take = [&o](size_t bytes) { const size_t at = o; o += align_up(bytes, 256); return at; };
  w.rec = take((size_t)max_slots(M, k, E) * sizeof(SlotRec));
  w.h = take(pairs * I * sizeof(uint16_t));
  w.hlo = take(pairs * I * sizeof(uint16_t));
  if (mfma_path(M, H, I)) {
    w.xq_hi = take((size_t)M * H);
    w.xq_lo = take((size_t)M * H);
    w.xq_shi = take((size_t)M * H / 32);
    w.xq_slo = take((size_t)M * H / 32);
    w.hq_hi = take(pairs * I);
    w.hq_lo = take(pairs * I);
    w.hq_shi = take(pairs * I / 32);
    w.hq_slo = take(pairs * I / 32);
    w.items = take((size_t)mfma_max_items(M, k) * sizeof(int2));
  }
  if (combine_rows(M, k, H)) {
    w.yp = take(pairs * H * sizeof(float));
    w.inv = take((size_t)M * k * sizeof(int));
  }
  if (M > kRoutedMaxTokens) w.lists = take(2 * (size_t)max_slots(M, k, E) * sizeof(int));
  w.xdq = take((size_t)M * H * sizeof(uint16_t));   // W4A8: the experts' MXFP8 x as bf16 values
  w.total = o;
  return w;
}

// Optional epilogue of the sort: slot records for the forward kernels, the
// MFMA work items, and the path counters in the workspace header.
struct RecOut {
  SlotRec* rec;               // null: no records
  const float* topk_weights;  // [M][k]
  int M, k, has_shared;
  int mfma_min;               // experts with at least this many tokens go to MFMA
  int2* items;                // MFMA work items (null when the path is off)
  WorkspaceHeader* hdr;
  int mt_min, mt_max;         // few-token matrix-core range (mt_min = INT_MAX: off)
  int* inv;                   // null, or [M*k]: sorted position of each flattened pair (-1: dropped)
  int* lists;                 // null, or [2][max_slots]: slots of the GEMV / few-token experts
};

// Routing done inside the gate/up kernel (decode batches): where the logits
// are and where the routing results go.
struct RouteOut {
  const float* logits;        // [M][E] fp32
  int* topk_ids;              // [M][k]
  float* topk_weights;        // [M][k]
  int* offsets;               // [E+1]
  int* sorted_pairs;          // [M*k]
  int* active;                // [E]
  int* num_active;            // [1]
  SlotRec* rec;               // slot records for the down kernel
  int ebits;                  // bits of an expert id
};
constexpr int kRoutedMaxPairs = kRoutedMaxTokens * MOE_MAX_TOPK;

// Batches of at least this many tokens take the matrix-core router (weights
// split exactly into three bf16 parts).
constexpr int kRouterGemmMinTokens = 64;
hipError_t launch_router_logits(const uint16_t* x, const float* w_router, const float* bias,
                                int64_t bias_stride, int M, int H, int E, float* logits, hipStream_t s);
// Fused top-k + sort in one workgroup for batches of at most this many tokens.
constexpr int kTopkSortMaxTokens = 8;
int expert_bits(int E);
bool topk_sort_fits_one_block(int M);
hipError_t launch_topk_sort_small(const float* logits, int M, int E, int k, int* ids, float* weights,
                                  int* offsets, int* sorted_pairs, int* active, int* num_active,
                                  hipStream_t s, RecOut ro);
hipError_t launch_topk_softmax(const float* logits, int M, int E, int k, int* ids, float* weights,
                               hipStream_t s);
hipError_t launch_sort_by_expert(const int* ids, int N, int E, int* offsets, int* sorted_pairs,
                                 int* active, int* num_active, hipStream_t s,
                                 RecOut ro = RecOut{nullptr, nullptr, 0, 0, 0, 0, nullptr, nullptr, 0, 0, nullptr, nullptr});
// Timing events bound to the GEMV gate/up and down kernels' own begin and
// end timestamps (hipExtLaunchKernelGGL); null: none.
struct Timing {
  hipEvent_t gu_start, gu_stop, dn_start, dn_stop;
};
inline Timing timing_of(const moe_exec_opts* o) {
  if (!o) return Timing{};
  return Timing{(hipEvent_t)o->gateup_events[0], (hipEvent_t)o->gateup_events[1], (hipEvent_t)o->down_events[0],
                (hipEvent_t)o->down_events[1]};
}
// GEMV experts: gate/up (which zeroes y; `zeroed`, if given, is recorded on s
// right after it), then down.
hipError_t launch_forward(const ForwardArgs& a, hipStream_t s, const Timing& tm = Timing{},
                          hipEvent_t zeroed = nullptr);
// Gate/up with the top-k and the expert sort done in every block from the
// logits (M <= kRoutedMaxTokens), then down.  W4A8 (act8): rows of at most
// this many elements are rounded to MXFP8 as the kernel stages x (a.x is the
// bf16 x); longer rows need a.x to hold the MXFP8 values already.
bool routed_stages_x(int H);
// The decode path of decode.hip (M <= kRoutedMaxTokens, the shapes it is
// built for): routed gate/up kernel with 128-bit loads, then down; with
// `probe`, the instances that stamp each workgroup's phases into a.probe.
bool decode_fast_fits(int M, int H, int I);
// Stamps the measurement instances write: 8 per workgroup of the larger grid.
size_t decode_probe_stamps(int M, int k, int E, int H, int I, int has_shared);
hipError_t launch_decode(const ForwardArgs& a, const RouteOut& r, hipStream_t s, const Timing& tm, bool probe);
// Batches at H = 2560, I = 768 whose GEMV experts (one or two tokens) run on
// the decode kernels' slot code (records from the sort epilogue's list).
bool batch_decode_fits(const ForwardArgs& a);
hipError_t launch_decode_batch(const ForwardArgs& a, hipStream_t s, const Timing& tm, hipEvent_t zeroed, int cus);

// Read-bandwidth floor (moe_read_probe): one workgroup per 16 KB chunk of each
// byte range, every load in flight at once.
constexpr int64_t kReadProbeChunk = MOE_READ_PROBE_CHUNK;
inline int64_t read_probe_chunks(int64_t max_bytes) { return (max_bytes + kReadProbeChunk - 1) / kReadProbeChunk; }
hipError_t launch_read_probe(const uint64_t* addrs, const int64_t* sizes, int n, int64_t max_bytes, uint32_t* out,
                             hipEvent_t start, hipEvent_t stop, hipStream_t s);
hipError_t launch_forward_routed(const ForwardArgs& a, const RouteOut& r, hipStream_t s,
                                 const Timing& tm = Timing{});
// MFMA path (mfma.hip): two-term MXFP8 quantisation of x, the dense gate/up
// and down products of the experts listed in the work items.
hipError_t launch_forward_mfma_front(const ForwardArgs& a, hipStream_t s);   // x quantisation
hipError_t launch_gateup_mfma(const ForwardArgs& a, hipStream_t s);
// Few-token matrix-core path (mt.hip).
hipError_t launch_gateup_mt(const ForwardArgs& a, hipStream_t s);
hipError_t launch_down_mt(const ForwardArgs& a, hipStream_t s);
hipError_t launch_down_mfma(const ForwardArgs& a, hipStream_t s);
// Slot records and MFMA items from the sort outputs (one workgroup).
hipError_t launch_records(const int* offsets, const int* sorted_pairs, const int* active, const int* num_active,
                          int E, RecOut ro, hipStream_t s);
// y[t] = sum over s of yp[inv[t*k + s]] (+ yp[M*k + t] for the shared expert).
hipError_t launch_combine_rows(const ForwardArgs& a, hipStream_t s);
hipError_t launch_dequant(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols, float* out,
                          hipStream_t st);
// MXFP8 quantisation of bf16 rows [rows][K] (mxfp8.hip): codes, scale bytes
// and the codes' values as bf16, each optional.
hipError_t launch_mxfp8_quantize(const uint16_t* src, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                                 uint16_t* deq, hipStream_t s);
// MXFP8 round trip (codes' values, as bf16) of h rows [rows][K] carried as
// two bf16 terms, quantised from hi + lo, the result in hi; and of the h rows
// of one path's experts (path 0: GEMV, 1: few-token) the same way.
hipError_t launch_mxfp8_round_trip_rows(uint16_t* hi, const uint16_t* lo, int64_t rows, int K, hipStream_t s);
hipError_t launch_h_round_trip(const ForwardArgs& a, int path, hipStream_t s);
// Expert prefetch (prefetch.hip).  The chosen arrays of one expert (gate/up
// codes, gate/up scales, down codes, down scales: those whose part is
// chosen) are its regions; region q of expert e is the bytes[q] bytes at
// base[q] + e * bytes[q].  The launcher fills per_block and blk_end.
struct PrefetchArgs {
  const uint8_t* base[4];
  int64_t bytes[4];         // bytes per expert (a multiple of 4)
  int blk_end[4];           // cumulative blocks per list entry, by region
  int per_block;            // 64-byte lines per block (a multiple of 1024)
  int nreg;                 // regions in use (2 or 4)
  int nbank;                // bank entries (E + shared)
  const int* ids;           // [max_ids] list entries
  const int* num_live;      // live entries (device), or null: all max_ids
  int max_ids;
  uint32_t* checksums;      // [max_ids], each entry's line-word sum is added
};
// Draft heat map -> prefetch list (one workgroup); keys need heat < 2^20.
constexpr int kPrefetchMaxIds = MOE_PREFETCH_MAX_DRAFT_IDS;
constexpr int kPrefetchMaxList = MOE_PREFETCH_MAX_LIST;    // list entries: one grid row each
hipError_t launch_prefetch_select(const int* ids, int n_ids, int E, int has_shared, int max_n, int* out,
                                  int* num_out, hipStream_t s);
hipError_t launch_prefetch(PrefetchArgs a, hipStream_t s);
// FP8 LM head (lmhead.hip).
hipError_t launch_lmhead_quantize(const uint16_t* w, int V, int H, uint8_t* codes, float* scales, hipStream_t s);
hipError_t launch_lmhead_fp8(const uint16_t* x, const uint8_t* codes, const float* scales, int M, int V, int H,
                             float* logits, hipStream_t s);

}  // namespace moe
