// Internal launch interface between the C ABI (capi.hip) and the kernels.
#pragma once

#include "common.h"

namespace moe {

// Per-expert work record written by the sort epilogue of moe_layer: one 64-byte
// load gives an expert kernel its expert, token count and first tokens, instead
// of a chain of dependent loads through num_active, active, offsets and pairs.
constexpr int kRecTokens = 4;
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
  WorkspaceHeader* hdr;       // workspace header
  const SlotRec* rec;         // slot records, or null (then resolved from the sort outputs)
  int M, k, E, H, I, has_shared;
};

// Workspace: header | slot records (one per possible active expert + shared) | h.
__host__ __device__ inline int max_slots(int M, int k, int E) { return (E < M * k ? E : M * k) + 1; }
inline size_t workspace_rec_offset() { return sizeof(WorkspaceHeader); }
inline size_t workspace_h_offset(int M, int k, int E) {
  return workspace_rec_offset() + align_up((size_t)max_slots(M, k, E) * sizeof(SlotRec), 256);
}
inline size_t workspace_bytes(int M, int k, int E, int I) {
  return workspace_h_offset(M, k, E) + align_up((size_t)(M * (size_t)k + M) * I * sizeof(uint16_t), 256);
}

// Optional epilogue of the sort: slot records for the forward kernels.
struct RecOut {
  SlotRec* rec;               // null: no records
  const float* topk_weights;  // [M][k]
  int M, k, has_shared;
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
// Largest batch whose routing runs inside every gate/up block: an expert then
// has at most kRecTokens tokens, all of them in its slot record.
constexpr int kRoutedMaxTokens = kRecTokens;
constexpr int kRoutedMaxPairs = kRoutedMaxTokens * MOE_MAX_TOPK;

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
                                 RecOut ro = RecOut{nullptr, nullptr, 0, 0, 0});
hipError_t launch_forward(const ForwardArgs& a, hipStream_t s, hipEvent_t start = nullptr,
                          hipEvent_t stop = nullptr);
// Gate/up with the top-k and the expert sort done in every block from the
// logits (M <= kRoutedMaxTokens), then down.
hipError_t launch_forward_routed(const ForwardArgs& a, const RouteOut& r, hipStream_t s,
                                 hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
hipError_t launch_dequant(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols, float* out,
                          hipStream_t st);

}  // namespace moe
