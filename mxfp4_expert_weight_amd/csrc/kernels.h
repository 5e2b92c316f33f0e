// Internal launch interface between the C ABI (capi.hip) and the kernels.
#pragma once

#include "common.h"

namespace moe {

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
  int M, k, E, H, I, has_shared;
};

// Workspace layout of moe_mxfp4_forward: header, then h.
inline size_t workspace_h_offset() { return sizeof(WorkspaceHeader); }
inline size_t workspace_bytes(int M, int k, int I) {
  return workspace_h_offset() + align_up((size_t)(M * (size_t)k + M) * I * sizeof(uint16_t), 256);
}

hipError_t launch_router_logits(const uint16_t* x, const float* w_router, const float* bias,
                                int64_t bias_stride, int M, int H, int E, float* logits, hipStream_t s);
hipError_t launch_topk_softmax(const float* logits, int M, int E, int k, int* ids, float* weights,
                               hipStream_t s);
hipError_t launch_sort_by_expert(const int* ids, int N, int E, int* offsets, int* sorted_pairs,
                                 int* active, int* num_active, hipStream_t s);
hipError_t launch_forward(const ForwardArgs& a, hipStream_t s, hipEvent_t start = nullptr,
                          hipEvent_t stop = nullptr);
hipError_t launch_dequant(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols, float* out,
                          hipStream_t st);

}  // namespace moe
