// Wavefront top-k with the renormalised softmax (device routine).
#pragma once

#include "common.h"

namespace moe {

// ------------------------------------------------------------- top-k --
// Order-preserving map of an fp32 onto uint32 (-0 is folded onto +0 first so
// equal values tie on the index, as the definition asks).  0 is never the
// image of a number, so it marks an empty or already-taken slot.
__device__ __forceinline__ uint32_t f32_orderable(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_orderable(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Load one token's logits as orderable keys: lane l holds experts
// [l*kPer, l*kPer + kPer), missing ones as 0.  The loads are unconditional
// with clamped addresses: a guarded load would become a branch with its own
// wait, serialising the round trips.
template <int kPer>
__device__ __forceinline__ void load_logit_keys(const float* row, int E, uint32_t (&val)[kPer]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int e0 = lane * kPer;
  if ((E & 3) == 0 && (reinterpret_cast<uintptr_t>(row) & 15) == 0) {
    const float4* r4 = reinterpret_cast<const float4*>(row);
    const int last = E / 4 - 1;
#pragma unroll
    for (int j = 0; j < kPer; j += 4) {
      const float4 v = r4[min((e0 + j) / 4, last)];
      val[j + 0] = (e0 + j + 0 < E) ? f32_orderable(v.x) : 0u;
      val[j + 1] = (e0 + j + 1 < E) ? f32_orderable(v.y) : 0u;
      val[j + 2] = (e0 + j + 2 < E) ? f32_orderable(v.z) : 0u;
      val[j + 3] = (e0 + j + 3 < E) ? f32_orderable(v.w) : 0u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t v = f32_orderable(row[min(e0 + j, E - 1)]);
      val[j] = (e0 + j < E) ? v : 0u;
    }
  }
}

// Best and second-best key of a lane's entries (first index among equals),
// skipping entries whose bit is set in `taken`.
template <int kPer>
__device__ __forceinline__ void lane_top2(const uint32_t (&val)[kPer], uint32_t taken, uint32_t& b1, int& j1,
                                          uint32_t& b2, int& j2) {
  b1 = 0u; b2 = 0u; j1 = 0; j2 = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t v = ((taken >> j) & 1u) ? 0u : val[j];
    const bool gt1 = v > b1, gt2 = v > b2;
    b2 = gt1 ? b1 : (gt2 ? v : b2);
    j2 = gt1 ? j1 : (gt2 ? j : j2);
    b1 = gt1 ? v : b1;
    j1 = gt1 ? j : j1;
  }
}

// Top-k of one token's logits by one full wave (all 64 lanes active, E <=
// 64*kPer).  Each round takes the wave maximum of the lanes' best keys; the
// lowest lane holding it owns the lowest expert index with that value (a
// lane's experts are contiguous and precede the next lane's, and inside a lane
// the first of equal keys is kept), so ties go to the lower index with one
// ballot instead of a second reduction.  A lane keeps its two best keys, so
// the winner just promotes its second; only a lane that wins twice rescans its
// entries.  Round i's winner lands in lane i, which returns its expert and the
// weight exp(l_i - l_0) / sum over the kept experts; other lanes return 0.
template <int kPer>
__device__ __forceinline__ void wave_topk_softmax(const float* row, int E, int k, int& out_id,
                                                  float& out_w) {
  static_assert(kPer % 4 == 0 && kPer <= 32, "kPer");
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t val[kPer];
  load_logit_keys<kPer>(row, E, val);
  uint32_t b1, b2, taken = 0u;
  int j1, j2;
  lane_top2<kPer>(val, 0u, b1, j1, b2, j2);
  bool second = true;                 // b2 is still this lane's next-best entry

  int my_id = 0;
  uint32_t my_val = 0u, top_val = 0u;
  for (int i = 0; i < k; ++i) {
    const uint32_t vmax = wave_max_u32(b1);
    const uint64_t holders = __ballot(b1 == vmax);
    const int wl = (int)__builtin_ctzll(holders);                    // wave-uniform
    const int wj = __builtin_amdgcn_readlane(j1, wl);
    if (i == 0) top_val = vmax;
    my_id = (lane == i) ? wl * kPer + wj : my_id;
    my_val = (lane == i) ? vmax : my_val;
    const bool hit = lane == wl;
    taken |= hit ? (1u << j1) : 0u;
    if (__ballot(hit && !second)) {   // the winner already used its second: rescan
      if (hit) {
        lane_top2<kPer>(val, taken, b1, j1, b2, j2);
        second = true;
      }
    } else {
      b1 = hit ? b2 : b1;
      j1 = hit ? j2 : j1;
      second = hit ? false : second;
    }
  }
  const float ex = (lane < k) ? expf(f32_from_orderable(my_val) - f32_from_orderable(top_val)) : 0.f;
  const float sum = group_sum<kWave>(ex);
  out_id = my_id;
  out_w = (lane < k) ? ex / sum : 0.f;
}

// Experts per lane for a bank of E experts (E <= MOE_MAX_EXPERTS).
__host__ __device__ constexpr int topk_lane_experts(int E) { return E <= 512 ? 8 : 16; }

}  // namespace moe
