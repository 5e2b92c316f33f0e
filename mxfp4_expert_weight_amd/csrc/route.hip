// Router of the MoE layer: fp32 logits GEMV and the wavefront top-k with the
// renormalised softmax.  The gate network scores every expert and only the
// top-k are kept ("NVIDIA three-layer optimisation ... 42.5%" news rewrite,
// paragraph on sparse activation and expert routing); it stays in fp32 because
// the softmax is sensitive to quantisation error (MoE-SpeQ article, 2.1).
#include "kernels.h"
#include "sort_dev.h"
#include "topk_dev.h"

namespace moe {

// ------------------------------------------------------------- logits --
// One wave per expert row.  Lane l holds float4 number (l + 64 i) of the
// fp32 router row in registers (coalesced 16-byte loads, 1 KiB per wave
// instruction) and reuses it for every token; up to TB tokens are processed
// per pass with all their activation loads issued together.
// logits[t][e] = x_t . W_r[e] (+ bias): exact bf16 * fp32 products, fp32 sums.
template <int VMAX, int TB>
__global__ __launch_bounds__(128) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ w_router,
                                                            const float* __restrict__ bias,
                                                            int64_t bias_stride, int M, int H, int E,
                                                            float* __restrict__ logits) {
  const int lane = threadIdx.x & (kWave - 1);
  const int e = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (e >= E) return;
  const int nvec = H / 4;
  const float4* wrow = reinterpret_cast<const float4*>(w_router + (size_t)e * H);
  float4 w[VMAX];
#pragma unroll
  for (int i = 0; i < VMAX; ++i) {       // clamped loads, zeroed past the row (no branches)
    const int v = lane + kWave * i;
    const float4 t = wrow[min(v, nvec - 1)];
    w[i] = (v < nvec) ? t : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int t0 = 0; t0 < M; t0 += TB) {
    uint2 xv[TB][VMAX];
#pragma unroll
    for (int q = 0; q < TB; ++q) {
      const uint2* xrow = reinterpret_cast<const uint2*>(x + (size_t)min(t0 + q, M - 1) * H);
#pragma unroll
      for (int i = 0; i < VMAX; ++i) {
        const int v = lane + kWave * i;
        const uint2 t = xrow[min(v, nvec - 1)];
        xv[q][i] = (v < nvec) ? t : make_uint2(0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < TB; ++q) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < VMAX; ++i) {
        acc = fmaf(bf16_bits_to_f32(xv[q][i].x & 0xFFFFu), w[i].x, acc);
        acc = fmaf(bf16_bits_to_f32(xv[q][i].x >> 16), w[i].y, acc);
        acc = fmaf(bf16_bits_to_f32(xv[q][i].y & 0xFFFFu), w[i].z, acc);
        acc = fmaf(bf16_bits_to_f32(xv[q][i].y >> 16), w[i].w, acc);
      }
      acc = group_sum<kWave>(acc);
      const int t = t0 + q;
      if (lane == 0 && t < M) {
        if (bias) acc += bias[(size_t)t * bias_stride + e];
        logits[(size_t)t * E + e] = acc;
      }
    }
  }
}

// One wave per token.
template <int C>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits, int M, int E,
                                                           int k, int* __restrict__ topk_ids,
                                                           float* __restrict__ topk_weights) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= M) return;
  int id; float w;
  wave_topk_softmax<C>(logits + (size_t)t * E, E, k, id, w);
  if (lane < k) {
    topk_ids[(size_t)t * k + lane] = id;
    topk_weights[(size_t)t * k + lane] = w;
  }
}

// Small batches: one workgroup of M waves takes every token's top-k into LDS
// (and the outputs), then wave 0 sorts the M*k pairs by expert in LDS and the
// block writes the sort outputs and the slot records.
template <int C>
__global__ __launch_bounds__(64 * kTopkSortMaxTokens) void topk_sort_small_kernel(
    const float* __restrict__ logits, int M, int E, int k, int ebits, int* __restrict__ topk_ids,
    float* __restrict__ topk_weights, int* __restrict__ offsets, int* __restrict__ sorted_pairs,
    int* __restrict__ active, int* __restrict__ num_active, RecOut ro) {
  __shared__ SmallSortLds<C, kTopkSortMaxTokens * MOE_MAX_TOPK> L;
  const int N = M * k;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = threadIdx.x / kWave;
  int id; float w;
  wave_topk_softmax<C>(logits + (size_t)t * E, E, k, id, w);
  if (lane < k) {
    L.ids[t * k + lane] = id;
    L.w[t * k + lane] = w;
    L.tok[t * k + lane] = t;
  }
  __syncthreads();
  if (t == 0) wave_sort_small(L, N, E, ebits);
  __syncthreads();
  block_store_small_sort(L, N, E, topk_ids, topk_weights, offsets, sorted_pairs, active, num_active);
  if (ro.rec)
    for (int slot = threadIdx.x; slot < max_slots(M, k, E); slot += blockDim.x)
      ro.rec[slot] = small_slot_record(L, slot, M, k, E, ro.has_shared);
  if (ro.hdr && threadIdx.x == 0) {     // at most 8 tokens per expert: all on the GEMV path
    ro.hdr->gemv_experts = L.na + ro.has_shared;
    ro.hdr->mfma_experts = 0;
    ro.hdr->mfma_items = 0;
  }
}

hipError_t launch_router_logits(const uint16_t* x, const float* w_router, const float* bias,
                                int64_t bias_stride, int M, int H, int E, float* logits,
                                hipStream_t s) {
  const int waves_per_block = 2;
  dim3 grid((E + waves_per_block - 1) / waves_per_block), block(waves_per_block * kWave);
  if (H <= 2560) {
    if (M == 1)
      router_logits_kernel<10, 1><<<grid, block, 0, s>>>(x, w_router, bias, bias_stride, M, H, E, logits);
    else if (M <= 4)
      router_logits_kernel<10, 4><<<grid, block, 0, s>>>(x, w_router, bias, bias_stride, M, H, E, logits);
    else
      router_logits_kernel<10, 8><<<grid, block, 0, s>>>(x, w_router, bias, bias_stride, M, H, E, logits);
  } else {
    router_logits_kernel<32, 1><<<grid, block, 0, s>>>(x, w_router, bias, bias_stride, M, H, E, logits);
  }
  return hipGetLastError();
}

hipError_t launch_topk_softmax(const float* logits, int M, int E, int k, int* ids, float* weights,
                               hipStream_t s) {
  const int waves_per_block = 4;
  dim3 grid((M + waves_per_block - 1) / waves_per_block), block(waves_per_block * kWave);
  if (topk_lane_experts(E) == 8)
    topk_softmax_kernel<8><<<grid, block, 0, s>>>(logits, M, E, k, ids, weights);
  else
    topk_softmax_kernel<16><<<grid, block, 0, s>>>(logits, M, E, k, ids, weights);
  return hipGetLastError();
}

bool topk_sort_fits_one_block(int M) { return M <= kTopkSortMaxTokens; }

hipError_t launch_topk_sort_small(const float* logits, int M, int E, int k, int* ids, float* weights,
                                  int* offsets, int* sorted_pairs, int* active, int* num_active,
                                  hipStream_t s, RecOut ro) {
  auto kern = topk_lane_experts(E) == 8 ? topk_sort_small_kernel<8> : topk_sort_small_kernel<16>;
  kern<<<1, M * kWave, 0, s>>>(logits, M, E, k, expert_bits(E), ids, weights, offsets, sorted_pairs, active,
                               num_active, ro);
  return hipGetLastError();
}

}  // namespace moe
