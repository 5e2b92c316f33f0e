// Router of the MoE layer: fp32 logits GEMV and the wavefront top-k with the
// renormalised softmax.  The gate network scores every expert and only the
// top-k are kept ("NVIDIA three-layer optimisation ... 42.5%" news rewrite,
// paragraph on sparse activation and expert routing); it stays in fp32 because
// the softmax is sensitive to quantisation error (MoE-SpeQ article, 2.1).
#include "kernels.h"

namespace moe {

// ------------------------------------------------------------- logits --
// One wave per expert row.  Lane l holds float4 number (l + 64 i) of the
// fp32 router row in registers (coalesced 16-byte loads, 1 KiB per wave
// instruction) and reuses it for every token: logits[t][e] = x_t . W_r[e]
// with exact bf16 * fp32 products accumulated in fp32, then a wave sum.
template <int VMAX>
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
  for (int i = 0; i < VMAX; ++i) {
    const int v = lane + kWave * i;
    w[i] = (v < nvec) ? wrow[v] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int t = 0; t < M; ++t) {
    const uint2* xrow = reinterpret_cast<const uint2*>(x + (size_t)t * H);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < VMAX; ++i) {
      const int v = lane + kWave * i;
      if (v < nvec) {
        const uint2 xv = xrow[v];
        acc = fmaf(bf16_bits_to_f32(xv.x & 0xFFFFu), w[i].x, acc);
        acc = fmaf(bf16_bits_to_f32(xv.x >> 16), w[i].y, acc);
        acc = fmaf(bf16_bits_to_f32(xv.y & 0xFFFFu), w[i].z, acc);
        acc = fmaf(bf16_bits_to_f32(xv.y >> 16), w[i].w, acc);
      }
    }
    acc = group_sum<kWave>(acc);
    if (lane == 0) {
      if (bias) acc += bias[(size_t)t * bias_stride + e];
      logits[(size_t)t * E + e] = acc;
    }
  }
}

// ------------------------------------------------------------- top-k --
// Order-preserving map of an fp32 onto uint32 (-0 is folded onto +0 first so
// equal values tie on the index, as the definition asks).
__device__ __forceinline__ uint32_t f32_orderable(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_orderable(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Key: orderable logit in the high word, (2^32-1 - expert) in the low word,
// so one unsigned max picks the largest logit and, among equal logits, the
// lower expert index.  0 never occurs for a real entry.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  return ((uint64_t)f32_orderable(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t lo = __shfl_xor((uint32_t)k, off);
    uint32_t hi = __shfl_xor((uint32_t)(k >> 32), off);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    k = (o > k) ? o : k;
  }
  return k;
}

// One wave per token; lane l owns experts l, l+64, ... (at most 16 of them).
// k rounds of "wave max, owner drops it"; round i's winner lands in lane i,
// which then forms its weight exp(l_i - l_0) / sum over the kept experts.
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits, int M, int E,
                                                           int k, int* __restrict__ topk_ids,
                                                           float* __restrict__ topk_weights) {
  constexpr int kPer = MOE_MAX_EXPERTS / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= M) return;
  const float* row = logits + (size_t)t * E;
  uint64_t key[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = lane + kWave * j;
    key[j] = (e < E) ? topk_key(row[e], e) : 0ull;
  }
  uint64_t best = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) best = key[j] > best ? key[j] : best;

  int my_id = 0;
  float my_val = 0.f;
  float top_val = 0.f;
  for (int i = 0; i < k; ++i) {
    const uint64_t win = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)win);
    const float v = f32_from_orderable((uint32_t)(win >> 32));
    if (i == 0) top_val = v;
    if (lane == i) { my_id = e; my_val = v; }
    if ((e & (kWave - 1)) == lane) {       // owner drops the winner, rescans
      best = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if (key[j] == win) key[j] = 0ull;
        best = key[j] > best ? key[j] : best;
      }
    }
  }
  const float ex = (lane < k) ? expf(my_val - top_val) : 0.f;
  const float sum = group_sum<kWave>(ex);
  if (lane < k) {
    topk_ids[(size_t)t * k + lane] = my_id;
    topk_weights[(size_t)t * k + lane] = ex / sum;
  }
}

hipError_t launch_router_logits(const uint16_t* x, const float* w_router, const float* bias,
                                int64_t bias_stride, int M, int H, int E, float* logits,
                                hipStream_t s) {
  const int waves_per_block = 2;
  dim3 grid((E + waves_per_block - 1) / waves_per_block), block(waves_per_block * kWave);
  if (H <= 2560)
    router_logits_kernel<10><<<grid, block, 0, s>>>(x, w_router, bias, bias_stride, M, H, E, logits);
  else
    router_logits_kernel<32><<<grid, block, 0, s>>>(x, w_router, bias, bias_stride, M, H, E, logits);
  return hipGetLastError();
}

hipError_t launch_topk_softmax(const float* logits, int M, int E, int k, int* ids, float* weights,
                               hipStream_t s) {
  const int waves_per_block = 4;
  dim3 grid((M + waves_per_block - 1) / waves_per_block), block(waves_per_block * kWave);
  topk_softmax_kernel<<<grid, block, 0, s>>>(logits, M, E, k, ids, weights);
  return hipGetLastError();
}

}  // namespace moe
