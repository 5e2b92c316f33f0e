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
  for (int t0 = blockIdx.y * TB; t0 < M; t0 += gridDim.y * TB) {   // grid rows split the tokens
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

// Batches: a tiled fp32 GEMM.  Workgroup = 32 tokens x TE experts, thread
// (ty, tx) of 16 x 16 owns tokens {ty, ty + 16} and experts {tx + 16 j}.
// K runs in 128-element chunks staged in LDS (x widened to fp32), double
// buffered, so each memory round trip carries 4 KB per thread row group.
// Each logit is summed in 16-product leaves, 16 leaves per group, then the
// groups in order: the longest chain of fp32 roundings is
// 16 + 16 + ceil(H/256) + 1 (bias), 43 at H = 2560 -- no longer than the
// small-batch kernel's H/64 + 6 + 1.
constexpr int RG_TT = 32, RG_KC = 128, RG_PITCH = RG_KC + 4;
template <int TE>
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ w_router,
                                                          const float* __restrict__ bias, int64_t bias_stride,
                                                          int M, int H, int E, float* __restrict__ logits) {
  constexpr int NE = TE / 16;
  constexpr int WQ = TE * RG_KC / 4 / 256;      // float4s of W each thread stages per chunk
  __shared__ __align__(16) float xs[2][RG_TT][RG_PITCH];
  __shared__ __align__(16) float wsh[2][TE][RG_PITCH];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int t0 = blockIdx.y * RG_TT, e0 = blockIdx.x * TE;
  // x staging: thread -> row tid/8, 16 bf16 at column (tid%8)*16
  const int xr_row = tid >> 3, xr_col = (tid & 7) * 16;
  const bool xv = t0 + xr_row < M;
  const uint4* xsrc = reinterpret_cast<const uint4*>(x + (size_t)min(t0 + xr_row, M - 1) * H + xr_col);
  // W staging: float4 number q = tid + 256 i of the TE x 128 tile: row q/32, column (q%32)*4
  const float4* wsrc[WQ];
  bool wv[WQ];
#pragma unroll
  for (int i = 0; i < WQ; ++i) {
    const int q = tid + 256 * i, row = q >> 5;
    wv[i] = e0 + row < E;
    wsrc[i] = reinterpret_cast<const float4*>(w_router + (size_t)min(e0 + row, E - 1) * H + (q & 31) * 4);
  }
  float tot[2][NE], grp[2][NE];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NE; ++j) { tot[i][j] = 0.f; grp[i][j] = 0.f; }
  const int nk = H / RG_KC;
  const int ktail = H - nk * RG_KC;              // < 128, multiple of 32: a last, partial chunk
  const int nchunks = nk + (ktail ? 1 : 0);
  uint4 xr0, xr1;
  float4 wr[WQ];
  auto load = [&](int kc) {
    const int kbase = kc * RG_KC;
    // columns past H read a clamped in-row address and are zeroed when staged
    const int off = min(kbase + xr_col, H - 16);
    xr0 = xsrc[(off - xr_col) / 8];
    xr1 = xsrc[(off - xr_col) / 8 + 1];
#pragma unroll
    for (int i = 0; i < WQ; ++i) {
      const int q = tid + 256 * i, col = (q & 31) * 4;
      wr[i] = wsrc[i][(min(kbase + col, H - 4) - col) / 4];
    }
  };
  auto store = [&](int buf, int kc) {
    const int kbase = kc * RG_KC;
    const bool in = xv && kbase + xr_col < H;
    const uint32_t w8[8] = {xr0.x, xr0.y, xr0.z, xr0.w, xr1.x, xr1.y, xr1.z, xr1.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float4 f = in ? make_float4(bf16_bits_to_f32(w8[2 * h] & 0xFFFFu), bf16_bits_to_f32(w8[2 * h] >> 16),
                                        bf16_bits_to_f32(w8[2 * h + 1] & 0xFFFFu),
                                        bf16_bits_to_f32(w8[2 * h + 1] >> 16))
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(&xs[buf][xr_row][xr_col + 4 * h]) = f;
    }
#pragma unroll
    for (int i = 0; i < WQ; ++i) {
      const int q = tid + 256 * i, row = q >> 5, col = (q & 31) * 4;
      *reinterpret_cast<float4*>(&wsh[buf][row][col]) =
          (wv[i] && kbase + col < H) ? wr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  load(0);
  store(0, 0);
  __syncthreads();
  int leaves = 0;
  for (int kc = 0; kc < nchunks; ++kc) {
    const int cur = kc & 1;
    if (kc + 1 < nchunks) load(kc + 1);
    const int klen = (kc < nk) ? RG_KC : ktail;
    for (int k0 = 0; k0 < klen; k0 += 16) {       // one 16-product leaf per step
      float leaf[2][NE];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NE; ++j) leaf[i][j] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 16; kk += 4) {
        const float4 a0 = *reinterpret_cast<const float4*>(&xs[cur][ty][k0 + kk]);
        const float4 a1 = *reinterpret_cast<const float4*>(&xs[cur][ty + 16][k0 + kk]);
#pragma unroll
        for (int j = 0; j < NE; ++j) {
          const float4 b = *reinterpret_cast<const float4*>(&wsh[cur][tx + 16 * j][k0 + kk]);
          leaf[0][j] = fmaf(a0.x, b.x, leaf[0][j]); leaf[0][j] = fmaf(a0.y, b.y, leaf[0][j]);
          leaf[0][j] = fmaf(a0.z, b.z, leaf[0][j]); leaf[0][j] = fmaf(a0.w, b.w, leaf[0][j]);
          leaf[1][j] = fmaf(a1.x, b.x, leaf[1][j]); leaf[1][j] = fmaf(a1.y, b.y, leaf[1][j]);
          leaf[1][j] = fmaf(a1.z, b.z, leaf[1][j]); leaf[1][j] = fmaf(a1.w, b.w, leaf[1][j]);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NE; ++j) grp[i][j] += leaf[i][j];
      if (++leaves == 16) {                        // a group is 16 leaves
        leaves = 0;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < NE; ++j) { tot[i][j] += grp[i][j]; grp[i][j] = 0.f; }
      }
    }
    if (kc + 1 < nchunks) store(cur ^ 1, kc + 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const int t = t0 + ty + 16 * i, e = e0 + tx + 16 * j;
      if (t < M && e < E) {
        float v = tot[i][j] + grp[i][j];
        if (bias) v += bias[(size_t)t * bias_stride + e];
        logits[(size_t)t * E + e] = v;
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
  __shared__ int n_mt;
  if (threadIdx.x == 0) n_mt = 0;
  __syncthreads();
  if (ro.rec)
    for (int slot = threadIdx.x; slot < max_slots(M, k, E); slot += blockDim.x) {
      const SlotRec r = small_slot_record(L, slot, M, k, E, ro.has_shared);
      ro.rec[slot] = r;
      if (r.e >= 0 && expert_path(r.n, ro.mt_min, ro.mt_max, ro.mfma_min) == 1) atomicAdd(&n_mt, 1);
    }
  __syncthreads();
  if (ro.hdr && threadIdx.x == 0) {     // at most 8 tokens per expert: no dense MFMA
    ro.hdr->gemv_experts = L.na + ro.has_shared - n_mt;
    ro.hdr->mt_experts = n_mt;
    ro.hdr->mfma_experts = 0;
    ro.hdr->mfma_items = 0;
  }
}

hipError_t launch_router_logits(const uint16_t* x, const float* w_router, const float* bias,
                                int64_t bias_stride, int M, int H, int E, float* logits,
                                hipStream_t s) {
  if (M >= kRouterGemmMinTokens) {
    const int tt = (M + RG_TT - 1) / RG_TT;
    if (M >= 256) {
      router_gemm_kernel<32><<<dim3((E + 31) / 32, tt), dim3(256), 0, s>>>(x, w_router, bias, bias_stride, M, H,
                                                                           E, logits);
    } else {
      router_gemm_kernel<16><<<dim3((E + 15) / 16, tt), dim3(256), 0, s>>>(x, w_router, bias, bias_stride, M, H,
                                                                           E, logits);
    }
    return hipGetLastError();
  }
  const int waves_per_block = 2;
  // one pass of up to 8 tokens per grid row, so a batch of up to 63 tokens
  // runs on up to 8x more waves instead of looping in one wave per expert
  // (long rows, H > 2560: one grid row, each wave loops over the tokens)
  const int rows = (H <= 2560) ? (M + 7) / 8 : 1;
  dim3 grid((E + waves_per_block - 1) / waves_per_block, rows), block(waves_per_block * kWave);
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
