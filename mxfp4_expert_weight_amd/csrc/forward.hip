// Expert kernels of moe_mxfp4_forward on the VALU GEMV path, plus the dequant
// export.  A block is (row tile, expert slot); slots past the active experts
// (and the shared expert) exit at once -- the grid is sized for the worst case
// because the number of active experts is only known on the device.
//
//   gateup_kernel:  h[p][j] = SiLU(x_t . Wg[j]) * (x_t . Wu[j])   (bf16 h)
//   down_kernel:    y[t][r] += w_p * (h[p] . Wd[r])               (fp32 atomics;
//                   gateup_kernel zeroes y first)
#include "gemv_dev.h"
#include "sort_dev.h"
#include "topk_dev.h"

#include <hip/hip_ext.h>

namespace moe {

constexpr int GU_NP = 2, GU_HC = 5, GU_WPB = 4;     // 4*NP = 8 rows per wave, 16 pairs per block
constexpr int DN_NR = 4, DN_HC = 3, DN_WPB = 4;     // 4*NR = 16 rows per wave, 64 rows per block
constexpr int GU_PAIRS_PER_BLOCK = GU_WPB * 2 * GU_NP;
constexpr int DN_ROWS_PER_BLOCK = DN_WPB * 4 * DN_NR;
constexpr int GU_LDS_PER_WAVE = 2 * 2 * GU_NP * (MOE_MAX_HIDDEN / 32);
constexpr int DN_LDS_PER_WAVE = 4 * DN_NR * (MOE_MAX_INTER / 32);
constexpr int GU_SHORT_H = 32 * GU_HC * 16;         // longest row the single-pass path holds (2560)
constexpr int DN_SHORT_I = 16 * DN_HC * 16;         // (768)

// Routing inside a gate/up block (decode batches, M <= kRoutedMaxTokens):
// wave t takes token t's top-k from the logits, wave 0 sorts the pairs by
// expert in LDS, and the block reads its own slot (blockIdx.y) from the result.
// Every block computes the same routing from the same logits; block (0, 0)
// writes the routing outputs and block (0, slot) the slot record the down
// kernel reads.  Returns false when the slot has no work.
template <int C>
__device__ __forceinline__ bool route_in_block(const ForwardArgs& a, const RouteOut& r, ExpertSlot& s,
                                               int& n_act) {
  __shared__ int ids_lds[kRoutedMaxPairs];
  __shared__ float w_lds[kRoutedMaxPairs];
  __shared__ int sp_lds[kRoutedMaxPairs];
  __shared__ int act_lds[kRoutedMaxPairs];
  __shared__ int sort_lds[wave_sort_lds_ints(C)];
  __shared__ int na_lds;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const int N = a.M * a.k;
  for (int t = wave; t < a.M; t += nw) {
    int id; float w;
    wave_topk_softmax<C>(r.logits + (size_t)t * a.E, a.E, a.k, id, w);
    if (lane < a.k) {
      ids_lds[t * a.k + lane] = id;
      w_lds[t * a.k + lane] = w;
    }
  }
  __syncthreads();
  int* off = sort_lds + kWave * C + 1;
  if (wave == 0) wave_sort_small<C>(ids_lds, N, a.E, r.ebits, sort_lds, off, sp_lds, act_lds, &na_lds);
  __syncthreads();
  const int D = na_lds;
  n_act = D;
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    block_store_sort(a.E, off, sp_lds, act_lds, D, r.offsets, r.sorted_pairs, r.active, r.num_active);
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
      r.topk_ids[i] = ids_lds[i];
      r.topk_weights[i] = w_lds[i];
    }
  }
  const SlotRec rec = make_slot_record(blockIdx.y, D, off, sp_lds, act_lds, w_lds, a.M, a.k, a.E,
                                       a.has_shared);
  if (blockIdx.x == 0 && threadIdx.x == 0) r.rec[blockIdx.y] = rec;
  s.e = rec.e; s.n = rec.n; s.pbeg = rec.pbeg; s.hrow0 = rec.hrow0;
#pragma unroll
  for (int q = 0; q < kRecTokens; ++q) { s.tok[q] = rec.tok[q]; s.w[q] = rec.w[q]; }
  return rec.e >= 0;
}

// at most 3 waves per SIMD: the codes, scales and staged activations of a wave
// stay in registers without spilling (M=1 needs under 2 waves per SIMD anyway).
// C > 0: the block routes itself (C = experts per lane of the top-k).
template <bool SHORT, int C>
__global__ __launch_bounds__(GU_WPB * kWave) __attribute__((amdgpu_waves_per_eu(1, 3)))
void gateup_kernel(ForwardArgs a, RouteOut r) {
  {   // every block zeroes a share of y for the down kernel's scatter-add
    const size_t nblk = (size_t)gridDim.x * gridDim.y;
    const size_t b = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    const size_t total = (size_t)a.M * a.H;
    for (size_t i = b * blockDim.x + threadIdx.x; i < total; i += nblk * blockDim.x) a.y[i] = 0.f;
  }
  ExpertSlot s;
  int n_act = 0;
  if constexpr (C > 0) {
    if (!route_in_block<C>(a, r, s, n_act)) return;     // uniform over the block
  } else {
    if (!resolve_slot(blockIdx.y, a, s)) return;
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    if constexpr (C == 0) n_act = *a.num_active;
    a.hdr->gemv_experts = n_act + a.has_shared;          // every expert runs on this path
    a.hdr->mfma_experts = 0;
  }
  __shared__ uint8_t s_lds[GU_WPB][GU_LDS_PER_WAVE];
  const int wave = threadIdx.x / kWave;
  const int jp0 = (blockIdx.x * GU_WPB + wave) * 2 * GU_NP;
  if (jp0 >= a.I) return;
  if constexpr (SHORT)
    gateup_short<GU_NP, GU_HC>(a, s, jp0, s_lds[wave]);
  else
    gateup_long<GU_NP, GU_HC>(a, s, jp0, s_lds[wave]);
}

template <bool SHORT>
__global__ __launch_bounds__(DN_WPB * kWave) void down_kernel(ForwardArgs a) {
  ExpertSlot s;
  if (!resolve_slot(blockIdx.y, a, s)) return;
  __shared__ uint8_t s_lds[DN_WPB][DN_LDS_PER_WAVE];
  const int wave = threadIdx.x / kWave;
  const int r0 = (blockIdx.x * DN_WPB + wave) * 4 * DN_NR;
  if (r0 >= a.H) return;
  if constexpr (SHORT)
    down_short<DN_NR, DN_HC>(a, s, r0, s_lds[wave]);
  else
    down_long<DN_NR, DN_HC>(a, s, r0, s_lds[wave]);
}

// ------------------------------------------------------------- dequant --
// One thread per 32-bit code word (8 elements): the same pair routine as the
// expert kernels, widened from bf16 to fp32 (exact).
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ q,
                                                      const uint8_t* __restrict__ s, int64_t rows,
                                                      int64_t cols, float* __restrict__ out) {
  const int64_t words_per_row = cols / 8;
  const int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (wi >= rows * words_per_row) return;
  const int64_t r = wi / words_per_row, w = wi % words_per_row;
  const uint32_t code = reinterpret_cast<const uint32_t*>(q + r * (cols / 2))[w];
  const float scale = e8m0_to_f32(s[r * (cols / 32) + (w * 8) / 32]);
  const bf16x2 p0 = mxfp4_pair_bf16<0>(code, scale), p1 = mxfp4_pair_bf16<1>(code, scale);
  const bf16x2 p2 = mxfp4_pair_bf16<2>(code, scale), p3 = mxfp4_pair_bf16<3>(code, scale);
  float4* o = reinterpret_cast<float4*>(out + r * cols + w * 8);
  o[0] = make_float4((float)p0.x, (float)p0.y, (float)p1.x, (float)p1.y);
  o[1] = make_float4((float)p2.x, (float)p2.y, (float)p3.x, (float)p3.y);
}

namespace {

hipError_t launch_pair(void (*gu)(ForwardArgs, RouteOut), const ForwardArgs& a, const RouteOut& r,
                       hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  const int slots = max_slots(a.M, a.k, a.E) - 1 + (a.has_shared ? 1 : 0);
  dim3 ggu((a.I + GU_PAIRS_PER_BLOCK - 1) / GU_PAIRS_PER_BLOCK, slots), bgu(GU_WPB * kWave);
  dim3 gdn((a.H + DN_ROWS_PER_BLOCK - 1) / DN_ROWS_PER_BLOCK, slots), bdn(DN_WPB * kWave);
  auto dn = (a.I <= DN_SHORT_I) ? down_kernel<true> : down_kernel<false>;
  // with events, they take the gate/up kernel's own begin/end timestamps
  hipExtLaunchKernelGGL(gu, ggu, bgu, 0, s, start, stop, 0, a, r);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipExtLaunchKernelGGL(dn, gdn, bdn, 0, s, nullptr, nullptr, 0, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const ForwardArgs& a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  const RouteOut none{};
  return launch_pair(a.H <= GU_SHORT_H ? gateup_kernel<true, 0> : gateup_kernel<false, 0>, a, none, s, start,
                     stop);
}

hipError_t launch_forward_routed(const ForwardArgs& a, const RouteOut& r, hipStream_t s, hipEvent_t start,
                                 hipEvent_t stop) {
  const bool short_h = a.H <= GU_SHORT_H;
  void (*gu)(ForwardArgs, RouteOut);
  if (topk_lane_experts(a.E) == 8)
    gu = short_h ? gateup_kernel<true, 8> : gateup_kernel<false, 8>;
  else
    gu = short_h ? gateup_kernel<true, 16> : gateup_kernel<false, 16>;
  return launch_pair(gu, a, r, s, start, stop);
}

hipError_t launch_dequant(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols, float* out,
                          hipStream_t st) {
  const int64_t words = rows * (cols / 8);
  const int64_t blocks = (words + 255) / 256;
  dequant_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(q, s, rows, cols, out);
  return hipGetLastError();
}

}  // namespace moe
