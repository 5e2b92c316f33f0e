// Expert kernels of the MoE layer on the VALU GEMV path: every active expert
// runs once over all of its tokens (MoE-SpeQ article, section 4.2), with its
// MXFP4 weights (digest "3 Ways to Improve MoE Inference on NVIDIA DGX Spark",
// sections 2-3) streamed from HBM exactly once and dequantised in registers.
//
//   gate/up:  h[p][j] = SiLU(x_t . Wg[j]) * (x_t . Wu[j])       (bf16 h)
//   down:     y[t][r] += w_p * (h[p] . Wd[r])                    (fp32 atomics)
//
// Data layout of a 64-lane wave.  A row is cut into 16-element half-chunks
// (8 code bytes, half a 32-element scale block).  In gate/up a row is owned by
// a 32-lane group, lane j taking half-chunks j, j+32, ...; each wave load
// instruction therefore reads two 256-byte contiguous row segments.  In down
// (K = I = 768 is short) a row is owned by a 16-lane group, lane j taking
// half-chunks j, j+16, j+32: four 128-byte segments per instruction.  Partial
// dot products are summed across the group with DPP moves.
#include "kernels.h"

#include <hip/hip_ext.h>

namespace moe {

// Which expert a (slot) block works on, and where its tokens come from.
struct ExpertSlot {
  int e;        // expert index in the bank (E = shared)
  int n;        // tokens
  int pbeg;     // first sorted position (routed) or -1 (shared: tokens 0..M-1)
};

__device__ __forceinline__ bool resolve_slot(int slot, const ForwardArgs& a, ExpertSlot& s) {
  const int n_act = *a.num_active;
  if (slot < n_act) {
    s.e = a.active[slot];
    s.pbeg = a.offsets[s.e];
    s.n = a.offsets[s.e + 1] - s.pbeg;
    return true;
  }
  if (slot == n_act && a.has_shared) {
    s.e = a.E;
    s.pbeg = -1;
    s.n = a.M;
    return true;
  }
  return false;
}

// Token row, routing weight and h row of the i-th token of an expert.
__device__ __forceinline__ void token_of(const ForwardArgs& a, const ExpertSlot& s, int i, int& t,
                                         float& wgt, int& hrow) {
  if (s.pbeg >= 0) {
    const int pair = a.sorted_pairs[s.pbeg + i];
    t = pair / a.k;
    wgt = a.topk_weights[pair];
    hrow = s.pbeg + i;
  } else {
    t = i;
    wgt = 1.f;
    hrow = a.M * a.k + i;
  }
}

// ------------------------------------------------------------- gate/up --
// Block: 4 waves x 2 row-pair slots x GU_ITER iterations = 16 row pairs.
constexpr int GU_ITER = 2;
constexpr int GU_PAIRS_PER_BLOCK = 4 * 2 * GU_ITER;
constexpr int GU_HC = 5;        // half-chunks per lane per K pass (32 lanes -> 2560 elements)
constexpr int GU_NT = 2;        // tokens per pass over the weights

__global__ __launch_bounds__(256) void gateup_kernel(ForwardArgs a) {
  // Every block zeroes a share of y for the down kernel's scatter-add.
  {
    const size_t nblk = (size_t)gridDim.x * gridDim.y;
    const size_t b = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    const size_t total = (size_t)a.M * a.H;
    for (size_t i = b * blockDim.x + threadIdx.x; i < total; i += nblk * blockDim.x) a.y[i] = 0.f;
  }
  ExpertSlot s;
  if (!resolve_slot(blockIdx.y, a, s)) return;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    a.hdr->gemv_experts = *a.num_active + a.has_shared;   // every expert runs on this path
    a.hdr->mfma_experts = 0;
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int grp = lane >> 5;           // row-pair slot in the wave
  const int j32 = lane & 31;
  const int H = a.H, I = a.I;
  const int KH = H / 16;               // half-chunks per row
  const size_t row_q = H / 2, row_s = H / 32;
  const uint8_t* wq = a.w13_q + (size_t)s.e * 2 * I * row_q;
  const uint8_t* ws = a.w13_s + (size_t)s.e * 2 * I * row_s;

  for (int it = 0; it < GU_ITER; ++it) {
    const int jp = blockIdx.x * GU_PAIRS_PER_BLOCK + it * 8 + wave * 2 + grp;
    if (jp >= I) break;
    const uint8_t* qg = wq + (size_t)jp * row_q;
    const uint8_t* qu = wq + (size_t)(I + jp) * row_q;
    const uint8_t* sg = ws + (size_t)jp * row_s;
    const uint8_t* su = ws + (size_t)(I + jp) * row_s;

    for (int t0 = 0; t0 < s.n; t0 += GU_NT) {
      int tok[GU_NT];
#pragma unroll
      for (int q = 0; q < GU_NT; ++q) {
        float wdummy; int hdummy;
        if (t0 + q < s.n) token_of(a, s, t0 + q, tok[q], wdummy, hdummy); else tok[q] = -1;
      }
      float accg[GU_NT], accu[GU_NT];
#pragma unroll
      for (int q = 0; q < GU_NT; ++q) { accg[q] = 0.f; accu[q] = 0.f; }

      for (int kb = 0; kb < KH; kb += 32 * GU_HC) {
        uint2 cg[GU_HC], cu[GU_HC];
        float scg[GU_HC], scu[GU_HC];
#pragma unroll
        for (int i = 0; i < GU_HC; ++i) {
          const int hc = kb + j32 + 32 * i;
          if (hc < KH) {
            cg[i] = *reinterpret_cast<const uint2*>(qg + hc * 8);
            cu[i] = *reinterpret_cast<const uint2*>(qu + hc * 8);
            scg[i] = e8m0_to_f32(sg[hc >> 1]);
            scu[i] = e8m0_to_f32(su[hc >> 1]);
          } else {
            cg[i] = make_uint2(0, 0); cu[i] = make_uint2(0, 0);
            scg[i] = 0.f; scu[i] = 0.f;
          }
        }
#pragma unroll
        for (int q = 0; q < GU_NT; ++q) {
          if (tok[q] < 0) continue;
          const uint4* xr = reinterpret_cast<const uint4*>(a.x + (size_t)tok[q] * H);
#pragma unroll
          for (int i = 0; i < GU_HC; ++i) {
            const int hc = kb + j32 + 32 * i;
            if (hc < KH) {
              const uint4 x0 = xr[2 * hc], x1 = xr[2 * hc + 1];
              const uint32_t xa[4] = {x0.x, x0.y, x0.z, x0.w};
              const uint32_t xb[4] = {x1.x, x1.y, x1.z, x1.w};
              accg[q] = dot8_mxfp4_bf16(cg[i].x, scg[i], xa, accg[q]);
              accg[q] = dot8_mxfp4_bf16(cg[i].y, scg[i], xb, accg[q]);
              accu[q] = dot8_mxfp4_bf16(cu[i].x, scu[i], xa, accu[q]);
              accu[q] = dot8_mxfp4_bf16(cu[i].y, scu[i], xb, accu[q]);
            }
          }
        }
      }
#pragma unroll
      for (int q = 0; q < GU_NT; ++q) {
        const float g = group_sum<32>(accg[q]);
        const float u = group_sum<32>(accu[q]);
        if (tok[q] >= 0 && j32 == 0) {
          int t; float wgt; int hrow;
          token_of(a, s, t0 + q, t, wgt, hrow);
          a.h[(size_t)hrow * I + jp] = (uint16_t)f32_to_bf16_bits(silu(g) * u);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- down --
// Block: 4 waves x 4 row slots x DN_ITER iterations = 64 output rows.
constexpr int DN_ITER = 4;
constexpr int DN_ROWS_PER_BLOCK = 4 * 4 * DN_ITER;
constexpr int DN_HC = 3;        // half-chunks per lane per K pass (16 lanes -> 768 elements)
constexpr int DN_NT = 2;

__global__ __launch_bounds__(256) void down_kernel(ForwardArgs a) {
  ExpertSlot s;
  if (!resolve_slot(blockIdx.y, a, s)) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int grp = lane >> 4;
  const int j16 = lane & 15;
  const int H = a.H, I = a.I;
  const int KH = I / 16;
  const size_t row_q = I / 2, row_s = I / 32;
  const uint8_t* wq = a.w2_q + (size_t)s.e * H * row_q;
  const uint8_t* ws = a.w2_s + (size_t)s.e * H * row_s;

  for (int it = 0; it < DN_ITER; ++it) {
    const int r = blockIdx.x * DN_ROWS_PER_BLOCK + it * 16 + wave * 4 + grp;
    if (r >= H) break;
    const uint8_t* q = wq + (size_t)r * row_q;
    const uint8_t* sc = ws + (size_t)r * row_s;
    for (int t0 = 0; t0 < s.n; t0 += DN_NT) {
      int tok[DN_NT], hrow[DN_NT];
      float wgt[DN_NT], acc[DN_NT];
#pragma unroll
      for (int m = 0; m < DN_NT; ++m) {
        acc[m] = 0.f;
        if (t0 + m < s.n) token_of(a, s, t0 + m, tok[m], wgt[m], hrow[m]); else tok[m] = -1;
      }
      for (int kb = 0; kb < KH; kb += 16 * DN_HC) {
        uint2 c[DN_HC];
        float scl[DN_HC];
#pragma unroll
        for (int i = 0; i < DN_HC; ++i) {
          const int hc = kb + j16 + 16 * i;
          if (hc < KH) {
            c[i] = *reinterpret_cast<const uint2*>(q + hc * 8);
            scl[i] = e8m0_to_f32(sc[hc >> 1]);
          } else {
            c[i] = make_uint2(0, 0); scl[i] = 0.f;
          }
        }
#pragma unroll
        for (int m = 0; m < DN_NT; ++m) {
          if (tok[m] < 0) continue;
          const uint4* hr = reinterpret_cast<const uint4*>(a.h + (size_t)hrow[m] * I);
#pragma unroll
          for (int i = 0; i < DN_HC; ++i) {
            const int hc = kb + j16 + 16 * i;
            if (hc < KH) {
              const uint4 h0 = hr[2 * hc], h1 = hr[2 * hc + 1];
              const uint32_t ha[4] = {h0.x, h0.y, h0.z, h0.w};
              const uint32_t hb[4] = {h1.x, h1.y, h1.z, h1.w};
              acc[m] = dot8_mxfp4_bf16(c[i].x, scl[i], ha, acc[m]);
              acc[m] = dot8_mxfp4_bf16(c[i].y, scl[i], hb, acc[m]);
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < DN_NT; ++m) {
        const float v = group_sum<16>(acc[m]);
        if (tok[m] >= 0 && j16 == 0) unsafeAtomicAdd(&a.y[(size_t)tok[m] * H + r], wgt[m] * v);
      }
    }
  }
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

hipError_t launch_forward(const ForwardArgs& a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  const int slots = (a.E < a.M * a.k ? a.E : a.M * a.k) + (a.has_shared ? 1 : 0);
  dim3 block(256);
  dim3 ggu((a.I + GU_PAIRS_PER_BLOCK - 1) / GU_PAIRS_PER_BLOCK, slots);
  dim3 gdn((a.H + DN_ROWS_PER_BLOCK - 1) / DN_ROWS_PER_BLOCK, slots);
  if (start || stop) {
    // the events take the kernels' own begin/end timestamps
    hipExtLaunchKernelGGL(gateup_kernel, ggu, block, 0, s, start, nullptr, 0, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipExtLaunchKernelGGL(down_kernel, gdn, block, 0, s, nullptr, stop, 0, a);
    return hipGetLastError();
  }
  gateup_kernel<<<ggu, block, 0, s>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  down_kernel<<<gdn, block, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols, float* out,
                          hipStream_t st) {
  const int64_t words = rows * (cols / 8);
  const int64_t blocks = (words + 255) / 256;
  dequant_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(q, s, rows, cols, out);
  return hipGetLastError();
}

}  // namespace moe
