// MXFP8 quantisation of bf16 rows for the W4A8 variant: the baseline
// deployment in "3 Ways to Improve MoE Inference on NVIDIA DGX Spark" (digest,
// section 2) runs the MXFP4 experts with 8-bit activations.  Blocks of 32
// consecutive elements along a row share one E8M0 scale (OCP microscaling,
// rule in common.h); the elements are E4M3 codes.
#include <climits>

#include "kernels.h"

namespace moe {

// One thread per 32-element block of src [rows][K] (bf16): codes [rows][K]
// and scale bytes [rows][K/32] (either may be null), and the value of every
// code as bf16 [rows][K] (may be null).
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const uint16_t* __restrict__ src, int64_t nblocks,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales,
                                                             uint16_t* __restrict__ deq) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const uint4* p = reinterpret_cast<const uint4*>(src + b * 32);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = p[i];
    w[4 * i] = u.x; w[4 * i + 1] = u.y; w[4 * i + 2] = u.z; w[4 * i + 3] = u.w;
  }
  uint32_t m = 0u;                                   // |v| as bf16 bits: ordered like the values
#pragma unroll
  for (int i = 0; i < 16; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  const int e = mxfp8_exponent(__uint_as_float(m << 16));
  uint32_t c[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    int v = mxfp8_pack2<false>(bf16_bits_to_f32(w[2 * q] & 0xFFFFu), bf16_bits_to_f32(w[2 * q] >> 16), e, 0);
    v = mxfp8_pack2<true>(bf16_bits_to_f32(w[2 * q + 1] & 0xFFFFu), bf16_bits_to_f32(w[2 * q + 1] >> 16), e, v);
    c[q] = (uint32_t)v;
  }
  if (codes) {
    uint4* d = reinterpret_cast<uint4*>(codes + b * 32);
    d[0] = make_uint4(c[0], c[1], c[2], c[3]);
    d[1] = make_uint4(c[4], c[5], c[6], c[7]);
  }
  if (scales) scales[b] = (uint8_t)(e + 127);
  if (deq) {   // the values by the arithmetic rounding the down kernels use (checked against the codes)
    uint32_t o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      o[i] = f32_to_bf16_bits(mxfp8_round_value(bf16_bits_to_f32(w[i] & 0xFFFFu), e)) |
             (f32_to_bf16_bits(mxfp8_round_value(bf16_bits_to_f32(w[i] >> 16), e)) << 16);
    uint4* d = reinterpret_cast<uint4*>(deq + b * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  }
}

hipError_t launch_mxfp8_quantize(const uint16_t* src, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                                 uint16_t* deq, hipStream_t s) {
  const int64_t nb = rows * (K / 32);
  mxfp8_quantize_kernel<<<dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s>>>(src, nb, codes, scales, deq);
  return hipGetLastError();
}

// 16 elements of h (two bf16 terms, hi + lo) rounded to MXFP8 from their
// value; the codes' values replace hi.  Threads 2b and 2b + 1 share block b.
__device__ __forceinline__ void h_round_trip16(uint16_t* hi, const uint16_t* lo) {
  uint4* q = reinterpret_cast<uint4*>(hi);
  const uint4* l = reinterpret_cast<const uint4*>(lo);
  const uint4 u0 = q[0], u1 = q[1], v0 = l[0], v1 = l[1];
  uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
  const uint32_t r[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  mxfp8_round_trip16_2t(w, r);
  q[0] = make_uint4(w[0], w[1], w[2], w[3]);
  q[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// MXFP8 round trip of h rows [rows][K] (hi + lo) in place, 16 elements per
// thread.
__global__ __launch_bounds__(256) void mxfp8_round_trip_kernel(uint16_t* __restrict__ hi,
                                                               const uint16_t* __restrict__ lo, int64_t nblocks) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if ((t >> 1) >= nblocks) return;                  // whole pairs exit together
  h_round_trip16(hi + t * 16, lo + t * 16);
}

hipError_t launch_mxfp8_round_trip_rows(uint16_t* hi, const uint16_t* lo, int64_t rows, int K, hipStream_t s) {
  const int64_t nb = rows * (K / 32);
  mxfp8_round_trip_kernel<<<dim3((unsigned)((2 * nb + 255) / 256)), dim3(256), 0, s>>>(hi, lo, nb);
  return hipGetLastError();
}

// The h rows of one path's experts (batches): grid row y takes the path's
// y-th expert from the slot list (without a list, slot y if its expert is on
// the path); its n rows from hrow0 are rounded in place.
template <int PATH>   // 0: GEMV experts, 1: few-token matrix-core experts
__global__ __launch_bounds__(256) void h_round_trip_kernel(ForwardArgs a) {
  SlotRec r;
  const int y = blockIdx.y;
  if (a.lists) {
    if (y >= (PATH == 0 ? a.hdr->gemv_experts : a.hdr->mt_experts)) return;
    r = a.rec[a.lists[(PATH == 0 ? 0 : max_slots(a.M, a.k, a.E)) + y]];
  } else {
    r = a.rec[y];
    if (r.e < 0 || r.n >= a.mfma_min) return;
    const bool mt = r.n >= a.mt_min && r.n <= a.mt_max;
    if (mt != (PATH == 1)) return;
  }
  const int64_t nb = (int64_t)r.n * (a.I / 32);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if ((t >> 1) >= nb) return;                       // whole pairs exit together
  const int64_t o = (int64_t)r.hrow0 * a.I + t * 16;
  h_round_trip16(a.h + o, a.hlo + o);
}

hipError_t launch_h_round_trip(const ForwardArgs& a, int path, hipStream_t s) {
  const int slots = max_slots(a.M, a.k, a.E) - 1 + (a.has_shared ? 1 : 0);
  const bool mt_on = a.mt_min != INT_MAX, mfma_on = a.mfma_min != INT_MAX;
  // most tokens an expert of the path can have
  const int nmax = path == 1 ? kMtMaxTokens : (mt_on ? a.mt_min - 1 : (mfma_on ? a.mfma_min - 1 : a.M));
  const int64_t threads = 2 * (int64_t)min(nmax, a.M) * (a.I / 32);
  const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)slots);
  if (path == 0)
    h_round_trip_kernel<0><<<grid, dim3(256), 0, s>>>(a);
  else
    h_round_trip_kernel<1><<<grid, dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
