// Device helpers shared by the gfx950 kernels of the MXFP4 MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_mxfp4.h"

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- MXFP4 --
// E8M0 byte s -> 2^(s-127) as an fp32 bit pattern; exact for s in [1, 254].
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) { return __uint_as_float(s << 23); }

// Two E2M1 elements (one code byte: element 2j in the low nibble, 2j+1 in the
// high nibble) -> two bf16 values times the block scale.  `sel` picks the byte
// of `codes`.  E2M1 * 2^(s-127) has at most two significant bits, so the bf16
// result is exact for scale bytes in [2, 252].  Every kernel that reads MXFP4
// weights goes through this one routine (CDNA4 v_cvt_scalef32_pk_bf16_fp4).
template <int sel>
__device__ __forceinline__ bf16x2 mxfp4_pair_bf16(uint32_t codes, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, sel);
}

// 8 E2M1 elements of one 32-bit code word dotted with 8 bf16 activations
// (four packed pairs, element order matching the nibble order) into an fp32
// accumulator.  bf16*bf16 products are exact in fp32.
__device__ __forceinline__ float dot8_mxfp4_bf16(uint32_t codes, float scale, const uint32_t a[4],
                                                 float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(mxfp4_pair_bf16<0>(codes, scale), __builtin_bit_cast(bf16x2, a[0]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(mxfp4_pair_bf16<1>(codes, scale), __builtin_bit_cast(bf16x2, a[1]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(mxfp4_pair_bf16<2>(codes, scale), __builtin_bit_cast(bf16x2, a[2]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(mxfp4_pair_bf16<3>(codes, scale), __builtin_bit_cast(bf16x2, a[3]), acc, false);
  return acc;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// SiLU(g) = g * sigmoid(g) without overflow for large |g|.
__device__ __forceinline__ float silu(float g) {
  float e = __expf(-fabsf(g));                 // in (0, 1]
  float sig = (g >= 0.f) ? 1.f / (1.f + e) : e / (1.f + e);
  return g * sig;
}

// -------------------------------------------------------- DPP reductions --
// Sums across aligned groups of N lanes (N = 2, 4, 8, 16) with DPP moves that
// stay inside a 16-lane row: quad_perm swaps, then half-row and row mirrors.
__device__ __forceinline__ float dpp_add_quad_xor1(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_add_quad_xor2(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_add_half_mirror(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_add_row_mirror(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
}

// Sum over each aligned group of N lanes; every lane of the group gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  if constexpr (N >= 2) v = dpp_add_quad_xor1(v);
  if constexpr (N >= 4) v = dpp_add_quad_xor2(v);
  if constexpr (N >= 8) v = dpp_add_half_mirror(v);
  if constexpr (N >= 16) v = dpp_add_row_mirror(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

// ------------------------------------------------------------- workspace --
// Header at the start of the forward workspace; device-written counters that
// tell the caller which path ran (no global state in the library).
struct WorkspaceHeader {
  int32_t gemv_experts;   // expert passes on the VALU GEMV path in the last call
  int32_t mfma_experts;   // expert passes on the MFMA path in the last call
  int32_t reserved[62];
};
static_assert(sizeof(WorkspaceHeader) == 256, "header size");

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace moe
