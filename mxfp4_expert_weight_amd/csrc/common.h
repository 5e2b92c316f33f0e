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

// ------------------------------------------------------- wave reductions --
// Cross-lane steps without LDS: DPP moves inside a 16-lane row (quad_perm
// swaps, half-row and row mirrors), then the CDNA4 row swaps
// v_permlane16_swap (rows 0<->1, 2<->3) and v_permlane32_swap (halves).
// Every lane of the reduced group ends up holding the result.
__device__ __forceinline__ uint32_t dpp_quad_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_quad_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_half_mirror(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_row_mirror(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);
}
// The partner row's value (lanes l and l^16) / partner half's value (l and l^32):
// a swap leaves one copy of each operand in the two results.
struct Pair { uint32_t a, b; };
__device__ __forceinline__ Pair swap16(uint32_t v) {
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return {r[0], r[1]};
}
__device__ __forceinline__ Pair swap32(uint32_t v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return {r[0], r[1]};
}

// Sum over each aligned group of N lanes (N = 1..64, power of two).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  if constexpr (N >= 2) v += __uint_as_float(dpp_quad_xor1(__float_as_uint(v)));
  if constexpr (N >= 4) v += __uint_as_float(dpp_quad_xor2(__float_as_uint(v)));
  if constexpr (N >= 8) v += __uint_as_float(dpp_half_mirror(__float_as_uint(v)));
  if constexpr (N >= 16) v += __uint_as_float(dpp_row_mirror(__float_as_uint(v)));
  if constexpr (N >= 32) { Pair p = swap16(__float_as_uint(v)); v = __uint_as_float(p.a) + __uint_as_float(p.b); }
  if constexpr (N >= 64) { Pair p = swap32(__float_as_uint(v)); v = __uint_as_float(p.a) + __uint_as_float(p.b); }
  return v;
}

// Unsigned max / min over the whole wave; every lane gets the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_quad_xor1(v));
  v = max(v, dpp_quad_xor2(v));
  v = max(v, dpp_half_mirror(v));
  v = max(v, dpp_row_mirror(v));
  Pair p = swap16(v); v = max(p.a, p.b);
  p = swap32(v); return max(p.a, p.b);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_quad_xor1(v));
  v = min(v, dpp_quad_xor2(v));
  v = min(v, dpp_half_mirror(v));
  v = min(v, dpp_row_mirror(v));
  Pair p = swap16(v); v = min(p.a, p.b);
  p = swap32(v); return min(p.a, p.b);
}

// Workgroup barrier that orders LDS only: it does not wait for outstanding
// global loads (gfx950 barriers do not imply a memory wait), so prefetched
// weights stay in flight across it.  (__syncthreads waits for all of them.)
__device__ __forceinline__ void block_barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------- workspace --
// Header at the start of the forward workspace; device-written counters that
// tell the caller which path ran (no global state in the library).
struct WorkspaceHeader {
  int32_t gemv_experts;   // expert passes on the VALU GEMV path in the last call
  int32_t mfma_experts;   // expert passes on the MFMA path in the last call
  int32_t mfma_items;     // (expert slot, token tile) work items of the MFMA kernels
  int32_t mt_experts;     // expert passes on the few-token matrix-core path
  int32_t reserved[60];
};
static_assert(sizeof(WorkspaceHeader) == 256, "header size");

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace moe
