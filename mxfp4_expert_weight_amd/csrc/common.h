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

// The same against activations carried as two bf16 terms (v = hi + lo, ~16
// significant bits): the codes are decoded once; both products are exact in
// fp32 and go into the one accumulator.
__device__ __forceinline__ float dot8_mxfp4_bf16_2t(uint32_t codes, float scale, const uint32_t hi[4],
                                                    const uint32_t lo[4], float acc) {
#define MOE_DOT2_2T(sel)                                                                           \
  {                                                                                                \
    const bf16x2 w = mxfp4_pair_bf16<sel>(codes, scale);                                           \
    acc = __builtin_amdgcn_fdot2_f32_bf16(w, __builtin_bit_cast(bf16x2, hi[sel]), acc, false);    \
    acc = __builtin_amdgcn_fdot2_f32_bf16(w, __builtin_bit_cast(bf16x2, lo[sel]), acc, false);    \
  }
  MOE_DOT2_2T(0) MOE_DOT2_2T(1) MOE_DOT2_2T(2) MOE_DOT2_2T(3)
#undef MOE_DOT2_2T
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

// ---------------------------------------------------------------- MXFP8 --
// OCP microscaling with E4M3 elements over 32-element blocks (the 8-bit
// activations of the W4A8 variant): block exponent e = floor(log2 amax) - 8
// (8 is the exponent of E4M3's largest power of two), clamped to the E8M0
// range [-127, 127], -127 for an all-zero block; element code = E4M3 nearest
// to v * 2^-e clamped to +-448, ties to even.  From the fp32 bits: a zero or
// subnormal amax (< 2^-126) gives -127.
__device__ __forceinline__ int mxfp8_exponent(float amax) {
  const int f = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return f == 0 ? -127 : max(f - 135, -127);
}
// Codes of a and b into bytes 0-1 (HI = false) or 2-3 (HI = true) of `word`.
// v * 2^-e is exact (v_ldexp_f32); v_cvt_pk_fp8_f32 rounds to nearest even.
template <bool HI>
__device__ __forceinline__ int mxfp8_pack2(float a, float b, int e, int word) {
  const float qa = fminf(fmaxf(ldexpf(a, -e), -448.f), 448.f);
  const float qb = fminf(fmaxf(ldexpf(b, -e), -448.f), 448.f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(qa, qb, word, HI);
}
// MXFP8 round trip of one value of a block with exponent e, in fp32
// arithmetic: clamp to +-448 * 2^e, then round to nearest even at the E4M3
// quantum of the value's binade (3 fraction bits; below 2^(e-6), the fixed
// subnormal quantum 2^(e-9)).  Gives the value of the code the converter
// above produces, without the conversion instructions.
__device__ __forceinline__ float mxfp8_round_value(float v, int e) {
  const float lim = ldexpf(448.f, e);
  const float c = fminf(fmaxf(v, -lim), lim);
  const int f = (int)((__float_as_uint(c) >> 23) & 0xFFu) - 127;   // floor(log2 |c|) (-127 for 0 / subnormal)
  const int qe = max(f, e - 6) - 3;
  return ldexpf(__builtin_rintf(ldexpf(c, -qe)), qe);
}
// MXFP8 round trip of 16 values carried as two bf16 terms, v = hi + lo (the
// sum is exact in fp32: lo is the rounding residual of hi), quantised from
// that value; the result (a code's value, exact in bf16) replaces hi.  The
// 16 values are half of a 32-element block whose other half lane ^ 1 holds
// and passes at the same time (DPP quad swap: lane ^ 1 must be active).
__device__ __forceinline__ void mxfp8_round_trip16_2t(uint32_t (&hi)[8], const uint32_t (&lo)[8]) {
  float v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = bf16_bits_to_f32(hi[i] & 0xFFFFu) + bf16_bits_to_f32(lo[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_bits_to_f32(hi[i] >> 16) + bf16_bits_to_f32(lo[i] >> 16);
  }
  uint32_t m = 0u;                                   // |v| as fp32 bits: ordered like the values
#pragma unroll
  for (int i = 0; i < 16; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  m = max(m, dpp_quad_xor1(m));
  const int e = mxfp8_exponent(__uint_as_float(m));
#pragma unroll
  for (int i = 0; i < 8; ++i)
    hi[i] = f32_to_bf16_bits(mxfp8_round_value(v[2 * i], e)) |
            (f32_to_bf16_bits(mxfp8_round_value(v[2 * i + 1], e)) << 16);
}

// MXFP8 round trip of 8 bf16 values (one uint4) that are a quarter of a
// 32-element block held by the four lanes of a DPP quad (all four active).
__device__ __forceinline__ void mxfp8_round_trip8_quad(uint4& u) {
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  m = max(m, dpp_quad_xor1(m));
  m = max(m, dpp_quad_xor2(m));
  const int e = mxfp8_exponent(__uint_as_float(m << 16));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = mxfp8_round_value(bf16_bits_to_f32(w[i] & 0xFFFFu), e);
    const float hi = mxfp8_round_value(bf16_bits_to_f32(w[i] >> 16), e);
    w[i] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
  }
  u = make_uint4(w[0], w[1], w[2], w[3]);
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
