// FP8 LM head: online quantisation of the bf16 head to OCP E4M3 with one fp32
// scale per vocabulary row, and the decode projection logits = x . W^T read
// from the FP8 codes (half the bytes of the bf16 head: "3 Ways to Improve MoE
// Inference on NVIDIA DGX Spark" digest, section 4; the head projects the
// 2,560-wide hidden state onto 157,184 tokens, section 2).
//
// Arithmetic: E4M3 decodes exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8 with
// scale 1), x is bf16, so every product is exact in fp32 (v_dot2_f32_bf16
// accumulates in fp32); the row sum is then multiplied by the row's scale.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr float kE4M3Max = 448.f;

// ------------------------------------------------------------ quantise --
// One wave per row: amax over the row, s = amax / 448 (fp32; 1 for a zero
// row), code = E4M3 nearest to clamp(w / s, -448, 448), ties to even
// (v_cvt_pk_fp8_f32 rounds to nearest even; the clamp makes saturation
// explicit).  Lane l handles 8 consecutive elements per 512-element step.
__global__ __launch_bounds__(256) void lmhead_quantize_kernel(const uint16_t* __restrict__ w, int V, int H,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int v = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (v >= V) return;                               // uniform over the wave
  const uint16_t* row = w + (size_t)v * H;
  uint32_t amax_bits = 0u;                          // |w| as fp32 bits: ordered like the values
  for (int c = lane * 8; c < H; c += kWave * 8) {
    const uint4 u = *reinterpret_cast<const uint4*>(row + c);
    const uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax_bits = max(amax_bits, (p[i] << 16) & 0x7FFFFFFFu);
      amax_bits = max(amax_bits, p[i] & 0x7FFF0000u);
    }
  }
  amax_bits = wave_max_u32(amax_bits);
  const float amax = __uint_as_float(amax_bits);
  const float s = amax > 0.f ? amax / kE4M3Max : 1.f;
  if (lane == 0) scales[v] = s;
  for (int c = lane * 8; c < H; c += kWave * 8) {
    const uint4 u = *reinterpret_cast<const uint4*>(row + c);
    const uint32_t p[4] = {u.x, u.y, u.z, u.w};
    float q[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[2 * i] = fminf(fmaxf(__uint_as_float(p[i] << 16) / s, -kE4M3Max), kE4M3Max);
      q[2 * i + 1] = fminf(fmaxf(__uint_as_float(p[i] & 0xFFFF0000u) / s, -kE4M3Max), kE4M3Max);
    }
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
    *reinterpret_cast<uint2*>(codes + (size_t)v * H + c) = make_uint2((uint32_t)lo, (uint32_t)hi);
  }
}

// ---------------------------------------------------------- projection --
// Workgroup = 4 waves x LH_RB rows each; the tokens' x rows are staged in LDS
// once per workgroup.  A wave issues the 16-byte code loads of all LH_RB rows
// (lane l takes 16-byte chunks l, l + 64, ... of each row) before any product,
// so each wave keeps LH_RB * H bytes in flight; each chunk's codes are decoded
// once and used by every token (up to MM tokens in registers); then the
// per-lane sums are summed across the wave (DPP) and scaled.  (Waves that walk
// several row groups with the next group's loads rolling in behind the decode
// measured slower: fewer resident waves, and a tail of long-lived waves.)
constexpr int LH_RB = 4;
constexpr int LH_WAVES = 4;
constexpr int LH_MAX_CHUNKS = (MOE_MAX_HIDDEN / 16 + kWave - 1) / kWave;   // per lane and row (8)

template <int CH, int MM>   // CH: chunks per lane and row, ceil(H / 16 / 64); MM: tokens, at least M
__global__ __launch_bounds__(LH_WAVES * kWave) void lmhead_fp8_kernel(const uint16_t* __restrict__ x,
                                                                      const uint8_t* __restrict__ codes,
                                                                      const float* __restrict__ scales, int M,
                                                                      int V, int H, float* __restrict__ logits) {
  extern __shared__ uint4 xs[];                     // [M][H] bf16
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nx = M * H / 8;
  for (int i = threadIdx.x; i < nx; i += blockDim.x) xs[i] = reinterpret_cast<const uint4*>(x)[i];
  __syncthreads();
  const int v0 = (blockIdx.x * LH_WAVES + wave) * LH_RB;
  if (v0 >= V) return;                              // uniform over the wave (no barrier follows)
  const int nch = H / 16;
  uint4 cw[LH_RB][CH];
#pragma unroll
  for (int r = 0; r < LH_RB; ++r) {
    const uint4* row = reinterpret_cast<const uint4*>(codes + (size_t)min(v0 + r, V - 1) * H);
#pragma unroll
    for (int i = 0; i < CH; ++i) cw[r][i] = row[min(lane + kWave * i, nch - 1)];   // clamped; masked below
  }
  float acc[LH_RB][MM];
#pragma unroll
  for (int r = 0; r < LH_RB; ++r)
#pragma unroll
    for (int t = 0; t < MM; ++t) acc[r][t] = 0.f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int ch = lane + kWave * i;
    if (ch < nch) {
      bf16x2 wb[LH_RB][8];                          // the chunk's 16 weights of each row, as bf16 pairs
#pragma unroll
      for (int r = 0; r < LH_RB; ++r) {
        const uint32_t c4[4] = {cw[r][i].x, cw[r][i].y, cw[r][i].z, cw[r][i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          wb[r][2 * q] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c4[q], 1.f, false);
          wb[r][2 * q + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c4[q], 1.f, true);
        }
      }
#pragma unroll
      for (int t = 0; t < MM; ++t) {
        if (t < M) {
          const uint4* xr = xs + (size_t)t * (H / 8) + 2 * ch;
          const uint4 x0 = xr[0], x1 = xr[1];       // 16 bf16 of the chunk
          const uint32_t xa[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int r = 0; r < LH_RB; ++r)
#pragma unroll
            for (int q = 0; q < 8; ++q)
              acc[r][t] = __builtin_amdgcn_fdot2_f32_bf16(wb[r][q], __builtin_bit_cast(bf16x2, xa[q]), acc[r][t],
                                                          false);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MM; ++t) {
    if (t < M) {
#pragma unroll
      for (int r = 0; r < LH_RB; ++r) {
        const float sum = group_sum<kWave>(acc[r][t]);
        if (lane == 0 && v0 + r < V) logits[(size_t)t * V + v0 + r] = sum * scales[v0 + r];
      }
    }
  }
}

// Two to MOE_LMHEAD_MAX_TOKENS tokens, H a multiple of 256: the bf16 matrix
// cores (v_mfma_f32_16x16x32_bf16) take the products, so each code is decoded
// once and no per-token dot instructions are issued.  The vocabulary rows are
// the A rows (16-row tiles) and the tokens the B columns (columns past M
// repeat the last token and are not stored).  A group of 4 waves takes RT
// tiles, its waves the four quarters of K; a workgroup holds RG groups, which
// share one LDS stage of x (at H = 2560: 2 tiles per wave, 2 groups, 64 rows
// per workgroup; the stage is a quarter of the codes' bytes per workgroup).  A
// wave issues all of its code loads first: for load p, lane (r, g) reads the
// 16 codes K = k0 + 64 p + 16 g .. + 15 of row r, which are matrix-core steps
// 2p and 2p + 1 (K slots 8g .. 8g + 7 of each), and the B fragments take the
// same K elements of the staged x rows, so every pairing is the definition's.
// Each step's 32-product dot starts from zero (a leaf) and adds into the
// wave's sum in K order; the four waves' sums are added in K order through
// LDS, then the scale multiplies: a logit's longest rounding chain is
// 32 + H / 128 + 3 + 1.
constexpr int LM_WAVES = 4, LM_MAX_LOADS = MOE_MAX_HIDDEN / 4 / 64;   // 16-byte loads per lane (32)
constexpr int LM_RT = 2;                                                 // 16-row tiles per wave (H = 2560)
constexpr int LM_RG = 2;                                                 // 4-wave row groups per workgroup (H = 2560)
typedef __bf16 lv8bf __attribute__((ext_vector_type(8)));
typedef float lv4f __attribute__((ext_vector_type(4)));
template <int NL, bool EXACT, int RT, int RG>   // NL 16-byte code loads per lane and row tile: H = 256 NL
                                                // (EXACT), or any H up to that; RT 16-row tiles per wave,
                                                // RG groups of 4 waves (each its own rows) per workgroup
__global__ __launch_bounds__(LM_WAVES * RG * kWave) void lmhead_mfma_kernel(const uint16_t* __restrict__ x,
                                                                      const uint8_t* __restrict__ codes,
                                                                      const float* __restrict__ scales, int M,
                                                                      int V, int H, float* __restrict__ logits) {
  extern __shared__ uint4 xs[];                     // [M][H] bf16
  __shared__ float red[LM_WAVES][16 * RT * RG][17];
  const int lane = threadIdx.x & (kWave - 1), wave = (threadIdx.x / kWave) % LM_WAVES;
  const int grp = threadIdx.x / (kWave * LM_WAVES);
  const int r = lane & 15, g = lane >> 4;
  const int vb = blockIdx.x * 16 * RT * RG, v0 = vb + grp * 16 * RT;
  const int kw = wave * (H / LM_WAVES);             // this wave's quarter of K
  const int nl = EXACT ? NL : H / 256;
  uint4 cw[RT][NL];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const uint4* row = reinterpret_cast<const uint4*>(codes + (size_t)min(v0 + 16 * i + r, V - 1) * H + kw) + g;
#pragma unroll
    for (int p = 0; p < NL; ++p) cw[i][p] = row[4 * min(p, nl - 1)];   // issued before the x stage is waited for
  }
  const int nx = M * H / 8;
  for (int i = threadIdx.x; i < nx; i += blockDim.x) xs[i] = reinterpret_cast<const uint4*>(x)[i];
  block_barrier_lds();
  const uint16_t* xt = reinterpret_cast<const uint16_t*>(xs) + (size_t)min(r, M - 1) * H + kw + 16 * g;
  const lv4f zero = {0.f, 0.f, 0.f, 0.f};
  lv4f acc[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) acc[i] = zero;
#pragma unroll
  for (int p = 0; p < NL; ++p) {
    if (p < nl) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {                   // codes 8s .. 8s + 7 of the lane's 16
        const lv8bf b = __builtin_bit_cast(lv8bf, *reinterpret_cast<const uint4*>(xt + 64 * p + 8 * s));
#pragma unroll
        for (int i = 0; i < RT; ++i) {
        const uint32_t c4[4] = {cw[i][p].x, cw[i][p].y, cw[i][p].z, cw[i][p].w};
        const bf16x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c4[2 * s], 1.f, false);
        const bf16x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c4[2 * s], 1.f, true);
        const bf16x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c4[2 * s + 1], 1.f, false);
        const bf16x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c4[2 * s + 1], 1.f, true);
        lv8bf a;
        a[0] = w0.x; a[1] = w0.y; a[2] = w1.x; a[3] = w1.y;
        a[4] = w2.x; a[5] = w2.y; a[6] = w3.x; a[7] = w3.y;
        acc[i] += __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, zero, 0, 0, 0);
        }
      }
    }
  }
  // lane (r, g) holds D[4 g + q][r]: vocabulary row v0 + 4 g + q, token r
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][16 * RT * grp + 16 * i + 4 * g + q][r] = acc[i][q];
  __syncthreads();
  for (int o = threadIdx.x; o < 256 * RT * RG; o += LM_WAVES * RG * kWave) {
    const int vr = o >> 4, t = o & 15, v = vb + vr;
    float sum = red[0][vr][t];
#pragma unroll
    for (int w = 1; w < LM_WAVES; ++w) sum += red[w][vr][t];
    if (t < M && v < V) logits[(size_t)t * V + v] = sum * scales[v];
  }
}

hipError_t launch_lmhead_quantize(const uint16_t* w, int V, int H, uint8_t* codes, float* scales,
                                  hipStream_t s) {
  lmhead_quantize_kernel<<<(V + 3) / 4, 256, 0, s>>>(w, V, H, codes, scales);
  return hipGetLastError();
}

hipError_t launch_lmhead_fp8(const uint16_t* x, const uint8_t* codes, const float* scales, int M, int V, int H,
                             float* logits, hipStream_t s) {
  const int ch = (H / 16 + kWave - 1) / kWave;
  const unsigned grid = (V + LH_WAVES * LH_RB - 1) / (LH_WAVES * LH_RB);
  const size_t shmem = (size_t)M * H * sizeof(uint16_t);
  void (*k)(const uint16_t*, const uint8_t*, const float*, int, int, int, float*);
  if (M >= 2 && H % 256 == 0) {
    k = H == 2560 ? lmhead_mfma_kernel<10, true, LM_RT, LM_RG> : lmhead_mfma_kernel<LM_MAX_LOADS, false, 1, 1>;
    const int rows = H == 2560 ? 16 * LM_RT * LM_RG : 16, waves = H == 2560 ? LM_WAVES * LM_RG : LM_WAVES;
    k<<<(V + rows - 1) / rows, waves * kWave, shmem, s>>>(x, codes, scales, M, V, H, logits);
    return hipGetLastError();
  }
  if (M == 1) {
    switch (ch) {
      case 1: k = lmhead_fp8_kernel<1, 1>; break;
      case 2: k = lmhead_fp8_kernel<2, 1>; break;
      case 3: k = lmhead_fp8_kernel<3, 1>; break;
      case 4: k = lmhead_fp8_kernel<4, 1>; break;
      default: k = lmhead_fp8_kernel<LH_MAX_CHUNKS, 1>; break;
    }
  } else if (M <= 4) {
    switch (ch) {
      case 1: k = lmhead_fp8_kernel<1, 4>; break;
      case 2: k = lmhead_fp8_kernel<2, 4>; break;
      case 3: k = lmhead_fp8_kernel<3, 4>; break;
      case 4: k = lmhead_fp8_kernel<4, 4>; break;
      default: k = lmhead_fp8_kernel<LH_MAX_CHUNKS, 4>; break;
    }
  } else {
    switch (ch) {
      case 1: k = lmhead_fp8_kernel<1, 8>; break;
      case 2: k = lmhead_fp8_kernel<2, 8>; break;
      case 3: k = lmhead_fp8_kernel<3, 8>; break;
      case 4: k = lmhead_fp8_kernel<4, 8>; break;
      default: k = lmhead_fp8_kernel<LH_MAX_CHUNKS, 8>; break;   // M >= 5 and M * H <= 32768: H <= 6528
    }
  }
  k<<<grid, LH_WAVES * kWave, shmem, s>>>(x, codes, scales, M, V, H, logits);
  return hipGetLastError();
}

}  // namespace moe
