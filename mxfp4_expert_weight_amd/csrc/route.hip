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

// Batches of more than 8 and fewer than kRouterGemmMinTokens tokens with
// rows of at most 2560: a workgroup of RL_WAVES waves takes RL_WAVES expert
// rows (one per wave, in registers as above) and passes of RL_TOK tokens
// whose x rows it stages in LDS once for all of its waves, so x is read from
// L2 once per workgroup instead of once per wave.  Same products and sums, in
// the same order, as router_logits_kernel.
constexpr int RL_WAVES = 8, RL_TOK = 8;
__global__ __launch_bounds__(RL_WAVES * kWave) void router_lds_kernel(const uint16_t* __restrict__ x,
                                                                     const float* __restrict__ w_router,
                                                                     const float* __restrict__ bias,
                                                                     int64_t bias_stride, int M, int H, int E,
                                                                     float* __restrict__ logits) {
  constexpr int VMAX = 10;                         // H <= 2560
  __shared__ uint2 xs[RL_TOK][VMAX * kWave];       // 4 bf16 per entry; entries past the row are zero
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int e = blockIdx.x * RL_WAVES + wave;
  const int nvec = H / 4;
  const float4* wrow = reinterpret_cast<const float4*>(w_router + (size_t)min(e, E - 1) * H);
  float4 w[VMAX];
#pragma unroll
  for (int i = 0; i < VMAX; ++i) {
    const int v = lane + kWave * i;
    const float4 t = wrow[min(v, nvec - 1)];
    w[i] = (v < nvec) ? t : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int t0 = blockIdx.y * RL_TOK; t0 < M; t0 += gridDim.y * RL_TOK) {
    // stage RL_TOK rows (clamped to the last token), 8 bf16 per thread step
    // (all loads of a thread are issued before its first store, so the
    // round trips overlap)
    constexpr int kPairs = RL_TOK * VMAX * kWave / 2;    // uint4 entries of the stage
    constexpr int kSteps = kPairs / (RL_WAVES * kWave);
    static_assert(kPairs % (RL_WAVES * kWave) == 0, "the stage is a whole number of thread steps");
    uint4 u[kSteps];
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const int i = threadIdx.x + j * RL_WAVES * kWave;
      const int q = i / (VMAX * kWave / 2), v2 = i - q * (VMAX * kWave / 2);   // uint2 entries 2 v2, 2 v2 + 1
      const uint4* xrow = reinterpret_cast<const uint4*>(x + (size_t)min(t0 + q, M - 1) * H);
      u[j] = xrow[min(v2, nvec / 2 - 1)];
    }
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const int i = threadIdx.x + j * RL_WAVES * kWave;
      const int q = i / (VMAX * kWave / 2), v2 = i - q * (VMAX * kWave / 2);
      const bool in0 = 2 * v2 < nvec, in1 = 2 * v2 + 1 < nvec;
      xs[q][2 * v2] = in0 ? make_uint2(u[j].x, u[j].y) : make_uint2(0, 0);
      xs[q][2 * v2 + 1] = in1 ? make_uint2(u[j].z, u[j].w) : make_uint2(0, 0);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < RL_TOK; ++q) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < VMAX; ++i) {
        const uint2 xv = xs[q][lane + kWave * i];
        acc = fmaf(bf16_bits_to_f32(xv.x & 0xFFFFu), w[i].x, acc);
        acc = fmaf(bf16_bits_to_f32(xv.x >> 16), w[i].y, acc);
        acc = fmaf(bf16_bits_to_f32(xv.y & 0xFFFFu), w[i].z, acc);
        acc = fmaf(bf16_bits_to_f32(xv.y >> 16), w[i].w, acc);
      }
      acc = group_sum<kWave>(acc);
      const int t = t0 + q;
      if (lane == 0 && t < M && e < E) {
        if (bias) acc += bias[(size_t)t * bias_stride + e];
        logits[(size_t)t * E + e] = acc;
      }
    }
    __syncthreads();                               // the stage is rewritten by the next pass
  }
}

// Batches on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16).  Each fp32
// router weight is split exactly into three bf16 parts by truncation:
// w1 = w with its low 16 bits cleared, w2 = (w - w1) the same way, w3 = the
// rest (at most 8 significant bits, so exact in bf16; for w = 0 and
// |w| >= 2^-102, where the parts stay normal).  x is bf16, so every
// product x * w_j is exact in fp32 and the logit is the plain sum of 3H exact
// products; only the summation order differs from the fp32 definition.  Each
// 32-product matrix-core dot starts from zero (a leaf); per weight part, 16
// leaves add into a group; the groups add into the total in K order, and the
// last partial groups and the bias follow, so a logit's longest rounding chain
// is 32 (leaf) + 16 (group) + 3 ceil(H / 512) (total) + 3 + 1.
// Workgroup = 32 tokens x 32 experts, wave w = the 16 x 16 tile
// (tokens 16 (w / 2), experts 16 (w % 2)); K runs in LDS-staged chunks of
// 256, double-buffered (70 KB of LDS: one workgroup per CU).
typedef __bf16 rv8bf __attribute__((ext_vector_type(8)));
typedef float rv4f __attribute__((ext_vector_type(4)));
constexpr int RM_T = 32, RM_E = 32, RM_KC = 256, RM_PITCH = RM_KC + 8;   // bf16 elements per LDS row
constexpr int RM_WAVES = 4, RM_THREADS = RM_WAVES * 64;
constexpr int RM_TPR = RM_THREADS / RM_T;      // staging threads per row (8)
constexpr int RM_G = RM_KC / 8 / RM_TPR;       // 8-element groups per staging thread and chunk (4)
// NK > 0: H is exactly NK chunks and the chunk loop is unrolled (the waits
// for the prefetched chunks are then exact; a runtime loop makes the compiler
// wait for every outstanding load at its back edge).  NK = 0: any H.
template <int NK>
__global__ __launch_bounds__(RM_THREADS) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ w_router,
                                                          const float* __restrict__ bias, int64_t bias_stride,
                                                          int M, int H, int E, float* __restrict__ logits) {
  __shared__ __align__(16) uint16_t xs[2][RM_T][RM_PITCH];
  __shared__ __align__(16) uint16_t wsp[2][3][RM_E][RM_PITCH];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int t0 = blockIdx.y * RM_T, e0 = blockIdx.x * RM_E;
  // staging thread = (row tid / RM_TPR, RM_G groups of 8 elements at columns
  // (tid % RM_TPR) * 8 + 8 RM_TPR g): 16-byte x loads, 32-byte W loads
  const int srow = tid / RM_TPR, scol = (tid % RM_TPR) * 8;
  const bool xin = t0 + srow < M, win = e0 + srow < E;
  const uint16_t* xrow = x + (size_t)min(t0 + srow, M - 1) * H;
  const float* wrow = w_router + (size_t)min(e0 + srow, E - 1) * H;
  const int nk = NK > 0 ? NK : (H + RM_KC - 1) / RM_KC;
  // chunks kc+1 and kc+2 are in registers while chunk kc is computed (each
  // chunk is one round trip to L2); the two register sets alternate, so no
  // register copy waits on a load
  struct Stage { uint4 x[RM_G]; float4 w[RM_G][2]; };
  Stage sa{}, sb{};
  auto load = [&](Stage& g, int kc) {
#pragma unroll
    for (int q = 0; q < RM_G; ++q) {
      const int col = min(kc * RM_KC + scol + 8 * RM_TPR * q, H - 8);   // clamped in-row address; zeroed when staged
      g.x[q] = *reinterpret_cast<const uint4*>(xrow + col);
      g.w[q][0] = *reinterpret_cast<const float4*>(wrow + col);
      g.w[q][1] = *reinterpret_cast<const float4*>(wrow + col + 4);
    }
  };
  auto store = [&](int buf, int kc, const Stage& g) {
#pragma unroll
    for (int q = 0; q < RM_G; ++q) {
      const int c = scol + 8 * RM_TPR * q;
      const bool ok = kc * RM_KC + c < H;
      const uint32_t mx = (ok && xin) ? 0xFFFFFFFFu : 0u, mw = (ok && win) ? 0xFFFFFFFFu : 0u;
      const uint4 xr = g.x[q];
      *reinterpret_cast<uint4*>(&xs[buf][srow][c]) = make_uint4(xr.x & mx, xr.y & mx, xr.z & mx, xr.w & mx);
      const float f[8] = {g.w[q][0].x, g.w[q][0].y, g.w[q][0].z, g.w[q][0].w,
                          g.w[q][1].x, g.w[q][1].y, g.w[q][1].z, g.w[q][1].w};
      uint32_t p1[4], p2[4], p3[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t h[3][2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const uint32_t u = __float_as_uint(f[2 * i + r]) & mw;
          const uint32_t a1 = u & 0xFFFF0000u;
          const float r1 = __uint_as_float(u) - __uint_as_float(a1);          // exact
          const uint32_t a2 = __float_as_uint(r1) & 0xFFFF0000u;
          const float r2 = r1 - __uint_as_float(a2);                           // exact, <= 8 bits
          h[0][r] = a1 >> 16;
          h[1][r] = a2 >> 16;
          h[2][r] = __float_as_uint(r2) >> 16;
        }
        p1[i] = h[0][0] | (h[0][1] << 16);
        p2[i] = h[1][0] | (h[1][1] << 16);
        p3[i] = h[2][0] | (h[2][1] << 16);
      }
      *reinterpret_cast<uint4*>(&wsp[buf][0][srow][c]) = make_uint4(p1[0], p1[1], p1[2], p1[3]);
      *reinterpret_cast<uint4*>(&wsp[buf][1][srow][c]) = make_uint4(p2[0], p2[1], p2[2], p2[3]);
      *reinterpret_cast<uint4*>(&wsp[buf][2][srow][c]) = make_uint4(p3[0], p3[1], p3[2], p3[3]);
    }
  };
  const int tw = wave >> 1, ew = wave & 1;
  const int fr = lane & 15, fk = 8 * (lane >> 4);   // fragment row / column and K offset
  const rv4f zero = {0.f, 0.f, 0.f, 0.f};
  rv4f tot = zero, grp[3] = {zero, zero, zero};    // one group per weight part: three independent chains
  int leaves = 0;
  auto step = [&](int cur, int st) {
    const rv8bf a = __builtin_bit_cast(rv8bf, *reinterpret_cast<const uint4*>(&xs[cur][16 * tw + fr][32 * st + fk]));
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const rv8bf b =
          __builtin_bit_cast(rv8bf, *reinterpret_cast<const uint4*>(&wsp[cur][p][16 * ew + fr][32 * st + fk]));
      grp[p] += __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, zero, 0, 0, 0);
    }
    if (++leaves == 16) {                            // 16 leaves per group, then into the total
      leaves = 0;
#pragma unroll
      for (int p = 0; p < 3; ++p) { tot += grp[p]; grp[p] = zero; }
    }
  };
  auto compute = [&](int kc) {
    const int cur = kc & 1;
    if constexpr (NK > 0) {
#pragma unroll
      for (int st = 0; st < RM_KC / 32; ++st) step(cur, st);
    } else {
      const int steps = min(RM_KC, H - kc * RM_KC) / 32;
      for (int st = 0; st < steps; ++st) step(cur, st);
    }
  };
  {
    Stage s0;
    load(s0, 0);
    if (nk > 1) load(sa, 1);
    if (nk > 2) load(sb, 2);
    store(0, 0, s0);
  }
  __syncthreads();
  auto two_chunks = [&](int kc) {                 // chunk kc from buffer 0, kc + 1 from buffer 1
    compute(kc);
    if (kc + 1 < nk) store(1, kc + 1, sa);
    if (kc + 3 < nk) load(sa, kc + 3);
    block_barrier_lds();                             // the prefetches stay in flight
    if (kc + 1 >= nk) return;
    compute(kc + 1);
    if (kc + 2 < nk) store(0, kc + 2, sb);
    if (kc + 4 < nk) load(sb, kc + 4);
    block_barrier_lds();
  };
  if constexpr (NK > 0) {
#pragma unroll
    for (int kc = 0; kc < NK; kc += 2) two_chunks(kc);
  } else {
    for (int kc = 0; kc < nk; kc += 2) two_chunks(kc);
  }
  const int e = e0 + 16 * ew + fr;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + 16 * tw + 4 * (lane >> 4) + r;
    if (t < M && e < E) {
      float v = tot[r] + grp[0][r];
      v += grp[1][r];
      v += grp[2][r];
      if (bias) v += bias[(size_t)t * bias_stride + e];
      logits[(size_t)t * E + e] = v;
    }
  }
}

// Batches with rows a multiple of 128 on the bf16 matrix cores, without LDS
// staging: workgroup = 64 tokens x 16 experts, and its four waves take the
// four quarters of K (whole 128-element blocks), so there are four times as
// many waves as output tiles of this size and each wave holds a 64 x 16 tile
// (4 token fragments on one expert fragment, so each weight is split once for
// 64 tokens) whose operands come straight from global memory.  In
// step j of a block, lane (r, g) of a 16-row fragment holds K elements
// 32 j + 8 g .. + 7 of its row, the same for x and the weights, so every
// pairing of the matrix product is the one of the definition; the four lanes
// of a row read one contiguous run (64 bytes of x, 128 of the weights), so a
// load instruction touches 16 rows' lines, not 64 scattered pieces.  The
// weights are split exactly into three bf16 parts as in router_mfma_kernel.
// A step's leaf is three chained matrix-core dots, smallest part first from
// zero: the accumulator carried into the next dot is at most 2^-7 of the
// products it meets (|w2| < 2^-7 |w|, |w3| < 2^-14 |w|), so the leaf's error
// is within 33 u of the sum of |x w| over its 32 elements (32 roundings for
// the last dot's own sum, whatever its order).  Leaves add into the wave's
// sum in K order, then the four waves' sums in K order through LDS, then the
// bias: a logit's longest rounding chain is 33 + 4 ceil(H / 512) + 3 + 1.
// QB > 0: every wave has exactly QB blocks (H = 512 QB) and the block loop is
// unrolled; QB = 0: any multiple of 128.
constexpr int RS_TT = 4, RS_ET = 1;                              // 16-row fragments per wave: tokens, experts
constexpr int RS_T = 16 * RS_TT, RS_E = 16 * RS_ET, RS_KB = 128, RS_WAVES = 4, RS_PITCH = RS_E + 4;
__device__ __forceinline__ void router_split3(const float4& lo, const float4& hi, uint4& p1, uint4& p2, uint4& p3) {
  const float f[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t q1[4], q2[4], q3[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t u[3][2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const float w = f[2 * i + r];
      const float r1 = w - __uint_as_float(__float_as_uint(w) & 0xFFFF0000u);       // exact
      const float r2 = r1 - __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);     // exact, <= 8 bits
      u[0][r] = __float_as_uint(w);
      u[1][r] = __float_as_uint(r1);
      u[2][r] = __float_as_uint(r2);
    }
    // the high halves of a pair (bytes 2, 3 of each word): element 2i low, 2i + 1 high
    q1[i] = __builtin_amdgcn_perm(u[0][1], u[0][0], 0x07060302u);
    q2[i] = __builtin_amdgcn_perm(u[1][1], u[1][0], 0x07060302u);
    q3[i] = __builtin_amdgcn_perm(u[2][1], u[2][0], 0x07060302u);
  }
  p1 = make_uint4(q1[0], q1[1], q1[2], q1[3]);
  p2 = make_uint4(q2[0], q2[1], q2[2], q2[3]);
  p3 = make_uint4(q3[0], q3[1], q3[2], q3[3]);
}

struct RouterBlock {
  uint4 x[RS_TT][4];      // the token rows: 8 bf16 per step
  float4 w[RS_ET][8];     // the expert rows: 8 fp32 per step
};

template <int QB>
__global__ __launch_bounds__(RS_WAVES * kWave) void router_split_kernel(const uint16_t* __restrict__ x,
                                                                       const float* __restrict__ w_router,
                                                                       const float* __restrict__ bias,
                                                                       int64_t bias_stride, int M, int H, int E,
                                                                       float* __restrict__ logits) {
  __shared__ float red[RS_WAVES][RS_T][RS_PITCH];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int t0 = blockIdx.y * RS_T, e0 = blockIdx.x * RS_E;
  const int fr = lane & 15, g = lane >> 4;
  const int nb = H / RS_KB, qb = QB > 0 ? QB : (nb + RS_WAVES - 1) / RS_WAVES;
  const int b0 = min(wave * qb, nb), nbw = min(b0 + qb, nb) - b0;   // this wave's blocks (may be none)
  const int ba0 = min(b0, nb - 1);                                    // addressed block: inside the row
  const uint16_t* xr[RS_TT];
  const float* wr[RS_ET];
#pragma unroll
  for (int i = 0; i < RS_TT; ++i) xr[i] = x + (size_t)min(t0 + 16 * i + fr, M - 1) * H + (size_t)ba0 * RS_KB + 8 * g;
#pragma unroll
  for (int i = 0; i < RS_ET; ++i)
    wr[i] = w_router + (size_t)min(e0 + 16 * i + fr, E - 1) * H + (size_t)ba0 * RS_KB + 8 * g;
  auto load = [&](RouterBlock& B, int b) {     // block b of this wave (clamped: always in the row)
    const int o = min(b, max(nbw - 1, 0)) * RS_KB;
#pragma unroll
    for (int i = 0; i < RS_TT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) B.x[i][j] = *reinterpret_cast<const uint4*>(xr[i] + o + 32 * j);
#pragma unroll
    for (int i = 0; i < RS_ET; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) B.w[i][j] = *reinterpret_cast<const float4*>(wr[i] + o + 32 * (j >> 1) + 4 * (j & 1));
  };
  const rv4f zero = {0.f, 0.f, 0.f, 0.f};
  rv4f acc[RS_TT][RS_ET];
#pragma unroll
  for (int i = 0; i < RS_TT; ++i)
#pragma unroll
    for (int k = 0; k < RS_ET; ++k) acc[i][k] = zero;
  auto compute = [&](const RouterBlock& B) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 bw[RS_ET][3];
#pragma unroll
      for (int k = 0; k < RS_ET; ++k) router_split3(B.w[k][2 * j], B.w[k][2 * j + 1], bw[k][0], bw[k][1], bw[k][2]);
#pragma unroll
      for (int i = 0; i < RS_TT; ++i) {
        const rv8bf a = __builtin_bit_cast(rv8bf, B.x[i][j]);
#pragma unroll
        for (int k = 0; k < RS_ET; ++k) {
          rv4f t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(rv8bf, bw[k][2]), zero, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(rv8bf, bw[k][1]), t, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(rv8bf, bw[k][0]), t, 0, 0, 0);
          acc[i][k] += t;
        }
      }
    }
  };
  // two register sets alternate: block b + 1 is in flight while block b is multiplied
  RouterBlock ba, bb;
  if constexpr (QB > 0) {
    load(ba, 0);
#pragma unroll
    for (int b = 0; b < QB; b += 2) {
      if (b + 1 < QB) load(bb, b + 1);
      compute(ba);
      if (b + 1 < QB) {
        if (b + 2 < QB) load(ba, b + 2);
        compute(bb);
      }
    }
  } else {
    load(ba, 0);
    for (int b = 0; b < nbw; b += 2) {
      load(bb, b + 1);
      compute(ba);
      if (b + 1 >= nbw) break;
      load(ba, b + 2);
      compute(bb);
    }
  }
  // lane (r, g) holds D[4 g + q][r] of fragment (i, k): token 16 i + 4 g + q, expert 16 k + r
#pragma unroll
  for (int i = 0; i < RS_TT; ++i)
#pragma unroll
    for (int k = 0; k < RS_ET; ++k)
#pragma unroll
      for (int q = 0; q < 4; ++q) red[wave][16 * i + 4 * g + q][16 * k + fr] = acc[i][k][q];
  __syncthreads();
  for (int o = threadIdx.x; o < RS_T * RS_E; o += RS_WAVES * kWave) {
    const int tt = o / RS_E, ee = o % RS_E, t = t0 + tt, e = e0 + ee;
    float v = red[0][tt][ee];
#pragma unroll
    for (int w = 1; w < RS_WAVES; ++w) v += red[w][tt][ee];
    if (t < M && e < E) {
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
  if (M >= kRouterGemmMinTokens && H % RS_KB == 0) {
    auto kern = (H == 5 * RS_WAVES * RS_KB) ? router_split_kernel<5> : router_split_kernel<0>;
    kern<<<dim3((E + RS_E - 1) / RS_E, (M + RS_T - 1) / RS_T), dim3(RS_WAVES * kWave), 0, s>>>(
        x, w_router, bias, bias_stride, M, H, E, logits);
    return hipGetLastError();
  }
  if (M >= kRouterGemmMinTokens) {
    auto kern = (H == 10 * RM_KC) ? router_mfma_kernel<10> : router_mfma_kernel<0>;
    kern<<<dim3((E + RM_E - 1) / RM_E, (M + RM_T - 1) / RM_T), dim3(RM_THREADS), 0, s>>>(
        x, w_router, bias, bias_stride, M, H, E, logits);
    return hipGetLastError();
  }
  if (M > 8 && H <= 2560 && H % 8 == 0) {
    const dim3 grid((E + RL_WAVES - 1) / RL_WAVES, (M + RL_TOK - 1) / RL_TOK);
    router_lds_kernel<<<grid, RL_WAVES * kWave, 0, s>>>(x, w_router, bias, bias_stride, M, H, E, logits);
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
