// Dense path for experts with many tokens: the expert products run on the
// gfx950 scaled matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4) with the
// MXFP4 weights as the FP4 operand, read straight from their row-major layout
// with their own E8M0 block scales.  The choice of kernel by problem shape
// follows the MoE-SpeQ article, section 3.3 (many tokens per expert make the
// work a dense contraction).
//
// The other operand must be FP8/FP6/FP4, so activations are carried as two
// MXFP8 (E4M3) terms per 32-element block: v ~ hi * 2^sh + lo * 2^sl, where lo
// encodes the residual of hi.  Each term keeps 4 significant bits, so the
// pair keeps about 8, and the two products accumulate into one fp32 tile.
//
// The W4A8 variant carries x and h as one MXFP8 term (OCP rule, common.h),
// so each K chunk takes one scaled MFMA instead of two.
//
// Operand layout of the instruction (16 x 16 output tile, K = 128), lane l:
//   FP4 A:   row l%16, K = 32*(l/16) + p for nibble p of 16 bytes (low nibble first)
//   FP8 B:   column l%16, K = 64*(p/16) + 16*(l/16) + p%16 for byte p of 32 bytes
//   scales:  byte 0 of lane l's scale register covers row/column l%16 and the
//            K block [32*(l/16), +32), for both operands
//   output:  register r of lane l is D[4*(l/16) + r][l%16]
#include "kernels.h"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int MF_TT = kMfmaTileTokens;   // tokens per work item (4 sub-tiles of 16)
constexpr int MF_J = 32;                 // intermediate indices per gate/up workgroup
constexpr int MF_R = 64;                 // output rows per down workgroup
constexpr int MF_PITCH = 144;            // LDS bytes per staged 128-element row (+16 spreads banks)
constexpr int MF_WAVES = 4;

// ------------------------------------------------------- two-term MXFP8 --
// E8M0 exponent e with amax * 2^-e in [128, 256): the block's largest value
// uses the top normal binades of E4M3 (max 448) and never saturates.
__device__ __forceinline__ int mx_exponent(float amax) {
  return (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 7;
}
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Encode 32 fp32 values.  Blocks whose largest value is below 2^-100 encode
// as zero (scale byte 0).
__device__ __forceinline__ void encode_two_term(const float (&v)[32], uint32_t (&hi)[8], uint32_t (&lo)[8],
                                                uint32_t& shi, uint32_t& slo) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  if (!(amax >= 0x1p-100f)) {
#pragma unroll
    for (int q = 0; q < 8; ++q) { hi[q] = 0u; lo[q] = 0u; }
    shi = slo = 0u;
    return;
  }
  const int e1 = mx_exponent(amax);
  const float inv1 = pow2f(-e1), sc1 = pow2f(e1);
  float r[32];
  float ramax = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * q] * inv1, v[4 * q + 1] * inv1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * q + 2] * inv1, v[4 * q + 3] * inv1, w, true);
    hi[q] = (uint32_t)w;
    // the residual is exact in fp32 (hi * 2^e1 is within a factor 2^-4 of v)
    r[4 * q + 0] = v[4 * q + 0] - __builtin_amdgcn_cvt_f32_fp8(w, 0) * sc1;
    r[4 * q + 1] = v[4 * q + 1] - __builtin_amdgcn_cvt_f32_fp8(w, 1) * sc1;
    r[4 * q + 2] = v[4 * q + 2] - __builtin_amdgcn_cvt_f32_fp8(w, 2) * sc1;
    r[4 * q + 3] = v[4 * q + 3] - __builtin_amdgcn_cvt_f32_fp8(w, 3) * sc1;
#pragma unroll
    for (int i = 0; i < 4; ++i) ramax = fmaxf(ramax, fabsf(r[4 * q + i]));
  }
  shi = (uint32_t)(e1 + 127);
  if (!(ramax >= 0x1p-100f)) {
#pragma unroll
    for (int q = 0; q < 8; ++q) lo[q] = 0u;
    slo = 0u;
    return;
  }
  const int e2 = mx_exponent(ramax);
  const float inv2 = pow2f(-e2);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * q] * inv2, r[4 * q + 1] * inv2, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * q + 2] * inv2, r[4 * q + 3] * inv2, w, true);
    lo[q] = (uint32_t)w;
  }
  slo = (uint32_t)(e2 + 127);
}

// One thread per 32-element block of x [M][H] (bf16).
__global__ __launch_bounds__(256) void quantize_x_kernel(const uint16_t* __restrict__ x, int M, int H,
                                                         uint8_t* __restrict__ hi, uint8_t* __restrict__ lo,
                                                         uint8_t* __restrict__ shi, uint8_t* __restrict__ slo) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nb = (int64_t)M * (H / 32);
  if (b >= nb) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = src[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
      v[8 * i + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
    }
  }
  uint32_t h[8], l[8], sh, sl;
  encode_two_term(v, h, l, sh, sl);
  uint4* dh = reinterpret_cast<uint4*>(hi + b * 32);
  uint4* dl = reinterpret_cast<uint4*>(lo + b * 32);
  dh[0] = make_uint4(h[0], h[1], h[2], h[3]);
  dh[1] = make_uint4(h[4], h[5], h[6], h[7]);
  dl[0] = make_uint4(l[0], l[1], l[2], l[3]);
  dl[1] = make_uint4(l[4], l[5], l[6], l[7]);
  shi[b] = (uint8_t)sh;
  slo[b] = (uint8_t)sl;
}

// W4A8: 32 values -> one MXFP8 term (codes, E8M0 byte), OCP block rule.
__device__ __forceinline__ void encode_one_term(const float (&v)[32], uint32_t (&c)[8], uint32_t& sb) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mxfp8_exponent(amax);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    int w = mxfp8_pack2<false>(v[4 * q], v[4 * q + 1], e, 0);
    w = mxfp8_pack2<true>(v[4 * q + 2], v[4 * q + 3], e, w);
    c[q] = (uint32_t)w;
  }
  sb = (uint32_t)(e + 127);
}

// ------------------------------------------------------ staging in LDS --
// A work item's 64 token rows of one 128-element chunk, both terms, are staged
// by the 256 threads of the workgroup: thread (row c, quarter q) moves bytes
// [32q, 32q + 32) of each term and the scale byte of block q.  Rows past the
// item's tokens are zero.
struct StageRegs {
  uint4 h0, h1, l0, l1;
  uint32_t sh, sl;
};

// Raw loads (clamped row); the mask for rows past the tile is applied when
// the registers are written to LDS, so the load's wait is not forced early.
template <bool ONE>
__device__ __forceinline__ void stage_load(StageRegs& st, const uint8_t* qhi, const uint8_t* qlo,
                                           const uint8_t* shi, const uint8_t* slo, int64_t row, int K, int kc,
                                           int q) {
  const uint4* ph = reinterpret_cast<const uint4*>(qhi + row * K + kc * kMfmaK + 32 * q);
  st.h0 = ph[0]; st.h1 = ph[1];
  st.sh = shi[row * (K / 32) + kc * 4 + q];
  if constexpr (!ONE) {
    const uint4* pl = reinterpret_cast<const uint4*>(qlo + row * K + kc * kMfmaK + 32 * q);
    st.l0 = pl[0]; st.l1 = pl[1];
    st.sl = slo[row * (K / 32) + kc * 4 + q];
  }
}

struct __align__(16) StageBuf {
  uint8_t hi[MF_TT * MF_PITCH];
  uint8_t lo[MF_TT * MF_PITCH];
  uint8_t shi[MF_TT * 4];
  uint8_t slo[MF_TT * 4];
};

template <bool ONE>
__device__ __forceinline__ void stage_store(StageBuf& b, const StageRegs& st, int c, int q, bool valid) {
  // mask word by word (a select of whole vectors goes through scratch memory)
  const uint32_t m = valid ? 0xFFFFFFFFu : 0u;
  uint4* dh = reinterpret_cast<uint4*>(b.hi + c * MF_PITCH + 32 * q);
  dh[0] = make_uint4(st.h0.x & m, st.h0.y & m, st.h0.z & m, st.h0.w & m);
  dh[1] = make_uint4(st.h1.x & m, st.h1.y & m, st.h1.z & m, st.h1.w & m);
  b.shi[c * 4 + q] = (uint8_t)(st.sh & m);
  if constexpr (!ONE) {
    uint4* dl = reinterpret_cast<uint4*>(b.lo + c * MF_PITCH + 32 * q);
    dl[0] = make_uint4(st.l0.x & m, st.l0.y & m, st.l0.z & m, st.l0.w & m);
    dl[1] = make_uint4(st.l1.x & m, st.l1.y & m, st.l1.z & m, st.l1.w & m);
    b.slo[c * 4 + q] = (uint8_t)(st.sl & m);
  }
}

// B operand of token sub-tile s for lane (g, j): bytes [16g, +16) and
// [64 + 16g, +16) of row 16s + j, and the scale of block g of that row.
__device__ __forceinline__ v8i frag_b(const uint8_t* rows, int s, int g, int j) {
  const uint8_t* r = rows + (16 * s + j) * MF_PITCH;
  const uint4 a = *reinterpret_cast<const uint4*>(r + 16 * g);
  const uint4 b = *reinterpret_cast<const uint4*>(r + 64 + 16 * g);
  v8i v;
  v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
  v[4] = (int)b.x; v[5] = (int)b.y; v[6] = (int)b.z; v[7] = (int)b.w;
  return v;
}


// Expert `rec`, token tile t0..t0+nt: one 16-row x 64-token product per wave
// over K, both activation terms into the same accumulators.  The weight
// operand is prefetched MF_ADEPTH chunks ahead in a register ring (the HBM
// round trip is several chunks of products long); the activation chunks go
// through two LDS buffers one chunk ahead.  Barriers order LDS only, so the
// prefetched weights stay in flight across them.
constexpr int MF_ADEPTH = 8;
static_assert(MF_ADEPTH % 2 == 0, "the staging registers alternate by chunk parity");
template <bool ONE>
__device__ __forceinline__ void mfma_tile(v4f (&acc)[4], const uint8_t* row_q, const uint8_t* row_s,
                                          const uint8_t* qhi, const uint8_t* qlo, const uint8_t* shi,
                                          const uint8_t* slo, const int64_t stage_row, bool stage_valid, int K,
                                          StageBuf (&buf)[2]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4, j = lane & 15;
  const int c = threadIdx.x >> 2, q = threadIdx.x & 3;
  const int nk = K / kMfmaK;
#pragma unroll
  for (int s = 0; s < 4; ++s) acc[s] = v4f{0.f, 0.f, 0.f, 0.f};
  uint4 ar[MF_ADEPTH];
  uint32_t sr[MF_ADEPTH];
#pragma unroll
  for (int d = 0; d < MF_ADEPTH; ++d) {           // chunks past the end re-read the last (unused)
    const int kc = min(d, nk - 1);
    ar[d] = *reinterpret_cast<const uint4*>(row_q + kc * (kMfmaK / 2) + 16 * g);
    sr[d] = row_s[4 * kc + g];
  }
  // activation chunks: loaded two chunks ahead into st[chunk & 1], written to
  // LDS one chunk ahead (chunks past the end repeat the last: never read)
  StageRegs st[2];
  stage_load<ONE>(st[0], qhi, qlo, shi, slo, stage_row, K, 0, q);
  stage_store<ONE>(buf[0], st[0], c, q, stage_valid);
  stage_load<ONE>(st[1], qhi, qlo, shi, slo, stage_row, K, min(1, nk - 1), q);
  block_barrier_lds();
  for (int kb = 0; kb < nk; kb += MF_ADEPTH) {
#pragma unroll
    for (int d = 0; d < MF_ADEPTH; ++d) {
      const int kc = kb + d;
      if (kc < nk) {                               // uniform
        const int cur = kc & 1;                    // == d & 1 (MF_ADEPTH is even)
        stage_load<ONE>(st[d & 1], qhi, qlo, shi, slo, stage_row, K, min(kc + 2, nk - 1), q);
        v8i a;
        a[0] = (int)ar[d].x; a[1] = (int)ar[d].y; a[2] = (int)ar[d].z; a[3] = (int)ar[d].w;
        a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
        const int sa = (int)sr[d];
        {                                          // refill this ring slot with chunk kc + MF_ADEPTH
          const int kn = min(kc + MF_ADEPTH, nk - 1);
          ar[d] = *reinterpret_cast<const uint4*>(row_q + kn * (kMfmaK / 2) + 16 * g);
          sr[d] = row_s[4 * kn + g];
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const v8i bh = frag_b(buf[cur].hi, s, g, j);
          const int sbh = buf[cur].shi[(16 * s + j) * 4 + g];
          acc[s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bh, acc[s], 4, 0, 0, sa, 0, sbh);
          if constexpr (!ONE) {
            const v8i bl = frag_b(buf[cur].lo, s, g, j);
            const int sbl = buf[cur].slo[(16 * s + j) * 4 + g];
            acc[s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bl, acc[s], 4, 0, 0, sa, 0, sbl);
          }
        }
        stage_store<ONE>(buf[cur ^ 1], st[(d + 1) & 1], c, q, stage_valid);
        block_barrier_lds();
      }
    }
  }
}

// Token index of the expert's token number tt (sorted order).
__device__ __forceinline__ int item_token(const ForwardArgs& a, const SlotRec& r, int tt) {
  return r.pbeg >= 0 ? a.sorted_pairs[r.pbeg + tt] / a.k : tt;
}

// ------------------------------------------------------------- gate/up --
// Workgroup (32 intermediate indices, items): waves 0-1 take the 32 gate
// rows, waves 2-3 the 32 up rows, each over the item's 64 tokens.  Epilogue:
// h = SiLU(g) * u through LDS, then one thread per token encodes its 32
// h values (one MXFP8 block along the down projection's K) in two terms
// (ONE, W4A8: h rounded to bf16, then one MXFP8 term).
template <bool ONE>
__global__ __launch_bounds__(MF_WAVES * kWave) void gateup_mfma_kernel(ForwardArgs a) {
  __shared__ StageBuf buf[2];
  __shared__ float ul[MF_TT][MF_J + 1];
  const int n_items = a.hdr->mfma_items;
  const int j0 = blockIdx.x * MF_J;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4, j = lane & 15;
  const int half = wave & 1, is_up = wave >> 1;
  const int c = threadIdx.x >> 2;
  for (int it = blockIdx.y; it < n_items; it += gridDim.y) {
    const int2 item = a.items[it];
    const SlotRec rec = a.rec[item.x];
    const int t0 = item.y * MF_TT;
    const int nt = min(MF_TT, rec.n - t0);
    const int64_t row = (int64_t)rec.e * 2 * a.I + (is_up ? a.I : 0) + j0 + 16 * half + j;
    const uint8_t* row_q = a.w13_q + row * (a.H / 2);
    const uint8_t* row_s = a.w13_s + row * (a.H / 32);
    const bool sv = c < nt;
    const int64_t srow = sv ? item_token(a, rec, t0 + c) : 0;
    v4f acc[4];
    mfma_tile<ONE>(acc, row_q, row_s, a.xq_hi, a.xq_lo, a.xq_shi, a.xq_slo, srow, sv, a.H, buf);
    // acc[s][r] = (gate or up) row 16*half + 4g + r, token 16s + j
    if (is_up) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) ul[16 * s + j][16 * half + 4 * g + r] = acc[s][r];
    }
    block_barrier_lds();
    if (!is_up) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int jl = 16 * half + 4 * g + r, tc = 16 * s + j;
          ul[tc][jl] = silu(acc[s][r]) * ul[tc][jl];
        }
    }
    block_barrier_lds();
    if (threadIdx.x < nt) {
      const int tc = threadIdx.x;
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = ul[tc][i];
      const int64_t hrow = rec.hrow0 + t0 + tc;
      if constexpr (ONE) {   // W4A8: one MXFP8 term, quantised from the fp32 h
        uint32_t h[8], sh;
        encode_one_term(v, h, sh);
        uint4* dh = reinterpret_cast<uint4*>(a.hq_hi + hrow * a.I + j0);
        dh[0] = make_uint4(h[0], h[1], h[2], h[3]);
        dh[1] = make_uint4(h[4], h[5], h[6], h[7]);
        a.hq_shi[hrow * (a.I / 32) + j0 / 32] = (uint8_t)sh;
      } else {
        uint32_t h[8], l[8], sh, sl;
        encode_two_term(v, h, l, sh, sl);
        uint4* dh = reinterpret_cast<uint4*>(a.hq_hi + hrow * a.I + j0);
        uint4* dl = reinterpret_cast<uint4*>(a.hq_lo + hrow * a.I + j0);
        dh[0] = make_uint4(h[0], h[1], h[2], h[3]);
        dh[1] = make_uint4(h[4], h[5], h[6], h[7]);
        dl[0] = make_uint4(l[0], l[1], l[2], l[3]);
        dl[1] = make_uint4(l[4], l[5], l[6], l[7]);
        a.hq_shi[hrow * (a.I / 32) + j0 / 32] = (uint8_t)sh;
        a.hq_slo[hrow * (a.I / 32) + j0 / 32] = (uint8_t)sl;
      }
    }
    block_barrier_lds();
  }
}

// ---------------------------------------------------------------- down --
// Workgroup (64 output rows, items): wave w takes rows 16w..16w+15 over the
// item's 64 tokens; the epilogue adds w_token * result into y (fp32 atomics,
// as the GEMV path's combine).  ONE (W4A8): h is one MXFP8 term.
template <bool ONE>
__global__ __launch_bounds__(MF_WAVES * kWave) void down_mfma_kernel(ForwardArgs a) {
  __shared__ StageBuf buf[2];
  const int n_items = a.hdr->mfma_items;
  const int r0 = blockIdx.x * MF_R;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4, j = lane & 15;
  const int c = threadIdx.x >> 2;
  for (int it = blockIdx.y; it < n_items; it += gridDim.y) {
    const int2 item = a.items[it];
    const SlotRec rec = a.rec[item.x];
    const int t0 = item.y * MF_TT;
    const int nt = min(MF_TT, rec.n - t0);
    const int64_t row = (int64_t)rec.e * a.H + r0 + 16 * wave + j;
    const uint8_t* row_q = a.w2_q + row * (a.I / 2);
    const uint8_t* row_s = a.w2_s + row * (a.I / 32);
    const bool sv = c < nt;
    const int64_t srow = sv ? (int64_t)rec.hrow0 + t0 + c : 0;
    v4f acc[4];
    mfma_tile<ONE>(acc, row_q, row_s, a.hq_hi, a.hq_lo, a.hq_shi, a.hq_slo, srow, sv, a.I, buf);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int tc = 16 * s + j;
      if (tc < nt) {
        int t;
        float w;
        if (rec.pbeg >= 0) {
          const int pair = a.sorted_pairs[rec.pbeg + t0 + tc];
          t = pair / a.k;
          w = a.topk_weights[pair];
        } else {
          t = t0 + tc;
          w = 1.f;
        }
        if (a.yp) {
          float* yr = a.yp + ((int64_t)rec.hrow0 + t0 + tc) * a.H + r0 + 16 * wave + 4 * g;
          *reinterpret_cast<float4*>(yr) = make_float4(w * acc[s][0], w * acc[s][1], w * acc[s][2], w * acc[s][3]);
        } else {
          float* yr = a.y + (int64_t)t * a.H + r0 + 16 * wave + 4 * g;
#pragma unroll
          for (int r = 0; r < 4; ++r) unsafeAtomicAdd(yr + r, w * acc[s][r]);
        }
      }
    }
  }
}

namespace {
// Rows of persistent workgroups: enough to fill the chip a few times over.
unsigned item_rows(int row_tiles, int M, int k) {
  const int want = (4 * 256 + row_tiles - 1) / row_tiles;
  const int cap = mfma_max_items(M, k);
  return (unsigned)(want < cap ? (want > 0 ? want : 1) : cap);
}
}  // namespace

hipError_t launch_forward_mfma_front(const ForwardArgs& a, hipStream_t s) {
  const int64_t nb = (int64_t)a.M * (a.H / 32);
  quantize_x_kernel<<<dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s>>>(a.x, a.M, a.H, a.xq_hi, a.xq_lo,
                                                                            a.xq_shi, a.xq_slo);
  return hipGetLastError();
}

hipError_t launch_gateup_mfma(const ForwardArgs& a, hipStream_t s) {
  const int tiles = a.I / MF_J;
  const dim3 grid(tiles, item_rows(tiles, a.M, a.k)), block(MF_WAVES * kWave);
  if (a.act8)
    gateup_mfma_kernel<true><<<grid, block, 0, s>>>(a);
  else
    gateup_mfma_kernel<false><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_mfma(const ForwardArgs& a, hipStream_t s) {
  const int tiles = a.H / MF_R;
  const dim3 grid(tiles, item_rows(tiles, a.M, a.k)), block(MF_WAVES * kWave);
  if (a.act8)
    down_mfma_kernel<true><<<grid, block, 0, s>>>(a);
  else
    down_mfma_kernel<false><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
