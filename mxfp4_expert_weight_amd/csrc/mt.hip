// Experts with a few tokens (from kMtMinTokens up to one 16-token tile) in
// batches of more than kRoutedMaxTokens tokens.  The per-token VALU GEMV
// decodes every weight once per token; here a workgroup decodes each MXFP4
// weight once (v_cvt_scalef32_pk_bf16_fp4, exact) and the products with all
// of the expert's tokens run on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16): bf16 x bf16 products are exact and accumulate
// in fp32, the same arithmetic as the GEMV path.  The expert still runs once
// over all of its tokens (MoE-SpeQ article, section 4.2).
//
// Operand layout (16 x 16 x 32): lane l holds row (A) / column (B) l%16 and
// 8 consecutive K values of lane group l/16; output register r of lane l is
// D[4*(l/16) + r][l%16].  Only the pairing of A and B values matters, so in
// step s of a 256-element chunk lane group g takes chunk elements
// 64g + 8s .. 64g + 8s + 7: a lane's weight codes for the whole chunk are 32
// contiguous bytes (two 16-byte loads) and cover scale blocks 2g and 2g + 1.
#include "gemv_dev.h"

namespace moe {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int MT_KC = 256;                 // K per staged chunk (8 steps of 32)
constexpr int MT_TOK = 16;                 // token columns of one tile
constexpr int MT_PITCH = MT_KC * 2 + 16;   // LDS bytes per staged token row (+16 spreads banks)
constexpr int MT_WAVES = 4;
constexpr int MT_GU_J = 16 * MT_WAVES;     // intermediate indices per gate/up workgroup
constexpr int MT_DN_R = 32 * MT_WAVES;     // output rows per down workgroup

struct MtStage {
  __align__(16) uint8_t rows[2][MT_TOK * MT_PITCH];
};

// Token number c (sorted order) of the expert: its row of x, routing weight and h row.
__device__ __forceinline__ void mt_token(const ForwardArgs& a, const SlotRec& r, int c, int& t, float& w) {
  if (r.pbeg >= 0) {
    const int pair = a.sorted_pairs[r.pbeg + c];
    t = pair / a.k;
    w = a.topk_weights[pair];
  } else {
    t = c;
    w = 1.f;
  }
}

// The record of grid row y, if its expert is on this path: with the slot
// list, row y takes the y-th few-token expert (rows past them exit); without
// it, row y is slot y.
__device__ __forceinline__ bool mt_slot(const ForwardArgs& a, int y, SlotRec& r) {
  if (a.lists) {
    if (y >= a.hdr->mt_experts) return false;
    r = a.rec[a.lists[max_slots(a.M, a.k, a.E) + y]];
    return true;
  }
  r = a.rec[y];
  return r.e >= 0 && r.n >= a.mt_min && r.n <= a.mt_max && r.n < a.mfma_min;
}

// Weight codes and scales of one row for chunk kc: 32 code bytes and the two
// scale bytes of lane group g.
struct MtRowChunk {
  uint4 c0, c1;
  uint32_t s0, s1;
};
__device__ __forceinline__ MtRowChunk mt_load_row(const uint8_t* row_q, const uint8_t* row_s, int kc, int g) {
  MtRowChunk m;
  const uint4* q = reinterpret_cast<const uint4*>(row_q + kc * (MT_KC / 2) + 32 * g);
  m.c0 = q[0];
  m.c1 = q[1];
  m.s0 = row_s[kc * (MT_KC / 32) + 2 * g];
  m.s1 = row_s[kc * (MT_KC / 32) + 2 * g + 1];
  return m;
}

// A operand of step s: the 8 weights of code word s, decoded to bf16.
__device__ __forceinline__ v8bf mt_frag_a(const MtRowChunk& m, int s) {
  const uint32_t w = (s & 3) == 0 ? ((s < 4) ? m.c0.x : m.c1.x)
                   : (s & 3) == 1 ? ((s < 4) ? m.c0.y : m.c1.y)
                   : (s & 3) == 2 ? ((s < 4) ? m.c0.z : m.c1.z)
                                  : ((s < 4) ? m.c0.w : m.c1.w);
  const float sc = e8m0_to_f32(s < 4 ? m.s0 : m.s1);
  const bf16x2 p0 = mxfp4_pair_bf16<0>(w, sc), p1 = mxfp4_pair_bf16<1>(w, sc);
  const bf16x2 p2 = mxfp4_pair_bf16<2>(w, sc), p3 = mxfp4_pair_bf16<3>(w, sc);
  v8bf v;
  v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
  v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
  return v;
}

// B operand of step s: 8 activations of token column j from the staged chunk.
__device__ __forceinline__ v8bf mt_frag_b(const uint8_t* rows, int s, int g, int j) {
  const uint4 u = *reinterpret_cast<const uint4*>(rows + j * MT_PITCH + (64 * g + 8 * s) * 2);
  return __builtin_bit_cast(v8bf, u);
}

// Staging of token rows: thread (row tid/16, part tid%16) moves 16 bf16 of
// its token's 256-element chunk.  Rows past the expert's tokens are zero.
__device__ __forceinline__ void mt_stage_load(uint4& u0, uint4& u1, const uint16_t* src_row, bool valid, int kc,
                                              int part) {
  const uint4* p = reinterpret_cast<const uint4*>(src_row + kc * MT_KC + 16 * part);
  const uint4 a = p[0], b = p[1];
  const uint32_t m = valid ? 0xFFFFFFFFu : 0u;   // word masks: no vector selects (they go through scratch)
  u0 = make_uint4(a.x & m, a.y & m, a.z & m, a.w & m);
  u1 = make_uint4(b.x & m, b.y & m, b.z & m, b.w & m);
}
__device__ __forceinline__ void mt_stage_store(uint8_t* rows, int row, int part, uint4 u0, uint4 u1) {
  uint4* d = reinterpret_cast<uint4*>(rows + row * MT_PITCH + 32 * part);
  d[0] = u0;
  d[1] = u1;
}

// Workgroup -> (slot, column).  Workgroups are handed to the chip's 8 XCDs
// in turn by their linear index, and each XCD has its own L2: with the grid
// laid out so that linear index L goes to XCD L mod 8 and an XCD's k-th
// workgroup takes column k mod C of slot 8 (k / C) + XCD, every column of a
// slot runs on one XCD and the slot's activations are fetched into one L2
// instead of up to eight.  The grid is 1-D, C x (slots rounded up to 8).
constexpr int kXcds = 8;
__device__ __forceinline__ int mt_slots(const ForwardArgs& a) { return max_slots(a.M, a.k, a.E) - 1 + a.has_shared; }
__device__ __forceinline__ void mt_tile(int cols, int& slot, int& col) {
  const int L = (int)blockIdx.x, xcd = L % kXcds, k = L / kXcds;
  slot = (k / cols) * kXcds + xcd;
  col = k % cols;
}

// ------------------------------------------------------------- gate/up --
// Workgroup (64 intermediate indices, slot): wave w takes indices
// j0 + 16w .. + 15 as a gate tile and an up tile over the expert's tokens, so
// h = SiLU(g) * u is formed in registers.
__global__ __launch_bounds__(MT_WAVES * kWave) void gateup_mt_kernel(ForwardArgs a) {
  SlotRec rec;
  int slot, col;
  mt_tile(a.I / MT_GU_J, slot, col);
  if (slot >= mt_slots(a) || !mt_slot(a, slot, rec)) return;  // uniform over the workgroup
  __shared__ MtStage st;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int g = lane >> 4, j = lane & 15;
  const int jw = col * MT_GU_J + 16 * wave;
  const int H = a.H, I = a.I;
  const int64_t grow = (int64_t)rec.e * 2 * I + jw + j;      // this lane's gate row; up row is + I
  const uint8_t* gq = a.w13_q + grow * (H / 2);
  const uint8_t* gs = a.w13_s + grow * (H / 32);
  const uint8_t* uq = gq + (int64_t)I * (H / 2);
  const uint8_t* us = gs + (int64_t)I * (H / 32);
  const int srow = threadIdx.x >> 4, part = threadIdx.x & 15;
  int stok = 0;
  float sw;
  const bool sv = srow < rec.n;
  if (sv) mt_token(a, rec, srow, stok, sw);
  const uint16_t* xsrc = a.x + (int64_t)stok * H;
  const int nk = H / MT_KC;
  uint4 x0, x1;
  mt_stage_load(x0, x1, xsrc, sv, 0, part);
  mt_stage_store(st.rows[0], srow, part, x0, x1);
  MtRowChunk wg = mt_load_row(gq, gs, 0, g), wu = mt_load_row(uq, us, 0, g);
  v4f accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int cur = kc & 1;
    const bool more = kc + 1 < nk;
    MtRowChunk ng = wg, nu = wu;
    if (more) {                                  // next chunk in flight during this one's products
      mt_stage_load(x0, x1, xsrc, sv, kc + 1, part);
      ng = mt_load_row(gq, gs, kc + 1, g);
      nu = mt_load_row(uq, us, kc + 1, g);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const v8bf b = mt_frag_b(st.rows[cur], s, g, j);
      accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mt_frag_a(wg, s), b, accg, 0, 0, 0);
      accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mt_frag_a(wu, s), b, accu, 0, 0, 0);
    }
    if (more) mt_stage_store(st.rows[cur ^ 1], srow, part, x0, x1);
    block_barrier_lds();                         // the next chunk's weights stay in flight
    wg = ng;
    wu = nu;
  }
  // lane (g, j): indices jw + 4g + r of token j
  if (j < rec.n) {   // h = hi + lo, two bf16 terms (W4A8: the MXFP8 round trip reads both)
    uint32_t hb[4], lb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = silu(accg[r]) * accu[r];
      hb[r] = f32_to_bf16_bits(v);
      lb[r] = f32_to_bf16_bits(v - bf16_bits_to_f32(hb[r]));
    }
    const int64_t o = ((int64_t)rec.hrow0 + j) * I + jw + 4 * g;
    *reinterpret_cast<uint2*>(a.h + o) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
    *reinterpret_cast<uint2*>(a.hlo + o) = make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
  }
}

// ---------------------------------------------------------------- down --
// Workgroup (128 output rows, slot): wave w takes rows r0 + 32w .. + 31 as two
// 16-row tiles over the expert's tokens; y[t][r] += w_t * (h_t . Wd[r]).
// h = hi + lo (two bf16 terms, each staged and multiplied); W4A8 layers carry
// their MXFP8 h in hi alone.
__global__ __launch_bounds__(MT_WAVES * kWave) void down_mt_kernel(ForwardArgs a) {
  SlotRec rec;
  int slot, col;
  mt_tile(a.H / MT_DN_R, slot, col);
  if (slot >= mt_slots(a) || !mt_slot(a, slot, rec)) return;
  __shared__ MtStage st, stl;
  const bool two = !a.act8;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int g = lane >> 4, j = lane & 15;
  const int rw = col * MT_DN_R + 32 * wave;
  const int H = a.H, I = a.I;
  const int64_t row0 = (int64_t)rec.e * H + rw + j;           // tile 0 row; tile 1 is + 16
  const uint8_t* q0 = a.w2_q + row0 * (I / 2);
  const uint8_t* s0 = a.w2_s + row0 * (I / 32);
  const uint8_t* q1 = q0 + 16 * (I / 2);
  const uint8_t* s1 = s0 + 16 * (I / 32);
  const int srow = threadIdx.x >> 4, part = threadIdx.x & 15;
  const bool sv = srow < rec.n;
  const uint16_t* hsrc = a.h + ((int64_t)rec.hrow0 + (sv ? srow : 0)) * I;
  const uint16_t* lsrc = a.hlo + ((int64_t)rec.hrow0 + (sv ? srow : 0)) * I;
  const int nk = I / MT_KC;
  uint4 x0, x1, l0 = make_uint4(0, 0, 0, 0), l1 = l0;
  mt_stage_load(x0, x1, hsrc, sv, 0, part);
  if (two) mt_stage_load(l0, l1, lsrc, sv, 0, part);
  mt_stage_store(st.rows[0], srow, part, x0, x1);
  if (two) mt_stage_store(stl.rows[0], srow, part, l0, l1);
  MtRowChunk w0 = mt_load_row(q0, s0, 0, g), w1 = mt_load_row(q1, s1, 0, g);
  v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int cur = kc & 1;
    const bool more = kc + 1 < nk;
    MtRowChunk n0 = w0, n1 = w1;
    if (more) {
      mt_stage_load(x0, x1, hsrc, sv, kc + 1, part);
      if (two) mt_stage_load(l0, l1, lsrc, sv, kc + 1, part);
      n0 = mt_load_row(q0, s0, kc + 1, g);
      n1 = mt_load_row(q1, s1, kc + 1, g);
    }
    if (two) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const v8bf b = mt_frag_b(st.rows[cur], s, g, j);
        const v8bf bl = mt_frag_b(stl.rows[cur], s, g, j);
        const v8bf a0 = mt_frag_a(w0, s), a1 = mt_frag_a(w1, s);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bl, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bl, acc1, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const v8bf b = mt_frag_b(st.rows[cur], s, g, j);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mt_frag_a(w0, s), b, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mt_frag_a(w1, s), b, acc1, 0, 0, 0);
      }
    }
    if (more) {
      mt_stage_store(st.rows[cur ^ 1], srow, part, x0, x1);
      if (two) mt_stage_store(stl.rows[cur ^ 1], srow, part, l0, l1);
    }
    block_barrier_lds();
    w0 = n0;
    w1 = n1;
  }
  if (j < rec.n) {
    int t;
    float w;
    mt_token(a, rec, j, t, w);
    if (a.yp) {
      float* yr = a.yp + ((int64_t)rec.hrow0 + j) * H + rw + 4 * g;
      *reinterpret_cast<float4*>(yr) = make_float4(w * acc0[0], w * acc0[1], w * acc0[2], w * acc0[3]);
      *reinterpret_cast<float4*>(yr + 16) = make_float4(w * acc1[0], w * acc1[1], w * acc1[2], w * acc1[3]);
    } else {
      float* yr = a.y + (int64_t)t * H + rw + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        unsafeAtomicAdd(yr + r, w * acc0[r]);
        unsafeAtomicAdd(yr + 16 + r, w * acc1[r]);
      }
    }
  }
}

hipError_t launch_gateup_mt(const ForwardArgs& a, hipStream_t s) {
  const int slots = max_slots(a.M, a.k, a.E) - 1 + (a.has_shared ? 1 : 0);
  const int slots8 = (slots + kXcds - 1) / kXcds * kXcds;
  gateup_mt_kernel<<<dim3((a.I / MT_GU_J) * slots8), dim3(MT_WAVES * kWave), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_mt(const ForwardArgs& a, hipStream_t s) {
  const int slots = max_slots(a.M, a.k, a.E) - 1 + (a.has_shared ? 1 : 0);
  const int slots8 = (slots + kXcds - 1) / kXcds * kXcds;
  down_mt_kernel<<<dim3((a.H / MT_DN_R) * slots8), dim3(MT_WAVES * kWave), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
