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
constexpr int MT_GU_WAVES = 8;             // gate/up workgroup: the staged x rows serve 8 waves
constexpr int MT_DN_WAVES = 8;             // down workgroup: the staged h rows serve 8 waves
constexpr int MT_GU_J = 16 * MT_GU_WAVES;  // intermediate indices per gate/up workgroup
constexpr int MT_DN_R = 32 * MT_DN_WAVES;  // output rows per down workgroup

struct MtStage {
  __align__(16) uint8_t rows[2][MT_TOK * MT_PITCH];
};

// Token number c (sorted order) of the expert: its row of x and routing
// weight.  Branch-free (c is clamped to the expert's tokens, and the shared
// expert, pbeg < 0, takes token c with weight 1), so the loads are not waited
// for where they are issued.
__device__ __forceinline__ void mt_token(const ForwardArgs& a, const SlotRec& r, int c, int& t, float& w) {
  const int cc = min(c, r.n - 1);
  const int pair0 = a.sorted_pairs[max(r.pbeg, 0) + cc];   // in bounds: cc < M <= M*k for the shared expert
  const int pair = r.pbeg >= 0 ? pair0 : 0;                 // its value is only trusted for routed experts
  const float pw = a.topk_weights[pair];
  t = r.pbeg >= 0 ? pair / a.k : cc;
  w = r.pbeg >= 0 ? pw : 1.f;
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

// Weight codes of one row for chunk kc: the 32 code bytes of lane group g.
struct MtRowChunk {
  uint4 c0, c1;
};
__device__ __forceinline__ MtRowChunk mt_load_row(const uint8_t* row_q, int kc, int g) {
  MtRowChunk m;
  const uint4* q = reinterpret_cast<const uint4*>(row_q + kc * (MT_KC / 2) + 32 * g);
  m.c0 = q[0];
  m.c1 = q[1];
  return m;
}

// The scales of a workgroup's weight rows sit in LDS for the whole kernel:
// a scale read per chunk and row from global memory costs a load instruction
// as dear as a code load (16 rows, one cache line each) for an eighth of the
// bytes.  The rows are two runs of consecutive rows (16-byte aligned, each a
// whole number of 16-byte words: half16 of them at src0, n16 - half16 at
// src1), copied as they are; four words per thread are in flight at once.
// Loads use clamped indices and stores past the end go to a spare word at
// dst[n16], so no load is moved into a branch and waited on there.
__device__ __forceinline__ int mt_scale_pitch(int K) { return K / 32; }
__device__ __forceinline__ void mt_stage_scales(uint8_t* dst, const uint8_t* src0, const uint8_t* src1, int half16,
                                                int n16) {
  const uint4* s0 = reinterpret_cast<const uint4*>(src0);
  const uint4* s1 = reinterpret_cast<const uint4*>(src1) - half16;
  uint4* d = reinterpret_cast<uint4*>(dst);
  for (int b = 0; b < n16; b += 4 * (int)blockDim.x) {
    uint4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = min(b + q * (int)blockDim.x + (int)threadIdx.x, n16 - 1);
      v[q] = (i < half16 ? s0 : s1)[i];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) d[min(b + q * (int)blockDim.x + (int)threadIdx.x, n16)] = v[q];
  }
}
// The two scale bytes of lane group g for chunk kc of a staged row (blocks
// 8 kc + 2g and 8 kc + 2g + 1).
__device__ __forceinline__ uint32_t mt_scales(const uint8_t* row_lds, int kc, int g) {
  return *reinterpret_cast<const uint16_t*>(row_lds + kc * (MT_KC / 32) + 2 * g);
}

// A operand of step s: the 8 weights of code word s, decoded to bf16 with
// the block scale (low byte of s01 for steps 0-3, high byte for 4-7).
__device__ __forceinline__ v8bf mt_frag_a(const MtRowChunk& m, uint32_t s01, int s) {
  const uint32_t w = (s & 3) == 0 ? ((s < 4) ? m.c0.x : m.c1.x)
                   : (s & 3) == 1 ? ((s < 4) ? m.c0.y : m.c1.y)
                   : (s & 3) == 2 ? ((s < 4) ? m.c0.z : m.c1.z)
                                  : ((s < 4) ? m.c0.w : m.c1.w);
  const float sc = e8m0_to_f32(s < 4 ? (s01 & 0xFFu) : (s01 >> 8));
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

// Staging of token rows: thread (row tid / 32, part tid % 32) moves 8 bf16
// (16 bytes) of its token's 256-element chunk.  Rows past the expert's tokens
// repeat a valid row: token column j of a product only reaches output column
// j, and those columns are never stored.
__device__ __forceinline__ void mt_stage_load1(uint4& u, const uint16_t* src_row, int kc, int part) {
  u = *reinterpret_cast<const uint4*>(src_row + kc * MT_KC + 8 * part);
}
__device__ __forceinline__ void mt_stage_store1(uint8_t* rows, int row, int part, uint4 u) {
  *reinterpret_cast<uint4*>(rows + row * MT_PITCH + 16 * part) = u;
}

// Products of one staged chunk with a wave's gate and up tiles (scale words
// sg, su of the lane's gate and up rows).
__device__ __forceinline__ void mt_gu_products(v4f& accg, v4f& accu, const MtRowChunk& wg, const MtRowChunk& wu,
                                               uint32_t sg, uint32_t su, const uint8_t* rows, int g, int j) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const v8bf b = mt_frag_b(rows, s, g, j);
    accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mt_frag_a(wg, sg, s), b, accg, 0, 0, 0);
    accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mt_frag_a(wu, su, s), b, accu, 0, 0, 0);
  }
}

// Products of one staged chunk of h with a wave's two down tiles: the hi
// term, and with `two` the lo term too (h = hi + lo).
__device__ __forceinline__ void mt_down_products(v4f& acc0, v4f& acc1, const MtRowChunk& w0, const MtRowChunk& w1,
                                                 uint32_t s0, uint32_t s1, const uint8_t* rows,
                                                 const uint8_t* rows_lo, bool two, int g, int j) {
  if (two) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const v8bf b = mt_frag_b(rows, s, g, j);
      const v8bf bl = mt_frag_b(rows_lo, s, g, j);
      const v8bf a0 = mt_frag_a(w0, s0, s), a1 = mt_frag_a(w1, s1, s);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bl, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bl, acc1, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const v8bf b = mt_frag_b(rows, s, g, j);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mt_frag_a(w0, s0, s), b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mt_frag_a(w1, s1, s), b, acc1, 0, 0, 0);
    }
  }
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
// Workgroup (MT_GU_J = 128 intermediate indices, slot): wave w takes indices
// j0 + 16w .. + 15 as a gate tile and an up tile over the expert's tokens, so
// h = SiLU(g) * u is formed in registers.
__global__ __launch_bounds__(MT_GU_WAVES * kWave) void gateup_mt_kernel(ForwardArgs a) {
  SlotRec rec;
  int slot, col;
  mt_tile(a.I / MT_GU_J, slot, col);
  if (slot >= mt_slots(a) || !mt_slot(a, slot, rec)) return;  // uniform over the workgroup
  __shared__ MtStage st;
  extern __shared__ __align__(16) uint8_t mt_scale_lds[];     // the gate rows, then the up rows
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int g = lane >> 4, j = lane & 15;
  const int jw = col * MT_GU_J + 16 * wave;
  const int H = a.H, I = a.I;
  const int64_t grow0 = (int64_t)rec.e * 2 * I + col * MT_GU_J;   // the workgroup's first gate row
  const int64_t grow = grow0 + 16 * wave + j;                     // this lane's gate row; up row is + I
  const uint8_t* gq = a.w13_q + grow * (H / 2);
  const uint8_t* uq = gq + (int64_t)I * (H / 2);
  const int sp = mt_scale_pitch(H);
  const uint8_t* gsl = mt_scale_lds + (16 * wave + j) * sp;
  const uint8_t* usl = gsl + MT_GU_J * sp;
  const int srow = threadIdx.x >> 5, part = threadIdx.x & 31;   // 16 rows x 32 parts of 16 bytes
  // prologue: the token lookup, the first chunk's weights and the scales
  // are all requested before any of them is waited for
  int stok;
  float sw;
  mt_token(a, rec, srow, stok, sw);   // rows past the expert's tokens repeat its last one
  MtRowChunk ga = mt_load_row(gq, 0, g), ua = mt_load_row(uq, 0, g), gb, ub;
  const uint16_t* xsrc = a.x + (int64_t)stok * H;
  const int nk = H / MT_KC;
  uint4 x0;
  mt_stage_load1(x0, xsrc, 0, part);
  mt_stage_scales(mt_scale_lds, a.w13_s + grow0 * (H / 32), a.w13_s + (grow0 + I) * (H / 32), MT_GU_J * sp / 16,
                  2 * MT_GU_J * sp / 16);
  mt_stage_store1(st.rows[0], srow, part, x0);
  v4f accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  // Chunks alternate between register sets (a, b) and LDS buffers (0, 1): the
  // next chunk's loads land in the idle set while this chunk is multiplied.
  // The steady-state loop issues its loads unconditionally (a load under a
  // branch would make every later wait cover it too), and a scheduling fence
  // keeps the products after them; the last one or two chunks are done after
  // the loop.
  int kc = 0;
  for (; kc + 2 < nk; kc += 2) {
    mt_stage_load1(x0, xsrc, kc + 1, part);
    gb = mt_load_row(gq, kc + 1, g);
    ub = mt_load_row(uq, kc + 1, g);
    __builtin_amdgcn_sched_barrier(0);
    mt_gu_products(accg, accu, ga, ua, mt_scales(gsl, kc, g), mt_scales(usl, kc, g), st.rows[0], g, j);
    mt_stage_store1(st.rows[1], srow, part, x0);
    block_barrier_lds();
    mt_stage_load1(x0, xsrc, kc + 2, part);
    ga = mt_load_row(gq, kc + 2, g);
    ua = mt_load_row(uq, kc + 2, g);
    __builtin_amdgcn_sched_barrier(0);
    mt_gu_products(accg, accu, gb, ub, mt_scales(gsl, kc + 1, g), mt_scales(usl, kc + 1, g), st.rows[1], g, j);
    mt_stage_store1(st.rows[0], srow, part, x0);
    block_barrier_lds();
  }
  if (kc + 1 < nk) {
    mt_stage_load1(x0, xsrc, kc + 1, part);
    gb = mt_load_row(gq, kc + 1, g);
    ub = mt_load_row(uq, kc + 1, g);
    mt_gu_products(accg, accu, ga, ua, mt_scales(gsl, kc, g), mt_scales(usl, kc, g), st.rows[0], g, j);
    mt_stage_store1(st.rows[1], srow, part, x0);
    block_barrier_lds();
    mt_gu_products(accg, accu, gb, ub, mt_scales(gsl, kc + 1, g), mt_scales(usl, kc + 1, g), st.rows[1], g, j);
  } else {
    mt_gu_products(accg, accu, ga, ua, mt_scales(gsl, kc, g), mt_scales(usl, kc, g), st.rows[0], g, j);
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
// Workgroup (MT_DN_R = 256 output rows, slot): wave w takes rows r0 + 32w ..
// + 31 as two 16-row tiles over the expert's tokens; y[t][r] += w_t * (h_t . Wd[r]).
// h = hi + lo (two bf16 terms, each staged and multiplied); W4A8 layers carry
// their MXFP8 h in hi alone.
__global__ __launch_bounds__(MT_DN_WAVES * kWave) void down_mt_kernel(ForwardArgs a) {
  SlotRec rec;
  int slot, col;
  mt_tile(a.H / MT_DN_R, slot, col);
  if (slot >= mt_slots(a) || !mt_slot(a, slot, rec)) return;
  __shared__ MtStage st, stl;
  extern __shared__ __align__(16) uint8_t mt_scale_lds[];     // the workgroup's rows
  const bool two = !a.act8;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int g = lane >> 4, j = lane & 15;
  const int rw = col * MT_DN_R + 32 * wave;
  const int H = a.H, I = a.I;
  const int64_t wrow0 = (int64_t)rec.e * H + col * MT_DN_R;       // the workgroup's first row
  const int64_t row0 = (int64_t)rec.e * H + rw + j;               // tile 0 row; tile 1 is + 16
  const uint8_t* q0 = a.w2_q + row0 * (I / 2);
  const uint8_t* q1 = q0 + 16 * (I / 2);
  const int sp = mt_scale_pitch(I);
  const uint8_t* s0l = mt_scale_lds + (32 * wave + j) * sp;
  const uint8_t* s1l = s0l + 16 * sp;
  const int srow = threadIdx.x >> 5, part = threadIdx.x & 31;   // 16 rows x 32 parts of 16 bytes
  const bool sv = srow < rec.n;
  const uint16_t* hsrc = a.h + ((int64_t)rec.hrow0 + (sv ? srow : 0)) * I;
  const uint16_t* lsrc = a.hlo + ((int64_t)rec.hrow0 + (sv ? srow : 0)) * I;
  const int nk = I / MT_KC;
  const uint4 z = make_uint4(0, 0, 0, 0);
  // prologue: the first chunk's weights and h rows, then the scales
  uint4 x0, l0 = z;
  MtRowChunk a0 = mt_load_row(q0, 0, g), a1 = mt_load_row(q1, 0, g), b0, b1;
  mt_stage_load1(x0, hsrc, 0, part);
  if (two) mt_stage_load1(l0, lsrc, 0, part);
  const uint8_t* ssrc = a.w2_s + wrow0 * (I / 32);
  mt_stage_scales(mt_scale_lds, ssrc, ssrc, MT_DN_R * sp / 16, MT_DN_R * sp / 16);
  mt_stage_store1(st.rows[0], srow, part, x0);
  if (two) mt_stage_store1(stl.rows[0], srow, part, l0);
  v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  // the same alternation as gate/up
  int kc = 0;
  for (; kc + 2 < nk; kc += 2) {
    mt_stage_load1(x0, hsrc, kc + 1, part);
    if (two) mt_stage_load1(l0, lsrc, kc + 1, part);
    b0 = mt_load_row(q0, kc + 1, g);
    b1 = mt_load_row(q1, kc + 1, g);
    __builtin_amdgcn_sched_barrier(0);
    mt_down_products(acc0, acc1, a0, a1, mt_scales(s0l, kc, g), mt_scales(s1l, kc, g), st.rows[0], stl.rows[0], two,
                     g, j);
    mt_stage_store1(st.rows[1], srow, part, x0);
    if (two) mt_stage_store1(stl.rows[1], srow, part, l0);
    block_barrier_lds();
    mt_stage_load1(x0, hsrc, kc + 2, part);
    if (two) mt_stage_load1(l0, lsrc, kc + 2, part);
    a0 = mt_load_row(q0, kc + 2, g);
    a1 = mt_load_row(q1, kc + 2, g);
    __builtin_amdgcn_sched_barrier(0);
    mt_down_products(acc0, acc1, b0, b1, mt_scales(s0l, kc + 1, g), mt_scales(s1l, kc + 1, g), st.rows[1],
                     stl.rows[1], two, g, j);
    mt_stage_store1(st.rows[0], srow, part, x0);
    if (two) mt_stage_store1(stl.rows[0], srow, part, l0);
    block_barrier_lds();
  }
  if (kc + 1 < nk) {
    mt_stage_load1(x0, hsrc, kc + 1, part);
    if (two) mt_stage_load1(l0, lsrc, kc + 1, part);
    b0 = mt_load_row(q0, kc + 1, g);
    b1 = mt_load_row(q1, kc + 1, g);
    mt_down_products(acc0, acc1, a0, a1, mt_scales(s0l, kc, g), mt_scales(s1l, kc, g), st.rows[0], stl.rows[0], two,
                     g, j);
    mt_stage_store1(st.rows[1], srow, part, x0);
    if (two) mt_stage_store1(stl.rows[1], srow, part, l0);
    block_barrier_lds();
    mt_down_products(acc0, acc1, b0, b1, mt_scales(s0l, kc + 1, g), mt_scales(s1l, kc + 1, g), st.rows[1],
                     stl.rows[1], two, g, j);
  } else {
    mt_down_products(acc0, acc1, a0, a1, mt_scales(s0l, kc, g), mt_scales(s1l, kc, g), st.rows[0], stl.rows[0], two,
                     g, j);
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

// Grid rows for the few-token experts: with the slot list, at most one expert
// per mt_min routed pairs (plus the shared one) can be on this path, so rows
// past that bound are not launched; without it, every slot.
static int mt_grid_slots(const ForwardArgs& a) {
  int routed = max_slots(a.M, a.k, a.E) - 1;
  if (a.lists) routed = std::min(routed, a.M * a.k / a.mt_min);
  const int slots = routed + (a.has_shared ? 1 : 0);
  return (slots + kXcds - 1) / kXcds * kXcds;
}

hipError_t launch_gateup_mt(const ForwardArgs& a, hipStream_t s) {
  const int slots8 = mt_grid_slots(a);
  const size_t shmem = (size_t)2 * MT_GU_J * (a.H / 32) + 16;   // gate and up rows' scales, a spare word
  gateup_mt_kernel<<<dim3((a.I / MT_GU_J) * slots8), dim3(MT_GU_WAVES * kWave), shmem, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_mt(const ForwardArgs& a, hipStream_t s) {
  const int slots8 = mt_grid_slots(a);
  const size_t shmem = (size_t)MT_DN_R * (a.I / 32) + 16;
  down_mt_kernel<<<dim3((a.H / MT_DN_R) * slots8), dim3(MT_DN_WAVES * kWave), shmem, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
