// Wave-level MXFP4 GEMV routines of the expert MLP (the VALU path for experts
// with few tokens).  Every active expert runs once over all of its tokens
// (MoE-SpeQ article, section 4.2) with its MXFP4 weights (digest "3 Ways to
// Improve MoE Inference on NVIDIA DGX Spark", sections 2-3) streamed from HBM
// once and dequantised in registers.
//
// Layout in a wave.  A weight row is cut into 16-element half-chunks (8 code
// bytes, half of a 32-element scale block).  Gate/up rows belong to 32-lane
// groups (lane j takes half-chunks j, j+32, ...: each load instruction reads two
// 256-byte row segments); down rows belong to 16-lane groups (lane j takes j,
// j+16, j+32: four 128-byte segments per instruction).  Loads complete in
// issue order, so a wave first issues the code loads of all of its rows (the
// HBM stream), then the block stages the expert's first activation rows in LDS
// and each wave its rows' scale bytes; partial sums meet across the group
// through DPP and row swaps.  Accumulation is fp32 over exact bf16 products.
#pragma once

#include "kernels.h"

namespace moe {

// Which expert a work item belongs to, and where its tokens come from.
struct ExpertSlot {
  int e;          // expert index in the bank (E = shared)
  int n;          // tokens
  int pbeg;       // first sorted position (routed) or -1 (shared: tokens 0..M-1)
  int hrow0;      // h row of the first token
  int tok[kRecTokens];
  float w[kRecTokens];
};

// From the slot record when there is one (a single 64-byte load), else from
// the sort outputs.
// Experts with at least a.mfma_min tokens belong to the MFMA kernels, those
// with a.mt_min..a.mt_max tokens to the few-token matrix-core kernels.
__device__ __forceinline__ bool resolve_slot(int slot, const ForwardArgs& a, ExpertSlot& s) {
  if (a.rec) {
    const SlotRec r = a.rec[slot];
    s.e = r.e; s.n = r.n; s.pbeg = r.pbeg; s.hrow0 = r.hrow0;
#pragma unroll
    for (int q = 0; q < kRecTokens; ++q) { s.tok[q] = r.tok[q]; s.w[q] = r.w[q]; }
    return r.e >= 0 && r.n < a.mfma_min && !(r.n >= a.mt_min && r.n <= a.mt_max);
  }
  const int n_act = *a.num_active;
  if (slot < n_act) {
    s.e = a.active[slot];
    s.pbeg = a.offsets[s.e];
    s.n = a.offsets[s.e + 1] - s.pbeg;
    s.hrow0 = s.pbeg;
  } else if (slot == n_act && a.has_shared) {
    s.e = a.E;
    s.pbeg = -1;
    s.n = a.M;
    s.hrow0 = a.M * a.k;
  } else {
    return false;
  }
#pragma unroll
  for (int q = 0; q < kRecTokens; ++q) {
    if (q < s.n && s.pbeg >= 0) {
      const int pair = a.sorted_pairs[s.pbeg + q];
      s.tok[q] = pair / a.k;
      s.w[q] = a.topk_weights[pair];
    } else {
      s.tok[q] = q;
      s.w[q] = 1.f;
    }
  }
  return true;
}

// s.tok[i] / s.w[i] for a runtime i < kRecTokens without indexing into the
// arrays (a dynamic index would move them to scratch memory).
__device__ __forceinline__ int rec_tok(const ExpertSlot& s, int i) {
  int t = s.tok[0];
#pragma unroll
  for (int q = 1; q < kRecTokens; ++q) t = (i == q) ? s.tok[q] : t;
  return t;
}
__device__ __forceinline__ float rec_w(const ExpertSlot& s, int i) {
  float w = s.w[0];
#pragma unroll
  for (int q = 1; q < kRecTokens; ++q) w = (i == q) ? s.w[q] : w;
  return w;
}

// Token row, routing weight and h row of the i-th token of an expert.
__device__ __forceinline__ void token_of(const ForwardArgs& a, const ExpertSlot& s, int i, int& t,
                                         float& wgt, int& hrow) {
  hrow = s.hrow0 + i;
  if (i < kRecTokens) {
    t = rec_tok(s, i);
    wgt = rec_w(s, i);
  } else if (s.pbeg >= 0) {
    const int pair = a.sorted_pairs[s.pbeg + i];
    t = pair / a.k;
    wgt = a.topk_weights[pair];
  } else {
    t = i;
    wgt = 1.f;
  }
}

// This lane's index, opaque to the optimiser: the per-lane offsets derived
// from it are then computed where they are used, not hoisted out of a caller's
// loop over experts into registers held across the whole loop.
__device__ __forceinline__ int opaque_lane() {
  int lane = threadIdx.x & (kWave - 1);
  asm volatile("" : "+v"(lane));
  return lane;
}

// Copy `nbytes` contiguous bytes from global to this wave's LDS slice.
__device__ __forceinline__ void wave_stage_bytes(const uint8_t* __restrict__ src, uint8_t* dst,
                                                 int nbytes, int lane) {
  if (((uintptr_t)src & 15u) == 0 && (nbytes & 15) == 0) {
    for (int o = lane * 16; o < nbytes; o += kWave * 16)
      *reinterpret_cast<uint4*>(dst + o) = *reinterpret_cast<const uint4*>(src + o);
  } else {
    for (int o = lane; o < nbytes; o += kWave) dst[o] = src[o];
  }
  __builtin_amdgcn_wave_barrier();
}

// Makes `v` opaque to the optimiser at this point, so values derived from it
// (the dequantised weights) are recomputed per token rather than hoisted out of
// the token loop into hundreds of live registers.  Emits no instruction.
__device__ __forceinline__ void keep_in_loop(uint2& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y));
}

__device__ __forceinline__ void unpack8(const uint4& v, uint32_t* a) {
  a[0] = v.x; a[1] = v.y; a[2] = v.z; a[3] = v.w;
}


// Activations of one token for one lane: half-chunk hc = 16 bf16 = two uint4.
__device__ __forceinline__ void act_from(const uint4* row, int hc, uint32_t* a8) {
  unpack8(row[2 * hc], a8);
  unpack8(row[2 * hc + 1], a8 + 4);
}

// --------------------------------------------------------------- gate/up --
// Short rows (H <= 32 * HC * 16): one wave computes h for 2*NP consecutive row
// pairs [jp0, jp0 + 2*NP) of expert s; lane group g = lane/32 takes pairs
// jp0 + g + 2p.  Waves are independent (no block barrier).  Loads complete in
// issue order, so a wave issues, in this order: the first token's activations
// (L2), its rows' scale bytes, then the weight codes chunk by chunk in the order
// the math consumes them -- each chunk is computed as soon as it has landed.
// XL: the tokens' activations come from LDS (xl = bf16 [M][H], staged by the
// caller), read chunk by chunk as the products need them, so they hold no
// registers while the weight codes are in flight.
template <int NP, int HC, bool XL = false>
__device__ __forceinline__ void gateup_short(const ForwardArgs& a, const ExpertSlot& s, int jp0,
                                             uint8_t* s_lds, const uint16_t* xl = nullptr) {
  const int lane = opaque_lane();
  const int grp = lane >> 5, j32 = lane & 31;
  const int H = a.H, I = a.I;
  const int KH = H / 16;
  const int row_q = H / 2, row_s = H / 32;
  const uint8_t* wq = a.w13_q + (size_t)s.e * 2 * I * row_q;
  const uint8_t* ws = a.w13_s + (size_t)s.e * 2 * I * row_s;
  const int npairs = 2 * NP;
  int hcc[HC];                                     // clamped: lanes past the row end get scale 0
#pragma unroll
  for (int i = 0; i < HC; ++i) hcc[i] = min(j32 + 32 * i, KH - 1);

  uint4 xv[HC][2];
  if constexpr (!XL) {
    const uint4* xr = reinterpret_cast<const uint4*>(a.x + (size_t)s.tok[0] * H);
#pragma unroll
    for (int i = 0; i < HC; ++i) { xv[i][0] = xr[2 * hcc[i]]; xv[i][1] = xr[2 * hcc[i] + 1]; }
  }
  const int sbytes = npairs * row_s;             // each of the gate and up row groups
  const bool svec = (sbytes & 15) == 0 && sbytes <= 8 * kWave;
  uint4 sraw = make_uint4(0, 0, 0, 0);
  if (svec) {
    const int nv = sbytes / 16;                  // lanes [0, nv): gate, [nv, 2nv): up
    const int l = min(lane, 2 * nv - 1);
    const uint8_t* src = (l < nv) ? ws + (size_t)jp0 * row_s : ws + (size_t)(I + jp0) * row_s - sbytes;
    sraw = reinterpret_cast<const uint4*>(src)[l];
  }
  uint2 cg[NP][HC], cu[NP][HC];
#pragma unroll
  for (int i = 0; i < HC; ++i)
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int jp = jp0 + 2 * p + grp;
      cg[p][i] = *reinterpret_cast<const uint2*>(wq + (size_t)jp * row_q + hcc[i] * 8);
      cu[p][i] = *reinterpret_cast<const uint2*>(wq + (size_t)(I + jp) * row_q + hcc[i] * 8);
    }
  if (svec) {
    if (lane * 16 < 2 * sbytes) *reinterpret_cast<uint4*>(s_lds + lane * 16) = sraw;
  } else {
    for (int o = lane; o < sbytes; o += kWave) {
      s_lds[o] = ws[(size_t)jp0 * row_s + o];
      s_lds[sbytes + o] = ws[(size_t)(I + jp0) * row_s + o];
    }
  }
  __builtin_amdgcn_wave_barrier();
  float sg[NP][HC], su[NP][HC];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = 2 * p + grp;
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      const bool ok = j32 + 32 * i < KH;
      sg[p][i] = ok ? e8m0_to_f32(s_lds[r * row_s + (hcc[i] >> 1)]) : 0.f;
      su[p][i] = ok ? e8m0_to_f32(s_lds[sbytes + r * row_s + (hcc[i] >> 1)]) : 0.f;
    }
  }
  for (int q = 0; q < s.n; ++q) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int i = 0; i < HC; ++i) { keep_in_loop(cg[p][i]); keep_in_loop(cu[p][i]); }
    int t, hrow; float wgt;
    token_of(a, s, q, t, wgt, hrow);
    if (!XL && q > 0) {                            // later tokens' activations (L2)
      const uint4* xr = reinterpret_cast<const uint4*>(a.x + (size_t)t * H);
#pragma unroll
      for (int i = 0; i < HC; ++i) { xv[i][0] = xr[2 * hcc[i]]; xv[i][1] = xr[2 * hcc[i] + 1]; }
    }
    const uint4* xlr = reinterpret_cast<const uint4*>(xl + (size_t)t * H);
    float accg[NP], accu[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) { accg[p] = 0.f; accu[p] = 0.f; }
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      uint32_t xa[8];
      if constexpr (XL) {
        unpack8(xlr[2 * hcc[i]], xa);
        unpack8(xlr[2 * hcc[i] + 1], xa + 4);
      } else {
        unpack8(xv[i][0], xa);
        unpack8(xv[i][1], xa + 4);
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        accg[p] = dot8_mxfp4_bf16(cg[p][i].x, sg[p][i], xa, accg[p]);
        accg[p] = dot8_mxfp4_bf16(cg[p][i].y, sg[p][i], xa + 4, accg[p]);
        accu[p] = dot8_mxfp4_bf16(cu[p][i].x, su[p][i], xa, accu[p]);
        accu[p] = dot8_mxfp4_bf16(cu[p][i].y, su[p][i], xa + 4, accu[p]);
      }
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float g = group_sum<32>(accg[p]);
      const float u = group_sum<32>(accu[p]);
      if (j32 == 0) {   // h = hi + lo, two bf16 terms (the down kernels, or W4A8's round trip, read both)
        const float v = silu(g) * u;
        const uint32_t hi = f32_to_bf16_bits(v);
        const size_t o = (size_t)hrow * I + jp0 + 2 * p + grp;
        a.h[o] = (uint16_t)hi;
        a.hlo[o] = (uint16_t)f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
      }
    }
  }
}

// Long rows (any H): K passes per token, codes re-read per token (edge shapes).
template <int NP, int HC>
__device__ __forceinline__ void gateup_long(const ForwardArgs& a, const ExpertSlot& s, int jp0,
                                            uint8_t* s_lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const int grp = lane >> 5, j32 = lane & 31;
  const int H = a.H, I = a.I;
  const int KH = H / 16;
  const int row_q = H / 2, row_s = H / 32;
  const uint8_t* wq = a.w13_q + (size_t)s.e * 2 * I * row_q;
  const uint8_t* ws = a.w13_s + (size_t)s.e * 2 * I * row_s;
  const int npairs = 2 * NP;
  wave_stage_bytes(ws + (size_t)jp0 * row_s, s_lds, npairs * row_s, lane);
  wave_stage_bytes(ws + (size_t)(I + jp0) * row_s, s_lds + npairs * row_s, npairs * row_s, lane);
  for (int q = 0; q < s.n; ++q) {
    int t, hrow; float wgt;
    token_of(a, s, q, t, wgt, hrow);
    const uint4* xr = reinterpret_cast<const uint4*>(a.x + (size_t)t * H);
    float accg[NP], accu[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) { accg[p] = 0.f; accu[p] = 0.f; }
    for (int kb = 0; kb < KH; kb += 32 * HC) {
#pragma unroll
      for (int i = 0; i < HC; ++i) {
        const int hc = kb + j32 + 32 * i;
        if (hc < KH) {
          uint32_t xa[8];
          act_from(xr, hc, xa);
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const int r = 2 * p + grp;
            const int jp = jp0 + r;
            const uint2 g2 = *reinterpret_cast<const uint2*>(wq + (size_t)jp * row_q + hc * 8);
            const uint2 u2 = *reinterpret_cast<const uint2*>(wq + (size_t)(I + jp) * row_q + hc * 8);
            const float sgv = e8m0_to_f32(s_lds[r * row_s + (hc >> 1)]);
            const float suv = e8m0_to_f32(s_lds[(npairs + r) * row_s + (hc >> 1)]);
            accg[p] = dot8_mxfp4_bf16(g2.x, sgv, xa, accg[p]);
            accg[p] = dot8_mxfp4_bf16(g2.y, sgv, xa + 4, accg[p]);
            accu[p] = dot8_mxfp4_bf16(u2.x, suv, xa, accu[p]);
            accu[p] = dot8_mxfp4_bf16(u2.y, suv, xa + 4, accu[p]);
          }
        }
      }
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float g = group_sum<32>(accg[p]);
      const float u = group_sum<32>(accu[p]);
      if (j32 == 0) {   // h = hi + lo, two bf16 terms (the down kernels, or W4A8's round trip, read both)
        const float v = silu(g) * u;
        const uint32_t hi = f32_to_bf16_bits(v);
        const size_t o = (size_t)hrow * I + jp0 + 2 * p + grp;
        a.h[o] = (uint16_t)hi;
        a.hlo[o] = (uint16_t)f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
      }
    }
  }
}

// ------------------------------------------------------------------ down --
// Short rows (I <= 16 * HC * 16): one wave computes rows [r0, r0 + 4*NR) of
// expert s's down projection for all of its tokens (lane group g = lane/16
// takes rows r0 + g + 4q) and adds w * (h . Wd[r]) into y[t][r].  Same issue
// order as gateup_short: first h row, scales, then codes chunk by chunk.
// ROWS: store into the pair's partial row of yp (combine by rows) instead of
// adding into y.
template <int NR, int HC, bool ROWS>
__device__ __forceinline__ void down_short(const ForwardArgs& a, const ExpertSlot& s, int r0,
                                           uint8_t* s_lds) {
  const int lane = opaque_lane();   // recomputed per call: nothing hoisted out of a slot loop
  const int grp = lane >> 4, j16 = lane & 15;
  const int H = a.H, I = a.I;
  const int KH = I / 16;
  const int row_q = I / 2, row_s = I / 32;
  const uint8_t* wq = a.w2_q + (size_t)s.e * H * row_q;
  const uint8_t* ws = a.w2_s + (size_t)s.e * H * row_s;
  const int nrows = 4 * NR;
  int hcc[HC];
#pragma unroll
  for (int i = 0; i < HC; ++i) hcc[i] = min(j16 + 16 * i, KH - 1);

  // h = hi + lo (two bf16 terms); W4A8 layers carry their MXFP8 h in hi alone
  const bool two = !a.act8;
  uint4 hv[HC][2], hl[HC][2];
  {
    const uint4* hr = reinterpret_cast<const uint4*>(a.h + (size_t)s.hrow0 * I);
    const uint4* lr = reinterpret_cast<const uint4*>(a.hlo + (size_t)s.hrow0 * I);
#pragma unroll
    for (int i = 0; i < HC; ++i) { hv[i][0] = hr[2 * hcc[i]]; hv[i][1] = hr[2 * hcc[i] + 1]; }
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      hl[i][0] = two ? lr[2 * hcc[i]] : make_uint4(0, 0, 0, 0);
      hl[i][1] = two ? lr[2 * hcc[i] + 1] : make_uint4(0, 0, 0, 0);
    }
  }
  const int sbytes = nrows * row_s;
  const bool svec = (sbytes & 15) == 0 && sbytes <= 16 * kWave;
  uint4 sraw = make_uint4(0, 0, 0, 0);
  if (svec) sraw = reinterpret_cast<const uint4*>(ws + (size_t)r0 * row_s)[min(lane, sbytes / 16 - 1)];
  uint2 c[NR][HC];
#pragma unroll
  for (int i = 0; i < HC; ++i)
#pragma unroll
    for (int q = 0; q < NR; ++q)
      c[q][i] = *reinterpret_cast<const uint2*>(wq + (size_t)(r0 + 4 * q + grp) * row_q + hcc[i] * 8);
  if (svec) {
    if (lane * 16 < sbytes) *reinterpret_cast<uint4*>(s_lds + lane * 16) = sraw;
  } else {
    for (int o = lane; o < sbytes; o += kWave) s_lds[o] = ws[(size_t)r0 * row_s + o];
  }
  __builtin_amdgcn_wave_barrier();
  float sc[NR][HC];
#pragma unroll
  for (int q = 0; q < NR; ++q)
#pragma unroll
    for (int i = 0; i < HC; ++i)
      sc[q][i] = (j16 + 16 * i < KH) ? e8m0_to_f32(s_lds[(4 * q + grp) * row_s + (hcc[i] >> 1)]) : 0.f;
  for (int m = 0; m < s.n; ++m) {
#pragma unroll
    for (int q = 0; q < NR; ++q)
#pragma unroll
      for (int i = 0; i < HC; ++i) keep_in_loop(c[q][i]);
    int t, hrow; float wgt;
    token_of(a, s, m, t, wgt, hrow);
    if (m > 0) {
      const uint4* hr = reinterpret_cast<const uint4*>(a.h + (size_t)hrow * I);
      const uint4* lr = reinterpret_cast<const uint4*>(a.hlo + (size_t)hrow * I);
#pragma unroll
      for (int i = 0; i < HC; ++i) { hv[i][0] = hr[2 * hcc[i]]; hv[i][1] = hr[2 * hcc[i] + 1]; }
#pragma unroll
      for (int i = 0; i < HC; ++i) {
        hl[i][0] = two ? lr[2 * hcc[i]] : make_uint4(0, 0, 0, 0);
        hl[i][1] = two ? lr[2 * hcc[i] + 1] : make_uint4(0, 0, 0, 0);
      }
    }
    float acc[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) acc[q] = 0.f;
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      uint32_t ha[8], hb[8];
      unpack8(hv[i][0], ha);
      unpack8(hv[i][1], ha + 4);
      unpack8(hl[i][0], hb);
      unpack8(hl[i][1], hb + 4);
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        acc[q] = dot8_mxfp4_bf16_2t(c[q][i].x, sc[q][i], ha, hb, acc[q]);
        acc[q] = dot8_mxfp4_bf16_2t(c[q][i].y, sc[q][i], ha + 4, hb + 4, acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const float v = group_sum<16>(acc[q]);
      if (j16 == 0) {
        if constexpr (ROWS)
          a.yp[(size_t)hrow * H + r0 + 4 * q + grp] = wgt * v;
        else
          unsafeAtomicAdd(&a.y[(size_t)t * H + r0 + 4 * q + grp], wgt * v);
      }
    }
  }
}

// Long rows (any I): K passes per token.
template <int NR, int HC, bool ROWS>
__device__ __forceinline__ void down_long(const ForwardArgs& a, const ExpertSlot& s, int r0,
                                          uint8_t* s_lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const int grp = lane >> 4, j16 = lane & 15;
  const int H = a.H, I = a.I;
  const int KH = I / 16;
  const int row_q = I / 2, row_s = I / 32;
  const uint8_t* wq = a.w2_q + (size_t)s.e * H * row_q;
  const uint8_t* ws = a.w2_s + (size_t)s.e * H * row_s;
  const int nrows = 4 * NR;
  wave_stage_bytes(ws + (size_t)r0 * row_s, s_lds, nrows * row_s, lane);
  for (int m = 0; m < s.n; ++m) {
    int t, hrow; float wgt;
    token_of(a, s, m, t, wgt, hrow);
    const uint4* hr = reinterpret_cast<const uint4*>(a.h + (size_t)hrow * I);
    const uint4* lr = reinterpret_cast<const uint4*>(a.hlo + (size_t)hrow * I);
    float acc[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) acc[q] = 0.f;
    for (int kb = 0; kb < KH; kb += 16 * HC) {
#pragma unroll
      for (int i = 0; i < HC; ++i) {
        const int hc = kb + j16 + 16 * i;
        if (hc < KH) {
          uint32_t ha[8], hb[8] = {0, 0, 0, 0, 0, 0, 0, 0};
          act_from(hr, hc, ha);
          if (!a.act8) act_from(lr, hc, hb);     // h = hi + lo; W4A8: hi alone
#pragma unroll
          for (int q = 0; q < NR; ++q) {
            const int r = 4 * q + grp;
            const uint2 c2 = *reinterpret_cast<const uint2*>(wq + (size_t)(r0 + r) * row_q + hc * 8);
            const float scv = e8m0_to_f32(s_lds[r * row_s + (hc >> 1)]);
            acc[q] = dot8_mxfp4_bf16_2t(c2.x, scv, ha, hb, acc[q]);
            acc[q] = dot8_mxfp4_bf16_2t(c2.y, scv, ha + 4, hb + 4, acc[q]);
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const float v = group_sum<16>(acc[q]);
      if (j16 == 0) {
        if constexpr (ROWS)
          a.yp[(size_t)hrow * H + r0 + 4 * q + grp] = wgt * v;
        else
          unsafeAtomicAdd(&a.y[(size_t)t * H + r0 + 4 * q + grp], wgt * v);
      }
    }
  }
}

}  // namespace moe
