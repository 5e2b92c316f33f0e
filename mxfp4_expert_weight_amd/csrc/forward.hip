// Expert kernels of moe_mxfp4_forward on the VALU GEMV path, plus the dequant
// export.  A block is (row tile, expert slot); slots past the active experts
// (and the shared expert) exit at once -- the grid is sized for the worst case
// because the number of active experts is only known on the device.
//
//   gateup_kernel:  h[p][j] = SiLU(x_t . Wg[j]) * (x_t . Wu[j])   (h = hi + lo,
//                   two bf16 terms)
//   down_kernel:    y[t][r] += w_p * (h[p] . Wd[r])               (fp32 atomics;
//                   gateup_kernel zeroes y first)
#include "gemv_dev.h"
#include "sort_dev.h"
#include "topk_dev.h"

#include <hip/hip_ext.h>

namespace moe {

constexpr int GU_NP = 2, GU_HC = 5, GU_WPB = 4;     // 4*NP = 8 rows per wave, 16 pairs per block
constexpr int DN_NR = 4, DN_HC = 3, DN_WPB = 4;     // 4*NR = 16 rows per wave, 64 rows per block
constexpr int GU_PAIRS_PER_BLOCK = GU_WPB * 2 * GU_NP;
constexpr int DN_ROWS_PER_BLOCK = DN_WPB * 4 * DN_NR;
constexpr int GU_LDS_PER_WAVE = 2 * 2 * GU_NP * (MOE_MAX_HIDDEN / 32);
constexpr int DN_LDS_PER_WAVE = 4 * DN_NR * (MOE_MAX_INTER / 32);
constexpr int GU_SHORT_H = 32 * GU_HC * 16;         // longest row the single-pass path holds (2560)
constexpr int DN_SHORT_I = 16 * DN_HC * 16;         // (768)
// Gate/up workgroups resident per CU (3 waves per SIMD, 4 waves a workgroup).
constexpr int kGateupBlocksPerCu = 3;
constexpr int kDownBlocksPerCu = 4;
// Hinted line touches of a decode gate/up workgroup: its 2 * 16 rows of H/2
// code bytes in 64-byte lines, kGuTouchLoads per lane of each idle wave
// (three idle waves at M = 1 cover the 640 lines of H = 2560).
constexpr int kGuLineBytes = 64;
constexpr int kGuTouchLoads = 4;

// Routing inside a gate/up block (decode batches, M <= kRoutedMaxTokens, so
// at most 128 pairs: two per lane).  route_prepare: every workgroup takes the
// top-k of token t in wave t, into LDS.  The workgroup at x = 0 of the extra
// last grid row is the writer: wave 0 sorts the pairs and the block writes the
// routing outputs and the header.  Every other workgroup needs only the slots
// it works on: each wave marks the chosen experts in its own LDS bitmap and
// counts the active experts with a popcount scan over the bitmap words (no
// barrier, no sort); route_slot then takes the slot-th set bit as the slot's
// expert and finds its pairs with ballots.  Every workgroup computes the same
// top-k from the same logits.
struct RouteState {           // per-wave: this wave's copy of the pairs and the bitmap scan
  int eA, eB, tA, tB;         // pair `lane` (A) and pair `lane + 64` (B): expert, token
  float wA, wB;               // their routing weights
  bool vA, vB;
  uint32_t word;              // bitmap word `lane` of the active experts
  int inc;                    // inclusive popcount scan over the words
  int D;                      // active experts
};

// Returns false for the writer (after writing the routing outputs).
// `before_barrier` runs in every thread after the top-k, before the block
// barrier that publishes it (the caller stores its staged activations there).
template <int C, class Pre>
__device__ __forceinline__ bool route_prepare(const ForwardArgs& a, const RouteOut& r, RouteState& rs,
                                              bool writer, Pre before_barrier) {
  constexpr int kWords = MOE_MAX_EXPERTS / 32;           // bitmap words; index kWords is a sink
  __shared__ SmallSortLds<C, kRoutedMaxPairs> L;
  __shared__ uint32_t bits[GU_WPB][kWords + 1];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const int N = a.M * a.k, E = a.E;
  if (lane <= kWords) bits[wave][lane] = 0u;
  for (int t = wave; t < a.M; t += nw) {
    int id; float w;
    wave_topk_softmax<C>(r.logits + (size_t)t * E, E, a.k, id, w);
    if (lane < a.k) {
      L.ids[t * a.k + lane] = id;
      L.w[t * a.k + lane] = w;
      L.tok[t * a.k + lane] = t;
    }
  }
  before_barrier();
  __syncthreads();
  if (writer) {
    if (wave == 0) wave_sort_small(L, N, E, r.ebits);
    __syncthreads();
    block_store_small_sort(L, N, E, r.topk_ids, r.topk_weights, r.offsets, r.sorted_pairs, r.active,
                           r.num_active);
    if (threadIdx.x == 0) {
      a.hdr->gemv_experts = L.na + a.has_shared;        // every expert runs on this path
      a.hdr->mfma_experts = 0;
      a.hdr->mfma_items = 0;
      a.hdr->mt_experts = 0;
    }
    return false;
  }
  const int pA = min(lane, N - 1), pB = min(lane + kWave, N - 1);
  rs.eA = L.ids[pA]; rs.eB = L.ids[pB];
  rs.tA = L.tok[pA]; rs.tB = L.tok[pB];
  rs.wA = L.w[pA]; rs.wB = L.w[pB];
  rs.vA = lane < N && (unsigned)rs.eA < (unsigned)E;
  rs.vB = lane + kWave < N && (unsigned)rs.eB < (unsigned)E;
  uint32_t* mb = bits[wave];
  atomicOr(&mb[rs.vA ? (rs.eA >> 5) : kWords], 1u << (rs.eA & 31));
  atomicOr(&mb[rs.vB ? (rs.eB >> 5) : kWords], 1u << (rs.eB & 31));
  wave_lds_fence();
  const int nwords = (E + 31) >> 5;
  rs.word = (lane < nwords) ? mb[min(lane, kWords - 1)] : 0u;
  rs.inc = wave_inclusive_scan(__popc(rs.word));
  rs.D = __builtin_amdgcn_readlane(rs.inc, kWave - 1);
  return true;
}

// Slot record of `slot`: slots [0, D) are the active experts in increasing
// order, slot D the shared expert, later slots have no work (e = -1).
__device__ __forceinline__ SlotRec route_slot(const ForwardArgs& a, const RouteState& rs, int slot) {
  SlotRec rec;
  rec.pad[0] = rec.pad[1] = rec.pad[2] = rec.pad[3] = 0;
#pragma unroll
  for (int q = 0; q < kRecTokens; ++q) { rec.tok[q] = 0; rec.w[q] = 0.f; }
  if (slot < rs.D) {
    const int wsel = (int)__builtin_ctzll(__ballot(rs.inc > slot));      // word holding the expert
    uint32_t wb = (uint32_t)__builtin_amdgcn_readlane((int)rs.word, wsel);
    int nth = slot - (__builtin_amdgcn_readlane(rs.inc, wsel) - __popc(wb));
    for (; nth > 0; --nth) wb &= wb - 1u;
    const int e = wsel * 32 + __builtin_ctz(wb);
    uint64_t mA = __ballot(rs.vA && rs.eA == e), mB = __ballot(rs.vB && rs.eB == e);
    rec.e = e;
    rec.n = __popcll(mA) + __popcll(mB);
    rec.pbeg = __popcll(__ballot(rs.vA && rs.eA < e)) + __popcll(__ballot(rs.vB && rs.eB < e));
    rec.hrow0 = rec.pbeg;
#pragma unroll
    for (int q = 0; q < kRecTokens; ++q) {             // the expert's pairs in order
      if (mA) {
        const int p = (int)__builtin_ctzll(mA);
        rec.tok[q] = __builtin_amdgcn_readlane(rs.tA, p);
        rec.w[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rs.wA), p));
        mA &= mA - 1;
      } else if (mB) {
        const int p = (int)__builtin_ctzll(mB);
        rec.tok[q] = __builtin_amdgcn_readlane(rs.tB, p);
        rec.w[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rs.wB), p));
        mB &= mB - 1;
      }
    }
  } else if (slot == rs.D && a.has_shared) {
    rec.e = a.E; rec.n = a.M; rec.pbeg = -1; rec.hrow0 = a.M * a.k;
#pragma unroll
    for (int q = 0; q < kRecTokens; ++q) { rec.tok[q] = q < a.M ? q : 0; rec.w[q] = 1.f; }
  } else {
    rec.e = -1; rec.n = 0; rec.pbeg = -1; rec.hrow0 = 0;
  }
  return rec;
}

// at most 3 waves per SIMD: the codes, scales and staged activations of a wave
// stay in registers without spilling (M=1 needs under 2 waves per SIMD anyway).
// C > 0: the block routes itself (C = experts per lane of the top-k).
// A8 (W4A8 decode, short rows): x goes through the MXFP8 round trip as it is
// staged (the four threads of a DPP quad hold one 32-element block).
// HINT (moe_layer_hinted): idle waves touch the hinted expert's rows during the
// routing; a separate instance, so the plain kernel carries none of it.
template <bool SHORT, int C, bool A8 = false, bool HINT = false>
__global__ __launch_bounds__(GU_WPB * kWave) __attribute__((amdgpu_waves_per_eu(1, 3)))
void gateup_kernel(ForwardArgs a, RouteOut r) {
  if (C > 0 || !a.yp) {   // every block zeroes a share of y for the down kernel's scatter-add
                          // (decode batches never combine by rows)
    const size_t nblk = (size_t)gridDim.x * gridDim.y;
    const size_t b = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    const size_t total = (size_t)a.M * a.H;
    for (size_t i = b * blockDim.x + threadIdx.x; i < total; i += nblk * blockDim.x) a.y[i] = 0.f;
  }
  ExpertSlot s;
  __shared__ uint8_t s_lds[GU_WPB][GU_LDS_PER_WAVE];
  const int wave = threadIdx.x / kWave;
  const int jp0 = (blockIdx.x * GU_WPB + wave) * 2 * GU_NP;
  if constexpr (C > 0) {
    // routed: rows 0 .. gridDim.y-3 loop over the slots (each workgroup routes
    // once, however many slots it takes); with a shared expert, the row before
    // last streams it without waiting for the routing (it needs none); the
    // last row is the writer
    const bool writer = blockIdx.y == gridDim.y - 1;
    const bool shared_row = a.has_shared && blockIdx.y == gridDim.y - 2;
    if (writer && blockIdx.x != 0) return;
    // short rows: every token's activations are staged in LDS for the GEMVs;
    // the loads are issued before the top-k, whose logits wait covers them
    constexpr int kXVec = kRoutedMaxTokens * GU_SHORT_H / 8;      // uint4 of x, at most
    constexpr int kXPer = (kXVec + GU_WPB * kWave - 1) / (GU_WPB * kWave);
    __shared__ uint4 s_x[SHORT ? kXVec : 1];
    uint4 xs[SHORT ? kXPer : 1];
    const int nxv = SHORT ? a.M * a.H / 8 : 0;
    if constexpr (SHORT) {
      const uint4* x4 = reinterpret_cast<const uint4*>(a.x);
#pragma unroll
      for (int q = 0; q < kXPer; ++q) xs[q] = x4[min((int)threadIdx.x + q * GU_WPB * kWave, nxv - 1)];
    }
    // With a hint, the waves that take no part in the top-k (wave >= M) touch
    // this workgroup's code lines of the hinted expert of its first slot (one
    // word per 64-byte line), so the stream after the routing finds them in
    // this XCD's L2.  The routing barrier is their only wait on these loads,
    // and it waits for the top-k anyway.
    uint32_t tw[kGuTouchLoads];
    bool touch = false;
    if constexpr (SHORT && HINT) {
      const int row_q = a.H / 2;
      const int lpr = row_q / kGuLineBytes;
      const int jbase = blockIdx.x * GU_PAIRS_PER_BLOCK;
      if (a.hint && !writer && !shared_row && wave >= a.M && row_q % kGuLineBytes == 0 && jbase < a.I) {
        const int y = blockIdx.y;
        const int eh = (y < *a.num_hint) ? a.hint[y] : -1;
        if ((unsigned)eh < (unsigned)a.E) {
          touch = true;
          const uint8_t* base = a.w13_q + (size_t)eh * 2 * a.I * row_q;
          const int nl = 2 * GU_PAIRS_PER_BLOCK * lpr;            // gate rows, then up rows
          const int nlanes = (GU_WPB - a.M) * kWave;
          const int l0 = (wave - a.M) * kWave + (threadIdx.x & (kWave - 1));
#pragma unroll
          for (int q = 0; q < kGuTouchLoads; ++q) {
            const int l = min(q * nlanes + l0, nl - 1);
            const int r = l / lpr, c = l - r * lpr;
            const int row = (r < GU_PAIRS_PER_BLOCK) ? jbase + r : a.I + jbase + (r - GU_PAIRS_PER_BLOCK);
            tw[q] = *reinterpret_cast<const uint32_t*>(base + (size_t)row * row_q + c * kGuLineBytes);
          }
        }
      }
    }
    auto stage_x = [&]() {
      if constexpr (SHORT) {
#pragma unroll
        for (int q = 0; q < kXPer; ++q) {
          const int i = threadIdx.x + q * GU_WPB * kWave;
          if constexpr (A8) mxfp8_round_trip8_quad(xs[q]);   // quads never straddle nxv (H % 32 == 0)
          if (i < nxv) s_x[i] = xs[q];
        }
      }
    };
    // this block's slots: blockIdx.y, + rows, + 2 rows, ...  Their records are
    // looked up first (one wave per slot) and parked in LDS, so no routing
    // state stays live in registers through the GEMVs.  The shared row parks
    // the shared expert's record and skips the routing.
    __shared__ SlotRec s_rec[kRoutedMaxPairs + 1];
    int mine = 1;
    if (shared_row) {
      if constexpr (SHORT) {
#pragma unroll
        for (int q = 0; q < kXPer; ++q) {
          const int i = threadIdx.x + q * GU_WPB * kWave;
          uint4 v = xs[q];
          if constexpr (A8) mxfp8_round_trip8_quad(v);
          if (i < nxv) s_x[i] = v;
        }
      }
      if (threadIdx.x == 0) {
        SlotRec rec;
        rec.e = a.E; rec.n = a.M; rec.pbeg = -1; rec.hrow0 = a.M * a.k;
        rec.pad[0] = rec.pad[1] = rec.pad[2] = rec.pad[3] = 0;
#pragma unroll
        for (int q = 0; q < kRecTokens; ++q) { rec.tok[q] = q < a.M ? q : 0; rec.w[q] = 1.f; }
        s_rec[0] = rec;
      }
    } else {
      RouteState rs;
      if (!route_prepare<C>(a, r, rs, writer, stage_x)) return;     // uniform over the block
      const int slots = max_slots(a.M, a.k, a.E) - 1 + a.has_shared;
      const int rows = gridDim.y - 1 - a.has_shared;
      mine = (slots - (int)blockIdx.y + rows - 1) / rows;
      const int lane = threadIdx.x & (kWave - 1);
      for (int i = wave; i < mine; i += GU_WPB) {
        const int slot = blockIdx.y + i * rows;
        const SlotRec rec = route_slot(a, rs, slot);
        if (lane == 0) {
          s_rec[i] = rec;
          if (blockIdx.x == 0) r.rec[slot] = rec;
        }
      }
    }
    __syncthreads();
    for (int i = 0; i < mine; ++i) {
      const SlotRec& rec = s_rec[i];
      // later slots are empty; the shared row streams the shared expert
      if (rec.e < 0 || (rec.e == a.E && a.has_shared && !shared_row)) break;
      s.e = rec.e; s.n = rec.n; s.pbeg = rec.pbeg; s.hrow0 = rec.hrow0;
#pragma unroll
      for (int q = 0; q < kRecTokens; ++q) { s.tok[q] = rec.tok[q]; s.w[q] = rec.w[q]; }
      if (jp0 < a.I) {
        if constexpr (SHORT)
          gateup_short<GU_NP, GU_HC, true>(a, s, jp0, s_lds[wave], reinterpret_cast<const uint16_t*>(s_x));
        else
          gateup_long<GU_NP, GU_HC>(a, s, jp0, s_lds[wave]);
      }
    }
    if (HINT && touch) {
      uint32_t t = 0u;
#pragma unroll
      for (int q = 0; q < kGuTouchLoads; ++q) t += tw[q];
      if (t == 0x9E3779B9u && a.M < 0) a.y[0] = 0.f;   // never true (M >= 1): keeps the touches live
    }
    return;
  } else {
    if (!a.rec && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
      a.hdr->gemv_experts = *a.num_active + a.has_shared;  // without records: every expert on this path
      a.hdr->mfma_experts = 0;
      a.hdr->mfma_items = 0;
      a.hdr->mt_experts = 0;
    }
    if (a.lists) {   // grid row y takes GEMV experts y, y + rows, ... (a grid sized to the
                     // chip, not to every possible slot: no flood of empty workgroups)
      if (jp0 >= a.I) return;
      const int n = a.hdr->gemv_experts;
      for (int y = blockIdx.y; y < n; y += gridDim.y) {
        resolve_slot(a.lists[y], a, s);
        if constexpr (SHORT)
          gateup_short<GU_NP, GU_HC>(a, s, jp0, s_lds[wave]);
        else
          gateup_long<GU_NP, GU_HC>(a, s, jp0, s_lds[wave]);
      }
      return;
    } else if (!resolve_slot(blockIdx.y, a, s)) {
      return;
    }
  }
  if (jp0 >= a.I) return;
  if constexpr (SHORT)
    gateup_short<GU_NP, GU_HC>(a, s, jp0, s_lds[wave]);
  else
    gateup_long<GU_NP, GU_HC>(a, s, jp0, s_lds[wave]);
}

template <bool SHORT, bool ROWS>
__global__ __launch_bounds__(DN_WPB * kWave) void down_kernel(ForwardArgs a) {
  ExpertSlot s;
  __shared__ uint8_t s_lds[DN_WPB][DN_LDS_PER_WAVE];
  const int wave = threadIdx.x / kWave;
  const int r0 = (blockIdx.x * DN_WPB + wave) * 4 * DN_NR;
  if (a.lists) {     // grid row y takes GEMV experts y, y + rows, ...
    if (r0 >= a.H) return;
    const int n = a.hdr->gemv_experts;
    for (int y = blockIdx.y; y < n; y += gridDim.y) {
      resolve_slot(a.lists[y], a, s);
      if constexpr (SHORT)
        down_short<DN_NR, DN_HC, ROWS>(a, s, r0, s_lds[wave]);
      else
        down_long<DN_NR, DN_HC, ROWS>(a, s, r0, s_lds[wave]);
    }
    return;
  } else if (!resolve_slot(gridDim.y - 1 - blockIdx.y, a, s)) {
    // decode: slots in reverse, so the shared expert (every token, the most
    // work; the last working slot) is dispatched before the routed ones
    return;
  }
  if (r0 >= a.H) return;
  if constexpr (SHORT)
    down_short<DN_NR, DN_HC, ROWS>(a, s, r0, s_lds[wave]);
  else
    down_long<DN_NR, DN_HC, ROWS>(a, s, r0, s_lds[wave]);
}

// ------------------------------------------------------------- combine --
// Combine by rows: thread (token t, 4 columns) sums the token's partial rows
// in a fixed order -- its k routed pairs in slot order, then the shared
// expert's row -- and writes y (deterministic, no atomics).
__global__ __launch_bounds__(256) void combine_rows_kernel(const float* __restrict__ yp,
                                                           const int* __restrict__ inv, int M, int k, int H,
                                                           int has_shared, float* __restrict__ y) {
  const int t = blockIdx.y;
  const int c4 = blockIdx.x * blockDim.x + threadIdx.x;
  if (c4 >= H / 4) return;
  const float4* p4 = reinterpret_cast<const float4*>(yp);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < k; ++s) {
    const int row = inv[(size_t)t * k + s];
    if (row < 0) continue;
    const float4 v = p4[(size_t)row * (H / 4) + c4];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (has_shared) {
    const float4 v = p4[((size_t)M * k + t) * (H / 4) + c4];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  reinterpret_cast<float4*>(y)[(size_t)t * (H / 4) + c4] = acc;
}

// ------------------------------------------------------------- dequant --
// One thread per 32-bit code word (8 elements): the same pair routine as the
// expert kernels, widened from bf16 to fp32 (exact).
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ q,
                                                      const uint8_t* __restrict__ s, int64_t rows,
                                                      int64_t cols, float* __restrict__ out) {
  const int64_t words_per_row = cols / 8;
  const int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (wi >= rows * words_per_row) return;
  const int64_t r = wi / words_per_row, w = wi % words_per_row;
  const uint32_t code = reinterpret_cast<const uint32_t*>(q + r * (cols / 2))[w];
  const float scale = e8m0_to_f32(s[r * (cols / 32) + (w * 8) / 32]);
  const bf16x2 p0 = mxfp4_pair_bf16<0>(code, scale), p1 = mxfp4_pair_bf16<1>(code, scale);
  const bf16x2 p2 = mxfp4_pair_bf16<2>(code, scale), p3 = mxfp4_pair_bf16<3>(code, scale);
  float4* o = reinterpret_cast<float4*>(out + r * cols + w * 8);
  o[0] = make_float4((float)p0.x, (float)p0.y, (float)p1.x, (float)p1.y);
  o[1] = make_float4((float)p2.x, (float)p2.y, (float)p3.x, (float)p3.y);
}

namespace {

// Compute units of the current device (queried per launch: no cached state).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// routed: the gate/up grid has one more row (the routing writer), and one more
// for the shared expert when the bank has one.
hipError_t launch_pair(void (*gu)(ForwardArgs, RouteOut), const ForwardArgs& a, const RouteOut& r,
                       bool routed, hipStream_t s, const Timing& tm, hipEvent_t mid = nullptr) {
  const int slots = max_slots(a.M, a.k, a.E) - 1 + (a.has_shared ? 1 : 0);
  const int gx = (a.I + GU_PAIRS_PER_BLOCK - 1) / GU_PAIRS_PER_BLOCK;
  int gy = slots;
  if (routed) {   // as many rows of slots as stay resident with the shared and writer rows; blocks loop
                  // over the rest
    const int extra = 1 + (a.has_shared ? 1 : 0);
    const int fit = kGateupBlocksPerCu * device_cus() / gx - extra;
    gy = (slots < fit ? slots : (fit > 1 ? fit : 1)) + extra;
  }
  const int dx = (a.H + DN_ROWS_PER_BLOCK - 1) / DN_ROWS_PER_BLOCK;
  int dy = slots;
  if (a.lists) {   // batches: the kernels loop over the GEMV experts; two residency rounds of rows
    const int cus = device_cus();
    const int gfit = (2 * kGateupBlocksPerCu * cus + gx - 1) / gx, dfit = (2 * kDownBlocksPerCu * cus + dx - 1) / dx;
    gy = gy < gfit ? gy : gfit;
    dy = dy < dfit ? dy : dfit;
  }
  dim3 ggu(gx, gy);
  dim3 bgu(GU_WPB * kWave);
  dim3 gdn(dx, dy), bdn(DN_WPB * kWave);
  auto dn = (a.I <= DN_SHORT_I) ? (a.yp ? down_kernel<true, true> : down_kernel<true, false>)
                                : (a.yp ? down_kernel<false, true> : down_kernel<false, false>);
  // with events, they take the gate/up kernel's own begin/end timestamps
  hipExtLaunchKernelGGL(gu, ggu, bgu, 0, s, tm.gu_start, tm.gu_stop, 0, a, r);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (mid && (err = hipEventRecord(mid, s)) != hipSuccess) return err;   // y is zeroed from here on
  // W4A8: h goes through the MXFP8 round trip once, in place, between the
  // two kernels (decode: every row; batches: the rows of this path's experts)
  if (a.act8) {
    err = routed ? launch_mxfp8_round_trip_rows(a.h, a.hlo, (int64_t)a.M * a.k + a.M, a.I, s)
                 : launch_h_round_trip(a, 0, s);
    if (err != hipSuccess) return err;
  }
  hipExtLaunchKernelGGL(dn, gdn, bdn, 0, s, tm.dn_start, tm.dn_stop, 0, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const ForwardArgs& a, hipStream_t s, const Timing& tm, hipEvent_t zeroed) {
  if (batch_decode_fits(a)) return launch_decode_batch(a, s, tm, zeroed, device_cus());
  const RouteOut none{};
  return launch_pair(a.H <= GU_SHORT_H ? gateup_kernel<true, 0> : gateup_kernel<false, 0>, a, none, false, s,
                     tm, zeroed);
}

bool routed_stages_x(int H) { return H <= GU_SHORT_H; }

hipError_t launch_forward_routed(const ForwardArgs& a, const RouteOut& r, hipStream_t s, const Timing& tm) {
  const bool short_h = a.H <= GU_SHORT_H;
  const bool a8x = a.act8 && short_h;                // x rounded while staged (else a.x is already MXFP8)
  void (*gu)(ForwardArgs, RouteOut);
  const bool hint = a.hint != nullptr && short_h && !a.act8;
  if (topk_lane_experts(a.E) == 8)
    gu = short_h ? (a8x ? gateup_kernel<true, 8, true>
                        : (hint ? gateup_kernel<true, 8, false, true> : gateup_kernel<true, 8>))
                 : gateup_kernel<false, 8>;
  else
    gu = short_h ? (a8x ? gateup_kernel<true, 16, true>
                        : (hint ? gateup_kernel<true, 16, false, true> : gateup_kernel<true, 16>))
                 : gateup_kernel<false, 16>;
  return launch_pair(gu, a, r, true, s, tm);
}

hipError_t launch_combine_rows(const ForwardArgs& a, hipStream_t s) {
  dim3 grid((a.H / 4 + 255) / 256, a.M);
  combine_rows_kernel<<<grid, dim3(256), 0, s>>>(a.yp, a.inv, a.M, a.k, a.H, a.has_shared, a.y);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols, float* out,
                          hipStream_t st) {
  const int64_t words = rows * (cols / 8);
  const int64_t blocks = (words + 255) / 256;
  dequant_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(q, s, rows, cols, out);
  return hipGetLastError();
}

}  // namespace moe
