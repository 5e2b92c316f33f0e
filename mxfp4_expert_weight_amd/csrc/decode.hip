// The decode layer's expert kernels (M <= 4 tokens: one decode step, or the
// 4-token verify window of speculative decoding, digest "3 Ways to Improve
// MoE Inference on NVIDIA DGX Spark", section 5) for hidden sizes that are a
// multiple of 512 and intermediate sizes that are a multiple of 256:
//
//   decode_gateup_kernel:  every workgroup routes the batch itself from the
//       router logits (top-k by threshold and rank, pairs deduplicated in
//       pair order), then streams its slice of one expert's MXFP4 gate and up
//       rows and writes h = SiLU(x Wg^T) * (x Wu^T) as two bf16 terms.
//   decode_down_kernel:    y[t][r] += w * (h . Wd[r]) for every expert's
//       tokens (fp32 atomics; the gate/up kernel zeroes y).
//
// Each expert runs once over all of its tokens (MoE-SpeQ article, 4.2).  One
// 16-byte load per lane is one 32-element MXFP4 block (16 code bytes, one
// E8M0 scale byte); a wave instruction reads four rows' 256-byte segments
// (gate/up) or eight rows' 128-byte segments (down).  The grid holds one
// workgroup per (row slice, slot) for every possible slot, so at M = 4 all of
// a layer's expert bytes are requested in one residency round.
//
// Slots: record 0 is the shared expert; records 1.. are the routed experts in
// the order of their first pair p = t*k + s.  A routed pair's h row is p; the
// shared expert's row for token t is M*k + t.  The sorted outputs of the ABI
// (expert_offsets, sorted_pairs, active_experts, num_active) and the top-k
// outputs are written by one extra workgroup, off the critical path.
#include "sort_dev.h"
#include "topk_dev.h"

#include <hip/hip_ext.h>

namespace moe {

// 128-bit values move as a native vector type: the HIP uint4 struct is copied
// with a memcpy, which keeps small arrays of it in memory instead of registers.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 ld128(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Matrix-core operands (v_mfma_f32_16x16x32_bf16): lane l holds row (A) or
// column (B) l % 16 and 8 consecutive K values of lane group l / 16; output
// register i of lane l is D[4 (l / 16) + i][l % 16].  Only the pairing of A
// and B values along K matters, so lane group kq of load i takes scale block
// 4 i + kq of its row: one 16-byte load per lane is one whole MXFP4 block, a
// row's four lanes read 64 contiguous bytes, and step m of the block is its
// m-th 32-bit code word (8 elements).
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// One code word (8 E2M1 elements) times the block scale, as 8 bf16 (exact).
__device__ __forceinline__ v8bf mxfp4_word_bf16x8(uint32_t w, float scale) {
  const bf16x2 p0 = mxfp4_pair_bf16<0>(w, scale), p1 = mxfp4_pair_bf16<1>(w, scale);
  const bf16x2 p2 = mxfp4_pair_bf16<2>(w, scale), p3 = mxfp4_pair_bf16<3>(w, scale);
  v8bf v;
  v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
  v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
  return v;
}

// The value a lane's partner in the other half of the wave (l ^ 32) holds.
__device__ __forceinline__ float half_partner(float v) {
  const Pair p = swap32(__float_as_uint(v));
  return __uint_as_float(p.a == __float_as_uint(v) ? p.b : p.a);   // equal values: either copy
}

constexpr int DC_THREADS = 256;                 // 4 waves per workgroup (both kernels)
constexpr int DC_WAVES = DC_THREADS / kWave;
constexpr int DC_MAXP = kRoutedMaxTokens * MOE_MAX_TOPK;   // pairs of a decode batch (128)
constexpr int DN_RG = 2;                        // down: 8-row groups per wave (16 rows)
constexpr int DN_ROWS_WG = DC_WAVES * 8 * DN_RG;            // 64 rows per workgroup

// Record of one expert of a decode batch (64 bytes: one load).
struct DecRec {
  int32_t e;                  // bank index (E = shared), -1: no work
  int32_t n;                  // tokens (<= kRoutedMaxTokens)
  int32_t tok[kRoutedMaxTokens];
  float w[kRoutedMaxTokens];
  int32_t hrow[kRoutedMaxTokens];
  int32_t pad[2];
};
static_assert(sizeof(DecRec) == 64, "decode record size");

// ------------------------------------------------------------- probes --
// Phase stamps (s_memrealtime, 100 MHz) of thread 0 of each workgroup, for
// the measurement entry point only; the product instances carry none of it.
constexpr int kProbeStamps = 16;
enum ProbeSlot {
  kGuEntry = 0, kGuKeys = 1, kGuThreshold = 2, kGuTopk = 3, kGuRouted = 4, kGuSlot = 5, kGuIssued = 6,
  kGuFirstData = 7, kGuDone = 8,
  kDnEntry = 9, kDnRecord = 10, kDnIssued = 11, kDnFirstData = 12, kDnDone = 13,
};
template <bool PROBE>
__device__ __forceinline__ void stamp(unsigned long long* probe, int slot) {
  if constexpr (PROBE) {
    if (threadIdx.x == 0) {
      const size_t wg = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
      probe[wg * kProbeStamps + slot] = __builtin_amdgcn_s_memrealtime();
    }
  }
}

// -------------------------------------------------------------- top-k --
// LDS scratch of one wave's top-k: the 64 lane maxima, the candidates (keys,
// ids; 4 entries of padding) and the ranked output.
struct TopkScratch {
  __align__(16) uint32_t lmax[kWave];
  __align__(16) uint32_t ckey[kWave + 4];
  __align__(16) int cid[kWave + 4];
  __align__(16) uint32_t okey[MOE_MAX_TOPK];
  __align__(16) int oid[MOE_MAX_TOPK];
};

// The candidates of one token's top-k and their ranks, by one full wave.
// Threshold: the lanes form groups of G (G = 4 for k <= 8, 2 for k <= 16,
// else 1); T = the largest group maximum that at least k group maxima reach.
// Those k maxima are k distinct logits >= T, so the k-th largest logit is
// >= T and every logit of the top-k is a candidate (logit >= T).  The
// candidates -- usually k plus a few -- are compacted into LDS and each is
// ranked against all of them (greater key, or equal key and lower index,
// counts: ties go to the lower expert index).  Lane i < C gets candidate i's
// key, expert and rank.  Returns C, or -1 (wave-uniform) when more than 64
// logits reach T (heavy ties).
template <int kPer, bool PROBE>
__device__ __forceinline__ int wave_topk_candidates(const float* row, int E, int k, TopkScratch& S, uint32_t& mk,
                                                    int& mi, int& rank, unsigned long long* probe) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t val[kPer];
  load_logit_keys<kPer>(row, E, val);
  uint32_t m = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) m = max(m, val[j]);
  stamp<PROBE>(probe, kGuKeys);
  const int G = k <= 8 ? 4 : (k <= 16 ? 2 : 1);   // wave-uniform
  if (G >= 2) m = max(m, dpp_quad_xor1(m));
  if (G >= 4) m = max(m, dpp_quad_xor2(m));
  const int NG = kWave / G;
  if ((lane & (G - 1)) == 0) S.lmax[lane / G] = m;
  wave_lds_fence();
  int cnt = 0;                                      // group maxima >= mine
  const uint4* l4 = reinterpret_cast<const uint4*>(S.lmax);
  for (int q = 0; q < NG / 4; ++q) {                // NG / 4 is 4, 8 or 16
    const uint4 v = l4[q];
    cnt += (int)(v.x >= m) + (int)(v.y >= m) + (int)(v.z >= m) + (int)(v.w >= m);
  }
  const uint32_t T = wave_max_u32(cnt >= k ? m : 0u);
  stamp<PROBE>(probe, kGuThreshold);
  int base = 0;                                     // compaction, in (j, lane) order
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const bool c = val[j] != 0u && val[j] >= T;   // key 0: no expert
    const uint64_t mask = __ballot(c);
    const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
    if (c && pos < kWave) {
      S.ckey[pos] = val[j];
      S.cid[pos] = lane * kPer + j;
    }
    base += (int)__popcll(mask);
  }
  if (base > kWave) return -1;
  const int C = base;
  if (lane < 4) {                                   // padding: key 0 never outranks a candidate
    S.ckey[C + lane] = 0u;
    S.cid[C + lane] = 0x7FFFFFFF;
  }
  wave_lds_fence();
  mk = (lane < C) ? S.ckey[lane] : 0u;
  mi = (lane < C) ? S.cid[lane] : 0x7FFFFFFF;
  rank = 0;
  for (int q = 0; q < C; q += 4) {                  // C is wave-uniform
    const uint4 kq = *reinterpret_cast<const uint4*>(&S.ckey[q]);
    const int4 iq = *reinterpret_cast<const int4*>(&S.cid[q]);
    rank += (int)(kq.x > mk || (kq.x == mk && iq.x < mi));
    rank += (int)(kq.y > mk || (kq.y == mk && iq.y < mi));
    rank += (int)(kq.z > mk || (kq.z == mk && iq.z < mi));
    rank += (int)(kq.w > mk || (kq.w == mk && iq.w < mi));
  }
  return C;
}

// Top-k of one token's logits by one full wave (ranks as above), and the
// weights exp(l_i - l_max) / sum over the kept.  Lane i < k returns the
// i-th expert and its weight.  Returns false (wave-uniform) in the heavy-tie
// case; nothing is returned then.
template <int kPer, bool PROBE = false>
__device__ __forceinline__ bool wave_topk_rank(const float* row, int E, int k, TopkScratch& S, int& out_id,
                                               float& out_w, unsigned long long* probe = nullptr) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t mk;
  int mi, rank;
  const int C = wave_topk_candidates<kPer, PROBE>(row, E, k, S, mk, mi, rank, probe);
  if (C < 0) return false;
  if (lane < C && rank < k) {
    S.okey[rank] = mk;
    S.oid[rank] = mi;
  }
  wave_lds_fence();
  const uint32_t my_key = (lane < k) ? S.okey[lane] : 0u;
  const uint32_t top_key = S.okey[0];
  out_id = (lane < k) ? S.oid[lane] : 0;
  const float ex = (lane < k) ? expf(f32_from_orderable(my_key) - f32_from_orderable(top_key)) : 0.f;
  const float sum = group_sum<kWave>(ex);
  out_w = (lane < k) ? ex / sum : 0.f;
  return true;
}

// One slot of a one-token batch: the expert of rank s (every lane gets it)
// and, if need_w, its weight, with the same arithmetic as wave_topk_rank
// (the kept experts' exponentials are moved to the lanes of their ranks, so
// the sum runs in the same order).
template <int kPer, bool PROBE>
__device__ __forceinline__ void wave_topk_pick(const float* row, int E, int k, int s, bool need_w, TopkScratch& S,
                                               int& out_e, float& out_w, unsigned long long* probe) {
  uint32_t mk;
  int mi, rank;
  const int C = wave_topk_candidates<kPer, PROBE>(row, E, k, S, mk, mi, rank, probe);
  if (C < 0) {                                      // heavy ties: the sequential top-k
    int id;
    float wt;
    wave_topk_softmax<kPer>(row, E, k, id, wt);
    out_e = __builtin_amdgcn_readlane(id, s);
    out_w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), s));
    return;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const bool kept = lane < C && rank < k;
  const uint64_t sel = __ballot(lane < C && rank == s);
  out_e = __builtin_amdgcn_readlane(mi, (int)__builtin_ctzll(sel));
  out_w = 0.f;
  if (need_w) {                                     // wave-uniform
    const uint32_t top_key = __builtin_amdgcn_readlane(mk, (int)__builtin_ctzll(__ballot(lane < C && rank == 0)));
    const float ex = kept ? expf(f32_from_orderable(mk) - f32_from_orderable(top_key)) : 0.f;
    // lane r receives the exponential of rank r; the other lanes go one to
    // one onto lanes k.. (every lane is written exactly once) and carry 0
    const uint64_t km = __ballot(kept);
    const int other = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(~km >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)~km, 0u));
    const float er = __int_as_float(
        __builtin_amdgcn_ds_permute((kept ? rank : k + other) * 4, kept ? __float_as_int(ex) : 0));
    const float exr = lane < k ? er : 0.f;
    const float sum = group_sum<kWave>(exr);
    out_w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(exr), s)) / sum;
  }
}

// The top-k of token t into ids[t*k ..], w[t*k ..] by wave t (all lanes).
template <int C, bool PROBE = false>
__device__ __forceinline__ void route_token(const float* logits, int t, int E, int k, TopkScratch& S, int* ids,
                                            float* w, int* tok, unsigned long long* probe = nullptr) {
  const int lane = threadIdx.x & (kWave - 1);
  int id;
  float wt;
  if (!wave_topk_rank<C, PROBE>(logits + (size_t)t * E, E, k, S, id, wt, probe))
    wave_topk_softmax<C>(logits + (size_t)t * E, E, k, id, wt);
  stamp<PROBE>(probe, kGuTopk);
  if (lane < k) {
    ids[t * k + lane] = id;
    w[t * k + lane] = wt;
    if (tok) tok[t * k + lane] = t;
  }
}

// --------------------------------------------------------------- slots --
// A record in registers: its four 16-byte words (the DecRec layout), so it
// is never an aggregate the compiler would copy through memory.
//   a = {e, n, tok0, tok1}, b = {tok2, tok3, w0, w1}, c = {w2, w3, hrow0, hrow1},
//   d = {hrow2, hrow3, 0, 0}
struct PRec {
  u32x4 a, b, c, d;
};
__device__ __forceinline__ int prec_e(const PRec& r) { return (int)r.a[0]; }
__device__ __forceinline__ int prec_n(const PRec& r) { return (int)r.a[1]; }
// token, weight and h row of the record's i-th token (i runtime, < 4)
__device__ __forceinline__ int prec_tok(const PRec& r, int i) {
  const unsigned t = i == 0 ? r.a[2] : i == 1 ? r.a[3] : i == 2 ? r.b[0] : r.b[1];
  return (int)t;
}
__device__ __forceinline__ float prec_w(const PRec& r, int i) {
  const unsigned w = i == 0 ? r.b[2] : i == 1 ? r.b[3] : i == 2 ? r.c[0] : r.c[1];
  return __uint_as_float(w);
}
__device__ __forceinline__ int prec_hrow(const PRec& r, int i) {
  const unsigned h = i == 0 ? r.c[2] : i == 1 ? r.c[3] : i == 2 ? r.d[0] : r.d[1];
  return (int)h;
}
__device__ __forceinline__ void prec_pack(PRec& r, int e, int n, const int (&tok)[4], const float (&w)[4],
                                          const int (&hrow)[4]) {
  r.a = u32x4{(unsigned)e, (unsigned)n, (unsigned)tok[0], (unsigned)tok[1]};
  r.b = u32x4{(unsigned)tok[2], (unsigned)tok[3], __float_as_uint(w[0]), __float_as_uint(w[1])};
  r.c = u32x4{__float_as_uint(w[2]), __float_as_uint(w[3]), (unsigned)hrow[0], (unsigned)hrow[1]};
  r.d = u32x4{(unsigned)hrow[2], (unsigned)hrow[3], 0u, 0u};
}
__device__ __forceinline__ void prec_store(DecRec* dst, const PRec& r) {
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  d[0] = r.a; d[1] = r.b; d[2] = r.c; d[3] = r.d;
}
__device__ __forceinline__ void prec_load(const DecRec* src, PRec& r) {
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  r.a = p[0]; r.b = p[1]; r.c = p[2]; r.d = p[3];
}

// Record of routed slot s (0-based) from the batch's pairs (ids, w in LDS),
// by one wave: distinct experts in the order of their first pair.  M = 1:
// pair s itself (a token's k experts are distinct).  Otherwise owner[e] (LDS,
// preset to INT_MAX) takes each expert's first pair by an LDS atomic min; the
// waves of a workgroup may run this together (each applies the same mins).
__device__ __forceinline__ void routed_record(const int* ids, const float* w, int* owner, int M, int k, int E,
                                              int s, PRec& out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int P = M * k;
  int e = -1, n = 0;
  int tok[4] = {0, 0, 0, 0}, hrow[4] = {0, 0, 0, 0};
  float wt[4] = {0.f, 0.f, 0.f, 0.f};
  if (M == 1) {
    const int ee = (s < P) ? ids[s] : -1;
    if ((unsigned)ee < (unsigned)E) {
      e = ee;
      n = 1;
      wt[0] = w[s];
      hrow[0] = s;
    }
    prec_pack(out, e, n, tok, wt, hrow);
    return;
  }
  const int pA = lane, pB = lane + kWave;           // P <= 128: two pairs per lane
  const int eA = ids[min(pA, P - 1)], eB = ids[min(pB, P - 1)];
  const bool vA = pA < P && (unsigned)eA < (unsigned)E;
  const bool vB = pB < P && (unsigned)eB < (unsigned)E;
  if (vA) atomicMin(&owner[eA], pA);
  if (vB) atomicMin(&owner[eB], pB);
  wave_lds_fence();
  const bool fA = vA && owner[vA ? eA : 0] == pA;
  const bool fB = vB && owner[vB ? eB : 0] == pB;
  const uint64_t mA = __ballot(fA), mB = __ballot(fB);
  const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mA >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mA, 0u));
  const int belowB = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mB >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mB, 0u));
  const int nA = (int)__popcll(mA);
  const uint64_t sA = __ballot(fA && below == s), sB = __ballot(fB && nA + belowB == s);
  if (sA || sB) {
    e = sA ? __builtin_amdgcn_readlane(eA, (int)__builtin_ctzll(sA))
           : __builtin_amdgcn_readlane(eB, (int)__builtin_ctzll(sB));
    uint64_t tA = __ballot(vA && eA == e), tB = __ballot(vB && eB == e);   // its pairs, in order
#pragma unroll
    for (int q = 0; q < kRoutedMaxTokens; ++q) {
      int p = -1;
      if (tA) { p = (int)__builtin_ctzll(tA); tA &= tA - 1; }
      else if (tB) { p = kWave + (int)__builtin_ctzll(tB); tB &= tB - 1; }
      if (p >= 0) {
        tok[q] = p / k;
        wt[q] = w[p];
        hrow[q] = p;
        n = q + 1;
      }
    }
  }
  prec_pack(out, e, n, tok, wt, hrow);
}

__device__ __forceinline__ void shared_record(int M, int k, int E, PRec& out) {
  int tok[4], hrow[4];
  float wt[4];
#pragma unroll
  for (int q = 0; q < kRoutedMaxTokens; ++q) {
    tok[q] = q < M ? q : 0;
    wt[q] = 1.f;
    hrow[q] = M * k + (q < M ? q : 0);
  }
  prec_pack(out, E, M, tok, wt, hrow);
}

// ------------------------------------------------------------ gate/up --
// x staged in LDS as [token][quarter][block] uint4: block b of a row is 32
// bf16 (four 16-byte quarters); lanes reading consecutive blocks of one
// quarter touch consecutive 16 bytes.
// The writer workgroup keeps its sort state where the others stage x.
template <int NB, int Q>
struct GateupLds {
  static constexpr int kBlocks = NB * 16;                   // H / 32
  u32x4 x[kRoutedMaxTokens * 4 * kBlocks];
  uint8_t scales[DC_WAVES][2 * 4 * Q][kBlocks];             // a wave's 4Q gate rows, then its 4Q up rows
  TopkScratch topk[DC_WAVES];
  int ids[DC_MAXP];
  float w[DC_MAXP];
  int owner[MOE_MAX_EXPERTS];
};

// Dot product of one 32-element MXFP4 block (16 code bytes, scale) with 32
// bf16 activations (four uint4 in element order).
__device__ __forceinline__ float dot_block(const u32x4& c, float scale, const u32x4 (&x)[4], float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a[4] = {x[i][0], x[i][1], x[i][2], x[i][3]};
    acc = dot8_mxfp4_bf16(c[i], scale, a, acc);
  }
  return acc;
}

// Makes a 128-bit register tuple opaque at this point (one operand, so the
// tuple stays whole): values derived from it are recomputed in each pass of a
// token loop, not hoisted out of it into many live registers.  No instruction.
__device__ __forceinline__ void keep_in_loop(u32x4& v) { asm volatile("" : "+v"(v)); }

// One slot's gate/up work for the rows of this workgroup: its x rows, scales
// and code words requested in consumption order, x and the scales staged in
// LDS, the products formed as the codes arrive, h written as two bf16 terms.
// Q: quads of row pairs per wave (a workgroup covers 16 Q intermediate
// indices); A8: W4A8 (x rounded to MXFP8 as it is staged); MF: the products on
// the matrix cores (Q = 2: a wave's 8 gate and 8 up rows are the 16 rows of
// one tile, the slot's tokens its columns), each weight decoded once for all
// of the slot's tokens; otherwise per-token v_dot2 products.
template <int NB, int Q, bool A8, bool PROBE, bool MF>
__device__ __forceinline__ void gateup_slot(const ForwardArgs& a, GateupLds<NB, Q>& L, const PRec& rec) {
  constexpr int KB = NB * 16;                      // 32-element blocks per row
  static_assert(!MF || Q == 2, "a matrix-core wave covers 8 row pairs");
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int H = a.H, I = a.I;
  const int rec_e = prec_e(rec), rec_n = prec_n(rec);
  // the slot's tokens' x rows (issued before the weights, consumed first);
  // stores are unconditional (a guarded one would make a branch that holds
  // the load): threads past the end rewrite the last element's own value
  constexpr int kXVec = kRoutedMaxTokens * KB * 4;            // uint4 of x, at most
  constexpr int kXPer = (kXVec + DC_THREADS - 1) / DC_THREADS;
  const int nxv = rec_n * KB * 4;
  u32x4 xs[kXPer];
#pragma unroll
  for (int q = 0; q < kXPer; ++q) {
    const int v = min((int)threadIdx.x + q * DC_THREADS, nxv - 1);
    const int n = v / (KB * 4), r = v - n * (KB * 4);
    xs[q] = ld128(a.x + (size_t)prec_tok(rec, n) * H + 8 * r);
  }
  __builtin_amdgcn_sched_barrier(0);
  // this wave's rows: intermediate indices jb + 4q + g (g = lane / 16)
  const int g = lane >> 4, j = lane & 15;
  const int jb = (blockIdx.x * DC_WAVES + wave) * 4 * Q;   // waves past I load clamped rows and skip the math
  const int row_q = H / 2, row_s = KB;
  const uint8_t* wq = a.w13_q + (size_t)rec_e * 2 * I * row_q;
  const uint8_t* ws = a.w13_s + (size_t)rec_e * 2 * I * row_s;
  // the wave's scale bytes: 4Q gate rows then 4Q up rows (rows past I are
  // clamped; their results are not written)
  constexpr int kSVec = 2 * 4 * Q * KB / 16;        // uint4 of scales
  u32x4 sv[(kSVec + kWave - 1) / kWave];
#pragma unroll
  for (int i = 0; i < (kSVec + kWave - 1) / kWave; ++i) {
    const int v = min(lane + i * kWave, kSVec - 1);
    const int half = v / (kSVec / 2), r = v - half * (kSVec / 2);      // r: 16-byte piece within 4Q rows
    const int row = min(jb + (r * 16) / KB, I - 1) + half * I;
    const int col = (r * 16) % KB;
    sv[i] = ld128(ws + (size_t)row * row_s + col);
  }
  __builtin_amdgcn_sched_barrier(0);                // the scale loads go out before the code stream
  // per-token products: lane (g, j) takes rows jb + 4q + g, blocks c * 16 + j;
  // matrix cores: lane (r, kq) takes row r of the tile (gate rows jb .. jb + 7,
  // then the same up rows), blocks 4 i + kq
  constexpr int kMfLoads = MF ? KB / 4 : 1;
  constexpr int kDotQ = MF ? 1 : Q, kDotNB = MF ? 1 : NB;
  u32x4 cg[kDotQ][kDotNB], cu[kDotQ][kDotNB], cm[kMfLoads];
  const int mr = lane & 15, kq = lane >> 4;
  if constexpr (MF) {
    const int idx = min(jb + (mr & 7), I - 1);
    const uint8_t* rq = wq + (size_t)((mr >> 3) * I + idx) * row_q + kq * 16;
#pragma unroll
    for (int i = 0; i < kMfLoads; ++i) {
      cm[i] = ld128(rq + i * 64);
      __builtin_amdgcn_sched_barrier(0);            // issued in the order the products consume them
    }
  } else {
#pragma unroll
    for (int c = 0; c < NB; ++c)
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int idx = min(jb + 4 * q + g, I - 1);
        cg[q][c] = ld128(wq + (size_t)idx * row_q + c * 256 + j * 16);
        cu[q][c] = ld128(wq + (size_t)(I + idx) * row_q + c * 256 + j * 16);
        __builtin_amdgcn_sched_barrier(0);          // issued in the order the products consume them
      }
  }
  stamp<PROBE>(a.probe, kGuIssued);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < kXPer; ++q) {                 // x[n] (the record's n-th token): block b, quarter i
    const int v = min((int)threadIdx.x + q * DC_THREADS, nxv - 1);
    const int n = v / (KB * 4), r = v - n * (KB * 4);
    u32x4 u = xs[q];
    if constexpr (A8) {                             // a quad of threads holds one 32-element block
      uint4 t4 = make_uint4(u[0], u[1], u[2], u[3]);
      mxfp8_round_trip8_quad(t4);
      u = u32x4{t4.x, t4.y, t4.z, t4.w};
    }
    L.x[(n * 4 + (r & 3)) * KB + (r >> 2)] = u;
  }
  uint8_t* sl = &L.scales[wave][0][0];
#pragma unroll
  for (int i = 0; i < (kSVec + kWave - 1) / kWave; ++i)
    reinterpret_cast<u32x4*>(sl)[min(lane + i * kWave, kSVec - 1)] = sv[i];
  block_barrier_lds();                              // x and the scales staged; the codes stay in flight
  if constexpr (MF) {
    if (jb >= I) return;
    // column c of the tile: the record's token c (columns past its tokens
    // repeat token 0 and are not stored)
    const int c = lane & 15;
    const u32x4* xb = L.x + (size_t)((c < rec_n ? c : 0) * 4) * KB + kq;
    const uint8_t* sb = sl + mr * KB + kq;
    v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMfLoads; ++i) {
      const float sc = e8m0_to_f32(sb[4 * i]);
#pragma unroll
      for (int m = 0; m < 4; m += 2) {               // two accumulators: no chain of dependent products
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mxfp4_word_bf16x8(cm[i][m], sc),
                                                       __builtin_bit_cast(v8bf, xb[m * KB + 4 * i]), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mxfp4_word_bf16x8(cm[i][m + 1], sc),
                                                       __builtin_bit_cast(v8bf, xb[(m + 1) * KB + 4 * i]), acc1, 0,
                                                       0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);            // one block's operands at a time
      if (i == 0) stamp<PROBE>(a.probe, kGuFirstData);
    }
    // lanes 0..31 hold gate rows jb + 4 kq + e, lanes 32..63 the same up rows
    float gv[4], uv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gv[e] = acc0[e] + acc1[e];
      uv[e] = half_partner(gv[e]);
    }
    if (kq < 2 && c < rec_n) {
      const size_t o = (size_t)prec_hrow(rec, c) * I + jb + 4 * kq;   // 4 consecutive h elements
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {                 // h = hi + lo, two bf16 terms
        const float v = silu(gv[e]) * uv[e];
        hi[e] = f32_to_bf16_bits(v);
        lo[e] = f32_to_bf16_bits(v - bf16_bits_to_f32(hi[e]));
      }
      *reinterpret_cast<uint2*>(a.h + o) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
      *reinterpret_cast<uint2*>(a.hlo + o) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
    }
    stamp<PROBE>(a.probe, kGuDone);
    return;
  } else {
  // token n of the record; the first token is computed as the codes arrive,
  // later ones (multi-token experts) after an opaque barrier on the codes so
  // their decoding is redone per token rather than held in registers
  auto token = [&](int n) __attribute__((always_inline)) {
    const int hrow = prec_hrow(rec, n);
    float ag[Q], au[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) { ag[q] = 0.f; au[q] = 0.f; }
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      const int b = c * 16 + j;
      u32x4 xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = L.x[(n * 4 + i) * KB + b];
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float sgv = e8m0_to_f32(sl[(4 * q + g) * KB + b]);
        const float suv = e8m0_to_f32(sl[(4 * Q + 4 * q + g) * KB + b]);
        ag[q] = dot_block(cg[q][c], sgv, xv, ag[q]);
        au[q] = dot_block(cu[q][c], suv, xv, au[q]);
      }
      // one block column at a time: the next column's LDS reads are not
      // hoisted above this one's products (they would hold NB x 16 registers)
      __builtin_amdgcn_sched_barrier(0);
      if (c == 0 && n == 0) stamp<PROBE>(a.probe, kGuFirstData);
    }
    float gs[Q], us[Q];                             // every group sum before the first store
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      gs[q] = group_sum<16>(ag[q]);
      us[q] = group_sum<16>(au[q]);
    }
    if (j == 0) {
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int idx = jb + 4 * q + g;
        if (idx < I) {                              // h = hi + lo, two bf16 terms
          const float v = silu(gs[q]) * us[q];
          const uint32_t hi = f32_to_bf16_bits(v);
          const size_t o = (size_t)hrow * I + idx;
          a.h[o] = (uint16_t)hi;
          a.hlo[o] = (uint16_t)f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
        }
      }
    }
  };
  if (jb >= I) return;
  token(0);
  for (int n = 1; n < rec_n; ++n) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int c = 0; c < NB; ++c) { keep_in_loop(cg[q][c]); keep_in_loop(cu[q][c]); }
    token(n);
  }
  stamp<PROBE>(a.probe, kGuDone);
  }
}

// Roles of the gate/up grid rows: [shared row] [writer row] [R routed rows]
// (the writer is dispatched early: its loads then go out before the weight
// stream fills the memory queues).  C: experts per lane of the top-k; NB:
// H / 512; Q, A8, MF as for gateup_slot.
template <int C, int NB, int Q, bool A8, bool PROBE, bool MF>
__global__ __launch_bounds__(DC_THREADS) __attribute__((amdgpu_waves_per_eu(Q >= 2 ? 3 : 4, Q >= 2 ? 3 : 4)))
void decode_gateup_kernel(ForwardArgs a, RouteOut ro) {
  static_assert(Q >= 1 && Q <= 4, "quads");
  static_assert(!MF || Q == 2, "a matrix-core wave covers 8 row pairs");
  using Lds = GateupLds<NB, Q>;
  static_assert(sizeof(SmallSortLds<C, DC_MAXP>) <= sizeof(Lds::x), "the writer's sort state fits the x area");
  __shared__ __align__(16) Lds L;
  stamp<PROBE>(a.probe, kGuEntry);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int M = a.M, k = a.k, E = a.E, H = a.H;
  const int srow = a.has_shared ? 1 : 0;
  const bool writer = blockIdx.y == srow;
  const bool shared_row = a.has_shared && blockIdx.y == 0;
  {                                                // every workgroup zeroes a share of y (down adds into it)
    const size_t nblk = (size_t)gridDim.x * gridDim.y;
    const size_t b = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    for (size_t i = b * DC_THREADS + threadIdx.x; i < (size_t)M * H; i += nblk * DC_THREADS) a.y[i] = 0.f;
  }
  DecRec* recs = reinterpret_cast<DecRec*>(const_cast<SlotRec*>(a.rec));

  if (writer) {
    // the ABI's routing outputs: top-k of every token, the stable sort by
    // expert, and the header's path counters
    if (blockIdx.x != 0) return;
    SmallSortLds<C, DC_MAXP>& W = *reinterpret_cast<SmallSortLds<C, DC_MAXP>*>(L.x);
    if (wave < M) route_token<C>(ro.logits, wave, E, k, L.topk[wave], W.ids, W.w, W.tok);
    __syncthreads();
    const int N = M * k;
    if (wave == 0) wave_sort_small(W, N, E, ro.ebits);
    __syncthreads();
    block_store_small_sort(W, N, E, ro.topk_ids, ro.topk_weights, ro.offsets, ro.sorted_pairs, ro.active,
                           ro.num_active);
    if (threadIdx.x == 0) {
      a.hdr->gemv_experts = W.na + a.has_shared;
      a.hdr->mfma_experts = 0;
      a.hdr->mfma_items = 0;
      a.hdr->mt_experts = 0;
      if (!a.has_shared) recs[0].e = -1;            // record 0 is the shared expert's
    }
    stamp<PROBE>(a.probe, kGuDone);
    return;
  }

  // routing first: the logits are each routing wave's first load
  const int slot = (int)blockIdx.y - srow - 1;      // routed rows
  if (M == 1) {
    // one token: slot s is its expert of rank s; only the record's writer
    // (block column 0) needs the weight
    if (!shared_row && wave == 0) {
      int e;
      float w;
      wave_topk_pick<C, PROBE>(ro.logits, E, k, slot, blockIdx.x == 0, L.topk[0], e, w, a.probe);
      if (lane == 0) {
        L.ids[0] = e;
        L.w[0] = w;
      }
    }
  } else {
    if (!shared_row)
      for (int i = threadIdx.x; i < E; i += DC_THREADS) L.owner[i] = 0x7FFFFFFF;
    if (!shared_row && wave < M)
      route_token<C, PROBE>(ro.logits, wave, E, k, L.topk[wave], L.ids, L.w, nullptr, wave == 0 ? a.probe : nullptr);
  }
  if (!shared_row) __syncthreads();
  stamp<PROBE>(a.probe, kGuRouted);
  PRec rec;
  if (shared_row) {
    shared_record(M, k, E, rec);
  } else if (M == 1) {
    const int tok[4] = {0, 0, 0, 0}, hrow[4] = {slot, 0, 0, 0};
    const float wt[4] = {L.w[0], 0.f, 0.f, 0.f};
    prec_pack(rec, L.ids[0], 1, tok, wt, hrow);
  } else {
    routed_record(L.ids, L.w, L.owner, M, k, E, slot, rec);
  }
  // record 0: the shared expert; record 1 + s: routed slot s (grid row srow + 1 + s)
  if (blockIdx.x == 0 && lane == 0 && wave == 0) prec_store(&recs[shared_row ? 0 : (int)blockIdx.y - srow], rec);
  stamp<PROBE>(a.probe, kGuSlot);
  if (prec_e(rec) < 0) return;                      // no expert in this slot (uniform over the block)
  gateup_slot<NB, Q, A8, PROBE, MF>(a, L, rec);
}

// --------------------------------------------------------------- down --
// Workgroup (64 output rows, record y); wave: 16 rows as two 8-row groups,
// lane (g8 = lane / 8, j8 = lane % 8) takes row r0 + 8 rg + g8, blocks
// j8 + 8c of its I / 32.  The record's h rows (hi and lo) are staged in LDS
// as [token][term][quarter][block] uint4.
template <int NBD>
struct DownLds {
  static constexpr int kBlocks = NBD * 8;                   // I / 32
  u32x4 h[kRoutedMaxTokens * 2 * 4 * kBlocks];
  uint8_t scales[DC_WAVES][8 * DN_RG][kBlocks];
};

// MF: the products on the matrix cores: a wave's 16 rows are the 16 rows of
// one tile; column t < 4 is token t's hi term of h, column 7 - t its lo term
// (so a half-row mirror adds the two), each weight decoded once for all
// tokens.  Otherwise per-token v_dot2 products.
// One record's down work for this workgroup's 64 output rows: h (both terms)
// and the scale bytes staged in LDS, the code words in flight, products as
// they arrive.  ROWS: each pair's weighted row goes to its own partial row of
// yp (hrow order; a combine kernel sums them); otherwise fp32 atomics into y.
template <int NBD, bool PROBE, bool MF, bool ROWS>
__device__ __forceinline__ void down_slot(const ForwardArgs& a, DownLds<NBD>& L, const PRec& rec) {
  constexpr int KB = NBD * 8;                      // blocks per row (I / 32)
  const int rec_e = prec_e(rec), rec_n = prec_n(rec);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int H = a.H, I = a.I;
  const int g8 = lane >> 3, j8 = lane & 7;
  const int r0 = blockIdx.x * DN_ROWS_WG + wave * 8 * DN_RG;
  const int row_q = I / 2, row_s = KB;
  const uint8_t* wq = a.w2_q + (size_t)rec_e * H * row_q;
  const uint8_t* ws = a.w2_s + (size_t)rec_e * H * row_s;
  // h of the record's tokens (hi, lo): issued first, consumed first
  constexpr int kHVec = kRoutedMaxTokens * 2 * KB * 4;
  constexpr int kHPer = (kHVec + DC_THREADS - 1) / DC_THREADS;
  const int nhv = rec_n * 2 * KB * 4;
  u32x4 hv[kHPer];
#pragma unroll
  for (int i = 0; i < kHPer; ++i) {
    const int v = min((int)threadIdx.x + i * DC_THREADS, nhv - 1);
    const int tq = v / (2 * KB * 4), r = v - tq * (2 * KB * 4);
    const int term = r / (KB * 4), u = r - term * (KB * 4);
    const uint16_t* src = (term ? a.hlo : a.h) + (size_t)prec_hrow(rec, tq) * I;
    hv[i] = ld128(src + 8 * u);
  }
  // scale bytes of the wave's 32 rows: one contiguous range (clamped to the
  // expert's last 16 bytes; rows past H are never used)
  constexpr int kSVec = 8 * DN_RG * KB / 16;
  u32x4 sv[(kSVec + kWave - 1) / kWave];
#pragma unroll
  for (int i = 0; i < (kSVec + kWave - 1) / kWave; ++i) {
    const size_t off = (size_t)r0 * row_s + 16 * (size_t)min(lane + i * kWave, kSVec - 1);
    sv[i] = ld128(ws + min(off, (size_t)H * row_s - 16));
  }
  __builtin_amdgcn_sched_barrier(0);                // h and the scales go out before the code stream
  constexpr int kMfLoads = MF ? KB / 4 : 1;
  u32x4 c[MF ? 1 : DN_RG][MF ? 1 : NBD], cm[kMfLoads];
  const int mr = lane & 15, kq = lane >> 4;
  if constexpr (MF) {                               // lane (mr, kq): row r0 + mr, blocks 4 i + kq
    const uint8_t* rq = wq + (size_t)min(r0 + mr, H - 1) * row_q + kq * 16;
#pragma unroll
    for (int i = 0; i < kMfLoads; ++i) {
      cm[i] = ld128(rq + i * 64);
      __builtin_amdgcn_sched_barrier(0);            // issued in the order the products consume them
    }
  } else {
#pragma unroll
    for (int cc = 0; cc < NBD; ++cc)
#pragma unroll
      for (int rg = 0; rg < DN_RG; ++rg) {
        const int row = min(r0 + 8 * rg + g8, H - 1);
        c[rg][cc] = ld128(wq + (size_t)row * row_q + cc * 128 + j8 * 16);
        __builtin_amdgcn_sched_barrier(0);          // issued in the order the products consume them
      }
  }
  stamp<PROBE>(a.probe, kDnIssued);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kHPer; ++i) {                 // unconditional stores (clamped, as the loads)
    const int v = min((int)threadIdx.x + i * DC_THREADS, nhv - 1);
    const int tq = v / (2 * KB * 4), r = v - tq * (2 * KB * 4);
    const int term = r / (KB * 4), u = r - term * (KB * 4);
    L.h[((tq * 2 + term) * 4 + (u & 3)) * KB + (u >> 2)] = hv[i];
  }
  uint8_t* sl = &L.scales[wave][0][0];
#pragma unroll
  for (int i = 0; i < (kSVec + kWave - 1) / kWave; ++i)
    reinterpret_cast<u32x4*>(sl)[min(lane + i * kWave, kSVec - 1)] = sv[i];
  block_barrier_lds();                              // h staged; the weight codes stay in flight
  if (r0 >= H) return;
  if constexpr (MF) {
    const int col = lane & 15;
    const bool lo_col = col >= 4 && col < 8;
    const int tq = min(col < 4 ? col : (lo_col ? 7 - col : 0), rec_n - 1);
    const u32x4* hb = L.h + (size_t)((tq * 2 + (lo_col ? 1 : 0)) * 4) * KB + kq;
    const uint8_t* sb = sl + mr * KB + kq;
    v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMfLoads; ++i) {
      const float sc = e8m0_to_f32(sb[4 * i]);
#pragma unroll
      for (int m = 0; m < 4; m += 2) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mxfp4_word_bf16x8(cm[i][m], sc),
                                                       __builtin_bit_cast(v8bf, hb[m * KB + 4 * i]), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mxfp4_word_bf16x8(cm[i][m + 1], sc),
                                                       __builtin_bit_cast(v8bf, hb[(m + 1) * KB + 4 * i]), acc1, 0,
                                                       0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (i == 0) stamp<PROBE>(a.probe, kDnFirstData);
    }
    float v[4];                                     // rows r0 + 4 kq + e: hi + lo of token col
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = acc0[e] + acc1[e];
      v[e] = d + __uint_as_float(dpp_half_mirror(__float_as_uint(d)));
    }
    if (col < rec_n) {
      const int t = prec_tok(rec, col);
      const float wt = prec_w(rec, col);
      if constexpr (ROWS) {                         // rows r0 + 4 kq .. + 3 of the pair's partial row
        float* yr = a.yp + (size_t)prec_hrow(rec, col) * H + r0 + 4 * kq;
        *reinterpret_cast<float4*>(yr) = make_float4(wt * v[0], wt * v[1], wt * v[2], wt * v[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = r0 + 4 * kq + e;
          if (row < H) unsafeAtomicAdd(&a.y[(size_t)t * H + row], wt * v[e]);
        }
      }
    }
    stamp<PROBE>(a.probe, kDnDone);
    return;
  } else {
  auto token = [&](int n) __attribute__((always_inline)) {   // as in the gate/up kernel

    const int t = prec_tok(rec, n);
    const float wt = prec_w(rec, n);
    float acc[DN_RG];
#pragma unroll
    for (int rg = 0; rg < DN_RG; ++rg) acc[rg] = 0.f;
#pragma unroll
    for (int cc = 0; cc < NBD; ++cc) {
      const int b = cc * 8 + j8;
      u32x4 hh[4], hl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hh[i] = L.h[((n * 2 + 0) * 4 + i) * KB + b];
        hl[i] = L.h[((n * 2 + 1) * 4 + i) * KB + b];
      }
#pragma unroll
      for (int rg = 0; rg < DN_RG; ++rg) {
        const float sc = e8m0_to_f32(sl[(8 * rg + g8) * KB + b]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t ah[4] = {hh[i][0], hh[i][1], hh[i][2], hh[i][3]};
          const uint32_t al[4] = {hl[i][0], hl[i][1], hl[i][2], hl[i][3]};
          acc[rg] = dot8_mxfp4_bf16_2t(c[rg][cc][i], sc, ah, al, acc[rg]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);            // one block column's h at a time
      if (cc == 0 && n == 0) stamp<PROBE>(a.probe, kDnFirstData);
    }
    // every group sum before the first store: a store's branch would
    // otherwise split the row groups' products apart and keep h live across it
    float v[DN_RG];
#pragma unroll
    for (int rg = 0; rg < DN_RG; ++rg) v[rg] = group_sum<8>(acc[rg]);
    if (j8 == 0) {
#pragma unroll
      for (int rg = 0; rg < DN_RG; ++rg) {
        const int row = r0 + 8 * rg + g8;
        if constexpr (ROWS) {
          if (row < H) a.yp[(size_t)prec_hrow(rec, n) * H + row] = wt * v[rg];
        } else {
          if (row < H) unsafeAtomicAdd(&a.y[(size_t)t * H + row], wt * v[rg]);
        }
      }
    }
  };
  token(0);
  for (int n = 1; n < rec_n; ++n) {
#pragma unroll
    for (int rg = 0; rg < DN_RG; ++rg)
#pragma unroll
      for (int cc = 0; cc < NBD; ++cc) keep_in_loop(c[rg][cc]);
    token(n);
  }
  stamp<PROBE>(a.probe, kDnDone);
  }
}

template <int NBD, bool PROBE, bool MF>
__global__ __launch_bounds__(DC_THREADS) __attribute__((amdgpu_waves_per_eu(6, 6)))
void decode_down_kernel(ForwardArgs a) {
  __shared__ __align__(16) DownLds<NBD> L;
  stamp<PROBE>(a.probe, kDnEntry);
  PRec rec;
  prec_load(reinterpret_cast<const DecRec*>(a.rec) + blockIdx.y, rec);
  if (prec_e(rec) < 0) return;
  stamp<PROBE>(a.probe, kDnRecord);
  down_slot<NBD, PROBE, MF, false>(a, L, rec);
}

// ------------------------------------------------------------- batches --
// Batch experts with one or two tokens (the GEMV list that the sort epilogue
// builds) at H = 2560, I = 768: the decode kernels' slot work, driven by the
// records instead of the routing.  Grid row y takes list entries y, y + rows,
// ...: a grid of two residency rounds, not one row per possible slot.

// The record of a batch slot (SlotRec: e, n, first sorted position, first h
// row, 4 tokens, 4 weights) as a decode record; h rows are consecutive.
__device__ __forceinline__ void prec_from_slot(const SlotRec* src, PRec& r) {
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  const u32x4 a = p[0], t = p[1], w = p[2];
  const unsigned h0 = a[3];
  r.a = u32x4{a[0], a[1], t[0], t[1]};
  r.b = u32x4{t[2], t[3], w[0], w[1]};
  r.c = u32x4{w[2], w[3], h0, h0 + 1u};
  r.d = u32x4{h0 + 2u, h0 + 3u, 0u, 0u};
}

template <int NB>
__global__ __launch_bounds__(DC_THREADS) __attribute__((amdgpu_waves_per_eu(3, 3)))
void batch_gateup_kernel(ForwardArgs a) {
  __shared__ __align__(16) GateupLds<NB, 2> L;
  if (!a.yp) {                                     // atomics into y: every workgroup zeroes a share
    const size_t nblk = (size_t)gridDim.x * gridDim.y;
    const size_t b = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    for (size_t i = b * DC_THREADS + threadIdx.x; i < (size_t)a.M * a.H; i += nblk * DC_THREADS) a.y[i] = 0.f;
  }
  const int n = a.hdr->gemv_experts;
  for (int y = blockIdx.y; y < n; y += gridDim.y) {
    PRec rec;
    prec_from_slot(a.rec + a.lists[y], rec);
    if (prec_e(rec) >= 0 && prec_n(rec) <= kRoutedMaxTokens)   // uniform over the workgroup
      gateup_slot<NB, 2, false, false, true>(a, L, rec);
    __syncthreads();                               // the next slot restages x and the scales
  }
}

template <int NBD, bool ROWS>
__global__ __launch_bounds__(DC_THREADS) __attribute__((amdgpu_waves_per_eu(6, 6)))
void batch_down_kernel(ForwardArgs a) {
  __shared__ __align__(16) DownLds<NBD> L;
  const int n = a.hdr->gemv_experts;
  for (int y = blockIdx.y; y < n; y += gridDim.y) {
    PRec rec;
    prec_from_slot(a.rec + a.lists[y], rec);
    if (prec_e(rec) >= 0 && prec_n(rec) <= kRoutedMaxTokens)
      down_slot<NBD, false, true, ROWS>(a, L, rec);
    __syncthreads();
  }
}

// -------------------------------------------------------------- launch --
namespace {

template <int C, int NB, int Q, bool PROBE>
void* gateup_instance(bool a8) {
  constexpr bool MF = Q == 2;                       // batches of 2-4 tokens: matrix cores
  return a8 ? reinterpret_cast<void*>(decode_gateup_kernel<C, NB, Q, true, PROBE, MF>)
            : reinterpret_cast<void*>(decode_gateup_kernel<C, NB, Q, false, PROBE, MF>);
}

// Instances: H = 2560 (5 blocks of 512 per row) with I = 768 (3 blocks of
// 256), the Ling layer; the routing takes 8 or 16 experts per lane.
template <bool PROBE>
void* pick_gateup(int E, int H, int Q, bool a8) {
  if (H != 2560) return nullptr;
  const bool c8 = topk_lane_experts(E) == 8;
  if (Q == 1) return c8 ? gateup_instance<8, 5, 1, PROBE>(a8) : gateup_instance<16, 5, 1, PROBE>(a8);
  return c8 ? gateup_instance<8, 5, 2, PROBE>(a8) : gateup_instance<16, 5, 2, PROBE>(a8);
}

// One token: per-token dot products (the matrix-core tile would be 1/16
// used); 2-4 tokens: matrix cores.
template <bool PROBE>
void* pick_down(int I, int M) {
  if (I != 768) return nullptr;
  return M >= 2 ? reinterpret_cast<void*>(decode_down_kernel<3, PROBE, true>)
                : reinterpret_cast<void*>(decode_down_kernel<3, PROBE, false>);
}

}  // namespace

bool decode_fast_fits(int M, int H, int I) {
  return M >= 1 && M <= kRoutedMaxTokens && pick_gateup<false>(512, H, 1, false) && pick_down<false>(I, M);
}

namespace {
int decode_quads(int M) { return M == 1 ? 1 : 2; }
dim3 decode_gateup_grid(int M, int k, int E, int I, int has_shared) {
  const int Q = decode_quads(M);
  return dim3((I + 16 * Q - 1) / (16 * Q), (has_shared ? 1 : 0) + (max_slots(M, k, E) - 1) + 1);
}
dim3 decode_down_grid(int M, int k, int E, int H) {
  return dim3((H + DN_ROWS_WG - 1) / DN_ROWS_WG, max_slots(M, k, E));
}
}  // namespace

size_t decode_probe_stamps(int M, int k, int E, int H, int I, int has_shared) {
  const dim3 g = decode_gateup_grid(M, k, E, I, has_shared), d = decode_down_grid(M, k, E, H);
  const size_t n = (size_t)g.x * g.y > (size_t)d.x * d.y ? (size_t)g.x * g.y : (size_t)d.x * d.y;
  return n * kProbeStamps;
}

bool batch_decode_fits(const ForwardArgs& a) {
  return a.lists != nullptr && a.H == 2560 && a.I == 768 && a.mt_min <= kRoutedMaxTokens + 1;
}

hipError_t launch_decode_batch(const ForwardArgs& a, hipStream_t s, const Timing& tm, hipEvent_t zeroed,
                               int cus) {
  const int slots = max_slots(a.M, a.k, a.E) - 1 + (a.has_shared ? 1 : 0);
  const dim3 b(DC_THREADS);
  const int gx = a.I / 32, dx = (a.H + DN_ROWS_WG - 1) / DN_ROWS_WG;
  const int gfit = (2 * 3 * cus + gx - 1) / gx, dfit = (2 * 6 * cus + dx - 1) / dx;   // two residency rounds
  const dim3 gg(gx, slots < gfit ? slots : gfit), gd(dx, slots < dfit ? slots : dfit);
  void* args[] = {const_cast<ForwardArgs*>(&a)};
  hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(batch_gateup_kernel<5>), gg, b, args, 0, s,
                                    tm.gu_start, tm.gu_stop, 0);
  if (e != hipSuccess) return e;
  if (zeroed && (e = hipEventRecord(zeroed, s)) != hipSuccess) return e;   // y is zeroed from here on
  if (a.act8 && (e = launch_h_round_trip(a, 0, s)) != hipSuccess) return e;
  const void* dn = a.yp ? reinterpret_cast<const void*>(batch_down_kernel<3, true>)
                        : reinterpret_cast<const void*>(batch_down_kernel<3, false>);
  return hipExtLaunchKernel(dn, gd, b, args, 0, s, tm.dn_start, tm.dn_stop, 0);
}

hipError_t launch_decode(const ForwardArgs& a, const RouteOut& r, hipStream_t s, const Timing& tm, bool probe) {
  const int Q = decode_quads(a.M);
  void* gu = probe ? pick_gateup<true>(a.E, a.H, Q, a.act8 != 0) : pick_gateup<false>(a.E, a.H, Q, a.act8 != 0);
  void* dn = probe ? pick_down<true>(a.I, a.M) : pick_down<false>(a.I, a.M);
  if (!gu || !dn) return hipErrorInvalidValue;
  // gate/up rows: [shared] [writer] [routed slots]; down rows: the records
  const dim3 ggu = decode_gateup_grid(a.M, a.k, a.E, a.I, a.has_shared), bgu(DC_THREADS);
  const dim3 gdn = decode_down_grid(a.M, a.k, a.E, a.H), bdn(DC_THREADS);
  void* gu_args[] = {const_cast<ForwardArgs*>(&a), const_cast<RouteOut*>(&r)};
  hipError_t e = hipExtLaunchKernel(gu, ggu, bgu, gu_args, 0, s, tm.gu_start, tm.gu_stop, 0);
  if (e != hipSuccess) return e;
  if (a.act8 && (e = launch_mxfp8_round_trip_rows(a.h, a.hlo, (int64_t)a.M * a.k + a.M, a.I, s)) != hipSuccess)
    return e;
  void* dn_args[] = {const_cast<ForwardArgs*>(&a)};
  return hipExtLaunchKernel(dn, gdn, bdn, dn_args, 0, s, tm.dn_start, tm.dn_stop, 0);
}

}  // namespace moe
