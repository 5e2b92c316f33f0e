// Stable counting sort of the (token, slot) pairs by expert (MoE-SpeQ article,
// section 4.2: gather every token's expert assignments, order them by expert
// id and run each expert once over its tokens).  One workgroup does it all in
// LDS: per-wave histograms, an exclusive scan over experts, then each wave
// places its own segment of pairs in order.  Stability comes from three
// facts: waves own consecutive segments, a wave walks its segment in order in
// 64-pair steps, and inside a step a pair's rank is the number of lower lanes
// holding the same expert (found with one ballot per expert-id bit).
#pragma once

#include "kernels.h"

namespace moe {

// Inclusive prefix sum over the wave: Hillis-Steele inside each 16-lane row
// with DPP row shifts (lanes whose source falls outside the row add 0), then
// the row totals carried across rows with readlane.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  if (lane >= 16) v += r0;
  if (lane >= 32) v += r1;
  if (lane >= 48) v += r2;
  return v;
}

// Ints of LDS block_sort_pairs needs with nw waves and E experts.
__host__ __device__ inline size_t sort_lds_ints(int nw, int E) { return (size_t)nw * E + E + 1 + 2 * nw; }

// Sort `N` pairs whose expert ids are ids[0..N) (global or LDS).  Uses
// sort_lds_ints(nw, E) ints of LDS at `lds`; every thread of the block calls it.
// With sp_lds / act_lds / na_lds non-null it also keeps sorted_pairs, the
// active list and D in LDS (for an epilogue in the same block); the pairs are
// then placed in LDS and sorted_pairs goes out in one coalesced copy (one
// workgroup's scattered 4-byte stores would queue behind each other in its
// CU's memory pipeline).  With inv_lds non-null, inv_lds[p] receives the
// sorted position of pair p (-1 for a dropped id).  The exclusive offsets
// (E + 1 of them) stay at lds + nw*E after the call.
__device__ inline void block_sort_pairs(const int* ids, int N, int E, int ebits, int* lds,
                                 int* __restrict__ offsets, int* __restrict__ sorted_pairs,
                                 int* __restrict__ active, int* __restrict__ num_active,
                                 int* sp_lds = nullptr, int* act_lds = nullptr, int* na_lds = nullptr,
                                 int* inv_lds = nullptr) {
  const int nw = blockDim.x / kWave;
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int bd = blockDim.x;
  int* cnt = lds;                 // [nw][E]: per-wave counts, then per-wave running bases
  int* off = cnt + nw * E;        // [E + 1]: exclusive offsets of each expert
  int* wtot = off + E + 1;        // [2 * nw]: per-wave scan totals

  for (int i = threadIdx.x; i < nw * E; i += bd) cnt[i] = 0;
  __syncthreads();

  const int seg = (N + nw - 1) / nw;
  const int beg = min(N, w * seg), end = min(N, beg + seg);
  for (int p = beg + lane; p < end; p += kWave) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[w * E + e], 1);   // invalid ids are dropped
  }
  __syncthreads();

  // Each thread owns a contiguous span of experts: total count per expert and
  // the exclusive prefix over waves (stored back in place as wave bases).
  const int per = (E + bd - 1) / bd;
  const int e0 = min(E, threadIdx.x * per), e1 = min(E, e0 + per);
  int csum = 0, asum = 0;
  for (int e = e0; e < e1; ++e) {
    int run = 0;
    for (int v = 0; v < nw; ++v) {
      const int c = cnt[v * E + e];
      cnt[v * E + e] = run;
      run += c;
    }
    off[e] = run;                  // total, turned into an offset below
    csum += run;
    asum += run > 0;
  }
  // Block-wide exclusive scan of (count, active flag) over the thread spans.
  const int cinc = wave_inclusive_scan(csum);
  const int ainc = wave_inclusive_scan(asum);
  if (lane == kWave - 1) { wtot[w] = cinc; wtot[nw + w] = ainc; }
  __syncthreads();
  int cbase = cinc - csum, abase = ainc - asum;
  for (int v = 0; v < w; ++v) { cbase += wtot[v]; abase += wtot[nw + v]; }
  for (int e = e0; e < e1; ++e) {
    const int c = off[e];
    off[e] = cbase;
    offsets[e] = cbase;
    if (c > 0) {
      if (act_lds) act_lds[abase] = e;
      active[abase++] = e;
    }
    cbase += c;
  }
  if (threadIdx.x == bd - 1) {
    offsets[E] = cbase;            // == number of valid pairs
    off[E] = cbase;
    *num_active = abase;
    if (na_lds) *na_lds = abase;
  }
  __syncthreads();

  // Placement: wave w walks its segment in order, 64 pairs per step.
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int base = beg; base < end; base += kWave) {
    const int p = base + lane;
    int e = (p < end) ? ids[p] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    if (!valid) e = 0;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(valid && bit);
      match &= bit ? bal : ~bal;
    }
    if (valid) {
      const int rank = __popcll(match & lt_mask);
      const int pos = off[e] + cnt[w * E + e] + rank;
      if (sp_lds)
        sp_lds[pos] = p;
      else
        sorted_pairs[pos] = p;
      if (inv_lds) inv_lds[p] = pos;
      __builtin_amdgcn_wave_barrier();
      if (rank == 0) cnt[w * E + e] += __popcll(match);
    } else if (inv_lds && p < end) {
      inv_lds[p] = -1;
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (sp_lds) {
    block_barrier_lds();
    const int nvalid = off[E];
    for (int i = threadIdx.x; i < nvalid; i += bd) sorted_pairs[i] = sp_lds[i];
  }
}

// Slot record of `slot` from a finished sort: slots [0, D) are the active
// experts in increasing order, slot D the shared expert (if any), later slots
// have no work (e = -1).  off = exclusive offsets (E+1 entries), sp = sorted
// pairs, act = active list, w = routing weights of the pairs (LDS or global).
__device__ __forceinline__ SlotRec make_slot_record(int slot, int D, const int* off, const int* sp,
                                                    const int* act, const float* w, int M, int k, int E,
                                                    int has_shared) {
  SlotRec r;
  r.pad[0] = r.pad[1] = r.pad[2] = r.pad[3] = 0;
  if (slot < D) {
    r.e = act[slot];
    r.pbeg = off[r.e];
    r.n = off[r.e + 1] - r.pbeg;
    r.hrow0 = r.pbeg;
#pragma unroll
    for (int q = 0; q < kRecTokens; ++q) {
      const int pair = (q < r.n) ? sp[r.pbeg + q] : 0;
      r.tok[q] = (q < r.n) ? pair / k : 0;
      r.w[q] = (q < r.n) ? w[pair] : 0.f;
    }
  } else if (slot == D && has_shared) {
    r.e = E; r.pbeg = -1; r.n = M; r.hrow0 = M * k;
#pragma unroll
    for (int q = 0; q < kRecTokens; ++q) { r.tok[q] = q < M ? q : 0; r.w[q] = 1.f; }
  } else {
    r.e = -1; r.pbeg = -1; r.n = 0; r.hrow0 = 0;
#pragma unroll
    for (int q = 0; q < kRecTokens; ++q) { r.tok[q] = 0; r.w[q] = 0.f; }
  }
  return r;
}

// Expert and token count of `slot` (the first fields of its record), without
// the per-token fields.
__device__ __forceinline__ void slot_expert_tokens(int slot, int D, const int* off, const int* act, int M, int E,
                                                   int has_shared, int& e, int& n) {
  if (slot < D) {
    e = act[slot];
    n = off[e + 1] - off[e];
  } else if (slot == D && has_shared) {
    e = E;
    n = M;
  } else {
    e = -1;
    n = 0;
  }
}

// Path of an expert with n tokens: 0 GEMV, 1 few-token matrix cores, 2 MFMA.
__device__ __forceinline__ int expert_path(int n, int mt_min, int mt_max, int mfma_min) {
  return n >= mfma_min ? 2 : (n >= mt_min && n <= mt_max) ? 1 : 0;
}

// Slot records from the finished sort (offsets with E + 1 entries, sorted
// pairs, active list and D: in LDS, or in global memory this block wrote and a
// barrier made visible).  Thread i handles a contiguous span of slots.  With
// ro.lists: the slots of the GEMV experts at lists[0..), of the few-token
// experts at lists[nslots..), in slot order.  Then the path counters in the header and, with the MFMA path on,
// its work items: (slot, 64-token tile) for every slot with at least
// ro.mfma_min tokens, in slot order.  `lds` holds 4 * waves + 4 ints.
// `inv_src` (optional): the sorted position of every pair (-1: dropped), as
// block_sort_pairs leaves it in LDS; ro.inv is then a coalesced copy of it.
__device__ inline void block_write_slot_records(const RecOut& ro, int E, int nslots,
                                                const int* __restrict__ offsets,
                                                const int* __restrict__ sorted_pairs,
                                                const int* __restrict__ active,
                                                const int* __restrict__ num_active, int* lds,
                                                const int* inv_src = nullptr) {
  const int D = *num_active;
  const int bd = blockDim.x, tid = threadIdx.x;
  if (ro.inv) {   // sorted position of every flattened pair (-1: dropped id)
    const int N = ro.M * ro.k;
    if (inv_src) {
      for (int i = tid; i < N; i += bd) ro.inv[i] = inv_src[i];
    } else {
      const int nvalid = offsets[E];
      for (int i = tid; i < N; i += bd) ro.inv[i] = -1;
      __threadfence_block();
      __syncthreads();
      for (int i = tid; i < nvalid; i += bd) ro.inv[sorted_pairs[i]] = i;
    }
  }
  const int per = (nslots + bd - 1) / bd;
  const int s0 = min(nslots, tid * per), s1 = min(nslots, s0 + per);
  int tiles = 0, cnt[3] = {0, 0, 0};
  for (int slot = s0; slot < s1; ++slot) {
    const SlotRec r = make_slot_record(slot, D, offsets, sorted_pairs, active, ro.topk_weights, ro.M, ro.k, E,
                                       ro.has_shared);
    ro.rec[slot] = r;
    if (r.e < 0) continue;
    const int path = expert_path(r.n, ro.mt_min, ro.mt_max, ro.mfma_min);
    ++cnt[path];
    if (path == 2) tiles += (r.n + kMfmaTileTokens - 1) / kMfmaTileTokens;
  }
  if (!ro.hdr) return;
  // block-wide exclusive scan of the tile counts (thread spans are in slot
  // order) and block sums of the path counts
  const int lane = tid & (kWave - 1), w = tid / kWave, nw = bd / kWave;
  const int inc = wave_inclusive_scan(tiles);
  int csum[3];
#pragma unroll
  for (int p = 0; p < 3; ++p) csum[p] = wave_inclusive_scan(cnt[p]);
  if (lane == kWave - 1) {
    lds[w] = inc;
#pragma unroll
    for (int p = 0; p < 3; ++p) lds[nw * (p + 1) + w] = csum[p];
  }
  __syncthreads();
  int base = inc - tiles, tot[3] = {0, 0, 0}, pbase[3];
#pragma unroll
  for (int p = 0; p < 3; ++p) pbase[p] = csum[p] - cnt[p];
  for (int v = 0; v < nw; ++v) {
    if (v < w) base += lds[v];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      tot[p] += lds[nw * (p + 1) + v];
      if (v < w) pbase[p] += lds[nw * (p + 1) + v];
    }
  }
  if (ro.lists) {   // the GEMV and few-token experts' slots, each list in slot order
    for (int slot = s0; slot < s1; ++slot) {
      int e, n;
      slot_expert_tokens(slot, D, offsets, active, ro.M, E, ro.has_shared, e, n);
      if (e < 0) continue;
      const int path = expert_path(n, ro.mt_min, ro.mt_max, ro.mfma_min);
      if (path == 0) ro.lists[pbase[0]++] = slot;
      if (path == 1) ro.lists[nslots + pbase[1]++] = slot;
    }
  }
  if (ro.items) {
    for (int slot = s0; slot < s1; ++slot) {
      int e, n;
      slot_expert_tokens(slot, D, offsets, active, ro.M, E, ro.has_shared, e, n);
      if (e < 0 || n < ro.mfma_min) continue;
      for (int t = 0; t * kMfmaTileTokens < n; ++t) ro.items[base++] = make_int2(slot, t);
    }
  }
  if (tid == bd - 1) {
    ro.hdr->mfma_items = ro.items ? base : 0;
    ro.hdr->gemv_experts = tot[0];
    ro.hdr->mt_experts = tot[1];
    ro.hdr->mfma_experts = tot[2];
  }
}

// LDS state of the small sort (decode batches): MAXP pairs at most, E <= 64*C.
// Lane l owns experts [l*C, l*C + C) of the per-expert arrays and moves them
// with 16-byte accesses (a 4-byte access at a stride of C words would hit a
// few banks only).  Index kSink of the per-pair arrays absorbs the writes of
// lanes with nothing to write.
template <int C, int MAXP>
struct SmallSortLds {
  static constexpr int kExp = kWave * C;   // experts covered (>= E)
  static constexpr int kSink = MAXP;
  __align__(16) int cur[kExp + 4];          // histogram, then running positions; [kExp] = sink
  __align__(16) int off[kExp + 4];          // exclusive offsets; off[E] = valid pairs
  __align__(16) int pslot[kExp + 4];        // active experts below each expert
  int ids[MAXP];                            // input: expert of each pair
  float w[MAXP];                            // input: routing weight of each pair
  int tok[MAXP];                            // input: token of each pair
  int sp[MAXP + 1];                         // sorted pairs
  int stok[MAXP + 1];                       // their tokens
  float sw[MAXP + 1];                       // their weights
  int act[MAXP];                            // active experts in increasing order
  int act_beg[MAXP];                        // first sorted position of each
  int act_n[MAXP];                          // pairs of each
  int na;                                   // active experts
  int nvalid;                               // pairs with a valid expert
};

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Stable counting sort of the N pairs in L.ids by one wave (N <= MAXP).  Lane
// l owns experts [l*C, l*C + C): histogram with LDS atomics, a per-lane scan
// of its counts, one wave scan of (count, present) packed in one int; pairs
// are then placed 64 at a time in order, a pair's rank among equal experts of
// its step coming from one ballot per expert-id bit, and the first pair of
// each expert writes its active-list entry.  Fills every other field of L.
template <int C, int MAXP>
__device__ inline void wave_sort_small(SmallSortLds<C, MAXP>& L, int N, int E, int ebits) {
  using S = SmallSortLds<C, MAXP>;
  static_assert(C % 4 == 0 && MAXP < 65536 && S::kExp < 65536, "packed scan");
  const int lane = threadIdx.x & (kWave - 1);
  int4* cur4 = reinterpret_cast<int4*>(&L.cur[lane * C]);
#pragma unroll
  for (int i = 0; i < C / 4; ++i) cur4[i] = make_int4(0, 0, 0, 0);
  wave_lds_fence();
  for (int base = 0; base < N; base += kWave) {
    const int p = base + lane;
    const int e = L.ids[min(p, N - 1)];
    const bool valid = p < N && (unsigned)e < (unsigned)E;        // invalid ids are dropped
    atomicAdd(&L.cur[valid ? e : S::kExp], 1);
  }
  wave_lds_fence();
  int c[C], tot = 0, pres = 0;
#pragma unroll
  for (int i = 0; i < C / 4; ++i) {
    const int4 v = cur4[i];
    c[4 * i] = v.x; c[4 * i + 1] = v.y; c[4 * i + 2] = v.z; c[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < C; ++i) { tot += c[i]; pres += c[i] > 0; }
  const int packed = tot | (pres << 16);
  const int inc = wave_inclusive_scan(packed);
  const int all = __builtin_amdgcn_readlane(inc, kWave - 1);
  int run = (inc - packed) & 0xFFFF, slot = (inc - packed) >> 16;
  int o[C], ps[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {     // experts past E have no pairs: their offset is the total
    o[i] = run;
    ps[i] = slot;
    run += c[i];
    slot += c[i] > 0;
  }
  int4* off4 = reinterpret_cast<int4*>(&L.off[lane * C]);
  int4* ps4 = reinterpret_cast<int4*>(&L.pslot[lane * C]);
#pragma unroll
  for (int i = 0; i < C / 4; ++i) {
    const int4 v = make_int4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    off4[i] = v;
    cur4[i] = v;
    ps4[i] = make_int4(ps[4 * i], ps[4 * i + 1], ps[4 * i + 2], ps[4 * i + 3]);
  }
  if (lane == 0) {
    L.off[S::kExp] = all & 0xFFFF;  // covers E == kExp
    L.na = all >> 16;
    L.nvalid = all & 0xFFFF;
  }
  wave_lds_fence();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int base = 0; base < N; base += kWave) {
    const int p = base + lane;
    const int pc = min(p, N - 1);
    const int e0 = L.ids[pc];
    const bool valid = p < N && (unsigned)e0 < (unsigned)E;
    const int e = valid ? e0 : 0;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(valid && bit);
      match &= bit ? bal : ~bal;
    }
    const int rank = __popcll(match & lt_mask);
    const int pos = L.cur[e] + rank;
    const int d = valid ? pos : S::kSink;
    L.sp[d] = p;
    L.stok[d] = L.tok[pc];
    L.sw[d] = L.w[pc];
    if (valid && pos == L.off[e]) {   // first pair of its expert
      const int sl = L.pslot[e];
      L.act[sl] = e;
      L.act_beg[sl] = pos;
      L.act_n[sl] = L.off[e + 1] - pos;
    }
    if (base + kWave < N) {         // later steps start after this step's pairs
      wave_lds_fence();
      const bool lead = valid && rank == 0;
      atomicAdd(&L.cur[lead ? e : S::kExp], lead ? __popcll(match) : 0);
      wave_lds_fence();
    }
  }
}

// Slot record of `slot` from a small sort (after the barrier that follows it).
template <int C, int MAXP>
__device__ __forceinline__ SlotRec small_slot_record(const SmallSortLds<C, MAXP>& L, int slot, int M, int k, int E,
                                                     int has_shared) {
  SlotRec r;
  r.pad[0] = r.pad[1] = r.pad[2] = r.pad[3] = 0;
  const int D = L.na;
  if (slot < D) {
    r.e = L.act[slot];
    r.pbeg = L.act_beg[slot];
    r.n = L.act_n[slot];
    r.hrow0 = r.pbeg;
#pragma unroll
    for (int q = 0; q < kRecTokens; ++q) {
      const int at = r.pbeg + min(q, r.n - 1);
      r.tok[q] = (q < r.n) ? L.stok[at] : 0;
      r.w[q] = (q < r.n) ? L.sw[at] : 0.f;
    }
  } else if (slot == D && has_shared) {
    r.e = E; r.pbeg = -1; r.n = M; r.hrow0 = M * k;
#pragma unroll
    for (int q = 0; q < kRecTokens; ++q) { r.tok[q] = q < M ? q : 0; r.w[q] = 1.f; }
  } else {
    r.e = -1; r.pbeg = -1; r.n = 0; r.hrow0 = 0;
#pragma unroll
    for (int q = 0; q < kRecTokens; ++q) { r.tok[q] = 0; r.w[q] = 0.f; }
  }
  return r;
}

// Copy a small sort and the top-k it sorted to the caller's arrays (every
// thread of the block, after the barrier that follows the sort).
template <int C, int MAXP>
__device__ inline void block_store_small_sort(const SmallSortLds<C, MAXP>& L, int N, int E,
                                              int* __restrict__ topk_ids, float* __restrict__ topk_weights,
                                              int* __restrict__ offsets, int* __restrict__ sorted_pairs,
                                              int* __restrict__ active, int* __restrict__ num_active) {
  const int nvalid = L.nvalid, D = L.na;
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    if (topk_ids) topk_ids[i] = L.ids[i];
    if (topk_weights) topk_weights[i] = L.w[i];
  }
  for (int i = threadIdx.x; i <= E; i += blockDim.x) offsets[i] = L.off[i];
  for (int i = threadIdx.x; i < nvalid; i += blockDim.x) sorted_pairs[i] = L.sp[i];
  for (int i = threadIdx.x; i < D; i += blockDim.x) active[i] = L.act[i];
  if (threadIdx.x == 0) *num_active = D;
}

}  // namespace moe
