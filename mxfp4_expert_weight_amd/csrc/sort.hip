// Stable counting sort of the (token, slot) pairs by expert (MoE-SpeQ article,
// section 4.2: gather every token's expert assignments, order them by expert
// id and run each expert once over its tokens).  One workgroup does it all in
// LDS: per-wave histograms, an exclusive scan over experts, then each wave
// places its own segment of pairs in order.  Stability comes from three
// facts: waves own consecutive segments, a wave walks its segment in order in
// 64-pair steps, and inside a step a pair's rank is the number of lower lanes
// holding the same expert (found with one ballot per expert-id bit).
#include "kernels.h"

namespace moe {

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

__global__ __launch_bounds__(512) void sort_by_expert_kernel(const int* __restrict__ ids, int N, int E,
                                                             int ebits, int* __restrict__ offsets,
                                                             int* __restrict__ sorted_pairs,
                                                             int* __restrict__ active,
                                                             int* __restrict__ num_active) {
  extern __shared__ int lds[];
  const int nw = blockDim.x / kWave;
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int bd = blockDim.x;
  int* cnt = lds;                 // [nw][E]: per-wave counts, then per-wave running bases
  int* off = cnt + nw * E;        // [E]: exclusive offsets of each expert
  int* wtot = off + E;            // [2 * nw]: per-wave scan totals

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
    if (c > 0) active[abase++] = e;
    cbase += c;
  }
  if (threadIdx.x == bd - 1) {
    offsets[E] = cbase;            // == N
    *num_active = abase;
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
      sorted_pairs[pos] = p;
      __builtin_amdgcn_wave_barrier();
      if (rank == 0) cnt[w * E + e] += __popcll(match);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_sort_by_expert(const int* ids, int N, int E, int* offsets, int* sorted_pairs,
                                 int* active, int* num_active, hipStream_t s) {
  int nw = (N + 511) / 512;
  nw = nw < 1 ? 1 : (nw > 8 ? 8 : nw);
  int ebits = 0;
  while ((1 << ebits) < E) ++ebits;
  const size_t shmem = sizeof(int) * ((size_t)nw * E + E + 2 * nw);
  sort_by_expert_kernel<<<1, nw * kWave, shmem, s>>>(ids, N, E, ebits, offsets, sorted_pairs, active,
                                                     num_active);
  return hipGetLastError();
}

}  // namespace moe
