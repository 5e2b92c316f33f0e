// Standalone sort kernel (the routine is in sort_dev.h).
#include "kernels.h"
#include "sort_dev.h"

namespace moe {

// Whether the sort's outputs and copies of its inputs (ids, and the routing
// weights the records carry) also fit in LDS next to its working set, for the
// records epilogue: then the epilogue reads nothing from global memory.  The
// budget is the 160 KiB a CDNA4 workgroup can hold.
constexpr size_t kSortLdsBytes = 160 * 1024;
__host__ __device__ inline size_t sort_lds_extra(int nw, int N, int E) { return 4 * (size_t)N + E + 4 * nw + 8; }
__host__ __device__ inline bool sort_keeps_lds(int nw, int N, int E) {
  return sizeof(int) * (sort_lds_ints(nw, E) + sort_lds_extra(nw, N, E)) <= kSortLdsBytes;
}

__global__ __launch_bounds__(1024) void sort_by_expert_kernel(const int* __restrict__ ids, int N, int E,
                                                             int ebits, int* __restrict__ offsets,
                                                             int* __restrict__ sorted_pairs,
                                                             int* __restrict__ active,
                                                             int* __restrict__ num_active,
                                                             RecOut ro) {
  extern __shared__ int lds[];
  const int nw = blockDim.x / kWave;
  const size_t base = sort_lds_ints(nw, E);
  if (ro.rec && sort_keeps_lds(nw, N, E)) {
    // the records epilogue reads the sort from LDS: sorted pairs, active list,
    // D and the offsets left at lds + nw*E, the ids, weights and each pair's
    // sorted position
    int* sp = lds + base;
    int* act = sp + N;
    int* na = act + E;
    int* scan = na + 1;
    int* ids_l = scan + 4 * nw + 4;                // N + 1 (a spare word)
    float* w_l = reinterpret_cast<float*>(ids_l + N + 1);   // N + 1
    int* inv_l = ids_l + 2 * (N + 1);                        // N
    // ids (read twice: histogram, placement) and weights: one coalesced copy
    // first, 8 loads per thread in flight; loads at clamped indices and
    // stores past the end to the spare word, so no load waits in a branch
    for (int i0 = 0; i0 < N; i0 += 8 * blockDim.x) {
      int v[8];
      float wv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = min(i0 + q * (int)blockDim.x + (int)threadIdx.x, N - 1);
        v[q] = ids[i];
        wv[q] = ro.topk_weights[i];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = min(i0 + q * (int)blockDim.x + (int)threadIdx.x, N);
        ids_l[i] = v[q];
        w_l[i] = wv[q];
      }
    }
    __syncthreads();
    block_sort_pairs(ids_l, N, E, ebits, lds, offsets, sorted_pairs, active, num_active, sp, act, na, inv_l);
    __syncthreads();
    RecOut r = ro;
    r.topk_weights = w_l;
    block_write_slot_records(r, E, max_slots(ro.M, ro.k, E), lds + (size_t)nw * E, sp, act, na, scan, inv_l);
    return;
  }
  block_sort_pairs(ids, N, E, ebits, lds, offsets, sorted_pairs, active, num_active);
  if (ro.rec) {
    __threadfence_block();
    __syncthreads();
    block_write_slot_records(ro, E, max_slots(ro.M, ro.k, E), offsets, sorted_pairs, active, num_active,
                             lds + base);
  }
}

// Slot records (and MFMA items) from sort outputs already in memory: the
// expert stage of moe_mxfp4_forward when the MFMA path is on.
__global__ __launch_bounds__(512) void records_kernel(const int* __restrict__ offsets,
                                                      const int* __restrict__ sorted_pairs,
                                                      const int* __restrict__ active,
                                                      const int* __restrict__ num_active, int E, RecOut ro) {
  __shared__ int lds[4 * (512 / kWave) + 4];
  block_write_slot_records(ro, E, max_slots(ro.M, ro.k, E), offsets, sorted_pairs, active, num_active, lds);
}

int expert_bits(int E) {
  int ebits = 0;
  while ((1 << ebits) < E) ++ebits;
  return ebits;
}

hipError_t launch_sort_by_expert(const int* ids, int N, int E, int* offsets, int* sorted_pairs,
                                 int* active, int* num_active, hipStream_t s, RecOut ro) {
  // 8 waves (the records epilogue has a slot per thread), 16 for long inputs
  // (each wave places half as many pairs)
  const int nw = N >= 1024 ? 16 : 8;
  const size_t shmem =
      sizeof(int) * (sort_lds_ints(nw, E) + (ro.rec && sort_keeps_lds(nw, N, E) ? sort_lds_extra(nw, N, E) : 4 * nw + 4));
  if (shmem > 65536) {                             // more than the default dynamic LDS of a launch
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(sort_by_expert_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  sort_by_expert_kernel<<<1, nw * kWave, shmem, s>>>(ids, N, E, expert_bits(E), offsets, sorted_pairs,
                                                     active, num_active, ro);
  return hipGetLastError();
}

hipError_t launch_records(const int* offsets, const int* sorted_pairs, const int* active, const int* num_active,
                          int E, RecOut ro, hipStream_t s) {
  records_kernel<<<1, 512, 0, s>>>(offsets, sorted_pairs, active, num_active, E, ro);
  return hipGetLastError();
}

}  // namespace moe
