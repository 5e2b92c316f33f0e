// Expert prefetch: rank the experts a draft pass picked for a layer, then read
// the chosen experts' MXFP4 weights ahead of the layer so that its own reads
// find them in the Infinity Cache (MoE-SpeQ article: 4.1 heat map of the
// draft's picks and the prefetch priority, 4.3 prefetch on a stream of its
// own that the verify pass waits on).
//
// On MI355X every layer's experts already sit in HBM; the level a prefetch can
// fill is the 256 MB memory-side Infinity Cache (the 4 MB L2 of each XCD is
// far smaller than one layer's active experts).  A prefetch is therefore a
// streaming read of the listed experts, reduced to a per-entry checksum so
// that every load is live and the bytes read can be checked.
#include <algorithm>

#include "kernels.h"

namespace moe {

namespace {

constexpr int kSelectThreads = 256;
constexpr int kIdxBits = 11;                     // expert index field of a rank key (E + 1 <= 2048)
constexpr int kLineBytes = 64;                   // a prefetch reads one word per line
constexpr int kPrefetchLoads = 16;               // lines in flight per lane
constexpr int kPrefetchStep = kWave * kPrefetchLoads;   // lines per wave iteration (64 KB)
constexpr int kPrefetchWaves = 1024;             // about one wave per SIMD of the chip
// Word 3 of a gfx9 buffer resource: 32-bit data format, raw (untyped) access.
constexpr int kBufferWord3 = 0x00020000;

// One workgroup.  heat[e] counts the draft pairs routed to e (LDS atomics);
// each picked expert gets the key heat << 11 | (2047 - e), so a larger key is
// a higher heat or, at equal heat, a lower index; an expert's place in the
// list is the number of picked keys above its own.
__global__ __launch_bounds__(kSelectThreads) void prefetch_select_kernel(const int* __restrict__ ids, int n_ids,
                                                                         int E, int has_shared, int max_n,
                                                                         int* __restrict__ out,
                                                                         int* __restrict__ num_out) {
  __shared__ int heat[MOE_MAX_EXPERTS];
  __shared__ int keys[MOE_MAX_EXPERTS];
  __shared__ int npicked;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kSelectThreads) heat[e] = 0;
  if (tid == 0) npicked = 0;
  __syncthreads();
  for (int i = tid; i < n_ids; i += kSelectThreads) {
    const int e = ids[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&heat[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kSelectThreads) {
    const int h = heat[e];
    if (h > 0) keys[atomicAdd(&npicked, 1)] = (h << kIdxBits) | ((1 << kIdxBits) - 1 - e);
  }
  __syncthreads();
  const int P = npicked;
  const int base = has_shared ? 1 : 0;
  for (int i = tid; i < P; i += kSelectThreads) {
    const int key = keys[i];
    int r = 0;
    for (int j = 0; j < P; ++j) r += keys[j] > key ? 1 : 0;
    if (base + r < max_n) out[base + r] = (1 << kIdxBits) - 1 - (key & ((1 << kIdxBits) - 1));
  }
  const int n = min(max_n, base + P);
  if (tid == 0) {
    *num_out = n;
    if (base && max_n > 0) out[0] = E;
  }
  for (int r = n + tid; r < max_n; r += kSelectThreads) out[r] = -1;
}

// Grid (blocks, list entries) of one-wave workgroups.  Block b of an entry
// covers lines [l0, l0 + per_block) of one region (the region and l0 follow
// from b alone, so they sit in scalar registers).  A lane reads the first
// 32-bit word of 16 lines per iteration, 64 lines apart, so one wave has
// 1,024 lines (64 KB) in flight for 16 VGPRs: a cache fill needs the lines
// fetched, not their bytes in registers.  Loads go through a buffer resource
// whose size is the expert's part of the region, so reads past its end
// return 0 and add nothing (per_block is a whole number of iterations, so
// only a region's last block reaches past it).  The kernel is held to 32
// VGPRs: the decode expert kernels keep three 160-VGPR waves on every SIMD,
// and a prefetch wave still fits beside them.
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_num_vgpr(32))) void prefetch_kernel(PrefetchArgs a) {
  const int r = blockIdx.y;
  const int live = a.num_live ? min(*a.num_live, a.max_ids) : a.max_ids;
  if (r >= live) return;
  const int e = a.ids[r];
  if ((unsigned)e >= (unsigned)a.nbank) return;
  const int b = blockIdx.x;
  const uint8_t* base = a.base[0];
  int64_t bytes = a.bytes[0];
  int b0 = 0;
#pragma unroll
  for (int q = 1; q < 4; ++q) {
    const bool in = q < a.nreg && b >= a.blk_end[q - 1];
    base = in ? a.base[q] : base;
    bytes = in ? a.bytes[q] : bytes;
    b0 = in ? a.blk_end[q - 1] : b0;
  }
  const int64_t lines = (bytes + kLineBytes - 1) / kLineBytes;
  const int64_t l0 = (int64_t)(b - b0) * a.per_block;
  if (l0 >= lines) return;
  const int64_t l1 = min(l0 + (int64_t)a.per_block, lines);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(base + (int64_t)e * bytes), 0, (int)bytes, kBufferWord3);
  const int lane = threadIdx.x;
  uint32_t s = 0;
  for (int64_t l = l0; l < l1; l += kPrefetchStep) {
    uint32_t v[kPrefetchLoads];
#pragma unroll
    for (int u = 0; u < kPrefetchLoads; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)((l + u * kWave + lane) * kLineBytes), 0, 0);
#pragma unroll
    for (int u = 0; u < kPrefetchLoads; ++u) s += v[u];
  }
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) s += (uint32_t)__shfl_xor((int)s, m, kWave);
  if (lane == 0) atomicAdd(&a.checksums[r], s);
}

}  // namespace

hipError_t launch_prefetch_select(const int* ids, int n_ids, int E, int has_shared, int max_n, int* out,
                                  int* num_out, hipStream_t s) {
  hipLaunchKernelGGL(prefetch_select_kernel, dim3(1), dim3(kSelectThreads), 0, s, ids, n_ids, E, has_shared,
                     max_n, out, num_out);
  return hipGetLastError();
}

hipError_t launch_prefetch(PrefetchArgs a, hipStream_t s) {
  if (a.max_ids <= 0 || a.nreg <= 0) return hipSuccess;
  int64_t lines[4], total = 0;
  for (int q = 0; q < a.nreg; ++q) {
    lines[q] = (a.bytes[q] + kLineBytes - 1) / kLineBytes;
    total += lines[q];
  }
  // lines per block: the list's lines over about kPrefetchWaves waves, a whole
  // number of wave iterations
  const int64_t want = (total * a.max_ids + kPrefetchWaves - 1) / kPrefetchWaves;
  const int64_t per = std::max<int64_t>(kPrefetchStep, (want + kPrefetchStep - 1) / kPrefetchStep * kPrefetchStep);
  a.per_block = (int)std::min<int64_t>(per, int64_t(1) << 30);
  int blocks = 0;
  for (int q = 0; q < a.nreg; ++q) {
    blocks += (int)((lines[q] + a.per_block - 1) / a.per_block);
    a.blk_end[q] = blocks;
  }
  hipLaunchKernelGGL(prefetch_kernel, dim3((unsigned)blocks, (unsigned)a.max_ids), dim3(kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
