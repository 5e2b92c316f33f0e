// Measurement hook: how long the chip takes just to read a set of byte
// ranges when every load of a workgroup is in flight at once, the way the
// decode kernels stream their expert weights (16 bytes per lane, each
// workgroup's chunk requested before any of it is used), in chunks small
// enough that even a few MB fill every compute unit.  Reading a layer's
// expert bytes this way, with nothing else in the kernel, is the floor that
// the expert kernels are measured against.  Each workgroup XORs the 32-bit
// words of its chunk, so every load is used and the bytes reached can be
// checked exactly.
#include <hip/hip_ext.h>

#include "kernels.h"

namespace moe {

namespace {

typedef unsigned rp_u32x4 __attribute__((ext_vector_type(4)));
constexpr int RP_THREADS = 256;
constexpr int RP_LOADS = kReadProbeChunk / (RP_THREADS * 16);   // 4 loads of 16 bytes per lane
static_assert(RP_LOADS * RP_THREADS * 16 == kReadProbeChunk, "chunk = whole loads");

// Workgroup (chunk x, range y).  Loads past the range's end are clamped to its
// last 16 bytes and left out of the XOR (unconditional loads: a guarded one
// would wait inside its branch).
__global__ __launch_bounds__(RP_THREADS) void read_probe_kernel(const uint64_t* __restrict__ addrs,
                                                                const int64_t* __restrict__ sizes,
                                                                uint32_t* __restrict__ out) {
  const int64_t size = sizes[blockIdx.y];
  const int64_t base = (int64_t)blockIdx.x * kReadProbeChunk;
  const size_t o = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
  if (base >= size) {                              // past this range's end (uniform)
    if (threadIdx.x == 0) out[o] = 0u;
    return;
  }
  const uint8_t* p = reinterpret_cast<const uint8_t*>(addrs[blockIdx.y]);
  rp_u32x4 v[RP_LOADS];
#pragma unroll
  for (int i = 0; i < RP_LOADS; ++i) {
    const int64_t off = base + ((int64_t)i * RP_THREADS + threadIdx.x) * 16;
    v[i] = *reinterpret_cast<const rp_u32x4*>(p + (off < size ? off : size - 16));
  }
  uint32_t x = 0u;
#pragma unroll
  for (int i = 0; i < RP_LOADS; ++i) {
    const int64_t off = base + ((int64_t)i * RP_THREADS + threadIdx.x) * 16;
    const uint32_t w = v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    x ^= off < size ? w : 0u;
  }
  // XOR over the workgroup: the wave by DPP row steps and row swaps, then LDS
  x ^= dpp_quad_xor1(x);
  x ^= dpp_quad_xor2(x);
  x ^= dpp_half_mirror(x);
  x ^= dpp_row_mirror(x);
  {
    const Pair a = swap16(x);
    x = a.a ^ a.b;
    const Pair b = swap32(x);
    x = b.a ^ b.b;
  }
  __shared__ uint32_t part[RP_THREADS / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0u;
#pragma unroll
    for (int w = 0; w < RP_THREADS / kWave; ++w) t ^= part[w];
    out[o] = t;
  }
}

}  // namespace

hipError_t launch_read_probe(const uint64_t* addrs, const int64_t* sizes, int n, int64_t max_bytes, uint32_t* out,
                             hipEvent_t start, hipEvent_t stop, hipStream_t s) {
  const dim3 grid((unsigned)read_probe_chunks(max_bytes), (unsigned)n), block(RP_THREADS);
  void* args[] = {const_cast<uint64_t**>(&addrs), const_cast<int64_t**>(&sizes), &out};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(read_probe_kernel), grid, block, args, 0, s, start, stop,
                            0);
}

}  // namespace moe
