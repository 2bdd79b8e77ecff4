// kv8_read_probe: the measured HBM read ceiling that the decode kernels are
// compared with.  A read-only kernel streams tiles of `tile_bytes` bytes,
// taken in the order a caller-supplied index list gives, out of a buffer
// far larger than the last-level cache: the access pattern of the paged
// decode (random 2 KB (block, KV head) tiles) with no arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv8_launch.h"

namespace kv8 {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeIters = 8;   // 8 x 4 KB per workgroup, all loads in flight at once

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ buf,
                                                                   const int32_t* __restrict__ tiles,
                                                                   int tile_u4,
                                                                   uint32_t* __restrict__ out) {
  const int t = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * kProbeIters * kProbeThreads;
  uint4 v[kProbeIters];
#pragma unroll
  for (int i = 0; i < kProbeIters; ++i) {
    const int64_t p = base + (int64_t)i * kProbeThreads + t;    // logical 16-byte position
    const int64_t tile = tiles[p / tile_u4];
    v[i] = buf[tile * tile_u4 + p % tile_u4];
  }
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < kProbeIters; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  out[(int64_t)blockIdx.x * kProbeThreads + t] = acc;
}

}  // namespace

int64_t read_probe_bytes_per_workgroup() { return (int64_t)kProbeIters * kProbeThreads * 16; }

int launch_read_probe(const void* buf, const int32_t* tiles, int tile_bytes, int64_t workgroups,
                      uint32_t* out, hipStream_t stream) {
  read_probe_kernel<<<dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream>>>(
      static_cast<const uint4*>(buf), tiles, tile_bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kv8
