// Measured HBM read ceilings that the decode kernels are compared with.
// Two read-only kernels with no arithmetic but an xor per thread, both
// persistent: `workgroups` workgroups take 32 KB chunks c = w, w +
// workgroups, ... and read them with nontemporal 16-byte loads (the data
// is read once, so it need not stay in the caches), 8 loads in flight per
// lane.  Measured on MI355X over 1 GiB: 6.9 TB/s this way, 6.1 TB/s with
// ordinary loads, 5.6-6.0 TB/s with one chunk per workgroup.
// - kv8_stream_read: chunk c is bytes [32 KB * c, 32 KB * (c + 1)) of buf;
// - kv8_read_probe: the access pattern of the paged decode, random tiles of
//   `tile_bytes` out of a buffer far larger than the last-level cache in the
//   order a caller-supplied index list gives.  A workgroup holds the tile
//   indices of its current chunk in LDS and loads those of its next chunk
//   while the current chunk's data loads are in flight.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv8_launch.h"

namespace kv8 {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeIters = 8;                           // 8 x 4 KB per chunk
constexpr int kChunkU4 = kProbeIters * kProbeThreads;    // 16-byte units per chunk

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t load_xor_nt(const uint4* p) {
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return w.x ^ w.y ^ w.z ^ w.w;
}

// TILED: position p of chunk c reads unit p % tile_u4 of tile
// tiles[c * (kChunkU4 / tile_u4) + p / tile_u4]; tile_u4 is a multiple of
// 16 that divides kChunkU4, so a chunk spans at most kProbeThreads / 2
// tiles and its first threads hold one index each.  Otherwise position p
// of chunk c reads unit c * kChunkU4 + p.
template <bool TILED>
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint4* __restrict__ buf,
                                                                   const int32_t* __restrict__ tiles,
                                                                   int tile_u4, int64_t n_chunks,
                                                                   uint32_t* __restrict__ out) {
  const int t = threadIdx.x;
  const int64_t stride = gridDim.x;
  uint32_t acc = 0;
  if constexpr (TILED) {
    __shared__ int s_tile[kProbeThreads];
    const int ntile = kChunkU4 / tile_u4;
    int64_t c = blockIdx.x;
    int next = (t < ntile && c < n_chunks) ? tiles[c * ntile + t] : 0;
    for (; c < n_chunks; c += stride) {
      __syncthreads();                         // the previous chunk's reads of s_tile are done
      if (t < ntile) s_tile[t] = next;
      __syncthreads();
      if (t < ntile && c + stride < n_chunks) next = tiles[(c + stride) * ntile + t];
      uint32_t x[kProbeIters];
#pragma unroll
      for (int i = 0; i < kProbeIters; ++i) {
        const int p = i * kProbeThreads + t;
        x[i] = load_xor_nt(buf + (int64_t)s_tile[p / tile_u4] * tile_u4 + p % tile_u4);
      }
#pragma unroll
      for (int i = 0; i < kProbeIters; ++i) acc ^= x[i];
    }
  } else {
    for (int64_t c = blockIdx.x; c < n_chunks; c += stride) {
      const uint4* base = buf + c * kChunkU4 + t;
      uint32_t x[kProbeIters];
#pragma unroll
      for (int i = 0; i < kProbeIters; ++i) x[i] = load_xor_nt(base + i * kProbeThreads);
#pragma unroll
      for (int i = 0; i < kProbeIters; ++i) acc ^= x[i];
    }
  }
  out[(int64_t)blockIdx.x * kProbeThreads + t] = acc;
}

}  // namespace

int64_t read_probe_chunk_bytes() { return (int64_t)kChunkU4 * 16; }

int launch_read_probe(const void* buf, const int32_t* tiles, int tile_bytes, int64_t n_bytes,
                      int64_t workgroups, uint32_t* out, hipStream_t stream) {
  const int64_t n_chunks = n_bytes / read_probe_chunk_bytes();
  if (tiles != nullptr)
    read_probe_kernel<true><<<dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream>>>(
        static_cast<const uint4*>(buf), tiles, tile_bytes / 16, n_chunks, out);
  else
    read_probe_kernel<false><<<dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream>>>(
        static_cast<const uint4*>(buf), nullptr, 0, n_chunks, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kv8
