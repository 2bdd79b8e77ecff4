// Measured HBM read ceilings that the decode kernels are compared with.
// Two read-only kernels with no arithmetic but an xor per thread, both
// persistent, each with the access pattern it measured fastest at on MI355X.
// - kv8_stream_read: plain streaming.  `workgroups` workgroups of 256
//   threads take 32 KB chunks c = w, w + workgroups, ... (chunk c is bytes
//   [32 KB * c, 32 KB * (c + 1)) of buf) with nontemporal 16-byte loads, 8
//   in flight per lane.  Over 1-2 GiB: 6.7-6.9 TB/s this way, 6.1 TB/s with
//   ordinary loads, 5.6-6.0 TB/s with one chunk per workgroup.
// - kv8_read_probe: the access pattern of the paged decode, random tiles of
//   `tile_bytes` out of a buffer far larger than the last-level cache, in
//   the order a caller-supplied index list gives.  Each wave streams its own
//   tiles (list entries v, v + waves, v + 2 waves, ...) as 1 KB rows (one
//   16-byte load per lane), 4 rows in flight, ordinary loads, no barriers;
//   the tile ids come 64 to a wave load, one batch ahead.  For 170 MB of
//   random 2 KB tiles per launch this measured 28-29 us (5.9-6.1 TB/s),
//   against 29-35 us with nontemporal loads or 8-16 KB in flight per wave,
//   and 34.6 us for the earlier chunked form (tile ids staged in LDS per
//   32 KB chunk, nontemporal loads).
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

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ buf,
                                                                    int64_t n_chunks,
                                                                    uint32_t* __restrict__ out) {
  const int t = threadIdx.x;
  uint32_t acc = 0;
  for (int64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const uint4* base = buf + c * kChunkU4 + t;
    uint32_t x[kProbeIters];
#pragma unroll
    for (int i = 0; i < kProbeIters; ++i) x[i] = load_xor_nt(base + i * kProbeThreads);
#pragma unroll
    for (int i = 0; i < kProbeIters; ++i) acc ^= x[i];
  }
  out[(int64_t)blockIdx.x * kProbeThreads + t] = acc;
}

constexpr int kRowU4 = 64;      // one row: 64 lanes x 16 bytes
constexpr int kTileRing = 4;    // rows in flight per wave

// Wave v (of nw) reads tiles[v], tiles[v + nw], ...: tile j of the wave is
// list entry v + j * nw, and its rows_per_tile rows are read in order, lane
// l reading unit l of each row.  Ring slots past the wave's last row load
// the first row of the buffer (in bounds) so that every slot always loads
// and the compiler's wait counts stay exact; their bytes are not xored.
__global__ __launch_bounds__(kProbeThreads) void tile_read_kernel(const uint4* __restrict__ buf,
                                                                  const int32_t* __restrict__ tiles,
                                                                  int rows_per_tile,
                                                                  int64_t n_tiles,
                                                                  uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (kProbeThreads / 64);
  const int64_t v = (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  const int64_t mine = v < n_tiles ? (n_tiles - 1 - v) / nw + 1 : 0;   // the wave's tiles
  const int64_t nrows = mine * rows_per_tile;
  uint32_t acc = 0;
  if (nrows > 0) {
    // tile ids of the wave's tiles j0 .. j0 + 63 (cur) and the next 64 (nxt)
    auto ids_at = [&](int64_t j0) {
      const int64_t j = j0 + lane;
      return j < mine ? tiles[v + j * nw] : 0;
    };
    int64_t j0 = 0;
    int cur = ids_at(0), nxt = ids_at(64);
    int64_t it = 0, ik = 0;                    // tile and row of the next issue
    uint4 x[kTileRing];
    auto issue = [&](int s) {
      const bool real = it < mine;             // wave-uniform
      if (real && it >= j0 + 64) {             // next batch of ids
        j0 += 64;
        cur = nxt;
        nxt = ids_at(j0 + 64);
      }
      const int64_t id = real ? __builtin_amdgcn_readlane(cur, (int)(it - j0)) : 0;
      const int64_t row = real ? id * rows_per_tile + ik : 0;
      x[s] = buf[row * kRowU4 + lane];
      if (real && ++ik == rows_per_tile) {
        ik = 0;
        ++it;
      }
    };
#pragma unroll
    for (int s = 0; s < kTileRing; ++s) issue(s);
    for (int64_t r0 = 0; r0 < nrows; r0 += kTileRing) {
#pragma unroll
      for (int s = 0; s < kTileRing; ++s) {
        if (r0 + s < nrows) acc ^= x[s].x ^ x[s].y ^ x[s].z ^ x[s].w;
        issue(s);
      }
    }
  }
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace

int64_t read_probe_chunk_bytes() { return (int64_t)kChunkU4 * 16; }

int launch_read_probe(const void* buf, const int32_t* tiles, int tile_bytes, int64_t n_bytes,
                      int64_t workgroups, uint32_t* out, hipStream_t stream) {
  if (tiles != nullptr)
    tile_read_kernel<<<dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream>>>(
        static_cast<const uint4*>(buf), tiles, tile_bytes / (kRowU4 * 16), n_bytes / tile_bytes,
        out);
  else
    stream_read_kernel<<<dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream>>>(
        static_cast<const uint4*>(buf), n_bytes / read_probe_chunk_bytes(), out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kv8
