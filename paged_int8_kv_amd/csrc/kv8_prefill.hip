// paged_prefill_chunk_attn_kv8 kernel: causal attention of a chunk of query
// rows over the paged INT8 cache, on the gfx950 matrix cores.
//
// Attention softmax(Q K^T * sm_scale) V ("KV Cache 优化全景解析", section
// 2.1) per GQA group (section 3.3), for a prefill chunk whose own K/V are
// already in the cache (chunked prefill, section 11.2): row i of a chunk of
// Lc rows sits at absolute position ctx - Lc + i and sees keys 0 .. that
// position.  K/V are restored on the fly from INT8 codes and per-token fp16
// scales ("KV-Cache 全栈优化系统" README, section 主要特性); softmax and all
// accumulation run in fp32 ("大模型推理加速：KV Cache与vLLM技术解析",
// section 4.1).
//
// Work split: one workgroup of 4 waves per (sequence b, KV head g, tile of
// 256 queries).  A query is a (chunk row, head of the group) pair with the
// G heads innermost, so every K/V byte staged by the workgroup serves all G
// heads of its group.  Each wave owns 64 queries: two 32-query column
// blocks of the MFMA output.
//
// Key tiles of 64 tokens (4 cache blocks) are staged once per workgroup in
// LDS, double-buffered (the next tile's codes are loaded into registers
// while the current tile is computed, one barrier per tile):
//   K  exact fp16 codes, row-major [key][channel] (rows padded by 16 bytes);
//   V  exact fp16 codes, transposed [channel][key] (rows padded), with the
//      keys of every 16-token group permuted so that the 8 keys one lane
//      feeds to the PV product are 16 contiguous bytes;
//   scales as fp32, k_scale premultiplied by sm_scale * log2(e); keys past
//      the workgroup's key range get scale 0.
// Codes become fp16 without a convert per code: u = c xor 0x80 under the
// fp16 high byte 0x64 is the value c + 1152, and one packed fp16 subtract
// of 1152 leaves c exactly.
//
// Per wave and key tile (v_mfma_f32_32x32x16_f16, fp32 accumulate):
//   S^T[key][query] = K_code . Q^T, with Q scaled per query by 2^e_q so that
//                     bf16 q is exact in fp16 (max |q| in [2^14, 2^15));
//   z = S^T * (k_scale[key] * sm_scale * log2(e)) * 2^-e_q; the last factor
//       is exact, so the largest z of a row gives 2^0 = 1 exactly;
//   online softmax in base 2: running max m_q and sum l_q per query; the
//   accumulator is rescaled only when some running max of the wave grew;
//   w = 2^(z - m_q) * v_scale[key], rounded to fp16;
//   O^T[channel][query] += V_code^T . W^T.
// The output is O / l (0 for a query with no visible key).
//
// The MFMA operand slot (lane / 32, element j) pairs an A element with a B
// element, so K/V rows and channels may be permuted freely as long as both
// operands agree: QK^T feeds channel (d/2)(lane/32) + 8s + j at k-step s,
// and PV feeds, for S^T output register r = 8j + jj of a lane, the key
// 8(r/4) + 4(lane/32) + r%4 of the 32-key block (the output layout of the
// 32x32 MFMA), which the V staging permutation makes contiguous.
#include "kv8_device.h"
#include "kv8_launch.h"

namespace kv8 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kQueriesPerWave = 64;
constexpr int kQueriesPerGroup = kWaves * kQueriesPerWave;   // 256
constexpr int kTileKeys = 64;                                // 4 cache blocks
constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct PrefillArgs {
  const uint16_t* q;
  const int32_t* q_start_loc;
  const int8_t* k_cache;
  const int8_t* v_cache;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  const int32_t* block_table;
  const int32_t* context_lens;
  float* out;
  int64_t total_q;
  int64_t num_blocks;
  int max_blocks_per_seq;
  int ctx_cap;
  int num_q_heads;
  int num_kv_heads;
  float sm_scale_log2;     // sm_scale * log2(e)
};

template <int D>
struct __attribute__((aligned(16))) Lds {
  static constexpr int kRow = D + 8;            // halves per K row (16-byte pad)
  static constexpr int kVRow = kTileKeys + 8;   // halves per V^T row
  _Float16 k[2][kTileKeys][kRow];
  _Float16 v[2][D][kVRow];
  float ks[2][kTileKeys];
  float vs[2][kTileKeys];
};

__device__ __forceinline__ half8_t as_half8(uint4 u) { return __builtin_bit_cast(half8_t, u); }

// Four int8 codes (one dword) -> two exact fp16 pairs.
__device__ __forceinline__ void codes_to_f16(uint32_t u, half2_t& lo, half2_t& hi) {
  const uint32_t x = u ^ kXor80;
  const half2_t bias = {(_Float16)kCodeBias, (_Float16)kCodeBias};
  lo = biased_pair_lo(x) - bias;
  hi = biased_pair_hi(x) - bias;
}

__device__ __forceinline__ uint32_t h2_bits(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ float wave_max32(float x) {   // max of lanes l and l ^ 32
  float a, b;
  swap32(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float wave_sum32(float x) {
  float a, b;
  swap32(x, a, b);
  return a + b;
}

// Registers holding one key tile's codes and scales on their way to LDS.
template <int D>
struct Stage {
  static constexpr int kKVec = D / 64;          // uint4 of K codes per thread
  static constexpr int kVTasks = 2 * D;         // (8-key group, channel quad) tasks
  uint4 k[kKVec];
  uint32_t v[8];
  uint16_t sc;
};

template <int D>
__device__ __forceinline__ int64_t block_base(const PrefillArgs& a, const int32_t* table_row,
                                              int blk_idx, int last_blk, int g) {
  int id = table_row[blk_idx < last_blk ? blk_idx : last_blk];
  id = id < 0 ? 0 : (id >= a.num_blocks ? (int)(a.num_blocks - 1) : id);
  return (int64_t)id * a.num_kv_heads + g;       // (block, KV head) slab index
}

template <int D>
__device__ __forceinline__ void stage_load(const PrefillArgs& a, const int32_t* table_row,
                                           int kt, int last_blk, int g, int tid,
                                           Stage<D>& st) {
  // K: key tid/4, channel part tid%4 of D/4 bytes
  {
    const int key = tid >> 2, part = tid & 3;
    const int64_t slab = block_base<D>(a, table_row, kt * 4 + (key >> 4), last_blk, g);
    const uint4* src = reinterpret_cast<const uint4*>(
        a.k_cache + slab * (kBlock * D) + (key & 15) * D + part * (D / 4));
#pragma unroll
    for (int i = 0; i < Stage<D>::kKVec; ++i) st.k[i] = src[i];
  }
  // V: 8 rows x 4 channels per task; rows 4hh+{0..3}, 8+4hh+{0..3} of group grp
  if (tid < Stage<D>::kVTasks) {
    const int cq = tid % (D / 4), kg = tid / (D / 4);
    const int grp = kg >> 1, hh = kg & 1;
    const int64_t slab = block_base<D>(a, table_row, kt * 4 + grp, last_blk, g);
    const int8_t* base = a.v_cache + slab * (kBlock * D) + cq * 4;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = 4 * hh + (r & 3) + 8 * (r >> 2);
      st.v[r] = *reinterpret_cast<const uint32_t*>(base + row * D);
    }
  }
  // scales: threads 0..63 K, 64..127 V
  if (tid < 2 * kTileKeys) {
    const int key = tid & 63;
    const int64_t slab = block_base<D>(a, table_row, kt * 4 + (key >> 4), last_blk, g);
    const uint16_t* s = tid < kTileKeys ? a.k_scale : a.v_scale;
    st.sc = s[slab * kBlock + (key & 15)];
  }
}

template <int D>
__device__ __forceinline__ void stage_store(Lds<D>& lds, int buf, int kt, int n_keys, int tid,
                                            float k_mult, const Stage<D>& st) {
  {
    const int key = tid >> 2, part = tid & 3;
    _Float16* dst = &lds.k[buf][key][part * (D / 4)];
#pragma unroll
    for (int i = 0; i < Stage<D>::kKVec; ++i) {
      const uint32_t w[4] = {st.k[i].x, st.k[i].y, st.k[i].z, st.k[i].w};
      uint32_t o[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        half2_t lo, hi;
        codes_to_f16(w[j], lo, hi);
        o[2 * j] = h2_bits(lo);
        o[2 * j + 1] = h2_bits(hi);
      }
      reinterpret_cast<uint4*>(dst)[2 * i] = make_uint4(o[0], o[1], o[2], o[3]);
      reinterpret_cast<uint4*>(dst)[2 * i + 1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
  if (tid < Stage<D>::kVTasks) {
    const int cq = tid % (D / 4), kg = tid / (D / 4);
    const int grp = kg >> 1, hh = kg & 1;
    // [r0.c, r1.c, r0.c', r1.c'] for the row pairs (0,1) (2,3) (4,5) (6,7)
    uint32_t plo[4], phi[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      plo[p] = interleave_lo(st.v[2 * p], st.v[2 * p + 1]) ^ kXor80;
      phi[p] = interleave_hi(st.v[2 * p], st.v[2 * p + 1]) ^ kXor80;
    }
    const half2_t bias = {(_Float16)kCodeBias, (_Float16)kCodeBias};
#pragma unroll
    for (int ci = 0; ci < 4; ++ci) {
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t src = (ci < 2) ? plo[p] : phi[p];
        const half2_t h = ((ci & 1) ? biased_pair_hi(src) : biased_pair_lo(src)) - bias;
        o[p] = h2_bits(h);
      }
      *reinterpret_cast<uint4*>(&lds.v[buf][cq * 4 + ci][grp * 16 + hh * 8]) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  if (tid < 2 * kTileKeys) {
    const int key = tid & 63;
    const float s = (kt * kTileKeys + key < n_keys) ? fp16_bits_to_f32(st.sc) : 0.0f;
    if (tid < kTileKeys) lds.ks[buf][key] = s * k_mult;
    else lds.vs[buf][key] = s;
  }
}

template <int D, int G>
__global__ void __launch_bounds__(kThreads, 1) prefill_kernel(PrefillArgs a) {
  constexpr int KS = D / 16;        // k-steps of the QK^T product
  constexpr int CB = D / 32;        // 32-channel blocks of the output
  constexpr int kRowsPerTile = kQueriesPerGroup / G;
  __shared__ Lds<D> lds;

  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int m = lane & 31, h = lane >> 5;

  int r0 = a.q_start_loc[b], r1 = a.q_start_loc[b + 1];
  r0 = r0 < 0 ? 0 : r0;
  r1 = r1 > a.total_q ? (int)a.total_q : r1;
  const int lc = r1 - r0;
  const int row_begin = tile * kRowsPerTile;
  if (row_begin >= lc) return;                                   // uniform
  int ctx = a.context_lens[b];
  ctx = ctx < a.ctx_cap ? ctx : a.ctx_cap;
  const int row_end = min(row_begin + kRowsPerTile, lc);         // exclusive
  const int pos0 = ctx - lc;                                     // position of row 0
  const int n_keys = min(ctx, pos0 + row_end);                   // keys any row sees
  const int nkt = n_keys > 0 ? (n_keys + kTileKeys - 1) / kTileKeys : 0;
  const int last_blk = n_keys > 0 ? (n_keys - 1) / kBlock : 0;
  const int32_t* table_row = a.block_table + (int64_t)b * a.max_blocks_per_seq;

  Stage<D> st;
  if (nkt > 0) stage_load<D>(a, table_row, 0, last_blk, g, tid, st);

  // ---- this lane's queries: load Q, exact fp16 after a power-of-two scale --
  half8_t qf[2][KS];
  float cq[2];
  int qpos[2], qrow[2], qhead[2];
  bool qvalid[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int nq = wave * kQueriesPerWave + qb * 32 + m;
    const int row = row_begin + nq / G;
    qrow[qb] = row;
    qhead[qb] = g * G + nq % G;
    qvalid[qb] = row < row_end;
    qpos[qb] = pos0 + row;
    uint4 raw[KS];
    if (qvalid[qb]) {
      const uint4* src = reinterpret_cast<const uint4*>(
          a.q + ((int64_t)(r0 + row) * a.num_q_heads + qhead[qb]) * D + (D / 2) * h);
#pragma unroll
      for (int s = 0; s < KS; ++s) raw[s] = src[s];
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) raw[s] = make_uint4(0, 0, 0, 0);
    }
    float mx = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t w[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mx = fmaxf(mx, fabsf(__builtin_bit_cast(float, w[j] << 16)));
        mx = fmaxf(mx, fabsf(__builtin_bit_cast(float, w[j] & 0xFFFF0000u)));
      }
    }
    mx = wave_max32(mx);
    int e = 0;
    if (mx > 0.0f) {
      int ex;
      frexpf(mx, &ex);                 // mx = f * 2^ex, f in [0.5, 1)
      e = 15 - ex;                     // mx * 2^e in [2^14, 2^15)
      e = e > 120 ? 120 : (e < -120 ? -120 : e);
    }
    cq[qb] = ldexpf(1.0f, -e);         // exact: z = x * cq rounds nowhere
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t w[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qf[qb][s][2 * j] =
            (_Float16)ldexpf(__builtin_bit_cast(float, w[j] << 16), e);
        qf[qb][s][2 * j + 1] =
            (_Float16)ldexpf(__builtin_bit_cast(float, w[j] & 0xFFFF0000u), e);
      }
    }
  }
  // wave-uniform causal bounds of this wave's valid queries
  const int wave_row_lo = row_begin + (wave * kQueriesPerWave) / G;
  const int wave_row_hi = min(row_begin + (wave * kQueriesPerWave + kQueriesPerWave - 1) / G,
                              row_end - 1);
  const bool wave_live = wave_row_lo <= wave_row_hi;
  const int wave_pos_lo = pos0 + wave_row_lo;   // smallest position of the wave
  const int wave_pos_hi = pos0 + wave_row_hi;   // largest

  f32x16_t acc[CB][2];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cb][qb][r] = 0.0f;
  float mrun[2] = {kNegInf, kNegInf}, lrun[2] = {0.0f, 0.0f};

  if (nkt > 0) stage_store<D>(lds, 0, 0, n_keys, tid, a.sm_scale_log2, st);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) stage_load<D>(a, table_row, kt + 1, last_blk, g, tid, st);

    const int key0 = kt * kTileKeys;
    if (wave_live && key0 <= wave_pos_hi) {
      const bool live1 = key0 + 32 <= wave_pos_hi;   // second 32-key block visible
      // ---- S^T = K . Q^T ---------------------------------------------------
      f32x16_t sacc[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][qb][r] = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && !live1) break;
        half8_t ka[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s)
          ka[s] = as_half8(*reinterpret_cast<const uint4*>(
              &lds.k[buf][kb * 32 + m][(D / 2) * h + 8 * s]));
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[s], qf[qb][s],
                                                                  sacc[kb][qb], 0, 0, 0);
      }
      // ---- online softmax (base 2) and fp16 weights, one query block at a time.
      // Lane keys of a 32-key block: 8a + 4h + i for register r = 4a + i.
      const bool need_mask = key0 + kTileKeys - 1 > wave_pos_lo;
      half8_t pw[2][2][2];     // [qb][kb][k-step]
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const float4 k4 =
                *reinterpret_cast<const float4*>(&lds.ks[buf][kb * 32 + 8 * a4 + 4 * h]);
            const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 4 * a4 + i;
              float x = sacc[kb][qb][r] * kv[i];
              if (need_mask) {
                const int key = key0 + kb * 32 + 8 * a4 + 4 * h + i;
                x = key > qpos[qb] ? kNegInf : x;
              }
              if (kb == 1 && !live1) x = kNegInf;
              sacc[kb][qb][r] = x;
              mx = fmaxf(mx, x);
            }
          }
        mx = wave_max32(mx);
        const float mnew = fmaxf(mrun[qb], mx * cq[qb]);
        if (__builtin_amdgcn_ballot_w64(mnew > mrun[qb]) != 0) {
          const float alpha = mnew == mrun[qb] ? 1.0f : __builtin_amdgcn_exp2f(mrun[qb] - mnew);
          lrun[qb] *= alpha;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[cb][qb][r] *= alpha;
          mrun[qb] = mnew;
        }
        const float muse = mrun[qb] == kNegInf ? 0.0f : mrun[qb];
        float lsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const float4 v4 =
                *reinterpret_cast<const float4*>(&lds.vs[buf][kb * 32 + 8 * a4 + 4 * h]);
            const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 4 * a4 + i;
              const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][qb][r], cq[qb], -muse));
              lsum += p;
              pw[qb][kb][r >> 3][r & 7] = (_Float16)(p * vv[i]);
            }
          }
        lrun[qb] += lsum;
      }
      // ---- O^T += V^T . W^T ----------------------------------------------------
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && !live1) break;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          half8_t va[CB];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            va[cb] = as_half8(*reinterpret_cast<const uint4*>(
                &lds.v[buf][cb * 32 + m][kb * 32 + 16 * j + 8 * h]));
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              acc[cb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[cb], pw[qb][kb][j],
                                                                   acc[cb][qb], 0, 0, 0);
        }
      }
    }

    if (more) stage_store<D>(lds, buf ^ 1, kt + 1, n_keys, tid, a.sm_scale_log2, st);
    __syncthreads();
  }

  // ---- epilogue: O / l, channel 32cb + 8(r/4) + 4h + r%4 --------------------
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = wave_sum32(lrun[qb]);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (!qvalid[qb]) continue;
    float* dst = a.out + ((int64_t)(r0 + qrow[qb]) * a.num_q_heads + qhead[qb]) * D + 4 * h;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int r = 4 * a4;
        *reinterpret_cast<float4*>(dst + cb * 32 + 8 * a4) =
            make_float4(acc[cb][qb][r] * inv, acc[cb][qb][r + 1] * inv,
                        acc[cb][qb][r + 2] * inv, acc[cb][qb][r + 3] * inv);
      }
  }
}

template <int D, int G>
int launch_dg(const PrefillArgs& a, int batch, int max_q_len, hipStream_t stream) {
  const int64_t tiles = ((int64_t)max_q_len * G + kQueriesPerGroup - 1) / kQueriesPerGroup;
  if (tiles > 0x7FFFFFFF) return -1;
  dim3 grid((unsigned)tiles, (unsigned)a.num_kv_heads, (unsigned)batch);
  hipLaunchKernelGGL((prefill_kernel<D, G>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int D>
int launch_d(const PrefillArgs& a, int G, int batch, int max_q_len, hipStream_t stream) {
  switch (G) {
    case 1: return launch_dg<D, 1>(a, batch, max_q_len, stream);
    case 2: return launch_dg<D, 2>(a, batch, max_q_len, stream);
    case 4: return launch_dg<D, 4>(a, batch, max_q_len, stream);
    case 8: return launch_dg<D, 8>(a, batch, max_q_len, stream);
    default: return -2;
  }
}

}  // namespace

int launch_prefill(const uint16_t* q, const int32_t* q_start_loc, int64_t total_q, int max_q_len,
                   const int8_t* k_cache, const int8_t* v_cache, const uint16_t* k_scale,
                   const uint16_t* v_scale, int64_t num_blocks, const int32_t* block_table,
                   int max_blocks_per_seq, const int32_t* context_lens, int ctx_cap, int batch,
                   int num_q_heads, int num_kv_heads, int head_dim, float sm_scale, float* out,
                   hipStream_t stream) {
  PrefillArgs a;
  a.q = q;
  a.q_start_loc = q_start_loc;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.out = out;
  a.total_q = total_q;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.ctx_cap = ctx_cap;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.sm_scale_log2 = sm_scale * kLog2e;
  const int G = num_q_heads / num_kv_heads;
  if (head_dim == 128) return launch_d<128>(a, G, batch, max_q_len, stream);
  if (head_dim == 64) return launch_d<64>(a, G, batch, max_q_len, stream);
  return -2;
}

}  // namespace kv8
