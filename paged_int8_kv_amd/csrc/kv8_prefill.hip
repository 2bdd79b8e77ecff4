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
// Work split: one workgroup of 8 waves per (sequence b, KV head g, tile of
// 256 queries).  A query is a (chunk row, head of the group) pair with the
// G heads innermost, so every K/V byte staged by the workgroup serves all G
// heads of its group.  Each wave owns 32 queries (one 32-column block of the
// MFMA output) and keeps their Q operands in registers; at two waves per
// SIMD one wave's softmax overlaps the other's matrix work.
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
// INT8 codes become fp16 without a convert per code: u = c xor 0x80 under
// the fp16 high byte 0x64 is the value c + 1152, and one packed fp16
// subtract of 1152 leaves c exactly.  The same kernel serves the FP8 (e4m3)
// cache ("KV Cache 优化全景解析", section 7.4), whose codes become exact
// fp16 pairs by one hardware convert, and the INT4 cache, whose nibble pairs
// become c + 1032 by a shift and one and-or with the fp16 pattern, and then c
// by the same kind of subtract; only the staging differs.
//
// Per wave and key tile (v_mfma_f32_32x32x16_f16, fp32 accumulate):
//   S^T[key][query] = K_code . Q^T, with Q scaled by one power of two 2^e
//                     per workgroup so that bf16 q is exact in fp16 (the
//                     workgroup's max |q| in [2^14, 2^15));
//   z = S^T * (k_scale[key] * sm_scale * log2(e) * 2^-e), the factor staged
//       with the scales; a row whose max moves gets 2^0 = 1 exactly;
//   online softmax in base 2: running max m_q and sum l_q per query; m_q
//   moves (and the accumulator is rescaled) only when the tile's max exceeds
//   it by more than kSlack, so 2^(z - m_q) <= 2^kSlack (exactly when the tile
//   holds a large v_scale);
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

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kQueriesPerWave = 32;
constexpr int kQueriesPerGroup = kWaves * kQueriesPerWave;   // 256
constexpr int kTileKeys = 64;                                // 4 cache blocks
constexpr float kLog2e = 1.4426950408889634f;
// A row's running max is moved (and the accumulator rescaled) only when the
// tile max exceeds it by more than kSlack (log2 units), so weights p may
// reach 2^kSlack.  Tiles holding a v_scale >= kBigVScale rescale exactly
// instead, so that p * v_scale always stays below the fp16 maximum.
constexpr float kSlack = 8.0f;
constexpr float kBigVScale = 128.0f;

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
  int batch;
  int tiles_per_pair;      // query tiles per (sequence, KV head)
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
  int big_vs[2];                                // some v_scale of the tile >= kBigVScale
  float qmax[kWaves];                           // per-wave max |q| (prologue)
};

// V^T rows hold 8 chunks of 8 keys (16 bytes); chunk c of row r is stored at
// c ^ vt_swizzle(r).  gfx950's LDS serves 32 consecutive lanes of a 16-byte
// read per pass over 128 banks of 4 bytes (a counter probe of access
// patterns); under that rule the operand reads here meet 2-way conflicts.
// A layout free of them (swizzle constant per 32-row group) cut the
// kernel's conflict cycles by a third and ran no faster: LDS is not what
// paces this kernel, so the layout stays.
__device__ __forceinline__ int vt_swizzle(int row) {
  return (((row >> 4) & 1) << 1) | ((row >> 5) & 1);
}

__device__ __forceinline__ half8_t as_half8(uint4 u) { return __builtin_bit_cast(half8_t, u); }

// Four codes (one dword) -> two exact fp16 pairs.
template <class C>
__device__ __forceinline__ void codes_to_f16(uint32_t u, half2_t& lo, half2_t& hi) {
  const uint32_t x = C::pre(u);
  lo = C::exact(C::lo(x));
  hi = C::exact(C::hi(x));
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
// K: thread t holds key t/8, channels (t%8)*d/8 ... +d/8.  V: task t (t < d,
// four per channel quad and 16-key group) holds 4 keys x 4 channels: the
// keys 16grp + 8a + 4hh + {0..3}, which sit at positions 8hh + 4a + {0..3}
// of their group in the transposed layout.  Scales: threads 0..63 K,
// 64..127 (wave 1) V.
// 4-bit codes (two per byte, element 2i in the low nibble of byte i) keep
// the same thread roles with half the bytes: K d/16 bytes per thread, V
// 2 bytes (4 channels) per row.
template <int D, bool NIB = false>
struct Stage {
  static constexpr int kKBytes = NIB ? D / 16 : D / 8;   // K code bytes per thread
  static constexpr int kVTasks = 4 * D;         // 512 (d=128) or 256 (d=64)
  uint32_t k[kKBytes / 4];
  uint32_t v[4];
  uint16_t sc;
};

// Cache block ids one thread's staging reads for a key tile (its K row's,
// its V rows', its scale's), loaded a tile ahead of the data loads that use
// them, so that those never wait on the block table.
struct TileIds {
  int k, v, s;
};

template <int D, bool NIB>
__device__ __forceinline__ TileIds load_ids(const int32_t* table_row, int kt, int last_blk,
                                            int tid) {
  auto at = [&](int j) {
    const int i = kt * 4 + j;
    return table_row[i < last_blk ? i : last_blk];
  };
  // unconditional (threads without a V row or a scale load an id they do
  // not use): no merge of loaded values across branches, which would wait
  // for every load in flight
  TileIds t;
  t.k = at(tid >> 7);                                            // key tid/8, block key/16
  t.v = at(((tid / (D / 4)) >> 2) & 3);
  t.s = at((tid & 63) >> 4);
  return t;
}

__device__ __forceinline__ int64_t slab_of(const PrefillArgs& a, int id, int g) {
  id = id < 0 ? 0 : (id >= a.num_blocks ? (int)(a.num_blocks - 1) : id);
  return (int64_t)id * a.num_kv_heads + g;       // (block, KV head) slab index
}

template <int D, bool NIB>
__device__ __forceinline__ void stage_load(const PrefillArgs& a, const TileIds& ids, int g,
                                           int tid, Stage<D, NIB>& st) {
  constexpr int RB = NIB ? D / 2 : D;           // code bytes per cache row
  constexpr int KB = Stage<D, NIB>::kKBytes;
  {
    const int key = tid >> 3, part = tid & 7;
    const int64_t slab = slab_of(a, ids.k, g);
    const int8_t* src = a.k_cache + slab * (kBlock * RB) + (key & 15) * RB + part * KB;
    if constexpr (KB == 16) {
      const uint4 u = *reinterpret_cast<const uint4*>(src);
      st.k[0] = u.x; st.k[1] = u.y; st.k[2] = u.z; st.k[3] = u.w;
    } else if constexpr (KB == 8) {
      const uint2 u = *reinterpret_cast<const uint2*>(src);
      st.k[0] = u.x; st.k[1] = u.y;
    } else {
      st.k[0] = *reinterpret_cast<const uint32_t*>(src);
    }
  }
  // Branch-free: threads past the V tasks and the scale threads load in-bounds
  // bytes they do not store, so that the loads of one tile always take one
  // path and their waits count exactly.
  {
    const int cq = tid % (D / 4), kq = (tid / (D / 4)) & 15;
    const int sub = kq & 3;
    const int64_t slab = slab_of(a, ids.v, g);
    const int8_t* base = a.v_cache + slab * (kBlock * RB) + cq * (NIB ? 2 : 4);
    const int row0 = 8 * (sub >> 1) + 4 * (sub & 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (NIB) st.v[r] = *reinterpret_cast<const uint16_t*>(base + (row0 + r) * RB);
      else st.v[r] = *reinterpret_cast<const uint32_t*>(base + (row0 + r) * RB);
    }
  }
  {
    const int key = tid & 63;
    const int64_t slab = slab_of(a, ids.s, g);
    const uint16_t* sp = (tid & kTileKeys) == 0 ? a.k_scale : a.v_scale;
    st.sc = sp[slab * kBlock + (key & 15)];
  }
}

template <int D, class C>
__device__ __forceinline__ void stage_store(Lds<D>& lds, int buf, int kt, int n_keys, int tid,
                                            float k_mult,
                                            const Stage<D, C::kBits == 4>& st) {
  constexpr bool NIB = C::kBits == 4;
  {
    const int key = tid >> 3, part = tid & 7;
    uint32_t o[D / 16];                         // the thread's d/8 channels as fp16 pairs
    if constexpr (NIB) {
      // dword j: channels 8j .. 8j+7 as nibbles; pair m (channels 2m, 2m+1)
      // takes byte m's low nibble from x and its high nibble from x >> 4
#pragma unroll
      for (int j = 0; j < Stage<D, true>::kKBytes / 4; ++j) {
        const uint32_t x = C::pre(st.k[j]), xs = x >> 4;
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          const uint32_t sel = 0x0C000C00u | ((4u + mm) << 16) | (uint32_t)mm;   // [x.b_m, 0, xs.b_m, 0]
          const uint32_t t = (__builtin_amdgcn_perm(xs, x, sel) & 0x000F000Fu) | 0x64006400u;
          o[4 * j + mm] = h2_bits(C::exact(__builtin_bit_cast(half2_t, t)));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < Stage<D>::kKBytes / 4; ++j) {
        half2_t lo, hi;
        codes_to_f16<C>(st.k[j], lo, hi);
        o[2 * j] = h2_bits(lo);
        o[2 * j + 1] = h2_bits(hi);
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(&lds.k[buf][key][part * (D / 8)]);
#pragma unroll
    for (int i = 0; i < D / 64; ++i)
      dst[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  }
  if constexpr (NIB) {
    if (tid < Stage<D, true>::kVTasks) {
      const int cq = tid % (D / 4), kq = tid / (D / 4);
      const int grp = kq >> 2, sub = kq & 3;
      const int a4 = sub >> 1, hh = sub & 1;
      // rows r, r+1 side by side: nibble ci of each half is channel ci of
      // that row, so nibble pair ci is (row r, row r+1) of channel 4 cq + ci
      const uint32_t u01 = C::pre(st.v[0] | (st.v[1] << 16));
      const uint32_t u23 = C::pre(st.v[2] | (st.v[3] << 16));
#pragma unroll
      for (int ci = 0; ci < 4; ++ci) {
        const half2_t p01 = C::exact(C::nib_pair(u01, ci));
        const half2_t p23 = C::exact(C::nib_pair(u23, ci));
        const int row = cq * 4 + ci;
        *reinterpret_cast<uint2*>(
            &lds.v[buf][row][8 * ((grp * 2 + hh) ^ vt_swizzle(row)) + 4 * a4]) =
            make_uint2(h2_bits(p01), h2_bits(p23));
      }
    }
  } else if (tid < Stage<D>::kVTasks) {
    const int cq = tid % (D / 4), kq = tid / (D / 4);
    const int grp = kq >> 2, sub = kq & 3;
    const int a4 = sub >> 1, hh = sub & 1;
    // 4 rows x 4 channel bytes -> per channel the 4 rows' codes
    const uint32_t t01l = C::pre(interleave_lo(st.v[0], st.v[1]));   // [r0c0 r1c0 r0c1 r1c1]
    const uint32_t t01h = C::pre(interleave_hi(st.v[0], st.v[1]));   // [r0c2 r1c2 r0c3 r1c3]
    const uint32_t t23l = C::pre(interleave_lo(st.v[2], st.v[3]));
    const uint32_t t23h = C::pre(interleave_hi(st.v[2], st.v[3]));
#pragma unroll
    for (int ci = 0; ci < 4; ++ci) {
      const uint32_t x01 = ci < 2 ? t01l : t01h, x23 = ci < 2 ? t23l : t23h;
      const half2_t p01 = C::exact((ci & 1) ? C::hi(x01) : C::lo(x01));
      const half2_t p23 = C::exact((ci & 1) ? C::hi(x23) : C::lo(x23));
      const int row = cq * 4 + ci;
      *reinterpret_cast<uint2*>(
          &lds.v[buf][row][8 * ((grp * 2 + hh) ^ vt_swizzle(row)) + 4 * a4]) =
          make_uint2(h2_bits(p01), h2_bits(p23));
    }
  }
  if (tid < 2 * kTileKeys) {
    const int key = tid & 63;
    const float s = (kt * kTileKeys + key < n_keys) ? fp16_bits_to_f32(st.sc) : 0.0f;
    if (tid < kTileKeys) {
      lds.ks[buf][key] = s * k_mult;
    } else {
      lds.vs[buf][key] = s;
      // threads 64..127 are exactly wave 1: one ballot covers the tile
      const bool big = __builtin_amdgcn_ballot_w64(!(s < kBigVScale)) != 0;
      if (key == 0) lds.big_vs[buf] = big;
    }
  }
}

// Online softmax of one 64-key tile for the lane's query.  ks holds
// k_scale * sm_scale * log2(e) * 2^-e (e: the workgroup's Q exponent), so
// z = S^T * ks is the logit in log2 units; vs holds v_scale.  Returns the
// fp16 weights 2^(z - m) * v_scale as the PV B operands.  The lane's keys in
// 32-key block kb are 32kb + 8a + 4h + i for S register r = 4a + i.
//
// Fast path (no causal mask, no large v_scale, every running max already
// set): p = 2^fma(S, ks, -m) with the current maxima, accepted when every
// lane's tile sum of p is <= 256, which bounds each p and keeps p * v_scale
// in fp16 range.  Otherwise the exact path runs: z = S * ks, the tile max,
// and the slack rule (a lane's max moves, rescaling its accumulator, when
// the tile max exceeds it by more than kSlack, or at all on a tile with a
// large v_scale).  A lane that moved its max uses 2^(z - m), so its largest
// weight is exactly 1; every other lane uses the fast path's formula, so a
// lane's result never depends on which path its wave took.
template <bool MASK, int CB>
__device__ __forceinline__ void softmax_tile(f32x16_t (&sc)[2], const float* ks, const float* vs,
                                             int h, int key0, int qpos, bool big_tile,
                                             float& mrun, float& lrun, f32x16_t (&acc)[CB],
                                             half8_t (&pw)[2][2]) {
  if (!MASK && !big_tile && __builtin_amdgcn_ballot_w64(mrun == kNegInf) == 0) {
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 k4 = *reinterpret_cast<const float4*>(ks + 32 * kb + 8 * a4 + 4 * h);
        const float4 v4 = *reinterpret_cast<const float4*>(vs + 32 * kb + 8 * a4 + 4 * h);
        const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
        const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * a4 + i;
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], kv[i], -mrun));
          lsum += p;
          pw[kb][r >> 3][r & 7] = (_Float16)(p * vv[i]);
        }
      }
    if (__builtin_amdgcn_ballot_w64(!(lsum <= 256.0f)) == 0) {
      lrun += lsum;
      return;
    }
  }
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const float4 k4 = *reinterpret_cast<const float4*>(ks + 32 * kb + 8 * a4 + 4 * h);
      const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = sc[kb][4 * a4 + i] * kv[i];
        if (MASK) x = (key0 + 32 * kb + 8 * a4 + 4 * h + i > qpos) ? kNegInf : x;
        mx = fmaxf(mx, x);
      }
    }
  mx = wave_max32(mx);
  const bool grow = mx > mrun + (big_tile ? 0.0f : kSlack);
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float mnew = grow ? mx : mrun;
    const float alpha = mnew == mrun ? 1.0f : __builtin_amdgcn_exp2f(mrun - mnew);
    lrun *= alpha;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
    mrun = mnew;
  }
  const float muse = mrun == kNegInf ? 0.0f : mrun;
  float lsum = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const float4 k4 = *reinterpret_cast<const float4*>(ks + 32 * kb + 8 * a4 + 4 * h);
      const float4 v4 = *reinterpret_cast<const float4*>(vs + 32 * kb + 8 * a4 + 4 * h);
      const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
      const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * a4 + i;
        const float sv = sc[kb][r];
        float exact;
        {
          // the rounded product, as the max saw it, minus the max: no fma
#pragma clang fp contract(off)
          exact = sv * kv[i] - muse;
        }
        float arg = grow ? exact : __builtin_fmaf(sv, kv[i], -muse);
        if (MASK) arg = (key0 + 32 * kb + 8 * a4 + 4 * h + i > qpos) ? kNegInf : arg;
        const float p = __builtin_amdgcn_exp2f(arg);
        lsum += p;
        pw[kb][r >> 3][r & 7] = (_Float16)(p * vv[i]);
      }
    }
  lrun += lsum;
}

template <int D, int G, class C>
__global__ void __launch_bounds__(kThreads) prefill_kernel(PrefillArgs a) {
  constexpr int KS = D / 16;        // k-steps of the QK^T product
  constexpr int CB = D / 32;        // 32-channel blocks of the output
  constexpr int kRowsPerTile = kQueriesPerGroup / G;
  __shared__ Lds<D> lds;

  // XCD-aware, longest-first order.  Workgroup id L runs on XCD L % 8; pair
  // p = (b, g) is served by the XCD p % 8, so all query tiles of a pair share
  // that XCD's L2 and its K/V is fetched from HBM about once.  Within an XCD
  // the k-th workgroup (k = L / 8) takes the pair of rank k / tiles when the
  // XCD's pairs are ordered by decreasing context length (longest first
  // balances the CUs), and its tiles from the last (most keys) down.  Every
  // workgroup computes the same ranks, so the map is a bijection.
  const int L = blockIdx.x;
  const int tiles = a.tiles_per_pair;
  const int npairs = a.batch * a.num_kv_heads;
  const int xcd = L & 7, kx = L >> 3;
  const int npx = (npairs - xcd + 7) >> 3;                      // pairs on this XCD
  const int prank = kx / tiles;
  const int tile = tiles - 1 - kx % tiles;
  if (prank >= npx) return;                                      // padding
  int pair = xcd + 8 * prank;
  if (npx > 1 && npx <= 64) {
    const int ln = threadIdx.x & 63;
    int cost = -1;
    if (ln < npx) {
      const int bb = (xcd + 8 * ln) / a.num_kv_heads;
      const int c = a.context_lens[bb];
      const bool has_rows = a.q_start_loc[bb + 1] > a.q_start_loc[bb];
      cost = has_rows ? (c < a.ctx_cap ? c : a.ctx_cap) : -1;
    }
    int rank = 0;
    for (int j = 0; j < npx; ++j) {
      const int cj = __builtin_amdgcn_readlane(cost, j);
      rank += (cj > cost || (cj == cost && j < ln)) ? 1 : 0;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(ln < npx && rank == prank);
    pair = xcd + 8 * (int)__builtin_ctzll(hit);
  }
  const int b = pair / a.num_kv_heads, g = pair % a.num_kv_heads;
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

  Stage<D, C::kBits == 4> st;
  TileIds ids_next = {0, 0, 0};
  if (nkt > 0) {
    const TileIds ids0 = load_ids<D, C::kBits == 4>(table_row, 0, last_blk, tid);
    stage_load<D>(a, ids0, g, tid, st);
    ids_next = load_ids<D, C::kBits == 4>(table_row, nkt > 1 ? 1 : 0, last_blk, tid);
  }

  // ---- this lane's query: load Q, exact fp16 after a power-of-two scale ----
  const int nq = wave * kQueriesPerWave + m;
  const int qrow = row_begin + nq / G;
  const int qhead = g * G + nq % G;
  const bool qvalid = qrow < row_end;
  const int qpos = pos0 + qrow;
  // One power-of-two exponent e for the whole workgroup: max |q| over its
  // 256 queries lands in [2^14, 2^15), so bf16 q is exact in fp16 (bits far
  // below the workgroup's largest element aside) and the factor 2^-e folds
  // into the staged k_scale.
  half8_t qf[KS];
  uint4 raw[KS];
  if (qvalid) {
    const uint4* src = reinterpret_cast<const uint4*>(
        a.q + ((int64_t)(r0 + qrow) * a.num_q_heads + qhead) * D + (D / 2) * h);
#pragma unroll
    for (int s = 0; s < KS; ++s) raw[s] = src[s];
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) raw[s] = make_uint4(0, 0, 0, 0);
  }
  {
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
    mx = across_groups_max(group8_max(mx));
    if (lane == 0) lds.qmax[wave] = mx;
  }
  // wave-uniform causal bounds of this wave's valid queries
  const int wave_row_lo = row_begin + (wave * kQueriesPerWave) / G;
  const int wave_row_hi = min(row_begin + (wave * kQueriesPerWave + kQueriesPerWave - 1) / G,
                              row_end - 1);
  const bool wave_live = wave_row_lo <= wave_row_hi;
  const int wave_pos_lo = pos0 + wave_row_lo;   // smallest position of the wave
  const int wave_pos_hi = pos0 + wave_row_hi;   // largest

  // V^T operand of row cb*32 + m, chunk 4kb + 2j + h: the row's swizzle is
  // 2 (m >> 4 & 1) + (cb & 1), so the chunk stored there is 4kb + 2(j ^ m4)
  // + (h ^ (cb & 1)); the lane-dependent part is one of four offsets.
  const _Float16* vlane = &lds.v[0][m][0];
  int vt_lane_off[2][2];
  {
    const int m4 = (m >> 4) & 1;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int c = 0; c < 2; ++c) vt_lane_off[j][c] = 16 * (j ^ m4) + 8 * (h ^ c);
  }

  f32x16_t acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.0f;
  float mrun = kNegInf, lrun = 0.0f;

  __syncthreads();
  float k_mult;
  {
    float mx = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, lds.qmax[w]);
    int e = 0;
    if (mx > 0.0f) {
      int ex;
      frexpf(mx, &ex);                 // mx = f * 2^ex, f in [0.5, 1)
      e = 15 - ex;                     // mx * 2^e in [2^14, 2^15)
      e = e > 120 ? 120 : (e < -120 ? -120 : e);
    }
    k_mult = ldexpf(a.sm_scale_log2, -e);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t w[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qf[s][2 * j] = (_Float16)ldexpf(__builtin_bit_cast(float, w[j] << 16), e);
        qf[s][2 * j + 1] = (_Float16)ldexpf(__builtin_bit_cast(float, w[j] & 0xFFFF0000u), e);
      }
    }
  }
  if (nkt > 0) stage_store<D, C>(lds, 0, 0, n_keys, tid, k_mult, st);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nkt;
    stage_load<D>(a, ids_next, g, tid, st);   // the last step's load is not stored
    ids_next = load_ids<D, C::kBits == 4>(table_row, kt + 2 < nkt ? kt + 2 : kt, last_blk, tid);

    const int key0 = kt * kTileKeys;
    if (wave_live && key0 <= wave_pos_hi) {
      const bool live1 = key0 + 32 <= wave_pos_hi;   // second 32-key block visible
      // ---- S^T = K . Q^T: 64 keys x 32 queries ------------------------------
      f32x16_t sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
      const _Float16* krow0 = &lds.k[buf][m][(D / 2) * h];
      const _Float16* krow1 = krow0 + 32 * Lds<D>::kRow;
      if (live1) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const half8_t k0 = *reinterpret_cast<const half8_t*>(krow0 + 8 * s);
          const half8_t k1 = *reinterpret_cast<const half8_t*>(krow1 + 8 * s);
          sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0, qf[s], sacc[0], 0, 0, 0);
          sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k1, qf[s], sacc[1], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const half8_t k0 = *reinterpret_cast<const half8_t*>(krow0 + 8 * s);
          sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0, qf[s], sacc[0], 0, 0, 0);
        }
      }
      // ---- online softmax and fp16 weights -------------------------------------
      const bool need_mask = key0 + kTileKeys - 1 > wave_pos_lo;
      const bool big_tile = lds.big_vs[buf] != 0;
      half8_t pw[2][2];     // [kb][k-step]
      if (need_mask)
        softmax_tile<true, CB>(sacc, lds.ks[buf], lds.vs[buf], h, key0, qpos, big_tile, mrun,
                               lrun, acc, pw);
      else
        softmax_tile<false, CB>(sacc, lds.ks[buf], lds.vs[buf], h, key0, qpos, big_tile, mrun,
                                lrun, acc, pw);
      // ---- O^T += V^T . W^T ------------------------------------------------------
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && !live1) break;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          half8_t va[CB];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            va[cb] = as_half8(*reinterpret_cast<const uint4*>(
                vlane + buf * (D * Lds<D>::kVRow) + vt_lane_off[j][cb & 1] +
                cb * 32 * Lds<D>::kVRow + 32 * kb));
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[cb], pw[kb][j], acc[cb], 0, 0, 0);
        }
      }
    }

    if (more) stage_store<D, C>(lds, buf ^ 1, kt + 1, n_keys, tid, k_mult, st);
    __syncthreads();
  }

  // ---- epilogue: O / l, channel 32cb + 8(r/4) + 4h + r%4 --------------------
  const float l = wave_sum32(lrun);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (qvalid) {
    float* dst = a.out + ((int64_t)(r0 + qrow) * a.num_q_heads + qhead) * D + 4 * h;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int r = 4 * a4;
        *reinterpret_cast<float4*>(dst + cb * 32 + 8 * a4) =
            make_float4(acc[cb][r] * inv, acc[cb][r + 1] * inv, acc[cb][r + 2] * inv,
                        acc[cb][r + 3] * inv);
      }
  }
}

template <int D, int G, class C>
int launch_dg(PrefillArgs a, int batch, int max_q_len, hipStream_t stream) {
  const int64_t tiles = ((int64_t)max_q_len * G + kQueriesPerGroup - 1) / kQueriesPerGroup;
  const int64_t pairs8 = ((int64_t)batch * a.num_kv_heads + 7) / 8 * 8;
  if (tiles * pairs8 > 0x7FFFFFFF) return -2;
  a.tiles_per_pair = (int)tiles;
  a.batch = batch;
  hipLaunchKernelGGL((prefill_kernel<D, G, C>), dim3((unsigned)(tiles * pairs8)), dim3(kThreads),
                     0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int D, class C>
int launch_d(const PrefillArgs& a, int G, int batch, int max_q_len, hipStream_t stream) {
  switch (G) {
    case 1: return launch_dg<D, 1, C>(a, batch, max_q_len, stream);
    case 2: return launch_dg<D, 2, C>(a, batch, max_q_len, stream);
    case 4: return launch_dg<D, 4, C>(a, batch, max_q_len, stream);
    case 8: return launch_dg<D, 8, C>(a, batch, max_q_len, stream);
    default: return -2;
  }
}

}  // namespace

int launch_prefill(const uint16_t* q, const int32_t* q_start_loc, int64_t total_q, int max_q_len,
                   const int8_t* k_cache, const int8_t* v_cache, const uint16_t* k_scale,
                   const uint16_t* v_scale, int64_t num_blocks, const int32_t* block_table,
                   int max_blocks_per_seq, const int32_t* context_lens, int ctx_cap, int batch,
                   int num_q_heads, int num_kv_heads, int head_dim, float sm_scale, float* out,
                   int fmt, hipStream_t stream) {
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
  if (fmt == kFmtInt4) {
    if (head_dim == 128) return launch_d<128, CodesInt4>(a, G, batch, max_q_len, stream);
    if (head_dim == 64) return launch_d<64, CodesInt4>(a, G, batch, max_q_len, stream);
    return -2;
  }
  const bool fp8 = fmt == kFmtFp8;
  if (head_dim == 128) return fp8 ? launch_d<128, CodesFp8>(a, G, batch, max_q_len, stream)
                                  : launch_d<128, CodesInt8>(a, G, batch, max_q_len, stream);
  if (head_dim == 64) return fp8 ? launch_d<64, CodesFp8>(a, G, batch, max_q_len, stream)
                                 : launch_d<64, CodesInt8>(a, G, batch, max_q_len, stream);
  return -2;
}

}  // namespace kv8
