// paged_decode_attn_kv8 kernel: split-K flash-decoding over the paged INT8
// cache for gfx950.
//
// Attention softmax(q K^T * sm_scale) V ("KV Cache 优化全景解析", section 2.1)
// per GQA group (section 3.3) over K/V restored on the fly from INT8 codes
// and per-token fp16 scales ("KV-Cache 全栈优化系统" README, section
// 主要特性), with fp32 softmax and accumulation ("大模型推理加速：KV Cache
// 与vLLM技术解析", section 4.1).  Split results are merged by log-sum-exp
// inside the same launch: the last workgroup of a (sequence, KV head) to
// finish merges the partials of all its splits.
//
// One workgroup (4 waves) serves one (sequence b, KV head g, split) and all
// G query heads of the group, so each cache byte is read from HBM once.
// Inside a wave, lane = 8 * slot + chunk: `chunk` picks d/8 channels and
// `slot` (0..7) picks tokens slot and slot+8 of a 16-token block, so one
// wave-wide load of d/8 bytes per lane reads half a block (8 rows of d
// bytes, contiguous in memory) and two loads read the whole block.
//
// The split is processed in two passes over its blocks (distributed
// round-robin over the 4 waves):
//   pass 1  K codes: z[t,h] = log2e * sm_scale * k_scale[t] * <q_h, k_code[t]>
//           for the G heads, written to LDS; running max per head.
//   middle  p[t,h] = 2^(z - M_h) <= 1, l_h = sum p, and the fp16 weight
//           w[t,h] = p * v_scale[t] packed as token pairs in LDS.
//   pass 2  V codes: acc[h,c] = sum_t w[t,h] * v_code[t,c].
// Because the exact split max is known before pass 2, no accumulator is
// ever rescaled and the largest weight of the split is exact.
//
// Dot products use v_dot2_f32_f16 on fp16 pairs.  A code c enters as the
// fp16 value c + 1152 built by one byte permute (see kv8_device.h); the
// bias is removed once per token (pass 1: 1152 * sum q_h) and once per
// output (pass 2: 1152 * sum w).  q enters as fp16 after an exact
// per-head power-of-two rescale (bf16 q is exact in fp16 then); an fp32 q
// is split into a high and a low fp16 part.
//
// Each wave keeps kPf blocks in flight in a register ring; the ring is
// branch-free around its loads so that the compiler's wait counts stay
// exact, and scheduling barriers keep later slots' waits from being hoisted.
#include <atomic>

#include "kv8_device.h"
#include "kv8_launch.h"

namespace kv8 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kPf = 4;        // blocks in flight per wave and pass
constexpr int kMergeBatch = 8;
constexpr float kLog2e = 1.4426950408889634f;

struct SplitArgs {
  const void* q;
  const int8_t* k_cache;
  const int8_t* v_cache;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  const int32_t* block_table;
  const int32_t* context_lens;
  float* out;
  float* o_part;
  float* lse_part;
  unsigned* counters;
  int64_t num_blocks;
  int max_blocks_per_seq;
  int ctx_cap;
  int num_q_heads;
  int num_kv_heads;
  int split_tokens;
  int n_split;
  int batch;
  int period;        // workgroups per dispatch round (the CU count)
  int snake_rounds;  // rounds resident at once (workgroups per CU)
  float qk_scale_log2;
};

__host__ __device__ constexpr int align16(int x) { return (x + 15) & ~15; }

struct SmemLayout {
  int blk_off, z_off, vs_off, pp_off, red_off, flag_off, total;
};

// LDS carve-up of one workgroup: block ids, logits (reused for the final
// cross-wave reduction), v scales, packed fp16 weights, per-head scalars,
// and the last-workgroup flag.
__host__ __device__ inline SmemLayout smem_layout(int split_tokens, int G, int D) {
  SmemLayout L{};
  const int zbytes = split_tokens * G * 4;
  const int finbytes = kWaves * G * D * 4;
  L.blk_off = 0;
  L.z_off = align16((split_tokens / kBlock) * 4);
  L.vs_off = L.z_off + align16(zbytes > finbytes ? zbytes : finbytes);
  L.pp_off = L.vs_off + align16(split_tokens * 2);
  L.red_off = L.pp_off + align16((split_tokens / 2) * G * 4);
  L.flag_off = L.red_off + align16(3 * kWaves * G * 4);
  L.total = L.flag_off + 16;
  return L;
}

template <int NDW> struct RowT;
template <> struct RowT<4> { using type = uint4; };
template <> struct RowT<2> { using type = uint2; };

__device__ __forceinline__ uint32_t dword(const uint4& r, int k) {
  return k == 0 ? r.x : k == 1 ? r.y : k == 2 ? r.z : r.w;
}
__device__ __forceinline__ uint32_t dword(const uint2& r, int k) { return k == 0 ? r.x : r.y; }

// One reduce-scatter step over lane pairs given by the DPP pattern CTRL:
// the lane flagged `upper` keeps the second half of its N values, its
// partner the first half, and each adds the partner's copy of the half it
// keeps.
template <int CTRL, int N>
__device__ __forceinline__ void rs_half(const float (&in)[N], float (&out)[N / 2], bool upper) {
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const float keep = upper ? in[k + N / 2] : in[k];
    const float send = upper ? in[k] : in[k + N / 2];
    out[k] = keep + dpp_f<CTRL>(send);
  }
}

// Reduce the N = 2G partial dot products v[t*G + h] (tokens t = 0, 1 of the
// lane's pair, heads h) over the 8 lanes of a token group.  Lane i of the
// group ends with NV = max(1, N/8) full sums: value j is v index
//   (i>>2)*(N/2) + ((i>>1)&1)*(N/4 if N>=4) + (i&1)*(N/8 if N>=8) + j,
// i.e. token i>>2.  The first step pairs lanes i and 7-i (half mirror),
// the next two are quad exchanges.
template <int G>
__device__ __forceinline__ void reduce_scatter8(const float (&v)[2 * G],
                                                float (&out)[(2 * G >= 8) ? (2 * G) / 8 : 1],
                                                int i) {
  constexpr int N = 2 * G;
  float a[N / 2];
  rs_half<kDppHalfMirror, N>(v, a, i >= 4);
  if constexpr (N / 2 >= 2) {
    float b[N / 4];
    rs_half<kDppQuadXor2, N / 2>(a, b, (i & 2) != 0);
    if constexpr (N / 4 >= 2) {
      rs_half<kDppQuadXor1, N / 4>(b, out, (i & 1) != 0);
    } else {
      out[0] = b[0] + dpp_f<kDppQuadXor1>(b[0]);
    }
  } else {
    float x = a[0] + dpp_f<kDppQuadXor2>(a[0]);
    out[0] = x + dpp_f<kDppQuadXor1>(x);
  }
}

// Head of value j after reduce_scatter8 on lane i of its group.
template <int G>
__device__ __forceinline__ int rs_head(int i, int j) {
  constexpr int N = 2 * G;
  int idx = ((i >> 1) & 1) * (N >= 4 ? N / 4 : 0) + (i & 1) * (N >= 8 ? N / 8 : 0) + j;
  return idx % G;
}

// Agent-scope relaxed accesses (coherent across the XCDs' L2 caches).
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Wait until every vector memory access of this wave has completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D, int G, bool QF32>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(SplitArgs a) {
  constexpr int CPL = D / 8;    // channels (= code bytes) per lane per token
  constexpr int NDW = CPL / 4;  // dwords per lane per token
  constexpr int NP = CPL / 2;   // fp16 pairs per lane per token
  constexpr int NV = (2 * G >= 8) ? (2 * G) / 8 : 1;   // logits stored per lane
  constexpr int M = G * CPL;    // accumulators per lane
  using Row = typename RowT<NDW>::type;

  extern __shared__ __align__(16) unsigned char smem[];
  const SmemLayout L = smem_layout(a.split_tokens, G, D);
  int* s_blk = reinterpret_cast<int*>(smem + L.blk_off);
  float* s_z = reinterpret_cast<float*>(smem + L.z_off);
  float* s_fin = s_z;
  uint16_t* s_vs = reinterpret_cast<uint16_t*>(smem + L.vs_off);
  uint32_t* s_pp = reinterpret_cast<uint32_t*>(smem + L.pp_off);
  float* s_red = reinterpret_cast<float*>(smem + L.red_off);   // [3][kWaves][G]
  int* s_flag = reinterpret_cast<int*>(smem + L.flag_off);

  const int tid = threadIdx.x, lane = tid & 63;
  // Work items are (sequence b, split, KV head g).  A sequence's n splits
  // share its blocks evenly (n = ceil(blocks / blocks_per_split)), so its
  // items are of one size and only the last block of the last split is
  // partial; a sequence with an empty context keeps one item, which writes
  // its zero output.  The grid is sized by the longest context and
  // workgroups past the last item exit.
  //
  // Item order.  The dispatcher places workgroup i on the CU that i mod
  // `period` names, as long as every workgroup of the first snake_rounds
  // rounds of `period` is resident at once.  With at most 64 sequences the
  // items are ranked longest first and dealt to those rounds in a snake
  // (even rounds forward, odd rounds backward), which evens out the tokens
  // per CU; later rounds keep the longest-first order, which the dispatcher
  // fills greedily as CUs free up.  With more sequences the items keep
  // sequence order.  Every wave locates its item itself.
  const int bps = a.split_tokens / kBlock;      // blocks per split at most
  int b = -1, g = 0, split = 0, nsplit = 1, nbt = 0;
  if (a.batch <= 64 && a.period > 0) {
    int key = -1, cnt = 0, nb = 0, n = 1;
    if (lane < a.batch) {
      const int cx = min(max(a.context_lens[lane], 0), a.ctx_cap);
      nb = (cx + kBlock - 1) / kBlock;
      n = max(1, (nb + bps - 1) / bps);
      key = ((nb + n - 1) / n) * 64 + (63 - lane);  // unique; larger goes first
      cnt = n * a.num_kv_heads;
    }
    int start = 0, total = 0;
    for (int j = 0; j < a.batch; ++j) {
      const int kj = __builtin_amdgcn_readlane(key, j);
      const int cj = __builtin_amdgcn_readlane(cnt, j);
      start += kj > key ? cj : 0;
      total += cj;
    }
    const int bid = (int)blockIdx.x;
    const int r = bid / a.period;
    int rank = bid;
    if (r < a.snake_rounds) {
      const int c = bid - r * a.period;
      rank = r * a.period + ((r & 1) ? a.period - 1 - c : c);
    }
    if (rank < total) {
      const uint64_t hit = __ballot(lane < a.batch && start <= rank && rank < start + cnt);
      b = (int)__builtin_ctzll(hit);
      const int j = rank - __builtin_amdgcn_readlane(start, b);
      split = j / a.num_kv_heads;
      g = j - split * a.num_kv_heads;
      nsplit = __builtin_amdgcn_readlane(n, b);
      nbt = __builtin_amdgcn_readlane(nb, b);
    }
  } else {
    const int sg = (int)blockIdx.x / a.num_kv_heads;     // global split index
    g = (int)blockIdx.x - sg * a.num_kv_heads;
    int base = 0;
    for (int c0 = 0; c0 < a.batch; c0 += 64) {
      const int bi = c0 + lane;
      int n = 0, nb = 0;
      if (bi < a.batch) {
        const int cx = min(max(a.context_lens[bi], 0), a.ctx_cap);
        nb = (cx + kBlock - 1) / kBlock;
        n = max(1, (nb + bps - 1) / bps);
      }
      const int incl = wave_incl_scan(n, lane);
      const int tot = __builtin_amdgcn_readlane(incl, 63);
      if (sg < base + tot) {
        const int idx = __builtin_popcountll(__ballot(base + incl <= sg));
        b = c0 + idx;
        nsplit = __builtin_amdgcn_readlane(n, idx);
        nbt = __builtin_amdgcn_readlane(nb, idx);
        split = sg - base - (__builtin_amdgcn_readlane(incl, idx) - nsplit);
        break;
      }
      base += tot;
    }
  }
  if (b < 0) return;                           // uniform: past the work list
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int slot = lane >> 3, chunk = lane & 7;
  const int64_t bh0 = (int64_t)b * a.num_q_heads + (int64_t)g * G;

  int ctx = a.context_lens[b];
  ctx = min(max(ctx, 0), a.ctx_cap);
  if (ctx == 0) {                              // uniform: empty context, zero output
    for (int e = tid; e < G * D; e += kThreads) a.out[bh0 * D + e] = 0.0f;
    return;
  }
  // blocks [jb0, jb0 + nblk) of the sequence: nbt blocks shared by nsplit
  const int bq = nbt / nsplit, brem = nbt - bq * nsplit;
  const int nblk = bq + (split < brem ? 1 : 0);
  const int jb0 = split * bq + min(split, brem);
  const int t0 = jb0 * kBlock;
  const int ntok = min(ctx - t0, nblk * kBlock);
  const int Hkv = a.num_kv_heads;
  const int nvalid = nsplit;

  if (tid < nblk) {
    int64_t id = a.block_table[(int64_t)b * a.max_blocks_per_seq + jb0 + tid];
    id = id < 0 ? 0 : (id >= a.num_blocks ? a.num_blocks - 1 : id);
    s_blk[tid] = (int)id;
  }

  // ---- q of the G heads: this lane's d/8 channels as fp16 pairs ----------
  half2_t qh[G][NP];
  half2_t ql[QF32 ? G : 1][QF32 ? NP : 1];
  float cz[G], qbias[G];
  {
    const int64_t qrow0 = bh0 * D + chunk * CPL;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x[CPL];
      if constexpr (QF32) {
        const float4* qp = reinterpret_cast<const float4*>(
            static_cast<const float*>(a.q) + qrow0 + (int64_t)h * D);
#pragma unroll
        for (int i = 0; i < CPL / 4; ++i) {
          const float4 v = qp[i];
          x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
        }
      } else {
        // CPL bf16 values = two Rows of NDW dwords
        const Row* qp = reinterpret_cast<const Row*>(
            static_cast<const uint16_t*>(a.q) + qrow0 + (int64_t)h * D);
        const Row r = qp[0], r2 = qp[1];
#pragma unroll
        for (int k = 0; k < NDW; ++k) {
          const uint32_t w = dword(r, k), w2 = dword(r2, k);
          x[2 * k] = __builtin_bit_cast(float, w << 16);
          x[2 * k + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
          x[2 * NDW + 2 * k] = __builtin_bit_cast(float, w2 << 16);
          x[2 * NDW + 2 * k + 1] = __builtin_bit_cast(float, w2 & 0xFFFF0000u);
        }
      }
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) m = fmaxf(m, fabsf(x[i]));
      m = group8_max(m);
      // power-of-two shift bringing the head's largest |q| into [2^14, 2^15)
      const int e = m > 0.0f ? ilogbf(m) - 14 : 0;
      float qsum = 0.0f;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const float a0 = ldexpf(x[2 * p], -e), a1 = ldexpf(x[2 * p + 1], -e);
        const _Float16 h0 = (_Float16)a0, h1 = (_Float16)a1;
        qh[h][p] = half2_t{h0, h1};
        qsum += (float)h0 + (float)h1;
        if constexpr (QF32) {
          const _Float16 l0 = (_Float16)(a0 - (float)h0), l1 = (_Float16)(a1 - (float)h1);
          ql[h][p] = half2_t{l0, l1};
          qsum += (float)l0 + (float)l1;
        }
      }
      qsum = group8_sum(qsum);
      cz[h] = ldexpf(a.qk_scale_log2, e);
      qbias[h] = kCodeBias * qsum;
    }
  }
  // per-lane constants of the logits this lane stores after the reduction
  const int tk = chunk >> 2;            // token of the pair: slot or slot+8
  int hv[NV];
  float czl[NV], qbl[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    hv[j] = rs_head<G>(chunk, j);
    czl[j] = cz[0];
    qbl[j] = qbias[0];
#pragma unroll
    for (int h = 1; h < G; ++h) {
      czl[j] = hv[j] == h ? cz[h] : czl[j];
      qbl[j] = hv[j] == h ? qbias[h] : qbl[j];
    }
  }
  __syncthreads();   // s_blk visible

  // Each wave owns blocks wave + i * kWaves, i = 0 .. nmine-1.
  const int nmine = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;
  const int last = nmine - 1;
  auto line_of = [&](int i) {
    return ((int64_t)s_blk[wave + i * kWaves] * Hkv + g) * kBlock + slot;
  };

  // ---- pass 1: logits ----------------------------------------------------
  float mloc[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) mloc[j] = kNegInf;
  if (nmine > 0) {
    Row r0[kPf], r1[kPf];
    uint16_t ks0[kPf], ks1[kPf], vs0[kPf], vs1[kPf];
    auto issue = [&](int s, int i) {
      const int64_t line = line_of(i);
      const int8_t* p = a.k_cache + line * D + chunk * CPL;
      r0[s] = *reinterpret_cast<const Row*>(p);
      r1[s] = *reinterpret_cast<const Row*>(p + 8 * D);
      ks0[s] = a.k_scale[line];
      ks1[s] = a.k_scale[line + 8];
      vs0[s] = a.v_scale[line];
      vs1[s] = a.v_scale[line + 8];
    };
    // Slots past the wave's last block re-read that block (L2 hits) and skip
    // the compute, so every load stays unconditional.
#pragma unroll
    for (int s = 0; s < kPf; ++s) issue(s, min(s, last));
    for (int base = 0; base < nmine; base += kPf) {
#pragma unroll
      for (int s = 0; s < kPf; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        const int i = base + s;
        if (i < nmine) {
          const Row w0 = r0[s], w1 = r1[s];
          float S[2 * G];
#pragma unroll
          for (int k = 0; k < 2 * G; ++k) S[k] = 0.0f;
#pragma unroll
          for (int k = 0; k < NDW; ++k) {
            const uint32_t x0 = dword(w0, k) ^ kXor80, x1 = dword(w1, k) ^ kXor80;
            const half2_t a0 = biased_pair_lo(x0), b0 = biased_pair_hi(x0);
            const half2_t a1 = biased_pair_lo(x1), b1 = biased_pair_hi(x1);
#pragma unroll
            for (int h = 0; h < G; ++h) {
              S[h] = fdot2(qh[h][2 * k], a0, S[h]);
              S[h] = fdot2(qh[h][2 * k + 1], b0, S[h]);
              S[G + h] = fdot2(qh[h][2 * k], a1, S[G + h]);
              S[G + h] = fdot2(qh[h][2 * k + 1], b1, S[G + h]);
              if constexpr (QF32) {
                S[h] = fdot2(ql[h][2 * k], a0, S[h]);
                S[h] = fdot2(ql[h][2 * k + 1], b0, S[h]);
                S[G + h] = fdot2(ql[h][2 * k], a1, S[G + h]);
                S[G + h] = fdot2(ql[h][2 * k + 1], b1, S[G + h]);
              }
            }
          }
          float R[NV];
          reduce_scatter8<G>(S, R, chunk);
          const int tl = (wave + i * kWaves) * kBlock + slot + 8 * tk;
          const bool ok = tl < ntok;
          const float ksc = fp16_bits_to_f32(tk ? ks1[s] : ks0[s]);
#pragma unroll
          for (int j = 0; j < NV; ++j) {
            const float z = ok ? (ksc * czl[j]) * (R[j] - qbl[j]) : kNegInf;
            s_z[tl * G + hv[j]] = z;
            mloc[j] = fmaxf(mloc[j], z);
          }
          s_vs[tl] = tk ? vs1[s] : vs0[s];
        }
        issue(s, min(i + kPf, last));
      }
    }
  }

  // V rows of the first kPf blocks are requested now, so that they arrive
  // while the workgroup finishes the logits and builds the weights.
  Row r0[kPf], r1[kPf];
  auto issue_v = [&](int s, int i) {
    const int8_t* p = a.v_cache + line_of(i) * D + chunk * CPL;
    r0[s] = *reinterpret_cast<const Row*>(p);
    r1[s] = *reinterpret_cast<const Row*>(p + 8 * D);
  };
  if (nmine > 0) {
#pragma unroll
    for (int s = 0; s < kPf; ++s) issue_v(s, min(s, last));
  }

  // max per head: lanes chunk and chunk^4 hold the two tokens of a head,
  // the eight token groups hold the other tokens
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float m = fmaxf(mloc[j], __shfl_xor(mloc[j], 4));
    m = across_groups_max(m);
    if (slot == 0) s_red[wave * G + hv[j]] = m;
  }
  __syncthreads();

  // ---- middle: weights ----------------------------------------------------
  {
    const int h = tid % G;
    float Mh = s_red[h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) Mh = fmaxf(Mh, s_red[w * G + h]);
    float lsum = 0.0f, psum = 0.0f;
    _Float16* pph = reinterpret_cast<_Float16*>(s_pp);
    const int total = nblk * kBlock * G;
    for (int e = tid; e < total; e += kThreads) {
      const int t = e / G;
      const float z = s_z[e];
      _Float16 p16 = (_Float16)0.0f;
      if (z != kNegInf) {
        const float p = __builtin_amdgcn_exp2f(z - Mh);
        p16 = (_Float16)(p * fp16_bits_to_f32(s_vs[t]));
        lsum += p;
        psum += (float)p16;
      }
      const int jj = t / kBlock, r = t % kBlock;
      pph[((jj * 8 + (r & 7)) * G + h) * 2 + (r >> 3)] = p16;
    }
#pragma unroll
    for (int off = G; off < 64; off <<= 1) {
      lsum += __shfl_xor(lsum, off);
      psum += __shfl_xor(psum, off);
    }
    if (lane < G) {
      s_red[kWaves * G + wave * G + lane] = lsum;
      s_red[2 * kWaves * G + wave * G + lane] = psum;
    }
  }
  __syncthreads();

  // ---- pass 2: weighted sum of V codes ------------------------------------
  float acc[M];
#pragma unroll
  for (int k = 0; k < M; ++k) acc[k] = 0.0f;
  for (int base = 0; base < nmine; base += kPf) {
#pragma unroll
    for (int s = 0; s < kPf; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      const int i = base + s;
      if (i < nmine) {
        const Row w0 = r0[s], w1 = r1[s];
        half2_t wp[G];
        const uint32_t* src = s_pp + ((wave + i * kWaves) * 8 + slot) * G;
#pragma unroll
        for (int h = 0; h < G; ++h) wp[h] = __builtin_bit_cast(half2_t, src[h]);
#pragma unroll
        for (int k = 0; k < NDW; ++k) {
          const uint32_t x0 = dword(w0, k) ^ kXor80, x1 = dword(w1, k) ^ kXor80;
          const uint32_t i01 = interleave_lo(x0, x1), i23 = interleave_hi(x0, x1);
          const half2_t f0 = biased_pair_lo(i01), f1 = biased_pair_hi(i01);
          const half2_t f2 = biased_pair_lo(i23), f3 = biased_pair_hi(i23);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h * CPL + 4 * k] = fdot2(wp[h], f0, acc[h * CPL + 4 * k]);
            acc[h * CPL + 4 * k + 1] = fdot2(wp[h], f1, acc[h * CPL + 4 * k + 1]);
            acc[h * CPL + 4 * k + 2] = fdot2(wp[h], f2, acc[h * CPL + 4 * k + 2]);
            acc[h * CPL + 4 * k + 3] = fdot2(wp[h], f3, acc[h * CPL + 4 * k + 3]);
          }
        }
      }
      issue_v(s, min(i + kPf, last));
    }
  }

  // ---- sum the eight token groups: a row step, then two reduce-scatter
  // steps on the row/half swaps.  Lane l keeps M/4 sums: value k is
  // accumulator k + (M/2)*(row of l is odd) + (M/4)*(l in upper half).
#pragma unroll
  for (int k = 0; k < M; ++k) acc[k] += dpp_f<kDppRowRor8>(acc[k]);
#pragma unroll
  for (int k = 0; k < M / 2; ++k) {
    float x, y;
    swap16_pair(acc[k], acc[k + M / 2], x, y);
    acc[k] = x + y;
  }
#pragma unroll
  for (int k = 0; k < M / 4; ++k) {
    float x, y;
    swap32_pair(acc[k], acc[k + M / 4], x, y);
    acc[k] = x + y;
  }
  if ((lane & 8) == 0) {               // the two groups of a row agree
    const int off = (M / 2) * ((lane >> 4) & 1) + (M / 4) * (lane >> 5);
#pragma unroll
    for (int k = 0; k < M / 4; ++k) {
      const int idx = k + off;
      s_fin[(wave * G + idx / CPL) * D + chunk * CPL + idx % CPL] = acc[k];
    }
  }
  __syncthreads();

  // ---- normalise; write the output or this split's partial ----------------
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, c = e % D;
    float s = s_fin[h * D + c];
    float Mh = s_red[h], Lh = s_red[kWaves * G + h], Ph = s_red[2 * kWaves * G + h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      s += s_fin[(w * G + h) * D + c];
      Mh = fmaxf(Mh, s_red[w * G + h]);
      Lh += s_red[kWaves * G + w * G + h];
      Ph += s_red[2 * kWaves * G + w * G + h];
    }
    const float o = (s - kCodeBias * Ph) / Lh;
    if (nvalid == 1) {
      a.out[(bh0 + h) * D + c] = o;
    } else {
      store_agent(a.o_part + ((bh0 + h) * a.n_split + split) * D + c, o);
      if (c == 0)
        store_agent(a.lse_part + (bh0 + h) * a.n_split + split, Mh + __builtin_amdgcn_logf(Lh));
    }
  }
  if (nvalid == 1) return;

  // ---- the last workgroup of (b, g) merges the splits by log-sum-exp ------
  // Partials travel through agent-scope stores and loads, which write
  // through / bypass the per-XCD L2, so no cache-wide writeback or
  // invalidate is needed: each wave waits for its stores to complete before
  // the barrier, and only then is the split counted.
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    unsigned* cnt = a.counters + (int64_t)b * Hkv + g;
    const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    const int is_last = prev == (unsigned)(nvalid - 1);
    if (is_last)                       // leave the counter zero for the next call
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_flag[0] = is_last;
  }
  __syncthreads();
  if (!s_flag[0]) return;
  // Partials are read in batches of kMergeBatch splits whose loads are all
  // issued before any is used (one memory round trip per batch), and folded
  // in by an online log-sum-exp update.
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, c = e % D;
    const int64_t bh = bh0 + h;
    const float* lse = a.lse_part + bh * a.n_split;
    const float* op = a.o_part + bh * a.n_split * D + c;
    float Mx = kNegInf, num = 0.0f, den = 0.0f;
    for (int s0 = 0; s0 < nvalid; s0 += kMergeBatch) {
      float lv[kMergeBatch], ov[kMergeBatch];
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const int s = min(s0 + u, nvalid - 1);
        lv[u] = load_agent(lse + s);
        ov[u] = load_agent(op + (int64_t)s * D);
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        if (s0 + u < nvalid) {
          const float mn = fmaxf(Mx, lv[u]);
          const float wo = __builtin_amdgcn_exp2f(Mx - mn);   // 0 while Mx = -inf
          const float wn = __builtin_amdgcn_exp2f(lv[u] - mn);
          num = num * wo + wn * ov[u];
          den = den * wo + wn;
          Mx = mn;
        }
      }
    }
    a.out[bh * D + c] = num / den;
  }
}

// Compute units of the current device (cached per device; 0 if unknown).
int device_cu_count() {
  static std::atomic<int> cache[64];   // 0 = not queried, -1 = unknown
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) v = -1;
    c = v > 0 ? v : -1;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c > 0 ? c : 0;
}

template <int D, int G, bool QF32>
bool launch_split(const SplitArgs& a, int batch, hipStream_t stream) {
  const SmemLayout L = smem_layout(a.split_tokens, G, D);
  int64_t grid = (int64_t)a.n_split * a.num_kv_heads * batch;
  SplitArgs args = a;
  args.period = 0;
  args.snake_rounds = 0;
  if (batch <= 64) {
    // resident workgroups per CU for this shared-memory size (cached)
    // (shared-memory bytes << 32 | workgroups); 0 until first computed
    static std::atomic<uint64_t> occ_cache{0};
    uint64_t oc = occ_cache.load(std::memory_order_relaxed);
    if ((oc >> 32) != (uint64_t)L.total) {
      int v = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &v, decode_split_kernel<D, G, QF32>, kThreads, L.total) != hipSuccess) v = 0;
      oc = ((uint64_t)L.total << 32) | (uint32_t)(v > 0 ? v : 0);
      occ_cache.store(oc, std::memory_order_relaxed);
    }
    const int occ = (int)(uint32_t)oc;
    const int cus = device_cu_count();
    if (cus > 0 && occ > 0) {
      args.period = cus;
      args.snake_rounds = occ;
      grid = (grid + cus - 1) / cus * cus;
    }
  }
  if (grid > 0x7FFFFFFF) return false;
  decode_split_kernel<D, G, QF32><<<dim3((unsigned)grid), dim3(kThreads), L.total, stream>>>(args);
  return true;
}

template <int D, bool QF32>
bool dispatch_g(int G, const SplitArgs& a, int batch, hipStream_t s) {
  switch (G) {
    case 1: return launch_split<D, 1, QF32>(a, batch, s);
    case 2: return launch_split<D, 2, QF32>(a, batch, s);
    case 4: return launch_split<D, 4, QF32>(a, batch, s);
    case 8: return launch_split<D, 8, QF32>(a, batch, s);
    default: return false;
  }
}

constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

bool plan_decode(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                 int max_context_len, int tokens_per_split, DecodePlan* plan) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0) return false;
  if (num_q_heads % num_kv_heads != 0) return false;
  const int G = num_q_heads / num_kv_heads;
  int tps = tokens_per_split;
  if (tps <= 0) {
    // Largest split whose grid bound (every sequence at max_context_len)
    // still reaches 1024 workgroups, about four per CU: the per-workgroup
    // prologue, cross-wave reductions, partials and merge are a fixed cost
    // that larger splits amortise (measured on the Llama-3.1-8B-shaped
    // batch: 1024-token splits 45.7 us, 512 51.0 us, 256 59.5 us).
    tps = 64;
    const int cands[] = {1024, 512, 256, 128};
    for (int c : cands) {
      const long long per_seq = max_context_len > 0 ? (max_context_len + c - 1) / c : 1;
      if ((long long)batch * num_kv_heads * per_seq >= 1024) { tps = c; break; }
    }
    while (tps > 64 && smem_layout(tps, G, head_dim).total > 64 * 1024) tps /= 2;
  } else if (tps % 64 != 0 || tps < 64 || tps > 2048) {
    return false;
  }
  if (smem_layout(tps, G, head_dim).total > 64 * 1024) return false;
  const int n_split = max_context_len > 0 ? (max_context_len + tps - 1) / tps : 1;
  plan->split_tokens = tps;
  plan->n_split = n_split;
  plan->counter_bytes = align256((size_t)batch * num_kv_heads * sizeof(unsigned));
  plan->o_bytes = align256((size_t)batch * num_q_heads * n_split * head_dim * sizeof(float));
  plan->lse_bytes = align256((size_t)batch * num_q_heads * n_split * sizeof(float));
  plan->total_bytes = plan->counter_bytes + plan->o_bytes + plan->lse_bytes;
  return true;
}

int launch_decode(const void* q, bool q_f32, const int8_t* k_cache, const int8_t* v_cache,
                  const uint16_t* k_scale, const uint16_t* v_scale, int64_t num_blocks,
                  const int32_t* block_table, int max_blocks_per_seq,
                  const int32_t* context_lens, int ctx_cap, int batch, int num_q_heads,
                  int num_kv_heads, int head_dim, float sm_scale, float* out,
                  void* workspace, const DecodePlan& plan, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  SplitArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.out = out;
  a.counters = reinterpret_cast<unsigned*>(ws);
  a.o_part = reinterpret_cast<float*>(ws + plan.counter_bytes);
  a.lse_part = reinterpret_cast<float*>(ws + plan.counter_bytes + plan.o_bytes);
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.ctx_cap = ctx_cap;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.split_tokens = plan.split_tokens;
  a.n_split = plan.n_split;
  a.batch = batch;
  a.qk_scale_log2 = sm_scale * kLog2e;
  const int G = num_q_heads / num_kv_heads;
  bool ok;
  if (head_dim == 128) ok = q_f32 ? dispatch_g<128, true>(G, a, batch, stream)
                                  : dispatch_g<128, false>(G, a, batch, stream);
  else ok = q_f32 ? dispatch_g<64, true>(G, a, batch, stream)
                  : dispatch_g<64, false>(G, a, batch, stream);
  if (!ok) return -2;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kv8
