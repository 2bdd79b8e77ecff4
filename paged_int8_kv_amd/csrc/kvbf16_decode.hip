// paged_decode_attn_bf16kv kernel: split-K flash-decoding over a paged
// bf16 (unquantised) KV cache for gfx950.
//
// The 16-bit reference point that KV8 attention is measured against at an
// equal memory budget ("KV-Cache 全栈优化系统" README, section 实验效果（摘要）):
// the same attention softmax(q K^T * sm_scale) V ("KV Cache 优化全景解析",
// sections 2.1 and 3.3) read through the same block table (section 4.2),
// with fp32 softmax and accumulation, but K and V stored as bf16 and no
// scales.  It shares the INT8 kernel's work items, item order, split spans,
// reductions and in-launch log-sum-exp merge (kv8_decode_common.h).
//
// One workgroup (4 waves) serves one (sequence b, split, KV head g) and all
// G query heads.  Inside a wave, lane = 8 * slot + chunk: `chunk` picks d/8
// channels (2d/8 bytes) and `slot` picks tokens slot and slot+8 of a
// 16-token block.  Two passes over the split's blocks (round-robin over
// the waves):
//   pass 1  z[t,h] = log2e * sm_scale * <q_h, k[t]> by v_dot2_f32_bf16 on
//           the cache's bf16 pairs, written to LDS; running max per head.
//   middle  p[t,h] = 2^(z - M_h) <= 1 (fp32, written over z), l_h = sum p.
//   pass 2  acc[h,c] += p[t,h] * v[t,c] in fp32 FMA.
// q enters as bf16 pairs: a bf16 q exactly, an fp32 q as the sum of three
// bf16 parts (hi, mid, lo), which hold its 24-bit significand.
#include "kv8_decode_common.h"
#include "kv8_device.h"
#include "kv8_launch.h"

namespace kv8 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kPf = 2;        // blocks in flight per wave and pass
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct Bf16Args {
  const void* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
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
  int period;
  int snake_rounds;
  float qk_scale_log2;
};

__host__ __device__ constexpr int align16b(int x) { return (x + 15) & ~15; }

struct Bf16Smem {
  int blk_off, z_off, fin_off, red_off, flag_off, total;
};

// LDS of one workgroup: block ids, logits (turned into weights in place),
// per-wave results of pass 2, per-head scalars and the last-workgroup flag.
__host__ __device__ inline Bf16Smem bf16_smem(int split_tokens, int G, int D) {
  Bf16Smem L{};
  L.blk_off = 0;
  L.z_off = align16b((split_tokens / kBlock) * 4);
  L.fin_off = L.z_off + align16b(split_tokens * G * 4);
  L.red_off = L.fin_off + align16b(kWaves * G * D * 4);
  L.flag_off = L.red_off + align16b(2 * kWaves * G * 4);
  L.total = L.flag_off + 16;
  return L;
}

// One token row of the lane: D/8 bf16 channels = D/16 dwords.
template <int NDW> struct Row16 { uint4 u[NDW / 4]; };

template <int NDW>
__device__ __forceinline__ uint32_t dw(const Row16<NDW>& r, int k) {
  const uint4& v = r.u[k >> 2];
  const int j = k & 3;
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_bits_f32(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}

template <int D, int G, bool QF32>
__global__ __launch_bounds__(kThreads) void decode_bf16_kernel(Bf16Args a) {
  constexpr int CPL = D / 8;    // channels per lane per token
  constexpr int NDW = CPL / 2;  // dwords (bf16 pairs) per lane per token
  constexpr int NV = (2 * G >= 8) ? (2 * G) / 8 : 1;   // logits stored per lane
  constexpr int M = G * CPL;    // accumulators per lane
  constexpr int NT = QF32 ? 3 : 1;                      // bf16 parts of q
  using Row = Row16<NDW>;

  extern __shared__ __align__(16) unsigned char smem[];
  const Bf16Smem L = bf16_smem(a.split_tokens, G, D);
  int* s_blk = reinterpret_cast<int*>(smem + L.blk_off);
  float* s_z = reinterpret_cast<float*>(smem + L.z_off);
  float* s_fin = reinterpret_cast<float*>(smem + L.fin_off);
  float* s_red = reinterpret_cast<float*>(smem + L.red_off);   // [2][kWaves][G]
  int* s_flag = reinterpret_cast<int*>(smem + L.flag_off);

  const int tid = threadIdx.x, lane = tid & 63;
  const Item it = locate_item(a.context_lens, a.batch, a.ctx_cap, a.num_kv_heads,
                              a.split_tokens, a.period, a.snake_rounds, lane);
  const int b = it.b, g = it.g, split = it.split;
  if (b < 0) return;                           // uniform: past the item list
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int slot = lane >> 3, chunk = lane & 7;
  const int64_t bh0 = (int64_t)b * a.num_q_heads + (int64_t)g * G;

  int ctx = a.context_lens[b];
  ctx = min(max(ctx, 0), a.ctx_cap);
  if (ctx == 0) {                              // uniform: empty context, zero output
    for (int e = tid; e < G * D; e += kThreads) a.out[bh0 * D + e] = 0.0f;
    return;
  }
  const Span sp = split_span(it, ctx);
  const int nblk = sp.nblk, jb0 = sp.jb0, ntok = sp.ntok;
  const int Hkv = a.num_kv_heads;

  if (tid < nblk) {
    int64_t id = a.block_table[(int64_t)b * a.max_blocks_per_seq + jb0 + tid];
    id = id < 0 ? 0 : (id >= a.num_blocks ? a.num_blocks - 1 : id);
    s_blk[tid] = (int)id;
  }

  // ---- q of the G heads: this lane's d/8 channels as bf16 pairs ----------
  uint32_t qp[NT][G][NDW];
  {
    const int64_t qrow0 = bh0 * D + chunk * CPL;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if constexpr (QF32) {
        const float4* src = reinterpret_cast<const float4*>(
            static_cast<const float*>(a.q) + qrow0 + (int64_t)h * D);
#pragma unroll
        for (int i = 0; i < CPL / 4; ++i) {
          const float4 v = src[i];
          const float x[4] = {v.x, v.y, v.z, v.w};
          uint32_t part[3][4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t hi = bf16_rne_bits(x[j]);
            const float r1 = x[j] - bf16_bits_f32(hi);          // exact
            const uint32_t mid = bf16_rne_bits(r1);
            const uint32_t lo = bf16_rne_bits(r1 - bf16_bits_f32(mid));
            part[0][j] = hi;
            part[1][j] = mid;
            part[2][j] = lo;
          }
#pragma unroll
          for (int t = 0; t < 3; ++t) {
            qp[t][h][2 * i] = part[t][0] | (part[t][1] << 16);
            qp[t][h][2 * i + 1] = part[t][2] | (part[t][3] << 16);
          }
        }
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(a.q) + qrow0 + (int64_t)h * D);
#pragma unroll
        for (int i = 0; i < NDW / 4; ++i) {
          const uint4 v = src[i];
          qp[0][h][4 * i] = v.x;
          qp[0][h][4 * i + 1] = v.y;
          qp[0][h][4 * i + 2] = v.z;
          qp[0][h][4 * i + 3] = v.w;
        }
      }
    }
  }
  const float cz = a.qk_scale_log2;
  const int tk = chunk >> 2;            // token of the pair: slot or slot+8
  int hv[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) hv[j] = rs_head<G>(chunk, j);
  __syncthreads();   // s_blk visible

  // Each wave owns blocks wave + i * kWaves, i = 0 .. nmine-1.
  const int nmine = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;
  const int last = nmine - 1;
  auto line_of = [&](int i) {
    return ((int64_t)s_blk[wave + i * kWaves] * Hkv + g) * kBlock + slot;
  };
  auto load_row = [&](const uint16_t* base, int64_t line, int tok_off) {
    Row r;
    const uint4* p = reinterpret_cast<const uint4*>(base + (line + tok_off) * D + chunk * CPL);
#pragma unroll
    for (int i = 0; i < NDW / 4; ++i) r.u[i] = p[i];
    return r;
  };

  // ---- pass 1: logits ----------------------------------------------------
  float mloc[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) mloc[j] = kNegInf;
  if (nmine > 0) {
    Row r0[kPf], r1[kPf];
    auto issue = [&](int s, int i) {
      const int64_t line = line_of(i);
      r0[s] = load_row(a.k_cache, line, 0);
      r1[s] = load_row(a.k_cache, line, 8);
    };
    // Slots past the wave's last block re-read that block (L2 hits) and skip
    // the compute, so every load stays unconditional.
#pragma unroll
    for (int s = 0; s < kPf; ++s) issue(s, min(s, last));
    for (int base = 0; base < nmine; base += kPf) {
      priority_by_remaining(2 * nmine - base);
#pragma unroll
      for (int s = 0; s < kPf; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        const int i = base + s;
        if (i < nmine) {
          float S[2 * G];
#pragma unroll
          for (int k = 0; k < 2 * G; ++k) S[k] = 0.0f;
#pragma unroll
          for (int k = 0; k < NDW; ++k) {
            const uint32_t x0 = dw(r0[s], k), x1 = dw(r1[s], k);
#pragma unroll
            for (int h = 0; h < G; ++h) {
#pragma unroll
              for (int t = 0; t < NT; ++t) {
                S[h] = dot2bf(qp[t][h][k], x0, S[h]);
                S[G + h] = dot2bf(qp[t][h][k], x1, S[G + h]);
              }
            }
          }
          float R[NV];
          reduce_scatter8<G>(S, R, chunk);
          const int tl = (wave + i * kWaves) * kBlock + slot + 8 * tk;
          const bool ok = tl < ntok;
#pragma unroll
          for (int j = 0; j < NV; ++j) {
            const float z = ok ? cz * R[j] : kNegInf;
            s_z[tl * G + hv[j]] = z;
            mloc[j] = fmaxf(mloc[j], z);
          }
        }
        issue(s, min(i + kPf, last));
      }
    }
  }

  // V rows of the first kPf blocks are requested now, so that they arrive
  // while the workgroup builds the weights.
  Row r0[kPf], r1[kPf];
  auto issue_v = [&](int s, int i) {
    const int64_t line = line_of(i);
    r0[s] = load_row(a.v_cache, line, 0);
    r1[s] = load_row(a.v_cache, line, 8);
  };
  if (nmine > 0) {
#pragma unroll
    for (int s = 0; s < kPf; ++s) issue_v(s, min(s, last));
  }

#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float m = fmaxf(mloc[j], __shfl_xor(mloc[j], 4));
    m = across_groups_max(m);
    if (slot == 0) s_red[wave * G + hv[j]] = m;
  }
  __syncthreads();

  // ---- middle: weights p = 2^(z - M) in place ----------------------------
  {
    const int h = tid % G;
    float Mh = s_red[h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) Mh = fmaxf(Mh, s_red[w * G + h]);
    float lsum = 0.0f;
    const int total = nblk * kBlock * G;
    for (int e = tid; e < total; e += kThreads) {
      const float p = __builtin_amdgcn_exp2f(s_z[e] - Mh);   // 0 for masked tokens
      s_z[e] = p;
      lsum += p;
    }
#pragma unroll
    for (int off = G; off < 64; off <<= 1) lsum += __shfl_xor(lsum, off);
    if (lane < G) s_red[kWaves * G + wave * G + lane] = lsum;
  }
  __syncthreads();

  // ---- pass 2: weighted sum of V rows -------------------------------------
  float acc[M];
#pragma unroll
  for (int k = 0; k < M; ++k) acc[k] = 0.0f;
  for (int base = 0; base < nmine; base += kPf) {
    priority_by_remaining(nmine - base);
#pragma unroll
    for (int s = 0; s < kPf; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      const int i = base + s;
      if (i < nmine) {
        const int t0 = (wave + i * kWaves) * kBlock + slot;
        float w0[G], w1[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          w0[h] = s_z[t0 * G + h];
          w1[h] = s_z[(t0 + 8) * G + h];
        }
        // rows past the context may hold anything (NaN included): zero them
        const bool ok0 = t0 < ntok, ok1 = t0 + 8 < ntok;
#pragma unroll
        for (int k = 0; k < NDW; ++k) {
          const uint32_t x0 = ok0 ? dw(r0[s], k) : 0u, x1 = ok1 ? dw(r1[s], k) : 0u;
          const float a0 = bf16_bits_f32(x0 & 0xFFFFu), b0 = bf16_bits_f32(x0 >> 16);
          const float a1 = bf16_bits_f32(x1 & 0xFFFFu), b1 = bf16_bits_f32(x1 >> 16);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h * CPL + 2 * k] = fmaf(w1[h], a1, fmaf(w0[h], a0, acc[h * CPL + 2 * k]));
            acc[h * CPL + 2 * k + 1] =
                fmaf(w1[h], b1, fmaf(w0[h], b0, acc[h * CPL + 2 * k + 1]));
          }
        }
      }
      issue_v(s, min(i + kPf, last));
    }
  }

  groups_to_lds<G, CPL, D>(acc, s_fin, wave, lane, chunk);
  __syncthreads();
  finish_split<G, D, kThreads, kWaves>(
      PartialArgs{a.out, a.o_part, a.lse_part, a.counters, a.n_split}, s_fin, s_red, s_flag,
      bh0, (int64_t)b * Hkv + g, split, it.nsplit, tid);
}

template <int D, int G, bool QF32>
bool launch_bf16(const Bf16Args& a, int batch, hipStream_t stream) {
  const Bf16Smem L = bf16_smem(a.split_tokens, G, D);
  Bf16Args args = a;
  const int64_t grid = item_grid<decode_bf16_kernel<D, G, QF32>>(
      kThreads, L.total, batch, (int64_t)a.n_split * a.num_kv_heads * batch, &args.period,
      &args.snake_rounds);
  if (grid > 0x7FFFFFFF) return false;
  decode_bf16_kernel<D, G, QF32><<<dim3((unsigned)grid), dim3(kThreads), L.total, stream>>>(args);
  return true;
}

template <int D, bool QF32>
bool dispatch_bf16(int G, const Bf16Args& a, int batch, hipStream_t s) {
  switch (G) {
    case 1: return launch_bf16<D, 1, QF32>(a, batch, s);
    case 2: return launch_bf16<D, 2, QF32>(a, batch, s);
    case 4: return launch_bf16<D, 4, QF32>(a, batch, s);
    case 8: return launch_bf16<D, 8, QF32>(a, batch, s);
    default: return false;
  }
}

}  // namespace

int launch_decode_bf16kv(const void* q, bool q_f32, const uint16_t* k_cache,
                         const uint16_t* v_cache, int64_t num_blocks,
                         const int32_t* block_table, int max_blocks_per_seq,
                         const int32_t* context_lens, int ctx_cap, int batch, int num_q_heads,
                         int num_kv_heads, int head_dim, float sm_scale, float* out,
                         void* workspace, const DecodePlan& plan, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  Bf16Args a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
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
  a.period = 0;
  a.snake_rounds = 0;
  a.qk_scale_log2 = sm_scale * kLog2e;
  const int G = num_q_heads / num_kv_heads;
  if (bf16_smem(plan.split_tokens, G, head_dim).total > 64 * 1024) return -2;
  bool ok;
  if (head_dim == 128) ok = q_f32 ? dispatch_bf16<128, true>(G, a, batch, stream)
                                  : dispatch_bf16<128, false>(G, a, batch, stream);
  else ok = q_f32 ? dispatch_bf16<64, true>(G, a, batch, stream)
                  : dispatch_bf16<64, false>(G, a, batch, stream);
  if (!ok) return -2;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kv8
