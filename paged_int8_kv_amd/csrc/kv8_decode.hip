// paged_decode_attn_kv8 kernels: split-K flash-decoding over the paged
// INT8 cache for gfx950.
//
// Attention softmax(q K^T * sm_scale) V ("KV Cache 优化全景解析", section 2.1)
// per GQA group (section 3.3) over K/V restored on the fly from INT8 codes
// and per-token fp16 scales ("KV-Cache 全栈优化系统" README, section
// 主要特性), with fp32 softmax and accumulation ("大模型推理加速：KV Cache
// 与vLLM技术解析", section 4.1).  Split results are merged by log-sum-exp.
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
#include "kv8_device.h"
#include "kv8_launch.h"

namespace kv8 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;

struct SplitArgs {
  const void* q;
  const int8_t* k_cache;
  const int8_t* v_cache;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  const int32_t* block_table;
  const int32_t* context_lens;
  float* o_part;
  float* lse_part;
  int64_t num_blocks;
  int max_blocks_per_seq;
  int ctx_cap;
  int num_q_heads;
  int num_kv_heads;
  int split_tokens;
  int n_split;
  float qk_scale_log2;
};

__host__ __device__ constexpr int align16(int x) { return (x + 15) & ~15; }

struct SmemLayout {
  int blk_off, z_off, vs_off, pp_off, red_off, total;
};

// LDS carve-up of one workgroup: block ids, logits (reused for the final
// cross-wave reduction), v scales, packed fp16 weights, per-head scalars.
__host__ __device__ inline SmemLayout smem_layout(int split_tokens, int G, int D) {
  SmemLayout L{};
  const int zbytes = split_tokens * G * 4;
  const int finbytes = kWaves * G * D * 4;
  L.blk_off = 0;
  L.z_off = align16((split_tokens / kBlock) * 4);
  L.vs_off = L.z_off + align16(zbytes > finbytes ? zbytes : finbytes);
  L.pp_off = L.vs_off + align16(split_tokens * 2);
  L.red_off = L.pp_off + align16((split_tokens / 2) * G * 4);
  L.total = L.red_off + align16(3 * kWaves * G * 4);
  return L;
}

template <int NDW> struct RowT;
template <> struct RowT<4> { using type = uint4; };
template <> struct RowT<2> { using type = uint2; };

__device__ __forceinline__ uint32_t dword(const uint4& r, int k) {
  return k == 0 ? r.x : k == 1 ? r.y : k == 2 ? r.z : r.w;
}
__device__ __forceinline__ uint32_t dword(const uint2& r, int k) { return k == 0 ? r.x : r.y; }

template <int D, int G, bool QF32>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(SplitArgs a) {
  constexpr int CPL = D / 8;    // channels (= code bytes) per lane per token
  constexpr int NDW = CPL / 4;  // dwords per lane per token
  constexpr int NP = CPL / 2;   // fp16 pairs per lane per token
  using Row = typename RowT<NDW>::type;

  extern __shared__ __align__(16) unsigned char smem[];
  const SmemLayout L = smem_layout(a.split_tokens, G, D);
  int* s_blk = reinterpret_cast<int*>(smem + L.blk_off);
  float* s_z = reinterpret_cast<float*>(smem + L.z_off);
  float* s_fin = s_z;
  uint16_t* s_vs = reinterpret_cast<uint16_t*>(smem + L.vs_off);
  uint32_t* s_pp = reinterpret_cast<uint32_t*>(smem + L.pp_off);
  float* s_red = reinterpret_cast<float*>(smem + L.red_off);   // [3][kWaves][G]

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = lane >> 3, chunk = lane & 7;

  int ctx = a.context_lens[b];
  ctx = min(max(ctx, 0), a.ctx_cap);
  const int t0 = split * a.split_tokens;
  if (t0 >= ctx) return;                       // uniform over the workgroup
  const int ntok = min(ctx - t0, a.split_tokens);
  const int nblk = (ntok + kBlock - 1) / kBlock;
  const int jb0 = t0 / kBlock;
  const int Hkv = a.num_kv_heads;

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
    const int64_t qrow0 = ((int64_t)b * a.num_q_heads + (int64_t)g * G) * D + chunk * CPL;
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
        const Row r = *reinterpret_cast<const Row*>(
            static_cast<const uint16_t*>(a.q) + qrow0 + (int64_t)h * D);
        // a Row of NDW dwords holds 2*NDW bf16 values; CPL = 4*NDW values
        // need two Rows
        const Row r2 = *(reinterpret_cast<const Row*>(
            static_cast<const uint16_t*>(a.q) + qrow0 + (int64_t)h * D) + 1);
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
  __syncthreads();   // s_blk visible

  // ---- pass 1: logits ----------------------------------------------------
  float mloc = kNegInf;
  {
    auto row_ptr = [&](const int8_t* base, int j) {
      const int64_t line = ((int64_t)s_blk[j] * Hkv + g) * kBlock;
      return base + (line + slot) * D + chunk * CPL;
    };
    auto scale_idx = [&](int j) { return ((int64_t)s_blk[j] * Hkv + g) * kBlock + slot; };

    int j = wave;
    Row w0{}, w1{};
    uint16_t ks0 = 0, ks1 = 0, vs0 = 0, vs1 = 0;
    if (j < nblk) {
      const int8_t* p = row_ptr(a.k_cache, j);
      w0 = *reinterpret_cast<const Row*>(p);
      w1 = *reinterpret_cast<const Row*>(p + 8 * D);
      const int64_t si = scale_idx(j);
      ks0 = a.k_scale[si]; ks1 = a.k_scale[si + 8];
      vs0 = a.v_scale[si]; vs1 = a.v_scale[si + 8];
    }
    for (; j < nblk; j += kWaves) {
      Row n0{}, n1{};
      uint16_t nks0 = 0, nks1 = 0, nvs0 = 0, nvs1 = 0;
      if (j + kWaves < nblk) {                 // prefetch the wave's next block
        const int8_t* p = row_ptr(a.k_cache, j + kWaves);
        n0 = *reinterpret_cast<const Row*>(p);
        n1 = *reinterpret_cast<const Row*>(p + 8 * D);
        const int64_t si = scale_idx(j + kWaves);
        nks0 = a.k_scale[si]; nks1 = a.k_scale[si + 8];
        nvs0 = a.v_scale[si]; nvs1 = a.v_scale[si + 8];
      }
      float S0[G], S1[G];
#pragma unroll
      for (int h = 0; h < G; ++h) { S0[h] = 0.0f; S1[h] = 0.0f; }
#pragma unroll
      for (int k = 0; k < NDW; ++k) {
        const uint32_t x0 = dword(w0, k) ^ kXor80, x1 = dword(w1, k) ^ kXor80;
        const half2_t a0 = biased_pair_lo(x0), b0 = biased_pair_hi(x0);
        const half2_t a1 = biased_pair_lo(x1), b1 = biased_pair_hi(x1);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          S0[h] = fdot2(qh[h][2 * k], a0, S0[h]);
          S0[h] = fdot2(qh[h][2 * k + 1], b0, S0[h]);
          S1[h] = fdot2(qh[h][2 * k], a1, S1[h]);
          S1[h] = fdot2(qh[h][2 * k + 1], b1, S1[h]);
          if constexpr (QF32) {
            S0[h] = fdot2(ql[h][2 * k], a0, S0[h]);
            S0[h] = fdot2(ql[h][2 * k + 1], b0, S0[h]);
            S1[h] = fdot2(ql[h][2 * k], a1, S1[h]);
            S1[h] = fdot2(ql[h][2 * k + 1], b1, S1[h]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) { S0[h] = group8_sum(S0[h]); S1[h] = group8_sum(S1[h]); }
      const int tl0 = j * kBlock + slot, tl1 = tl0 + 8;
      const bool ok0 = tl0 < ntok, ok1 = tl1 < ntok;
      const float k0 = fp16_bits_to_f32(ks0), k1 = fp16_bits_to_f32(ks1);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (chunk == h) {
          const float z0 = ok0 ? (k0 * cz[h]) * (S0[h] - qbias[h]) : kNegInf;
          const float z1 = ok1 ? (k1 * cz[h]) * (S1[h] - qbias[h]) : kNegInf;
          s_z[tl0 * G + h] = z0;
          s_z[tl1 * G + h] = z1;
          mloc = fmaxf(mloc, fmaxf(z0, z1));
        }
      }
      if (chunk == 0) { s_vs[tl0] = vs0; s_vs[tl1] = vs1; }
      w0 = n0; w1 = n1; ks0 = nks0; ks1 = nks1; vs0 = nvs0; vs1 = nvs1;
    }
  }
  mloc = across_groups_max(mloc);
  if (slot == 0 && chunk < G) s_red[wave * G + chunk] = mloc;
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
  float acc[G][CPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[h][c] = 0.0f;
  {
    auto row_ptr = [&](int j) {
      const int64_t line = ((int64_t)s_blk[j] * Hkv + g) * kBlock;
      return a.v_cache + (line + slot) * D + chunk * CPL;
    };
    int j = wave;
    Row w0{}, w1{};
    if (j < nblk) {
      const int8_t* p = row_ptr(j);
      w0 = *reinterpret_cast<const Row*>(p);
      w1 = *reinterpret_cast<const Row*>(p + 8 * D);
    }
    for (; j < nblk; j += kWaves) {
      Row n0{}, n1{};
      if (j + kWaves < nblk) {
        const int8_t* p = row_ptr(j + kWaves);
        n0 = *reinterpret_cast<const Row*>(p);
        n1 = *reinterpret_cast<const Row*>(p + 8 * D);
      }
      half2_t wp[G];
      const uint32_t* src = s_pp + (j * 8 + slot) * G;
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
          acc[h][4 * k] = fdot2(wp[h], f0, acc[h][4 * k]);
          acc[h][4 * k + 1] = fdot2(wp[h], f1, acc[h][4 * k + 1]);
          acc[h][4 * k + 2] = fdot2(wp[h], f2, acc[h][4 * k + 2]);
          acc[h][4 * k + 3] = fdot2(wp[h], f3, acc[h][4 * k + 3]);
        }
      }
      w0 = n0; w1 = n1;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[h][c] = across_groups_sum(acc[h][c]);
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < CPL; ++c) s_fin[(wave * G + h) * D + chunk * CPL + c] = acc[h][c];
  }
  __syncthreads();

  // ---- normalise and write this split's partial result ---------------------
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
    const int64_t bh = (int64_t)b * a.num_q_heads + (int64_t)g * G + h;
    a.o_part[(bh * a.n_split + split) * D + c] = (s - kCodeBias * Ph) / Lh;
    if (c == 0) a.lse_part[bh * a.n_split + split] = Mh + __builtin_amdgcn_logf(Lh);
  }
}

// Log-sum-exp merge of the split partials: one workgroup per (b, query
// head), one thread per channel.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    const int32_t* __restrict__ context_lens, int ctx_cap, int split_tokens, int n_split,
    int num_q_heads, float* __restrict__ out) {
  const int64_t bh = blockIdx.x;
  const int b = (int)(bh / num_q_heads);
  const int c = threadIdx.x;
  int ctx = context_lens[b];
  ctx = min(max(ctx, 0), ctx_cap);
  const int nv = (ctx + split_tokens - 1) / split_tokens;
  float* dst = out + bh * D + c;
  if (nv == 0) { *dst = 0.0f; return; }
  const float* lse = lse_part + bh * n_split;
  float M = kNegInf;
  for (int s = 0; s < nv; ++s) M = fmaxf(M, lse[s]);
  float num = 0.0f, den = 0.0f;
  for (int s = 0; s < nv; ++s) {
    const float w = __builtin_amdgcn_exp2f(lse[s] - M);
    den += w;
    num += w * o_part[(bh * n_split + s) * D + c];
  }
  *dst = num / den;
}

template <int D, int G, bool QF32>
bool launch_split(const SplitArgs& a, int batch, hipStream_t stream) {
  const SmemLayout L = smem_layout(a.split_tokens, G, D);
  decode_split_kernel<D, G, QF32><<<dim3(a.n_split, a.num_kv_heads, batch), dim3(kThreads),
                                    L.total, stream>>>(a);
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

int decode_smem_bytes(int split_tokens, int G, int D) {
  return smem_layout(split_tokens, G, D).total;
}

bool plan_decode(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                 int max_context_len, int tokens_per_split, DecodePlan* plan) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0) return false;
  if (num_q_heads % num_kv_heads != 0) return false;
  const int G = num_q_heads / num_kv_heads;
  int tps = tokens_per_split;
  if (tps <= 0) {
    // Largest split that still gives about 2048 workgroups over the grid;
    // larger splits amortise the per-split reductions and partial traffic.
    tps = 64;
    const int cands[] = {1024, 512, 256, 128};
    for (int c : cands) {
      const long long wgs = (long long)batch * num_kv_heads *
                            ((max_context_len + c - 1) / c > 0 ? (max_context_len + c - 1) / c : 1);
      if (wgs >= 2048) { tps = c; break; }
    }
    while (tps > 64 && smem_layout(tps, G, head_dim).total > 64 * 1024) tps /= 2;
  } else if (tps % 64 != 0 || tps < 64 || tps > 2048) {
    return false;
  }
  if (smem_layout(tps, G, head_dim).total > 64 * 1024) return false;
  const int n_split = max_context_len > 0 ? (max_context_len + tps - 1) / tps : 1;
  plan->split_tokens = tps;
  plan->n_split = n_split;
  plan->o_bytes = align256((size_t)batch * num_q_heads * n_split * head_dim * sizeof(float));
  plan->lse_bytes = align256((size_t)batch * num_q_heads * n_split * sizeof(float));
  plan->total_bytes = plan->o_bytes + plan->lse_bytes;
  return true;
}

int launch_decode(const void* q, bool q_f32, const int8_t* k_cache, const int8_t* v_cache,
                  const uint16_t* k_scale, const uint16_t* v_scale, int64_t num_blocks,
                  const int32_t* block_table, int max_blocks_per_seq,
                  const int32_t* context_lens, int ctx_cap, int batch, int num_q_heads,
                  int num_kv_heads, int head_dim, float sm_scale, float* out,
                  void* workspace, const DecodePlan& plan, hipStream_t stream) {
  SplitArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.o_part = static_cast<float*>(workspace);
  a.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.o_bytes);
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.ctx_cap = ctx_cap;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.split_tokens = plan.split_tokens;
  a.n_split = plan.n_split;
  a.qk_scale_log2 = sm_scale * kLog2e;
  const int G = num_q_heads / num_kv_heads;
  bool ok;
  if (head_dim == 128) ok = q_f32 ? dispatch_g<128, true>(G, a, batch, stream)
                                  : dispatch_g<128, false>(G, a, batch, stream);
  else ok = q_f32 ? dispatch_g<64, true>(G, a, batch, stream)
                  : dispatch_g<64, false>(G, a, batch, stream);
  if (!ok) return -2;
  const unsigned nbh = (unsigned)((int64_t)batch * num_q_heads);
  if (head_dim == 128)
    decode_merge_kernel<128><<<dim3(nbh), dim3(128), 0, stream>>>(
        a.o_part, a.lse_part, context_lens, ctx_cap, plan.split_tokens, plan.n_split,
        num_q_heads, out);
  else
    decode_merge_kernel<64><<<dim3(nbh), dim3(64), 0, stream>>>(
        a.o_part, a.lse_part, context_lens, ctx_cap, plan.split_tokens, plan.n_split,
        num_q_heads, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kv8
