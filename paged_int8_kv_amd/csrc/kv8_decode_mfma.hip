// Matrix-core forms of paged_decode_attn_kv8 / paged_decode_attn_fp8kv /
// paged_decode_attn_int4kv: split-K flash-decoding over the paged INT8 (or
// FP8 e4m3, or INT4) cache on gfx950, with both contractions of a block on
// MFMA.  Two kernels share the per-block layouts below:
//   decode_mfma2_kernel  two passes per split, as the dot-product kernel:
//                        logits of the whole split to LDS, the exact split
//                        max, fp16 weights to LDS, then the values;
//   decode_mfma1_kernel  one pass with an online softmax: the logit MFMA's
//                        output registers (token 4*(lane/16) + r, head
//                        lane % 16) are exactly the value MFMA's B-operand
//                        layout, so the weights never leave the registers
//                        and no LDS is used until the cross-wave merge; it
//                        also serves 4-bit codes at d = 128.
//
// Attention softmax(q K^T * sm_scale) V ("KV Cache 优化全景解析", section 2.1)
// per GQA group (section 3.3) over K/V restored from INT8 codes and
// per-token fp16 scales ("KV-Cache 全栈优化系统" README, section 主要特性),
// fp32 softmax and accumulation ("大模型推理加速：KV Cache与vLLM技术解析",
// section 4.1).  Work items, split spans, the two-pass softmax and the
// in-launch log-sum-exp merge are those of the dot-product kernel
// (kv8_decode.hip); only the per-block arithmetic differs.
//
// Why matrix cores here.  With G query heads per KV head, a 16-token block
// is a [16 x d] x [d x G] product (logits) and a [G x 16] x [16 x d] product
// (values).  As v_dot2 work every cache byte costs G/2 multiply-add issues
// per lane, so at G = 8 the vector unit, not HBM, sets the pace.  One
// 16x16 MFMA tile holds all G <= 16 heads at once: the columns past G are
// idle, which costs nothing that the memory stream would notice.
//
// Pass 1 (logits), per block, v_mfma_f32_16x16x32_f16 with
//   A = codes [token = lane % 16][8 channels of the lane's k group]
//   B = q     [same 8 channels][head = lane % 16]   (zero past G)
//   D[token 4*(lane/16) + r][head lane % 16], r = 0..3.
// Lane l loads 16-byte pieces of the row of token l % 16 at channel
// offsets 64u + 16*(l/16); MFMA j uses the 8 channels 64(j/2) + 16(l/16) +
// 8(j%2) ... + 7 on both sides, so A and B agree on every k slot.
//
// Pass 2 (values), per block, v_mfma_f32_16x16x16_f16 with
//   A = codes [channel row m = lane % 16][tokens 4*(lane/16) .. + 3]
//   B = w     [tokens 4*(lane/16) .. + 3][head = lane % 16]
//   tile j (j < d/16) holds channel (d/16)*m + j, so lane l reads d/16
//   contiguous bytes of each of the 4 token rows 4*(l/16) .. + 3 (one wave
//   load instruction covers 4 whole 128-byte rows).
//   D[row 4*(lane/16) + r][head lane % 16] = O[head][(d/16)(4(l/16)+r) + j].
//
// INT8 codes enter as the biased fp16 values c + 1152 (one byte permute per
// pair, kv8_device.h); the bias is removed from the logits by starting the
// accumulator at minus 1152 * sum(q_h), and from the V codes themselves, one
// packed fp16 subtract per pair, before they meet the weights.  FP8 codes
// become exact fp16 by one hardware convert per pair.  INT4 codes (d = 128,
// both kernels) enter both products as 1.5 + c/16 exactly: one shift and one
// three-input bit operation per nibble pair put the sign-flipped nibble into
// the top mantissa bits of 1.0.  The logits start their accumulator at minus
// 1.5 * sum(q_h) and take the 1/16 into the logit scale; the values keep the
// bias in their sums and take it off once per split through the weight sums
// that one more MFMA per block accumulates (value_unbias).  q enters as fp16
// after an exact per-head power-of-two rescale; an fp32 q is split into a
// high and a low fp16 part (two MFMAs).
#include "kv8_decode_common.h"
#include "kv8_device.h"
#include "kv8_launch.h"
#include "kv8_mfma_block.h"

namespace kv8 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kPf = 2;        // one-pass kernel: blocks (K and V tiles) in flight per wave
constexpr int kPfNib = 2;     // the same for 4-bit codes (4 measured slower: 29.5 vs 28.7 us)
constexpr int kPf2 = 3;       // two-pass kernel: blocks in flight per wave and pass

__host__ __device__ constexpr int align16m(int x) { return (x + 15) & ~15; }

struct M2Smem {
  int blk_off, z_off, vs_off, w_off, red_off, flag_off, total;
};

// LDS of a two-pass workgroup: block ids, logits [token][G] (reused for the
// cross-wave output sum [kWaves][G][D]), v scales per token, fp16 weights
// [block][G][16 tokens], per-head scalars, the last-workgroup flag.
__host__ __device__ inline M2Smem m2smem_layout(int split_tokens, int G, int D) {
  M2Smem L{};
  const int zbytes = split_tokens * G * 4;
  const int finbytes = kWaves * G * D * 4;
  L.blk_off = 0;
  L.z_off = align16m((split_tokens / kBlock) * 4);
  L.vs_off = L.z_off + align16m(zbytes > finbytes ? zbytes : finbytes);
  L.w_off = L.vs_off + align16m(split_tokens * 2);
  L.red_off = L.w_off + align16m(split_tokens * G * 2);
  L.flag_off = L.red_off + align16m(2 * kWaves * G * 4);
  L.total = L.flag_off + 16;
  return L;
}

struct MSmem {
  int fin_off, red_off, flag_off, total;
};

// LDS of a one-pass workgroup: the per-wave outputs [kWaves][G][D], per-wave head
// scalars (max, weight sum, fp16-weight sum) and the last-workgroup flag.
__host__ __device__ inline MSmem msmem_layout(int G, int D) {
  MSmem L{};
  L.fin_off = 0;
  L.red_off = align16m(kWaves * G * D * 4);
  L.flag_off = L.red_off + align16m(2 * kWaves * G * 4);
  L.total = L.flag_off + 16;
  return L;
}

template <int D, int G, bool QF32, class C>
__global__ __launch_bounds__(kThreads) void decode_mfma2_kernel(SplitArgs a) {
  static_assert(G >= 1 && G <= 16, "one 16-column tile of heads");
  constexpr bool NIB = C::kBits == 4;   // two 4-bit codes per byte
  static_assert(!NIB || D == 128, "4-bit codes: d = 128");
  constexpr int RB = NIB ? D / 2 : D;   // code bytes per cache row
  constexpr int NCH = NIB ? 1 : D / 64; // 16-byte K pieces per lane per block
  constexpr int NKM = D / 32;     // logit MFMAs per block (per q part)
  constexpr int NVT = D / 16;     // value tiles per block (= channels of a lane's V piece)
  constexpr int NVD = NIB ? 1 : NVT / 4;   // dwords of a lane's V row piece
  using VRow = typename VRowT<NVD>::type;

  extern __shared__ __align__(16) unsigned char smem[];
  const M2Smem L = m2smem_layout(a.split_tokens, G, D);
  int* s_blk = reinterpret_cast<int*>(smem + L.blk_off);
  float* s_z = reinterpret_cast<float*>(smem + L.z_off);
  float* s_fin = s_z;
  uint16_t* s_vs = reinterpret_cast<uint16_t*>(smem + L.vs_off);
  _Float16* s_w = reinterpret_cast<_Float16*>(smem + L.w_off);
  float* s_red = reinterpret_cast<float*>(smem + L.red_off);   // [2][kWaves][G]
  int* s_flag = reinterpret_cast<int*>(smem + L.flag_off);

  const int tid = threadIdx.x, lane = tid & 63;
  const Item it = locate_item(a.context_lens, a.batch, a.ctx_cap, a.num_kv_heads,
                              a.split_tokens, a.period, a.snake_rounds, lane);
  const int b = it.b, g = it.g, split = it.split;
  if (b < 0) return;                           // uniform: past the item list
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane & 15;                    // token (pass 1 A) / head (B, D) / channel row
  const int q4 = lane >> 4;                    // k group
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
  if constexpr (!NIB) {
    if (a.k_new != nullptr && split == it.nsplit - 1 && wave == 0)
      append_newest<D, C>(a, b, g, ctx, lane);
  }

  // ---- q of head hl as the B operand of the logit MFMAs ------------------
  half8_t qb[NKM], qlo[QF32 ? NKM : 1];
  float cz, nqb;
  q_operands<D, G, QF32, C>(a, bh0, hl, q4, qb, qlo, cz, nqb);
  __syncthreads();   // s_blk visible

  // Each wave owns blocks wave + i * kWaves, i = 0 .. nmine-1; lane i of
  // `mine` holds the id of the wave's block i.
  const int nmine = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;
  const int last = nmine - 1;
  const int mine = lane < nmine ? s_blk[wave + lane * kWaves] : 0;
  auto row0_of = [&](int i) {       // first cache row of block i (wave-uniform)
    const int id = __builtin_amdgcn_readlane(mine, i);
    return ((int64_t)id * Hkv + g) * kBlock;
  };

  // ---- pass 1: logits ----------------------------------------------------
  float mloc = kNegInf;
  if (nmine > 0) {
    uint4 rk[kPf2][NCH];
    uint2 ksc[kPf2], vsc[kPf2];
    // Slots past the wave's last block still load (so the compiler's wait
    // counts stay exact) but every lane reads the same bytes of the last
    // block, one cache line per instruction, and the compute skips them.
    auto issue = [&](int s, int i) {
      const bool real = i <= last;                 // wave-uniform
      const int64_t row0 = row0_of(min(i, last));
      const int8_t* p = a.k_cache + row0 * RB + (real ? hl * RB + 16 * q4 : 0);
      const int so = real ? 4 * q4 : 0;
#pragma unroll
      for (int u = 0; u < NCH; ++u) rk[s][u] = *reinterpret_cast<const uint4*>(p + 64 * u);
      ksc[s] = *reinterpret_cast<const uint2*>(a.k_scale + row0 + so);
      vsc[s] = *reinterpret_cast<const uint2*>(a.v_scale + row0 + so);
    };
#pragma unroll
    for (int s = 0; s < kPf2; ++s) issue(s, s);
    for (int base = 0; base < nmine; base += kPf2) {
      priority_by_remaining(2 * nmine - base);
#pragma unroll
      for (int s = 0; s < kPf2; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        const int i = base + s;
        if (i < nmine) {
          float4_t acc = {nqb, nqb, nqb, nqb};
#pragma unroll
          for (int j = 0; j < NKM; ++j) {
            const half8_t av = logit_operand<C>(rk[s], j);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qb[j], acc, 0, 0, 0);
            if constexpr (QF32) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qlo[j], acc, 0, 0, 0);
          }
          const int tb = (wave + i * kWaves) * kBlock + 4 * q4;   // first of the lane's 4 tokens
          const float k0 = fp16_bits_to_f32((uint16_t)ksc[s].x);
          const float k1 = fp16_bits_to_f32((uint16_t)(ksc[s].x >> 16));
          const float k2 = fp16_bits_to_f32((uint16_t)ksc[s].y);
          const float k3 = fp16_bits_to_f32((uint16_t)(ksc[s].y >> 16));
          const float kk[4] = {k0, k1, k2, k3};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float z = tb + r < ntok ? (kk[r] * cz) * acc[r] : kNegInf;
            if (hl < G) {
              s_z[(tb + r) * G + hl] = z;
              mloc = fmaxf(mloc, z);
            }
          }
          if (hl == 0) *reinterpret_cast<uint2*>(s_vs + tb) = vsc[s];
        }
        issue(s, i + kPf2);
      }
    }
  }

  // V rows of the first kPf2 blocks are requested now, so that they arrive
  // while the workgroup finishes the logits and builds the weights.
  VRow rv[kPf2][4];
  auto issue_v = [&](int s, int i) {
    const bool real = i <= last;                   // wave-uniform, as in pass 1
    const int8_t* p = a.v_cache + row0_of(min(i, last)) * RB +
                      (real ? 4 * q4 * RB + hl * (NIB ? NVT / 2 : NVT) : 0);
    const int stride = real ? RB : 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) rv[s][t] = *reinterpret_cast<const VRow*>(p + t * stride);
  };
  if (nmine > 0) {
#pragma unroll
    for (int s = 0; s < kPf2; ++s) issue_v(s, s);
  }

  // max per head over the four k groups of lanes
  {
    float m = fmaxf(mloc, __shfl_xor(mloc, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    if (lane < G) s_red[wave * G + lane] = m;
  }
  __syncthreads();

  // ---- middle: weights ----------------------------------------------------
  {
    const int h = tid % G;
    float Mh = s_red[h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) Mh = fmaxf(Mh, s_red[w * G + h]);
    float lsum = 0.0f;
    const int total = nblk * kBlock * G;
    for (int e = tid; e < total; e += kThreads) {
      const int t = e / G;
      const float z = s_z[e];
      _Float16 p16 = (_Float16)0.0f;
      if (z != kNegInf) {
        const float p = __builtin_amdgcn_exp2f(z - Mh);
        p16 = (_Float16)(p * fp16_bits_to_f32(s_vs[t]));
        lsum += p;
      }
      const int jj = t / kBlock, r = t % kBlock;
      s_w[(jj * G + h) * kBlock + r] = p16;
    }
#pragma unroll
    for (int off = G; off < 64; off <<= 1) lsum += __shfl_xor(lsum, off);
    if (lane < G) s_red[kWaves * G + wave * G + lane] = lsum;
  }
  __syncthreads();

  // ---- pass 2: weighted sum of V codes ------------------------------------
  float4_t acc[NVT];
  float4_t accw = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < NVT; ++j) acc[j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int base = 0; base < nmine; base += kPf2) {
    priority_by_remaining(nmine - base);
#pragma unroll
    for (int s = 0; s < kPf2; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      const int i = base + s;
      if (i < nmine) {
        half4_t wb = {(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
        if (hl < G)
          wb = *reinterpret_cast<const half4_t*>(
              s_w + ((wave + i * kWaves) * G + hl) * kBlock + 4 * q4);
        value_mfmas<C, NVT>(rv[s], wb, acc, accw);
      }
      issue_v(s, i + kPf2);
    }
  }
  value_unbias<C, NVT>(acc, accw);

  // this wave's [G][D] result to LDS (the logits are no longer needed)
  if (hl < G) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* dst = s_fin + (wave * G + hl) * D + NVT * (4 * q4 + r);
#pragma unroll
      for (int j = 0; j < NVT; ++j) dst[j] = acc[j][r];
    }
  }
  __syncthreads();
  finish_split<G, D, kThreads, kWaves>(
      PartialArgs{a.out, a.o_part, a.lse_part, a.counters, a.n_split}, s_fin, s_red, s_flag,
      bh0, (int64_t)b * Hkv + g, split, it.nsplit, tid);
}

template <int D, int G, bool QF32, class C>
__global__ __launch_bounds__(kThreads) void decode_mfma1_kernel(SplitArgs a) {
  static_assert(G >= 1 && G <= 16, "one 16-column tile of heads");
  constexpr bool NIB = C::kBits == 4;   // two 4-bit codes per byte
  static_assert(!NIB || D == 128, "4-bit codes: d = 128");
  constexpr int RB = NIB ? D / 2 : D;   // code bytes per cache row
  constexpr int NCH = D / 64;     // 16-byte K pieces per lane per block (byte codes)
  constexpr int NKM = D / 32;     // logit MFMAs per block (per q part)
  constexpr int NVT = D / 16;     // value tiles per block (= channels of a lane's V piece)
  constexpr int NVD = NIB ? 1 : NVT / 4;   // dwords of a lane's V row piece
  using VRow = typename VRowT<NVD>::type;
  constexpr int kPf = NIB ? kPfNib : ::kv8::kPf;

  extern __shared__ __align__(16) unsigned char smem[];
  const MSmem L = msmem_layout(G, D);
  float* s_fin = reinterpret_cast<float*>(smem + L.fin_off);   // [kWaves][G][D]
  float* s_red = reinterpret_cast<float*>(smem + L.red_off);   // [2][kWaves][G]
  int* s_flag = reinterpret_cast<int*>(smem + L.flag_off);

  const int tid = threadIdx.x, lane = tid & 63;
  const Item it = locate_item(a.context_lens, a.batch, a.ctx_cap, a.num_kv_heads,
                              a.split_tokens, a.period, a.snake_rounds, lane);
  const int b = it.b, g = it.g, split = it.split;
  if (b < 0) return;                           // uniform: past the item list
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane & 15;                    // token (logit A) / head (B, D) / channel row
  const int q4 = lane >> 4;                    // k group
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

  // Each wave owns blocks wave + i * kWaves, i = 0 .. nmine-1; lane i of
  // `mine` holds the id of the wave's block i, read straight from the table.
  const int nmine = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;
  const int last = nmine - 1;
  int mine = 0;
  if (lane < nmine) {
    int64_t id = a.block_table[(int64_t)b * a.max_blocks_per_seq + jb0 + wave + lane * kWaves];
    mine = (int)(id < 0 ? 0 : (id >= a.num_blocks ? a.num_blocks - 1 : id));
  }
  // Decode step with append: the wave that owns the split's last block (the
  // block of position ctx - 1) quantises and stores the newest token before
  // its own loads of that block, which are ordered after the stores' wait.
  if constexpr (!NIB) {
    if (a.k_new != nullptr && split == it.nsplit - 1 && wave == (nblk - 1) % kWaves)
      append_newest<D, C>(a, b, g, ctx, lane);
  }

  auto row0_of = [&](int i) {       // first cache row of block i (wave-uniform)
    const int id = __builtin_amdgcn_readlane(mine, i);
    return ((int64_t)id * Hkv + g) * kBlock;
  };

  // ---- the ring: K and V tiles of kPf blocks in flight -----------------------
  // Slots past the wave's last block still load (so the compiler's wait
  // counts stay exact) but every lane reads the same bytes of the last
  // block, one cache line per instruction, and the compute skips them.
  uint4 rk[kPf][NCH];
  uint2 ksc[kPf], vsc[kPf];
  VRow rv[kPf][4];
  auto issue = [&](int s, int i) {
    const bool real = i <= last;                   // wave-uniform
    const int64_t row0 = row0_of(min(i, last));
    const int8_t* pk = a.k_cache + row0 * RB + (real ? hl * RB + 16 * q4 : 0);
#pragma unroll
    for (int u = 0; u < (NIB ? 1 : NCH); ++u) rk[s][u] = *reinterpret_cast<const uint4*>(pk + 64 * u);
    const int so = real ? 4 * q4 : 0;
    ksc[s] = *reinterpret_cast<const uint2*>(a.k_scale + row0 + so);
    vsc[s] = *reinterpret_cast<const uint2*>(a.v_scale + row0 + so);
    const int8_t* pv = a.v_cache + row0 * RB + (real ? 4 * q4 * RB + hl * (NIB ? NVT / 2 : NVT) : 0);
    const int stride = real ? RB : 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) rv[s][t] = *reinterpret_cast<const VRow*>(pv + t * stride);
  };
  if (nmine > 0) {
#pragma unroll
    for (int s = 0; s < kPf; ++s) issue(s, s);
  }

  // ---- q of head hl as the B operand of the logit MFMAs (while the first
  // tiles are in flight) --------------------------------------------------------
  half8_t qb[NKM], qlo[QF32 ? NKM : 1];
  float cz, nqb;
  q_operands<D, G, QF32, C>(a, bh0, hl, q4, qb, qlo, cz, nqb);

  // ---- one pass: logits, online softmax, weighted values ---------------------
  // Lane l holds, for head hl, the running max m (the same in the four lanes
  // of the head), its partial weight sum l over its tokens, and
  // O[hl][channel (D/16)(4 q4 + r) + j] in acc[j][r].
  float m_run = kNegInf, l_run = 0.0f;
  float4_t acc[NVT];
  float4_t accw = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < NVT; ++j) acc[j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int base = 0; base < nmine; base += kPf) {
    priority_by_remaining(nmine - base);
#pragma unroll
    for (int s = 0; s < kPf; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      const int i = base + s;
      if (i < nmine) {
        // logits of tokens 4 q4 + r for head hl
        float4_t S = {nqb, nqb, nqb, nqb};
#pragma unroll
        for (int j = 0; j < NKM; ++j) {
          const half8_t av = logit_operand<C>(rk[s], j);
          S = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qb[j], S, 0, 0, 0);
          if constexpr (QF32) S = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qlo[j], S, 0, 0, 0);
        }
        const int tb = (wave + i * kWaves) * kBlock + 4 * q4;   // split-local token of r = 0
        const uint32_t kw[2] = {ksc[s].x, ksc[s].y};
        const uint32_t vw[2] = {vsc[s].x, vsc[s].y};
        float z[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ks = fp16_bits_to_f32((uint16_t)(kw[r / 2] >> (16 * (r % 2))));
          z[r] = tb + r < ntok ? (ks * cz) * S[r] : kNegInf;
        }
        // block max of the head over its four lanes; a new max rescales
        float bm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
        bm = rows_max(bm);
        if (__builtin_amdgcn_ballot_w64(bm > m_run)) {   // wave-uniform branch
          const float f = bm > m_run ? __builtin_amdgcn_exp2f(m_run - bm) : 1.0f;
          m_run = fmaxf(m_run, bm);
          l_run *= f;
#pragma unroll
          for (int j = 0; j < NVT; ++j) acc[j] *= f;
          accw *= f;
        }
        _Float16 w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(z[r] - m_run);   // 0 for masked tokens
          const float vs = fp16_bits_to_f32((uint16_t)(vw[r / 2] >> (16 * (r % 2))));
          w[r] = (_Float16)(tb + r < ntok ? p * vs : 0.0f);   // never reads a stale scale
          l_run += p;
        }
        const half4_t wb = {w[0], w[1], w[2], w[3]};
        value_mfmas<C, NVT>(rv[s], wb, acc, accw);
      }
      issue(s, i + kPf);
    }
  }
  value_unbias<C, NVT>(acc, accw);

  // ---- the four waves to one split result, all relative to the split max ----
  if (lane < G) s_red[wave * G + lane] = m_run;
  __syncthreads();
  {
    float M = s_red[hl < G ? hl : 0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_red[w * G + (hl < G ? hl : 0)]);
    // a wave without blocks holds m = -inf and nothing else: factor 0
    const float f = m_run == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m_run - M);
    float lw = l_run * f;
    lw += __shfl_xor(lw, 16);
    lw += __shfl_xor(lw, 32);
    if (lane < G) s_red[kWaves * G + wave * G + lane] = lw;
    if (hl < G) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* dst = s_fin + (wave * G + hl) * D + NVT * (4 * q4 + r);
#pragma unroll
        for (int j = 0; j < NVT; ++j) dst[j] = acc[j][r] * f;
      }
    }
  }
  __syncthreads();
  finish_split<G, D, kThreads, kWaves>(
      PartialArgs{a.out, a.o_part, a.lse_part, a.counters, a.n_split}, s_fin, s_red, s_flag,
      bh0, (int64_t)b * Hkv + g, split, it.nsplit, tid);
}

template <int D, int G, bool QF32, class C, bool ONEPASS>
constexpr auto pick_kernel() {
  if constexpr (ONEPASS) return decode_mfma1_kernel<D, G, QF32, C>;
  else return decode_mfma2_kernel<D, G, QF32, C>;
}

template <int D, int G, bool QF32, class C, bool ONEPASS>
bool launch_one(const SplitArgs& a, hipStream_t stream) {
  constexpr auto kernel = pick_kernel<D, G, QF32, C, ONEPASS>();
  const int smem = ONEPASS ? msmem_layout(G, D).total : m2smem_layout(a.split_tokens, G, D).total;
  SplitArgs args = a;
  const int64_t grid = item_grid<kernel>(kThreads, smem, a.batch,
                                         (int64_t)a.n_split * a.num_kv_heads * a.batch,
                                         &args.period, &args.snake_rounds);
  if (grid > 0x7FFFFFFF) return false;
  kernel<<<dim3((unsigned)grid), dim3(kThreads), smem, stream>>>(args);
  return true;
}

template <int D, bool QF32, class C, bool ONEPASS>
bool by_group(int G, const SplitArgs& a, hipStream_t s) {
  switch (G) {
    case 1: return launch_one<D, 1, QF32, C, ONEPASS>(a, s);
    case 2: return launch_one<D, 2, QF32, C, ONEPASS>(a, s);
    case 4: return launch_one<D, 4, QF32, C, ONEPASS>(a, s);
    case 8: return launch_one<D, 8, QF32, C, ONEPASS>(a, s);
    default: return false;
  }
}

template <class C, bool ONEPASS>
bool by_dim(int head_dim, bool q_f32, int G, const SplitArgs& a, hipStream_t s) {
  if (head_dim == 128)
    return q_f32 ? by_group<128, true, C, ONEPASS>(G, a, s) : by_group<128, false, C, ONEPASS>(G, a, s);
  if (head_dim == 64)
    return q_f32 ? by_group<64, true, C, ONEPASS>(G, a, s) : by_group<64, false, C, ONEPASS>(G, a, s);
  return false;
}

template <bool ONEPASS>
bool by_fmt(const SplitArgs& a, int head_dim, int G, bool q_f32, int fmt, hipStream_t stream) {
  if (fmt == kFmtFp8) return by_dim<CodesFp8, ONEPASS>(head_dim, q_f32, G, a, stream);
  if (fmt == kFmtInt8) return by_dim<CodesInt8, ONEPASS>(head_dim, q_f32, G, a, stream);
  if (fmt == kFmtInt4 && head_dim == 128)   // 4-bit codes: d = 128
    return q_f32 ? by_group<128, true, CodesInt4, ONEPASS>(G, a, stream)
                 : by_group<128, false, CodesInt4, ONEPASS>(G, a, stream);
  return false;
}

}  // namespace

int decode_mfma2_smem(int split_tokens, int G, int head_dim) {
  return m2smem_layout(split_tokens, G, head_dim).total;
}

bool launch_decode_mfma(const SplitArgs& a, int head_dim, int G, bool q_f32, int fmt,
                        bool one_pass, hipStream_t stream) {
  return one_pass ? by_fmt<true>(a, head_dim, G, q_f32, fmt, stream)
                  : by_fmt<false>(a, head_dim, G, q_f32, fmt, stream);
}

}  // namespace kv8
