// paged_decode_attn_kv8 / _fp8kv / _int4kv, v_dot2 form: split-K
// flash-decoding over the paged INT8 (or FP8 e4m3, or INT4) cache for
// gfx950.
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
// Dot products use v_dot2_f32_f16 on fp16 pairs.  An INT8 code c enters as
// the fp16 value c + 1152 built by one byte permute (see kv8_device.h); the
// bias is removed once per token in pass 1 (the sums start at minus 1152 *
// sum q_h) and from each V code pair in pass 2 (one packed fp16 subtract,
// exact).  The same kernel serves the FP8 (e4m3) cache ("KV Cache 优化全景
// 解析", section 7.4), whose codes become exact fp16 pairs by one hardware
// convert and carry no bias, and the INT4 cache, whose nibbles enter the
// logits as 1.5 + c/16 (one shift and one bit operation per pair; the sums
// start at minus 1.5 * sum q_h) and the values as c + 1032 less the bias,
// exactly.  q enters as fp16 after an exact per-head power-of-two rescale
// (bf16 q is exact in fp16 then); an fp32 q is split into a high and a low
// fp16 part.
//
// Each wave keeps kPf blocks in flight in a register ring; the ring is
// branch-free around its loads so that the compiler's wait counts stay
// exact, and scheduling barriers keep later slots' waits from being hoisted.
#include <mutex>

#include "kv8_decode_common.h"
#include "kv8_device.h"
#include "kv8_launch.h"

namespace kv8 {

// ---------------------------------------------------------------------------
// Scratch of the allocation-free decode entry (paged_decode_attn_kv8_noalloc):
// a fixed device array that stands in for the caller's workspace, laid out
// as a workspace is (the split counters first, then the partials).  Each
// device the library runs on holds its own copy until the process ends.
// Host code never passes the array's name to a kernel: decode_scratch
// resolves this device's address with hipGetSymbolAddress once, with the
// device current, and returns that address.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {

__global__ __launch_bounds__(256) void zero_words_kernel(unsigned* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

}  // namespace

void* decode_scratch(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p != nullptr) return p;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
    return nullptr;
  // The counters must start at zero: clear them once, by a kernel on the
  // caller's stream (ordered before the call's own launch), after which
  // every completed call leaves them at zero again.
  const int64_t words = (int64_t)(kCounterBytes / sizeof(unsigned));
  zero_words_kernel<<<dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream>>>(
      static_cast<unsigned*>(addr), words);
  if (hipGetLastError() != hipSuccess) return nullptr;
  g_scratch_ptr[dev].store(addr, std::memory_order_release);
  return addr;
}

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kPf = 4;        // blocks in flight per wave and pass
constexpr float kLog2e = 1.4426950408889634f;



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
  L.flag_off = L.red_off + align16(2 * kWaves * G * 4);
  L.total = L.flag_off + 16;
  return L;
}

template <int NDW> struct RowT;
template <> struct RowT<4> { using type = uint4; };
template <> struct RowT<2> { using type = uint2; };
template <> struct RowT<1> { using type = uint32_t; };

__device__ __forceinline__ uint32_t dword(const uint4& r, int k) {
  return k == 0 ? r.x : k == 1 ? r.y : k == 2 ? r.z : r.w;
}
__device__ __forceinline__ uint32_t dword(const uint2& r, int k) { return k == 0 ? r.x : r.y; }
__device__ __forceinline__ uint32_t dword(const uint32_t& r, int) { return r; }

template <int D, int G, bool QF32, class C>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(SplitArgs a) {
  constexpr int CPL = D / 8;    // channels (= code bytes) per lane per token
  constexpr int NDW = CPL / 4;  // dwords per lane per token of 8-bit codes (and of bf16 q / 2)
  constexpr int NP = CPL / 2;   // fp16 pairs per lane per token
  constexpr int NIB = C::kBits == 4;              // 4-bit codes: 8 per dword
  constexpr int NDC = NIB ? CPL / 8 : NDW;        // code dwords per lane per token
  constexpr int RB = NIB ? D / 2 : D;             // code bytes per cache row
  constexpr int NV = (2 * G >= 8) ? (2 * G) / 8 : 1;   // logits stored per lane
  constexpr int M = G * CPL;    // accumulators per lane
  using QRow = typename RowT<NDW>::type;         // CPL / 2 bf16 q values
  using Row = typename RowT<NDC>::type;          // the lane's codes of one token

  extern __shared__ __align__(16) unsigned char smem[];
  const SmemLayout L = smem_layout(a.split_tokens, G, D);
  int* s_blk = reinterpret_cast<int*>(smem + L.blk_off);
  float* s_z = reinterpret_cast<float*>(smem + L.z_off);
  float* s_fin = s_z;
  uint16_t* s_vs = reinterpret_cast<uint16_t*>(smem + L.vs_off);
  uint32_t* s_pp = reinterpret_cast<uint32_t*>(smem + L.pp_off);
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

  // ---- decode step with append (the newest token, in the last split) ----
  if (C::kBits == 8 && a.k_new != nullptr && split == it.nsplit - 1 && wave == 0)
    append_newest<D, C>(a, b, g, ctx, lane);

  // ---- q of the G heads: this lane's d/8 channels as fp16 pairs ----------
  half2_t qh[G][NP];
  half2_t ql[QF32 ? G : 1][QF32 ? NP : 1];
  float cz[G], nqb[G];          // nqb: minus the code bias of this lane's channels
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
        const QRow* qp = reinterpret_cast<const QRow*>(
            static_cast<const uint16_t*>(a.q) + qrow0 + (int64_t)h * D);
        const QRow r = qp[0], r2 = qp[1];
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
        // pair p: channels (2p, 2p+1) for byte codes; for 4-bit codes the
        // channels (j, j+4) of 8-channel group p/4, j = p%4, the pairs the
        // nibble extraction produces
        const int c0 = NIB ? 8 * (p / 4) + p % 4 : 2 * p, c1 = NIB ? c0 + 4 : 2 * p + 1;
        const float a0 = ldexpf(x[c0], -e), a1 = ldexpf(x[c1], -e);
        const _Float16 h0 = (_Float16)a0, h1 = (_Float16)a1;
        qh[h][p] = half2_t{h0, h1};
        qsum += (float)h0 + (float)h1;
        if constexpr (QF32) {
          const _Float16 l0 = (_Float16)(a0 - (float)h0), l1 = (_Float16)(a1 - (float)h1);
          ql[h][p] = half2_t{l0, l1};
          qsum += (float)l0 + (float)l1;
        }
      }
      cz[h] = ldexpf(a.qk_scale_log2, e) * (1.0f / C::kLogitStep);
      nqb[h] = -C::kLogitBias * qsum;
    }
  }
  // per-lane constants of the logits this lane stores after the reduction
  const int tk = chunk >> 2;            // token of the pair: slot or slot+8
  int hv[NV];
  float czl[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    hv[j] = rs_head<G>(chunk, j);
    czl[j] = cz[0];
#pragma unroll
    for (int h = 1; h < G; ++h) czl[j] = hv[j] == h ? cz[h] : czl[j];
  }
  __syncthreads();   // s_blk visible

  // Each wave owns blocks wave + i * kWaves, i = 0 .. nmine-1; lane i of
  // `mine` holds the id of the wave's block i, so a block's base address is
  // scalar (readlane) and each lane adds its own row and channel offset.
  const int nmine = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;
  const int last = nmine - 1;
  const int mine = lane < nmine ? s_blk[wave + lane * kWaves] : 0;
  auto row0_of = [&](int i) {       // first cache row of block i (wave-uniform)
    const int id = __builtin_amdgcn_readlane(mine, i);
    return ((int64_t)id * Hkv + g) * kBlock;
  };
  const int lane_row = slot * RB + chunk * (RB / 8);   // this lane's byte offset in a block

  // ---- pass 1: logits ----------------------------------------------------
  float mloc[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) mloc[j] = kNegInf;
  if (nmine > 0) {
    Row r0[kPf], r1[kPf];
    uint16_t ksc16[kPf], vsc16[kPf];
    const int tok_row = slot + 8 * tk;            // the token whose logits this lane stores
    auto issue = [&](int s, int i) {
      const int64_t row0 = row0_of(i);
      const int8_t* p = a.k_cache + row0 * RB + lane_row;
      r0[s] = *reinterpret_cast<const Row*>(p);
      r1[s] = *reinterpret_cast<const Row*>(p + 8 * RB);
      ksc16[s] = a.k_scale[row0 + tok_row];
      vsc16[s] = a.v_scale[row0 + tok_row];
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
          const Row w0 = r0[s], w1 = r1[s];
          // the sums start at minus the codes' logit bias times the lane's
          // q, so the 8-lane reduction yields the unbiased dot products
          float S[2 * G];
#pragma unroll
          for (int h = 0; h < G; ++h) S[h] = S[G + h] = nqb[h];
          if constexpr (NIB) {
#pragma unroll
            for (int k = 0; k < NDC; ++k) {
              const uint32_t x0 = dword(w0, k), x1 = dword(w1, k);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const half2_t a0 = C::logit_pair_raw(x0, j), a1 = C::logit_pair_raw(x1, j);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                  S[h] = fdot2(qh[h][4 * k + j], a0, S[h]);
                  S[G + h] = fdot2(qh[h][4 * k + j], a1, S[G + h]);
                  if constexpr (QF32) {
                    S[h] = fdot2(ql[h][4 * k + j], a0, S[h]);
                    S[G + h] = fdot2(ql[h][4 * k + j], a1, S[G + h]);
                  }
                }
              }
            }
          } else {
#pragma unroll
          for (int k = 0; k < NDW; ++k) {
            const uint32_t x0 = C::pre(dword(w0, k)), x1 = C::pre(dword(w1, k));
            const half2_t a0 = C::lo(x0), b0 = C::hi(x0);
            const half2_t a1 = C::lo(x1), b1 = C::hi(x1);
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
          }
          float R[NV];
          reduce_scatter8<G>(S, R, chunk);
          const int tl = (wave + i * kWaves) * kBlock + slot + 8 * tk;
          const bool ok = tl < ntok;
          const float ksc = fp16_bits_to_f32(ksc16[s]);
#pragma unroll
          for (int j = 0; j < NV; ++j) {
            const float z = ok ? (ksc * czl[j]) * R[j] : kNegInf;
            s_z[tl * G + hv[j]] = z;
            mloc[j] = fmaxf(mloc[j], z);
          }
          s_vs[tl] = vsc16[s];
        }
        issue(s, min(i + kPf, last));
      }
    }
  }

  // V rows of the first kPf blocks are requested now, so that they arrive
  // while the workgroup finishes the logits and builds the weights.
  Row r0[kPf], r1[kPf];
  auto issue_v = [&](int s, int i) {
    const int8_t* p = a.v_cache + row0_of(i) * RB + lane_row;
    r0[s] = *reinterpret_cast<const Row*>(p);
    r1[s] = *reinterpret_cast<const Row*>(p + 8 * RB);
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
    float lsum = 0.0f;
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
      }
      const int jj = t / kBlock, r = t % kBlock;
      pph[((jj * 8 + (r & 7)) * G + h) * 2 + (r >> 3)] = p16;
    }
#pragma unroll
    for (int off = G; off < 64; off <<= 1) lsum += __shfl_xor(lsum, off);
    if (lane < G) s_red[kWaves * G + wave * G + lane] = lsum;
  }
  __syncthreads();

  // ---- pass 2: weighted sum of V codes ------------------------------------
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
        const Row w0 = r0[s], w1 = r1[s];
        half2_t wp[G];
        const uint32_t* src = s_pp + ((wave + i * kWaves) * 8 + slot) * G;
#pragma unroll
        for (int h = 0; h < G; ++h) wp[h] = __builtin_bit_cast(half2_t, src[h]);
        if constexpr (NIB) {
          // bytes 0,1 (channels 8k..8k+3) and 2,3 (8k+4..8k+7) of the two
          // tokens side by side, so nibble pairs are (token t, token t+8)
#pragma unroll
          for (int k = 0; k < NDC; ++k) {
            const uint32_t u0 = dword(w0, k), u1 = dword(w1, k);
            const uint32_t lo = __builtin_amdgcn_perm(u1, u0, 0x05040100u);
            const uint32_t hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              // unbiased exactly here: biased sums over a long split would
              // cancel away too many bits
              const half2_t fl = C::exact(C::nib_pair_raw(lo, j));
              const half2_t fh = C::exact(C::nib_pair_raw(hi, j));
#pragma unroll
              for (int h = 0; h < G; ++h) {
                acc[h * CPL + 8 * k + j] = fdot2(wp[h], fl, acc[h * CPL + 8 * k + j]);
                acc[h * CPL + 8 * k + 4 + j] = fdot2(wp[h], fh, acc[h * CPL + 8 * k + 4 + j]);
              }
            }
          }
        } else {
#pragma unroll
        for (int k = 0; k < NDW; ++k) {
          const uint32_t x0 = C::pre(dword(w0, k)), x1 = C::pre(dword(w1, k));
          const uint32_t i01 = interleave_lo(x0, x1), i23 = interleave_hi(x0, x1);
          const half2_t f0 = C::exact(C::lo(i01)), f1 = C::exact(C::hi(i01));
          const half2_t f2 = C::exact(C::lo(i23)), f3 = C::exact(C::hi(i23));
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h * CPL + 4 * k] = fdot2(wp[h], f0, acc[h * CPL + 4 * k]);
            acc[h * CPL + 4 * k + 1] = fdot2(wp[h], f1, acc[h * CPL + 4 * k + 1]);
            acc[h * CPL + 4 * k + 2] = fdot2(wp[h], f2, acc[h * CPL + 4 * k + 2]);
            acc[h * CPL + 4 * k + 3] = fdot2(wp[h], f3, acc[h * CPL + 4 * k + 3]);
          }
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

template <int D, int G, bool QF32, class C>
bool launch_split(const SplitArgs& a, int batch, hipStream_t stream) {
  const SmemLayout L = smem_layout(a.split_tokens, G, D);
  SplitArgs args = a;
  const int64_t grid = item_grid<decode_split_kernel<D, G, QF32, C>>(
      kThreads, L.total, batch, (int64_t)a.n_split * a.num_kv_heads * batch, &args.period,
      &args.snake_rounds);
  if (grid > 0x7FFFFFFF) return false;
  decode_split_kernel<D, G, QF32, C><<<dim3((unsigned)grid), dim3(kThreads), L.total, stream>>>(
      args);
  return true;
}

template <int D, bool QF32, class C>
bool dispatch_g(int G, const SplitArgs& a, int batch, hipStream_t s) {
  switch (G) {
    case 1: return launch_split<D, 1, QF32, C>(a, batch, s);
    case 2: return launch_split<D, 2, QF32, C>(a, batch, s);
    case 4: return launch_split<D, 4, QF32, C>(a, batch, s);
    case 8: return launch_split<D, 8, QF32, C>(a, batch, s);
    default: return false;
  }
}

template <class C>
bool dispatch_fmt(int head_dim, bool q_f32, int G, const SplitArgs& a, int batch,
                  hipStream_t s) {
  if (head_dim == 128) return q_f32 ? dispatch_g<128, true, C>(G, a, batch, s)
                                    : dispatch_g<128, false, C>(G, a, batch, s);
  return q_f32 ? dispatch_g<64, true, C>(G, a, batch, s) : dispatch_g<64, false, C>(G, a, batch, s);
}

constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

// Automatic choice (measured on MI355X):
// - below G = 4: the v_dot2 kernel (the vector work per cache byte, G/2
//   v_dot2 issues per lane, still fits under the memory stream);
// - from G = 4, a grid bound of at most 1024 workgroups (one round at five
//   two-pass workgroups per CU) and a longest context in (2048, 8192]: the
//   two-pass matrix-core form, 3-7% ahead of stream-K there at G = 4 (37.3
//   against 41.6 us on the Llama-3.1-8B-shaped batch, 32 x 1024..4096
//   tokens; 39.3 against 42.2 us on 16 x 2048..8192) and 1-6% at G = 8
//   (42.0 against 44.5 us on 16 x 2048..8192);
// - otherwise the stream-K form.  With more work items
//   than one round the two-pass form falls behind by 5-18% (32 x
//   2048..8192: 79.3 against 66.8 us; 96 x 1024..4096: 117.5 against
//   95.9 us), and with short contexts it ties or loses (64 x 512..2048: 44.8
//   against 42.8 us).  Long contexts: 61.3 against 66.5 us per step for the
//   one-pass form on 4 sequences of 32768 tokens, 1488 against 1525 us on
//   15 sequences of 264192 tokens; 125.7 against 139.8 us per layer of the
//   Llama-3-70B-shaped sweep at G = 8.
// `grid_bound` is the workgroup count with every sequence at the longest
// context and 1024-token splits.
// - INT4 codes: the matrix-core forms serve d = 128 only (the v_dot2
//   kernel otherwise); from G = 4 the one-pass form (28.9 us on the
//   Llama-3.1-8B-shaped batch against 34.5 us for stream-K; 1911 against
//   2081 us on 31 sequences of 264192 tokens).
int decode_form(int requested, int fmt, int G, long long grid_bound, int max_context_len,
                int head_dim) {
  if (fmt == kFmtInt4 && head_dim != 128) return kDecodeKernelDot;
  if (requested != kDecodeKernelAuto) return requested;
  if (fmt == kFmtInt4) return G >= 4 ? kDecodeKernelMfmaOnePass : kDecodeKernelDot;
  if (G >= 4)
    return grid_bound <= 1024 && max_context_len > 2048 && max_context_len <= 8192
               ? kDecodeKernelMfma
               : kDecodeKernelStreamK;
  return kDecodeKernelDot;
}

bool plan_decode(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                 int max_context_len, int tokens_per_split, int form, DecodePlan* plan) {
  if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0) return false;
  if (num_q_heads % num_kv_heads != 0) return false;
  if ((int64_t)batch * num_kv_heads > kMaxDecodePairs) return false;
  const int G = num_q_heads / num_kv_heads;
  // LDS of one workgroup at a split size: the one-pass kernel's does not
  // grow with the split
  if (form == kDecodeKernelStreamK) {
    // units are counted in 32 bits: at most batch * Hkv * ceil(max_context_len / 16)
    if ((int64_t)batch * num_kv_heads * (((int64_t)max_context_len + 15) / 16) > 0x7FFFFFFF)
      return false;
    if (tokens_per_split < 0 || tokens_per_split > 2048 || tokens_per_split % 64 != 0)
      return false;
    plan->form = form;
    plan->split_tokens = 0;
    plan->n_split = 1;
    plan->counter_bytes = kCounterBytes;
    plan->o_bytes = align256((size_t)kSkMaxWorkgroups * 2 *
                             ((size_t)num_q_heads / num_kv_heads * head_dim +
                              2 * (size_t)(num_q_heads / num_kv_heads)) * sizeof(float));
    plan->lse_bytes = 0;
    plan->total_bytes = plan->counter_bytes + plan->o_bytes;
    return true;
  }
  auto smem = [&](int tps) {
    if (form == kDecodeKernelMfmaOnePass) return 0;
    if (form == kDecodeKernelMfma) return decode_mfma2_smem(tps, G, head_dim);
    return smem_layout(tps, G, head_dim).total;
  };
  int tps = tokens_per_split;
  if (tps <= 0) {
    // Largest split whose grid bound (every sequence at max_context_len)
    // still reaches 1024 workgroups, about four per CU: the per-workgroup
    // prologue, cross-wave reductions, partials and merge are a fixed cost
    // that larger splits amortise (measured on the Llama-3.1-8B-shaped
    // batch: 1024-token splits 45.7 us, 512 51.0 us, 256 59.5 us; on the
    // Llama-3-70B-shaped sweep with the one-pass kernel: 2048-token splits
    // 136.7 us per layer, 1024 152.6 us).  2048 only for the one-pass form.
    tps = 64;
    const int cands[] = {2048, 1024, 512, 256, 128};
    for (int c : cands) {
      if (c == 2048 && form != kDecodeKernelMfmaOnePass) continue;
      const long long per_seq = max_context_len > 0 ? (max_context_len + c - 1) / c : 1;
      if ((long long)batch * num_kv_heads * per_seq >= 1024) { tps = c; break; }
    }
    while (tps > 64 && smem(tps) > 64 * 1024) tps /= 2;
  } else if (tps % 64 != 0 || tps < 64 || tps > 2048) {
    return false;
  }
  if (smem(tps) > 64 * 1024) return false;
  const int n_split = max_context_len > 0 ? (max_context_len + tps - 1) / tps : 1;
  plan->form = form;
  plan->split_tokens = tps;
  plan->n_split = n_split;
  plan->counter_bytes = kCounterBytes;
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
                  void* workspace, const DecodePlan& plan, int fmt, const uint16_t* k_new,
                  const uint16_t* v_new, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  SplitArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.k_new = k_new;
  a.v_new = v_new;
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
  if (plan.form == kDecodeKernelStreamK) {
    a.period = decode_sk_workgroups();
    ok = launch_decode_sk(a, head_dim, G, q_f32, fmt, stream);
  } else if (plan.form != kDecodeKernelDot) {
    ok = launch_decode_mfma(a, head_dim, G, q_f32, fmt, plan.form == kDecodeKernelMfmaOnePass,
                            stream);
  } else if (fmt == kFmtFp8) ok = dispatch_fmt<CodesFp8>(head_dim, q_f32, G, a, batch, stream);
  else if (fmt == kFmtInt4) ok = dispatch_fmt<CodesInt4>(head_dim, q_f32, G, a, batch, stream);
  else ok = dispatch_fmt<CodesInt8>(head_dim, q_f32, G, a, batch, stream);
  if (!ok) return -2;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kv8
