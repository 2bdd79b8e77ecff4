// Stream-K form of paged_decode_attn_kv8 / _fp8kv / _int4kv on gfx950: the
// decode's work cut into equal contiguous ranges, one per workgroup, with
// the one-pass matrix-core arithmetic of kv8_decode_mfma.hip per block.
//
// Attention softmax(q K^T * sm_scale) V ("KV Cache 优化全景解析", section 2.1)
// per GQA group (section 3.3) over K/V restored from per-token quantised
// codes ("KV-Cache 全栈优化系统" README, section 主要特性), fp32 softmax and
// accumulation ("大模型推理加速：KV Cache与vLLM技术解析", section 4.1);
// partial results of one (sequence, KV head) are combined by log-sum-exp.
//
// Work units are the (sequence b, KV head g, block j) triples in that
// order: pair p = b * Hkv + g holds nb_b = ceil(ctx_b / 16) consecutive
// units.  With T units in all and NW workgroups (one per compute unit,
// kSkWaves = 8 waves each), workgroup w takes units [w T / NW, (w + 1) T /
// NW) and wave v of it the v-th of kSkWaves near-equal contiguous parts of
// that range.  A wave streams its units in order with the one-pass online
// softmax (K and V tiles of the next blocks in flight while the current
// block is computed), starting a new softmax state at every pair boundary,
// so its memory stream never waits on another wave: there are no per-item
// prologues, no mid-item barriers and no tail of unequal items.
//
// A pair wholly inside one wave's part is normalised and written by that
// wave.  A pair cut by wave boundaries leaves the state of each piece (sums
// relative to the piece's max, the max, the weight sum) in LDS; after one
// workgroup barrier the wave holding the pair's first piece merges them.  A
// pair cut by workgroup boundaries leaves one such merged state per
// workgroup in the workspace (slot 1 of the workgroup where the pair starts,
// slot 0 of every later one) and adds the number of the pair's units it
// holds to the pair's counter; the workgroup that brings the counter to the
// pair's block count merges the states, writes the output and clears the
// counter.
//
// In the decode step with append, the wave that owns a pair's last block
// quantises and stores the newest token of that pair before its loads of
// the block.
#include "kv8_decode_common.h"
#include "kv8_device.h"
#include "kv8_launch.h"
#include "kv8_mfma_block.h"

namespace kv8 {

namespace {

constexpr int kSkWaves = 8;
constexpr int kSkThreads = kSkWaves * 64;
constexpr int kSkPf = 2;        // blocks (K and V tiles) in flight per wave

// Unit of lane l of a wave's current batch of 64 units.
struct Unit {
  int id;    // physical block id (clamped into range)
  int bg;    // sequence b << 16 | KV head g
  int j;     // block of the pair
  int ctx;   // tokens of the sequence (the pair has ceil(ctx / 16) blocks)
};

// Blocks of sequence b's context (clamped as every decode clamps it).
__device__ __forceinline__ int seq_blocks(const SplitArgs& a, int b, int& ctx) {
  ctx = min(max(a.context_lens[b], 0), a.ctx_cap);
  return (ctx + kBlock - 1) / kBlock;
}

// The first 64 sequences' context lengths, block counts and their
// inclusive scan, kept from total_units for locate_units.
struct Chunk0 {
  int ctx, nb, incl, ntot;
};

// Total units T = Hkv * sum_b nb_b (every lane receives it).
__device__ __forceinline__ int64_t total_units(const SplitArgs& a, int lane, Chunk0& k0) {
  int64_t tot = 0;
  for (int c0 = 0; c0 < a.batch; c0 += 64) {
    int ctx = 0;
    const int nb = c0 + lane < a.batch ? seq_blocks(a, c0 + lane, ctx) : 0;
    const int incl = wave_incl_scan(nb, lane);
    const int n = __builtin_amdgcn_readlane(incl, 63);
    if (c0 == 0) k0 = Chunk0{ctx, nb, incl, n};
    tot += n;
  }
  return tot * a.num_kv_heads;
}

// Lane l's unit u = base + l, for lanes l < cnt (units are counted in 32
// bits: the host bounds their total below 2^31).  One ballot finds the
// sequence of the batch's first unit; a wave-uniform walk then takes the
// few sequences the batch spans in order, each giving its lanes' KV head and
// block by one division by the sequence's block count.
__device__ __forceinline__ Unit locate_units(const SplitArgs& a, int base, int cnt, int lane,
                                            const Chunk0& k0) {
  Unit x{0, 0, 0, 16};
  const int Hkv = a.num_kv_heads;
  const int u = base + lane;
  int before = 0;             // units of the sequences before chunk c0
  int c0 = 0, ctx = 0, nb = 0, incl = 0, ntot = 0;
  auto load_chunk = [&]() {
    if (c0 == 0) {            // wave-uniform: the first chunk is already at hand
      ctx = k0.ctx;
      nb = k0.nb;
      incl = k0.incl;
      ntot = k0.ntot;
      return;
    }
    ctx = 0;
    nb = c0 + lane < a.batch ? seq_blocks(a, c0 + lane, ctx) : 0;
    incl = wave_incl_scan(nb, lane);
    ntot = __builtin_amdgcn_readlane(incl, 63);
  };
  for (;;) {                  // the chunk of 64 sequences holding unit `base`
    load_chunk();
    if (base < before + ntot * Hkv || c0 + 64 >= a.batch) break;
    before += ntot * Hkv;
    c0 += 64;
  }
  int s = __builtin_popcountll(__builtin_amdgcn_ballot_w64(c0 + lane < a.batch &&
                                                           before + incl * Hkv <= base));
  int xb = 0;
  for (;;) {                  // wave-uniform walk over the sequences of the batch
    if (s >= 64) {
      if (c0 + 64 >= a.batch) break;
      before += ntot * Hkv;
      c0 += 64;
      s = 0;
      load_chunk();
    }
    if (c0 + s >= a.batch) break;
    const int nbs = __builtin_amdgcn_readlane(nb, s);
    const int start = before + (__builtin_amdgcn_readlane(incl, s) - nbs) * Hkv;
    const int end = start + nbs * Hkv;
    if (lane < cnt && u >= start && u < end) {
      const int r = u - start;
      const int g = r / nbs;
      xb = c0 + s;
      x.bg = (xb << 16) | g;
      x.j = r - g * nbs;
      x.ctx = __builtin_amdgcn_readlane(ctx, s);
    }
    if (end >= base + cnt) break;
    ++s;
  }
  if (lane < cnt) {
    const int64_t id = a.block_table[(int64_t)xb * a.max_blocks_per_seq + x.j];
    x.id = (int)(id < 0 ? 0 : (id >= a.num_blocks ? a.num_blocks - 1 : id));
  }
  return x;
}

// Workgroup whose range holds unit u: the largest w with floor(w T / NW) <= u.
__device__ __forceinline__ int wg_of(int64_t u, int64_t T, int nw) {
  return (int)(((u + 1) * nw - 1) / T);
}

template <int G, int D>
struct SkLds {
  float acc[kSkWaves][2][G * D];   // piece sums relative to the piece max
  float m[kSkWaves][2][G];         // piece max (log2 domain)
  float l[kSkWaves][2][G];         // piece weight sum
  int meta[kSkWaves][2][4];        // pair (-1: empty), flags (1: first block, 2: last), P0, nb
};

template <int D, int G, bool QF32, class C>
__global__ __launch_bounds__(kSkThreads) void decode_sk_kernel(SplitArgs a) {
  static_assert(G >= 1 && G <= 16, "one 16-column tile of heads");
  constexpr bool NIB = C::kBits == 4;
  static_assert(!NIB || D == 128, "4-bit codes: d = 128");
  constexpr int RB = NIB ? D / 2 : D;
  constexpr int NCH = D / 64;
  constexpr int NKM = D / 32;
  constexpr int NVT = D / 16;
  constexpr int NVD = NIB ? 1 : NVT / 4;
  using VRow = typename VRowT<NVD>::type;
  constexpr int SLOT = G * D + 2 * G;      // floats of one workspace partial
  constexpr int NE = G * D / 64;           // output elements per lane in the merges

  __shared__ SkLds<G, D> lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane & 15, q4 = lane >> 4;
  const int Hkv = a.num_kv_heads, Hq = a.num_q_heads;
  const int nw = a.period;
  const int w = blockIdx.x;

  if (lane < 2) lds.meta[wave][lane][0] = -1;

  // ---- sequences with an empty context: zero output (workgroup b % NW) ----
  if (wave == 0) {
    for (int c0 = 0; c0 < a.batch; c0 += 64) {
      const int b = c0 + lane;
      int ctx = 1;
      if (b < a.batch && b % nw == w) seq_blocks(a, b, ctx);
      uint64_t empty = __builtin_amdgcn_ballot_w64(ctx == 0);
      while (empty) {
        const int bb = c0 + __builtin_ctzll(empty);
        empty &= empty - 1;
        for (int e = lane; e < Hq * D; e += 64) a.out[(int64_t)bb * Hq * D + e] = 0.0f;
      }
    }
  }

  Chunk0 k0{0, 0, 0, 0};
  const int64_t T = total_units(a, lane, k0);
  const int64_t wu0 = (int64_t)w * T / nw, wu1 = (int64_t)(w + 1) * T / nw;
  // Wave parts: kSkWaves near-equal contiguous parts, each non-empty when
  // the workgroup holds at least kSkWaves units; with fewer, one unit for
  // each of the first waves.  Either way the empty parts come last, so the waves holding
  // pieces of one pair are consecutive.
  const int64_t n = wu1 - wu0;
  const int64_t u0 = wu0 + (n >= kSkWaves ? (int64_t)wave * n / kSkWaves : min((int64_t)wave, n));
  const int64_t u1 =
      wu0 + (n >= kSkWaves ? (int64_t)(wave + 1) * n / kSkWaves : min((int64_t)wave + 1, n));

  // ---- stream the wave's units ----------------------------------------------
  half8_t qb[NKM], qlo[QF32 ? NKM : 1];
  float cz = 0.0f, nqb = 0.0f;
  float m_run = kNegInf, l_run = 0.0f;
  float4_t acc[NVT];
  float4_t accw = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < NVT; ++j) acc[j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  int cur_b = -1, cur_g = 0, seg_flags = 0, seg_nb = 1, nseg = 0;
  int64_t seg_p0 = 0;

  // Ends the current piece: a whole pair is normalised and written out; a
  // piece of a pair goes to the wave's LDS slot (0: its first piece, 1: its
  // last one; only those can be cut).
  auto flush = [&]() {
    if constexpr (NIB) value_unbias<C, NVT>(acc, accw);
    float lw = l_run;
    lw += __shfl_xor(lw, 16);
    lw += __shfl_xor(lw, 32);
    const int64_t bh0 = (int64_t)cur_b * Hq + (int64_t)cur_g * G;
    if (seg_flags == 3) {
      if (hl < G) {
        const float inv = 1.0f / lw;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* dst = a.out + (bh0 + hl) * D + NVT * (4 * q4 + r);
#pragma unroll
          for (int j = 0; j < NVT; ++j) dst[j] = acc[j][r] * inv;
        }
      }
    } else {
      const int s = nseg == 0 ? 0 : 1;
      if (hl < G) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* dst = &lds.acc[wave][s][hl * D + NVT * (4 * q4 + r)];
#pragma unroll
          for (int j = 0; j < NVT; ++j) dst[j] = acc[j][r];
        }
        if (q4 == 0) {
          lds.m[wave][s][hl] = m_run;
          lds.l[wave][s][hl] = lw;
        }
      }
      if (lane == 0) {
        lds.meta[wave][s][0] = cur_b * Hkv + cur_g;
        lds.meta[wave][s][1] = seg_flags;
        lds.meta[wave][s][2] = (int)seg_p0;
        lds.meta[wave][s][3] = seg_nb;
      }
    }
    ++nseg;
  };

  for (int64_t base = u0; base < u1; base += 64) {
    const int cnt = (int)min((int64_t)64, u1 - base);
    const Unit un = locate_units(a, (int)base, cnt, lane, k0);

    // the decode step with append: the newest token of every pair whose
    // last block is in this batch, stored before the batch's loads
    if constexpr (!NIB) {
      if (a.k_new != nullptr) {
        uint64_t last = __builtin_amdgcn_ballot_w64(
            lane < cnt && un.j == (un.ctx + kBlock - 1) / kBlock - 1);
        while (last) {
          const int t = __builtin_ctzll(last);
          last &= last - 1;
          const int bg = __builtin_amdgcn_readlane(un.bg, t);
          append_newest<D, C>(a, bg >> 16, bg & 0xFFFF, __builtin_amdgcn_readlane(un.ctx, t),
                              lane);
        }
      }
    }

    uint4 rk[kSkPf][NCH];
    uint2 ksc[kSkPf], vsc[kSkPf];
    VRow rv[kSkPf][4];
    // Loads of unit i into ring slot sl (clamped to the batch's last unit:
    // the compute skips a clamped slot, the loads keep the compiler's wait
    // counts exact).  kSkPf blocks are in flight per wave: the K codes and
    // both scale rows of block i + kSkPf are requested once block i's
    // weights are formed, its V codes once block i's value MFMAs have read
    // theirs.  Codes are read once per call and come nontemporal (long
    // context: 62 -> 59 us per step; the 80-layer sweep 122 -> 115 us per
    // layer); the scales stay ordinary loads, one line serving several heads.
    auto row0_of = [&](int i, bool& real) {
      real = i < cnt;
      const int ii = real ? i : cnt - 1;
      const int id = __builtin_amdgcn_readlane(un.id, ii);
      const int g = __builtin_amdgcn_readlane(un.bg, ii) & 0xFFFF;
      return ((int64_t)id * Hkv + g) * kBlock;
    };
    auto issue_k = [&](int sl, int i) {
      bool real;
      const int64_t row0 = row0_of(i, real);
      const int8_t* pk = a.k_cache + row0 * RB + (real ? hl * RB + 16 * q4 : 0);
#pragma unroll
      for (int u = 0; u < (NIB ? 1 : NCH); ++u)
        rk[sl][u] = nt_load(reinterpret_cast<const uint4*>(pk + 64 * u));
      const int so = real ? 4 * q4 : 0;
      ksc[sl] = *reinterpret_cast<const uint2*>(a.k_scale + row0 + so);
      vsc[sl] = *reinterpret_cast<const uint2*>(a.v_scale + row0 + so);
    };
    auto issue_v = [&](int sl, int i) {
      bool real;
      const int64_t row0 = row0_of(i, real);
      const int8_t* pv =
          a.v_cache + row0 * RB + (real ? 4 * q4 * RB + hl * (NIB ? NVT / 2 : NVT) : 0);
      const int stride = real ? RB : 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) rv[sl][t] = nt_load(reinterpret_cast<const VRow*>(pv + t * stride));
    };
#pragma unroll
    for (int sl = 0; sl < kSkPf; ++sl) {
      issue_k(sl, sl);
      issue_v(sl, sl);
    }
    for (int i0 = 0; i0 < cnt; i0 += kSkPf) {
#pragma unroll
      for (int sl = 0; sl < kSkPf; ++sl) {
        __builtin_amdgcn_sched_barrier(0);
        const int i = i0 + sl;
        if (i < cnt) {                                  // wave-uniform
          const int bg = __builtin_amdgcn_readlane(un.bg, i);
          const int b = bg >> 16, g = bg & 0xFFFF;
          const int jb = __builtin_amdgcn_readlane(un.j, i);
          const int ctx = __builtin_amdgcn_readlane(un.ctx, i);
          const int nbp = (ctx + kBlock - 1) / kBlock;
          if (b != cur_b || g != cur_g) {                 // wave-uniform: a new pair
            if (cur_b >= 0) flush();
            cur_b = b;
            cur_g = g;
            seg_flags = jb == 0 ? 1 : 0;
            seg_p0 = base + i - jb;
            seg_nb = nbp;
            m_run = kNegInf;
            l_run = 0.0f;
#pragma unroll
            for (int j = 0; j < NVT; ++j) acc[j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (NIB) accw = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
            q_operands<D, G, QF32, C>(a, (int64_t)b * Hq + (int64_t)g * G, hl, q4, qb, qlo, cz, nqb);
          }
          if (jb == nbp - 1) seg_flags |= 2;
          const int nt = jb == nbp - 1 ? ctx - jb * kBlock : kBlock;   // tokens in the block

          float4_t S = {nqb, nqb, nqb, nqb};
#pragma unroll
          for (int j = 0; j < NKM; ++j) {
            const half8_t av = logit_operand<C>(rk[sl], j);
            S = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qb[j], S, 0, 0, 0);
            if constexpr (QF32) S = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qlo[j], S, 0, 0, 0);
          }
          float z[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t kw = r < 2 ? ksc[sl].x : ksc[sl].y;
            const float ks = fp16_bits_to_f32((uint16_t)(kw >> (16 * (r % 2))));
            z[r] = 4 * q4 + r < nt ? (ks * cz) * S[r] : kNegInf;
          }
          float bm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
          bm = rows_max(bm);
          if (__builtin_amdgcn_ballot_w64(bm > m_run)) {   // wave-uniform branch
            const float f = bm > m_run ? __builtin_amdgcn_exp2f(m_run - bm) : 1.0f;
            m_run = fmaxf(m_run, bm);
            l_run *= f;
#pragma unroll
            for (int j = 0; j < NVT; ++j) acc[j] *= f;
            if constexpr (NIB) accw *= f;
          }
          _Float16 wv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(z[r] - m_run);   // 0 for masked tokens
            const uint32_t vw = r < 2 ? vsc[sl].x : vsc[sl].y;
            const float vs = fp16_bits_to_f32((uint16_t)(vw >> (16 * (r % 2))));
            wv[r] = (_Float16)(4 * q4 + r < nt ? p * vs : 0.0f);     // never a stale scale
            l_run += p;
          }
          issue_k(sl, i + kSkPf);
          const half4_t wb = {wv[0], wv[1], wv[2], wv[3]};
          value_mfmas<C, NVT>(rv[sl], wb, acc, accw);
          issue_v(sl, i + kSkPf);
        } else {
          issue_k(sl, i + kSkPf);
          issue_v(sl, i + kSkPf);
        }
      }
    }
  }
  if (cur_b >= 0) flush();
  __syncthreads();

  // ---- pieces of pairs cut by wave boundaries: merge in LDS ------------------
  for (int s = 0; s < 2; ++s) {
    const int P = lds.meta[wave][s][0];
    if (P < 0) continue;                                          // wave-uniform
    if (s == 0 && wave > 0 &&
        (lds.meta[wave - 1][1][0] == P || lds.meta[wave - 1][0][0] == P))
      continue;                                                   // an earlier wave merges
    // this wave holds the pair's first piece in the workgroup: the pieces
    // are (wave, s) and slot 0 of the following waves while they hold P
    int vl = wave;
    while (vl + 1 < kSkWaves && lds.meta[vl + 1][0][0] == P) ++vl;
    const int flags_first = lds.meta[wave][s][1];
    const int flags_last = vl == wave ? flags_first : lds.meta[vl][0][1];
    const int64_t P0 = lds.meta[wave][s][2];
    const int nbp = lds.meta[wave][s][3];
    const int b = P / Hkv, g = P - (P / Hkv) * Hkv;
    const int64_t bh0 = (int64_t)b * Hq + (int64_t)g * G;
    const bool whole = (flags_first & 1) && (flags_last & 2);
    // combine the pieces: the per-head maxima, then per piece all of its
    // LDS reads issued together and folded in (a read waits only on its own
    // piece, not on the previous read).  Lane l holds elements e = l + 64 k,
    // of head 64 k / D (l < 64, D a multiple of 64).
    const int gslot = (flags_first & 1) ? 1 : 0;
    float* part = a.o_part + ((int64_t)w * 2 + gslot) * SLOT;
    float Mp[G], dp[G], np_[NE];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      Mp[h] = kNegInf;
      dp[h] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < NE; ++k) np_[k] = 0.0f;
    for (int v = wave; v <= vl; ++v) {
      const int sv = v == wave ? s : 0;
      float mv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) mv[h] = lds.m[v][sv][h];
#pragma unroll
      for (int h = 0; h < G; ++h) Mp[h] = fmaxf(Mp[h], mv[h]);
    }
    for (int v = wave; v <= vl; ++v) {
      const int sv = v == wave ? s : 0;
      float mv[G], lv[G], av[NE], f[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        mv[h] = lds.m[v][sv][h];
        lv[h] = lds.l[v][sv][h];
      }
#pragma unroll
      for (int k = 0; k < NE; ++k) av[k] = lds.acc[v][sv][lane + 64 * k];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        f[h] = mv[h] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mv[h] - Mp[h]);
        dp[h] += f[h] * lv[h];
      }
#pragma unroll
      for (int k = 0; k < NE; ++k) np_[k] += f[64 * k / D] * av[k];
    }
    if (whole) {
#pragma unroll
      for (int k = 0; k < NE; ++k) a.out[bh0 * D + lane + 64 * k] = np_[k] / dp[64 * k / D];
    } else {
#pragma unroll
      for (int k = 0; k < NE; ++k) store_agent(part + lane + 64 * k, np_[k]);
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          store_agent(part + G * D + h, Mp[h]);
          store_agent(part + G * D + G + h, dp[h]);
        }
      }
    }
    if (whole) continue;
    // ---- pairs cut by workgroup boundaries: the last workgroup merges -------
    // Each workgroup adds the pair's units it holds to the pair's counter;
    // the one that completes the pair's nbp units merges.  (Counting units,
    // not workgroups, stays right when some workgroups hold no units.)
    // The counters of pairs that finish together are spread one per
    // 128-byte line when the fixed counter region allows it, so that their
    // atomics do not queue on one line.
    wait_vmem();
    const int64_t P1 = P0 + nbp;
    const unsigned mine = (unsigned)(min(P1, wu1) - max(P0, wu0));
    const int cstride = min(32, (int)(kMaxDecodePairs / ((int64_t)a.batch * Hkv)));
    unsigned* cnt = a.counters + (int64_t)P * cstride;
    unsigned prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(cnt, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev + mine != (unsigned)nbp) continue;                   // not the last one
    if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int wf = wg_of(P0, T, nw), wl = wg_of(P1 - 1, T, nw);
    // The partial states travel through agent-scope (cross-XCD coherent)
    // accesses.  All loads of a batch of workgroups are issued before any is
    // used and folded in by an online log-sum-exp, so a batch costs one
    // memory round trip.  Lane l holds elements e = l + 64 k of the [G][D]
    // output, of head 64 k / D (l < 64, D a multiple of 64).
    constexpr int MB = 64 / (NE + 2 * G) < 1 ? 1 : (64 / (NE + 2 * G) > 8 ? 8 : 64 / (NE + 2 * G));
    auto holds_units = [&](int ww) {
      return ww <= wl && (int64_t)ww * T / nw != (int64_t)(ww + 1) * T / nw;
    };
    float Mx[G], den[G], num[NE];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      Mx[h] = kNegInf;
      den[h] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < NE; ++k) num[k] = 0.0f;
    for (int c = wf; c <= wl; c += MB) {
      float ov[MB][NE], lv[MB][G], mv[MB][G];
#pragma unroll
      for (int u = 0; u < MB; ++u) {
        const bool ok = holds_units(c + u);
        const float* pp = a.o_part + ((int64_t)(ok ? c + u : wf) * 2 + (c + u == wf ? 1 : 0)) * SLOT;
#pragma unroll
        for (int k = 0; k < NE; ++k) ov[u][k] = ok ? load_agent(pp + lane + 64 * k) : 0.0f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          mv[u][h] = ok ? load_agent(pp + G * D + h) : kNegInf;
          lv[u][h] = ok ? load_agent(pp + G * D + G + h) : 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < MB; ++u) {
        float fo[G], fn[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float mn = fmaxf(Mx[h], mv[u][h]);
          fo[h] = Mx[h] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(Mx[h] - mn);
          fn[h] = mv[u][h] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mv[u][h] - mn);
          den[h] = den[h] * fo[h] + lv[u][h] * fn[h];
          Mx[h] = mn;
        }
#pragma unroll
        for (int k = 0; k < NE; ++k) num[k] = num[k] * fo[64 * k / D] + ov[u][k] * fn[64 * k / D];
      }
    }
#pragma unroll
    for (int k = 0; k < NE; ++k) {
      a.out[bh0 * D + lane + 64 * k] = num[k] / den[64 * k / D];
    }
  }
}

template <int D, int G, bool QF32, class C>
bool launch_sk(const SplitArgs& a, hipStream_t stream) {
  decode_sk_kernel<D, G, QF32, C><<<dim3((unsigned)a.period), dim3(kSkThreads), 0, stream>>>(a);
  return true;
}

template <int D, bool QF32, class C>
bool sk_by_group(int G, const SplitArgs& a, hipStream_t s) {
  switch (G) {
    case 1: return launch_sk<D, 1, QF32, C>(a, s);
    case 2: return launch_sk<D, 2, QF32, C>(a, s);
    case 4: return launch_sk<D, 4, QF32, C>(a, s);
    case 8: return launch_sk<D, 8, QF32, C>(a, s);
    default: return false;
  }
}

template <class C>
bool sk_by_dim(int head_dim, bool q_f32, int G, const SplitArgs& a, hipStream_t s) {
  if (head_dim == 128)
    return q_f32 ? sk_by_group<128, true, C>(G, a, s) : sk_by_group<128, false, C>(G, a, s);
  if constexpr (C::kBits != 4) {   // 4-bit codes: d = 128 only
    if (head_dim == 64)
      return q_f32 ? sk_by_group<64, true, C>(G, a, s) : sk_by_group<64, false, C>(G, a, s);
  }
  return false;
}

}  // namespace

int decode_sk_workgroups() {
  const int cus = device_cu_count();
  const int n = cus > 0 ? cus : 256;
  return n < kSkMaxWorkgroups ? n : kSkMaxWorkgroups;
}

bool launch_decode_sk(const SplitArgs& a, int head_dim, int G, bool q_f32, int fmt,
                      hipStream_t stream) {
  if (fmt == kFmtFp8) return sk_by_dim<CodesFp8>(head_dim, q_f32, G, a, stream);
  if (fmt == kFmtInt8) return sk_by_dim<CodesInt8>(head_dim, q_f32, G, a, stream);
  if (fmt == kFmtInt4) return sk_by_dim<CodesInt4>(head_dim, q_f32, G, a, stream);
  return false;
}

}  // namespace kv8
