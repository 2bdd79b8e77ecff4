// Decode machinery shared by the paged-attention decode kernels of libkv8
// (INT8, FP8, INT4 and bf16 caches) on gfx950: the work items and their
// order, the span of blocks a split covers, the cross-lane reductions, and
// the end of a split (partial results and the in-launch log-sum-exp merge).
// Nothing here is used outside the HIP library.
#pragma once

#include <atomic>

#include "kv8_device.h"

namespace kv8 {

constexpr int kMergeBatch = 8;

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

// Issue priority of a wave from the blocks (K and V passes together) it
// still has to stream: more work left, higher priority.  Without it the
// hardware issues the oldest wave of a CU first, so a CU's first workgroup
// races ahead and its last one ends the launch streaming alone at a
// fraction of the CU's share of bandwidth; largest-remaining-first makes the
// workgroups that share a CU finish closer together.  s_setprio takes an
// immediate, hence the branches (uniform over the wave).
__device__ __forceinline__ void priority_by_remaining(int remaining_blocks) {
  if (remaining_blocks > 24) __builtin_amdgcn_s_setprio(3);
  else if (remaining_blocks > 16) __builtin_amdgcn_s_setprio(2);
  else if (remaining_blocks > 8) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Arguments of the INT8 / FP8 / INT4 decode kernels (both the dot-product
// and the matrix-core form).
struct SplitArgs {
  const void* q;
  const int8_t* k_cache;
  const int8_t* v_cache;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  const uint16_t* k_new;   // bf16 [B, Hkv, D] newest token per sequence, or null
  const uint16_t* v_new;
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

// Decode step with append: the newest token of sequence b sits at position
// ctx - 1, inside the sequence's last split, so that split's workgroup
// quantises the token's K and V rows of KV head g (as the append kernel
// does) and stores them before its passes read the block back.  A block id
// outside [0, num_blocks) stores nothing, as the append kernel skips such a
// slot (the reads that follow clamp it, as every read does).  Called by one
// whole wave; the stores complete (vmcnt 0) before it returns, so every load
// the workgroup issues after its next barrier sees the new codes.
template <int D, class C>
__device__ __forceinline__ void append_newest(const SplitArgs& a, int b, int g, int ctx,
                                              int lane) {
  constexpr int LPR = D / 8;          // lanes per row, 8 values each
  const int p = ctx - 1;
  const int64_t id = a.block_table[(int64_t)b * a.max_blocks_per_seq + p / kBlock];
  if (lane < LPR && id >= 0 && id < a.num_blocks) {
    const int Hkv = a.num_kv_heads;
    const int64_t line = (id * Hkv + g) * kBlock + p % kBlock;
    const int64_t src = ((int64_t)b * Hkv + g) * D + lane * 8;
    float kx[8], vx[8], ka, va;
    unpack8(*reinterpret_cast<const uint4*>(a.k_new + src), kx, ka);
    unpack8(*reinterpret_cast<const uint4*>(a.v_new + src), vx, va);
    ka = row_absmax<LPR>(ka);
    va = row_absmax<LPR>(va);
    const float ks = fp16_scale<C>(ka), vs = fp16_scale<C>(va);
    *reinterpret_cast<uint2*>(const_cast<int8_t*>(a.k_cache) + line * D + lane * 8) =
        quantise8<C>(kx, ks);
    *reinterpret_cast<uint2*>(const_cast<int8_t*>(a.v_cache) + line * D + lane * 8) =
        quantise8<C>(vx, vs);
    if (lane == 0) {
      const_cast<uint16_t*>(a.k_scale)[line] = __builtin_bit_cast(uint16_t, (_Float16)ks);
      const_cast<uint16_t*>(a.v_scale)[line] = __builtin_bit_cast(uint16_t, (_Float16)vs);
    }
  }
  wait_vmem();
}

// Matrix-core forms of the INT8 / FP8 decode (kv8_decode_mfma.hip): launch
// the one-pass or the two-pass split kernel for head dim D in {64, 128},
// group size G in {1, 2, 4, 8} and the given code format; false for a shape
// they do not serve.  decode_mfma2_smem: LDS bytes of a two-pass workgroup.
bool launch_decode_mfma(const SplitArgs& a, int head_dim, int G, bool q_f32, int fmt,
                        bool one_pass, hipStream_t stream);
// Stream-K form (kv8_decode_sk.hip): a.period workgroups, a.o_part the
// per-workgroup partial states.
bool launch_decode_sk(const SplitArgs& a, int head_dim, int G, bool q_f32, int fmt,
                      hipStream_t stream);
int decode_mfma2_smem(int split_tokens, int G, int head_dim);

struct Item {
  int b;        // sequence, -1 past the last item
  int g;        // KV head
  int split;    // split of the sequence
  int nsplit;   // splits of the sequence
  int nbt;      // blocks of the sequence
};

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
//
// XCD grouping.  Workgroup i runs on XCD i mod 8, and one 128-byte line of
// a block's scales holds 4 KV heads' rows.  So the ranks of each window of
// 8 * Hkv are transposed (position 8a + x takes item Hkv * x + a): the Hkv
// heads of one (sequence, split), of equal size and Hkv-aligned in the
// order, share a rank residue mod 8, hence one XCD and its L2, and a scale
// line comes from HBM once instead of once per head.  A last, partial
// window keeps its order.
__device__ __forceinline__ int xcd_group_rank(int rank, int total, int num_kv_heads) {
  const int win = 8 * num_kv_heads;
  const int w0 = rank - rank % win;
  if (w0 + win > total) return rank;            // partial last window
  const int p = rank - w0;
  return w0 + num_kv_heads * (p % 8) + p / 8;
}

__device__ __forceinline__ Item locate_item(const int32_t* context_lens, int batch, int ctx_cap,
                                            int num_kv_heads, int split_tokens, int period,
                                            int snake_rounds, int lane) {
  const int bps = split_tokens / kBlock;        // blocks per split at most
  Item it{-1, 0, 0, 1, 0};
  if (batch <= 64 && period > 0) {
    int key = -1, cnt = 0, nb = 0, n = 1;
    if (lane < batch) {
      const int cx = min(max(context_lens[lane], 0), ctx_cap);
      nb = (cx + kBlock - 1) / kBlock;
      n = max(1, (nb + bps - 1) / bps);
      key = ((nb + n - 1) / n) * 64 + (63 - lane);  // unique; larger goes first
      cnt = n * num_kv_heads;
    }
    int start = 0, total = 0;
    for (int j = 0; j < batch; ++j) {
      const int kj = __builtin_amdgcn_readlane(key, j);
      const int cj = __builtin_amdgcn_readlane(cnt, j);
      start += kj > key ? cj : 0;
      total += cj;
    }
    const int bid = (int)blockIdx.x;
    const int r = bid / period;
    int rank = bid;
    if (r < snake_rounds) {
      const int c = bid - r * period;
      rank = r * period + ((r & 1) ? period - 1 - c : c);
    }
    if (rank < total) {
      rank = xcd_group_rank(rank, total, num_kv_heads);
      const uint64_t hit = __ballot(lane < batch && start <= rank && rank < start + cnt);
      it.b = (int)__builtin_ctzll(hit);
      const int j = rank - __builtin_amdgcn_readlane(start, it.b);
      it.split = j / num_kv_heads;
      it.g = j - it.split * num_kv_heads;
      it.nsplit = __builtin_amdgcn_readlane(n, it.b);
      it.nbt = __builtin_amdgcn_readlane(nb, it.b);
    }
  } else {
    // the grid covers every item (extra workgroups exit), so grouping over
    // the grid size is a bijection onto the items and the empty tail
    const int idx0 = xcd_group_rank((int)blockIdx.x, (int)gridDim.x, num_kv_heads);
    const int sg = idx0 / num_kv_heads;                 // global split index
    it.g = idx0 - sg * num_kv_heads;
    int base = 0;
    for (int c0 = 0; c0 < batch; c0 += 64) {
      const int bi = c0 + lane;
      int n = 0, nb = 0;
      if (bi < batch) {
        const int cx = min(max(context_lens[bi], 0), ctx_cap);
        nb = (cx + kBlock - 1) / kBlock;
        n = max(1, (nb + bps - 1) / bps);
      }
      const int incl = wave_incl_scan(n, lane);
      const int tot = __builtin_amdgcn_readlane(incl, 63);
      if (sg < base + tot) {
        const int idx = __builtin_popcountll(__ballot(base + incl <= sg));
        it.b = c0 + idx;
        it.nsplit = __builtin_amdgcn_readlane(n, idx);
        it.nbt = __builtin_amdgcn_readlane(nb, idx);
        it.split = sg - base - (__builtin_amdgcn_readlane(incl, idx) - it.nsplit);
        break;
      }
      base += tot;
    }
  }
  return it;
}

// Blocks [jb0, jb0 + nblk) and tokens [t0, t0 + ntok) of the sequence that
// split it.split covers (ctx > 0 tokens, it.nbt blocks shared evenly by
// it.nsplit splits; every split gets at least one block).
struct Span {
  int jb0, nblk, t0, ntok;
};
__device__ __forceinline__ Span split_span(const Item& it, int ctx) {
  const int bq = it.nbt / it.nsplit, brem = it.nbt - bq * it.nsplit;
  Span s;
  s.nblk = bq + (it.split < brem ? 1 : 0);
  s.jb0 = it.split * bq + min(it.split, brem);
  s.t0 = s.jb0 * kBlock;
  s.ntok = min(ctx - s.t0, s.nblk * kBlock);
  return s;
}

// Sum the per-lane accumulators acc[h * CPL + i] (head h, channel
// chunk * CPL + i) over the eight token groups of the wave and write the
// wave's [G][D] result to s_fin[wave].  A row step, then two reduce-scatter
// steps on the row/half swaps; lane l keeps M/4 sums: value k is
// accumulator k + (M/2)*(row of l is odd) + (M/4)*(l in upper half).
template <int G, int CPL, int D>
__device__ __forceinline__ void groups_to_lds(float (&acc)[G * CPL], float* s_fin, int wave,
                                              int lane, int chunk) {
  constexpr int M = G * CPL;
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
}

struct PartialArgs {
  float* out;          // [B, Hq, D]
  float* o_part;       // [B, Hq, n_split, D]
  float* lse_part;     // [B, Hq, n_split], log2 domain
  unsigned* counters;  // [B, Hkv], zero between calls
  int n_split;
};

// Finish one split of (sequence, KV head) bg whose query heads start at bh0:
// combine the kWaves per-wave results (s_fin [kWaves][G][D]; s_red holds per
// wave and head the max, then the weight sum), then write the output (a
// single split) or the split's partial; the last workgroup of bg to finish
// merges the partials of all nvalid splits by log-sum-exp.
template <int G, int D, int kThreads, int kWaves>
__device__ __forceinline__ void finish_split(const PartialArgs& a, const float* s_fin,
                                             const float* s_red, int* s_flag, int64_t bh0,
                                             int64_t bg, int split, int nvalid, int tid) {
  // ---- normalise; write the output or this split's partial ----------------
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, c = e % D;
    float s = s_fin[h * D + c];
    float Mh = s_red[h], Lh = s_red[kWaves * G + h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      s += s_fin[(w * G + h) * D + c];
      Mh = fmaxf(Mh, s_red[w * G + h]);
      Lh += s_red[kWaves * G + w * G + h];
    }
    const float o = s / Lh;
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
    unsigned* cnt = a.counters + bg;
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

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// Compute units of the current device (cached per device; 0 if unknown).
inline int device_cu_count() {
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


// Grid of a decode launch over `bound` possible items (every sequence at the
// longest context) and the item-order parameters: with at most 64
// sequences, the CU count as the round width and the workgroups resident
// per CU as the snake rounds (cached per shared-memory size), and the grid
// rounded up to whole rounds.  Otherwise period = snake_rounds = 0 and the
// grid is the bound.
template <auto Kernel>
int64_t item_grid(int threads, int smem, int batch, int64_t bound, int* period,
                  int* snake_rounds) {
  *period = 0;
  *snake_rounds = 0;
  if (batch > 64) return bound;
  // (shared-memory bytes << 32 | workgroups); 0 until first computed
  static std::atomic<uint64_t> occ_cache{0};
  uint64_t oc = occ_cache.load(std::memory_order_relaxed);
  if ((oc >> 32) != (uint64_t)smem) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, Kernel, threads, smem) != hipSuccess)
      v = 0;
    oc = ((uint64_t)smem << 32) | (uint32_t)(v > 0 ? v : 0);
    occ_cache.store(oc, std::memory_order_relaxed);
  }
  const int occ = (int)(uint32_t)oc;
  const int cus = device_cu_count();
  if (cus <= 0 || occ <= 0) return bound;
  *period = cus;
  *snake_rounds = occ;
  return (bound + cus - 1) / cus * cus;
}

}  // namespace kv8
