/*
 * kv8.h - C ABI of the paged INT8-KV GQA attention library (libkv8.so),
 * written for AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * The attention layer keeps its K/V cache as INT8 codes obtained by dynamic
 * per-token quantisation and restores them on demand inside attention
 * ("KV-Cache 全栈优化系统" README, section 主要特性, item on low-bit linear
 * and KV-cache compression).  Attention itself is softmax(Q K^T / sqrt(d)) V
 * ("KV Cache 优化全景解析——从基础原理到工程实践", section 2.1 equation),
 * grouped so that every group of G = Hq / Hkv query heads shares one KV head
 * (same page, section 3.3), and the cache is paged: a per-sequence block
 * table maps logical 16-token blocks to physical blocks (same page, section
 * 4.2 and the 16/32-token blocks of section 6.3).
 *
 * Quantiser (per token n, KV head h, separately for K and V; x is bf16[d]):
 *   a = max_i |x_i|;  s = fp16(fp32(a / 127)) rounded to nearest even with
 *   gradual underflow, saturated to 65504 on overflow;
 *   code_i = clamp(round_half_even(fp32(x_i / s)), -127, 127), or 0 if s == 0;
 *   the restored value is code_i * s.
 *
 * Memory layout (all device memory, caller-owned)
 * ------------------------------------------------
 *   k_cache, v_cache : int8   [num_blocks, Hkv, 16, d]   codes of one
 *                      (block, head) are 16*d contiguous bytes
 *   k_scale, v_scale : uint16 [num_blocks, Hkv, 16]      fp16 bit patterns
 *   block_table      : int32  [B, max_blocks_per_seq]    physical block ids
 *   context_lens     : int32  [B]                        tokens to attend,
 *                      including any token just appended
 *   slot_mapping     : int32  [N]   physical slot = block * 16 + offset;
 *                      a negative slot skips the token
 *   bf16 / fp16 values are passed as their 16-bit patterns (uint16_t).
 * Query head hq reads KV head hq / G.  Logical token t of sequence b lives
 * in block block_table[b][t / 16] at offset t % 16.
 *
 * Conventions
 * -----------
 * - Ownership: the caller allocates every buffer, including the workspace;
 *   the library allocates nothing.  It keeps no setting between calls: what
 *   it does hold (the allocation-free decode's fixed scratch, cached device
 *   properties) never changes what a call computes.
 * - Ordering: each call validates its host arguments, enqueues its kernels
 *   on `stream` (a hipStream_t; NULL = the default stream) and returns
 *   without synchronising.
 * - Errors: every call returns a kv8_status.  Host validation runs before
 *   any HIP call and rejects null pointers, bad sizes, unsupported shapes,
 *   misaligned pointers and short workspaces; nothing is launched then.  A
 *   failed launch returns KV8_ERR_HIP.  No exception crosses the ABI and
 *   the library never aborts.
 * - Device data is not validated on the host.  Physical block ids outside
 *   [0, num_blocks) are clamped into range, so they never fault but give an
 *   undefined result.  context_lens values are clamped to
 *   [0, min(max_context_len, 16 * max_blocks_per_seq)].  Non-finite K/V/Q
 *   values give undefined results.  Slots at or beyond a sequence's context
 *   length are never read into a result, whatever they hold.
 * - Alignment: cache, scale, q, k_new/v_new and out base pointers must be
 *   16-byte aligned.
 * - Supported shapes: block_size == 16, d in {64, 128},
 *   G = Hq / Hkv in {1, 2, 4, 8}.
 */
#ifndef KV8_H
#define KV8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kv8_status {
  KV8_OK = 0,
  KV8_ERR_NULL = -1,        /* a required pointer is NULL                  */
  KV8_ERR_SHAPE = -2,       /* a size is negative, zero where it must not
                               be, or inconsistent (Hq % Hkv != 0, ...)    */
  KV8_ERR_UNSUPPORTED = -3, /* block_size != 16, d not in {64,128}, G not
                               in {1,2,4,8}, unknown dtype                  */
  KV8_ERR_ALIGN = -4,       /* a base pointer is not 16-byte aligned       */
  KV8_ERR_WORKSPACE = -5,   /* workspace missing or too small              */
  KV8_ERR_HIP = -6          /* the HIP runtime reported a launch error     */
} kv8_status;

typedef enum kv8_dtype {
  KV8_F32 = 0,              /* IEEE binary32                               */
  KV8_BF16 = 1              /* bfloat16 bit patterns in uint16_t           */
} kv8_dtype;

#define KV8_BLOCK_SIZE 16

/* Human-readable name of a kv8_status value (static string, never NULL). */
const char* kv8_status_string(int status);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int kv8_version(void);

/*
 * Decode kernel forms: the `kernel_form` argument of paged_decode_attn_kv8,
 * paged_decode_attn_kv8_append, paged_decode_attn_fp8kv and
 * paged_decode_attn_int4kv chooses, for that call only, which kernel runs:
 *   KV8_DECODE_AUTO (0): by group size G = Hq / Hkv and size (v_dot2 below
 *     G = 4; from G = 4 two-pass matrix-core for 2048 < max_context_len <=
 *     8192 with a grid bound, every sequence at max_context_len in
 *     1024-token splits, of at most 1024 workgroups, else stream-K; for the
 *     INT4 cache one-pass from G = 4 at d = 128, else v_dot2);
 *   KV8_DECODE_DOT (1): the v_dot2 kernel;
 *   KV8_DECODE_MFMA (2): the two-pass matrix-core kernel (logits of the
 *     split to LDS, then the weighted values; logits and values as 16x16
 *     MFMA tiles over all G heads of a group at once);
 *   KV8_DECODE_MFMA_ONEPASS (3): the one-pass matrix-core kernel (online
 *     softmax over K and V tiles streamed together, weights kept in
 *     registers);
 *   KV8_DECODE_STREAMK (4): the stream-K matrix-core kernel: the
 *     (sequence, KV head, block) units of the whole batch cut into equal
 *     contiguous ranges, one per compute unit and within it one per wave,
 *     each streamed with the one-pass arithmetic; pieces of one (sequence,
 *     KV head) are merged by log-sum-exp in LDS and, across workgroups,
 *     through the workspace in the same launch.  tokens_per_split does not
 *     apply to it (any valid value is accepted), and its output for a
 *     reordered batch agrees with the reordered output within the
 *     attention tolerance, not bitwise (the cuts move with the order).
 * The INT4 cache at d = 64 always runs the v_dot2 kernel.  All forms
 * compute the same attention (the same work items and in-launch merge);
 * results agree within the attention tolerance, not bitwise.  The form can
 * change the default split size, hence the workspace a call needs;
 * kv8_decode_workspace_size returns enough for every form.  Another value
 * returns KV8_ERR_UNSUPPORTED.  The library keeps no setting: two calls
 * with the same arguments run the same kernel.
 *
 * Split sizes.  tokens_per_split > 0 must be a multiple of 64 in
 * [64, 2048].  The v_dot2 and two-pass forms hold a split's logits in LDS,
 * so at G = 8 they accept at most 1280 tokens per split (a larger value
 * returns KV8_ERR_UNSUPPORTED); the one-pass form accepts every value.
 */
#define KV8_DECODE_AUTO 0
#define KV8_DECODE_DOT 1
#define KV8_DECODE_MFMA 2
#define KV8_DECODE_MFMA_ONEPASS 3
#define KV8_DECODE_STREAMK 4

/* Most (sequence, KV head) pairs, batch * num_kv_heads, of one decode
 * call; more returns KV8_ERR_SHAPE. */
#define KV8_DECODE_MAX_PAIRS 65536

/*
 * kv8_quant_append - quantise N new tokens' K and V and scatter them into
 * the paged cache (the quantise-on-write half of the KV8 method: "KV-Cache
 * 全栈优化系统" README, section 主要特性; slot addressing per the block
 * table of "KV Cache 优化全景解析", section 4.2).
 *
 *   k_new, v_new   device bf16 [n_tokens, num_kv_heads, head_dim]
 *   slot_mapping   device int32 [n_tokens]; slot = block*16 + offset;
 *                  slot < 0 or slot >= 16*num_blocks skips the token
 *   k_cache/v_cache/k_scale/v_scale  the cache (layout above); for every
 *                  kept token n and head h the 16-byte-aligned code row and
 *                  the fp16 scale of (slot, h) are overwritten
 *   stream         hipStream_t
 * Two tokens mapping to the same slot race (undefined which one wins).
 * n_tokens == 0 is a no-op returning KV8_OK.  KV8_ERR_SHAPE for a negative
 * n_tokens, num_kv_heads <= 0, or n_tokens * num_kv_heads >= 2^31 rows in
 * one call (more than 500 GB of bf16 K/V; split such a call).
 */
int kv8_quant_append(const uint16_t* k_new, const uint16_t* v_new,
                     const int32_t* slot_mapping, int64_t n_tokens,
                     int num_kv_heads, int head_dim, int block_size,
                     int64_t num_blocks,
                     int8_t* k_cache, int8_t* v_cache,
                     uint16_t* k_scale, uint16_t* v_scale,
                     void* stream);

/*
 * kv8_rope_quant_append - kv8_quant_append with the rotary position
 * embedding of K fused in front of the quantiser: K goes into the cache
 * after RoPE, then quantised, as on the cache-operator plane of the
 * "KV-Cache 全栈优化系统" README (section 系统架构概览).  Rotate-half
 * convention over the whole head: for j < d/2, with c = cos_sin[pos][j] and
 * s = cos_sin[pos][d/2 + j],
 *   k'_j = k_j c - k_{j+d/2} s,   k'_{j+d/2} = k_{j+d/2} c + k_j s,
 * each product and sum rounded to fp32; the rotated fp32 row is quantised
 * exactly as kv8_quant_append quantises a row.  V is appended unrotated.
 *
 *   k_new         device bf16 [n_tokens, Hkv, d], K before RoPE
 *   positions     device int32 [n_tokens], the token positions; values
 *                 outside [0, max_position) are clamped into it
 *   cos_sin       device fp32 [max_position, d], 16-byte aligned: row p
 *                 holds cos(p * theta_j) for j < d/2, then sin(p * theta_j)
 *   all other arguments as for kv8_quant_append
 * Returns KV8_OK, KV8_ERR_NULL, KV8_ERR_SHAPE (max_position <= 0 with
 * tokens to append), KV8_ERR_UNSUPPORTED, KV8_ERR_ALIGN or KV8_ERR_HIP.
 */
int kv8_rope_quant_append(const uint16_t* k_new, const uint16_t* v_new,
                          const int32_t* slot_mapping, const int32_t* positions,
                          const float* cos_sin, int max_position, int64_t n_tokens,
                          int num_kv_heads, int head_dim, int block_size,
                          int64_t num_blocks,
                          int8_t* k_cache, int8_t* v_cache,
                          uint16_t* k_scale, uint16_t* v_scale,
                          void* stream);

/*
 * kv8_decode_workspace_size - bytes of workspace paged_decode_attn_kv8
 * needs for these sizes, under any kernel form.  tokens_per_split: most
 * tokens one workgroup covers (a multiple of 64 in [64, 2048]), or <= 0 for
 * the library's choice, which depends on batch, num_kv_heads and
 * max_context_len only.  Returns 0 for invalid sizes (including
 * batch * num_kv_heads > KV8_DECODE_MAX_PAIRS).
 *
 * Workspace layout: the first 4 * KV8_DECODE_MAX_PAIRS bytes hold one
 * uint32 finished-split counter per (sequence b, KV head g), at index
 * b * num_kv_heads + g, whatever the call's shape; the partial results of
 * the splits follow.  Each call returns every counter it used to zero, so
 * a workspace zero-filled once is ready for every later call of any shape.
 */
size_t kv8_decode_workspace_size(int batch, int num_q_heads, int num_kv_heads,
                                 int head_dim, int max_context_len,
                                 int tokens_per_split);

/*
 * paged_decode_attn_kv8 - one query token per sequence attends to its
 * whole paged INT8 context (decode).  For every sequence b and query head
 * hq:  out[b,hq] = sum_t softmax_t(<q[b,hq], k_hat[b,g,t]> * sm_scale)
 * v_hat[b,g,t], t = 0 .. ctx_b - 1, g = hq / G, k_hat/v_hat the restored
 * codes ("KV Cache 优化全景解析", sections 2.1 and 3.3; dequantisation on
 * the fly per the KV8 item of the "KV-Cache 全栈优化系统" README).  The
 * softmax and all accumulation run in fp32 ("大模型推理加速：KV Cache与vLLM
 * 技术解析", section 4.1).  Split-K: a sequence's blocks are shared evenly
 * by ceil(ctx_b / tokens_per_split) splits; each workgroup covers one split
 * of one (sequence, KV head) for all G query heads, and the last workgroup
 * of each (sequence, KV head) to finish merges the partial results by
 * log-sum-exp inside the same launch.  Workgroups take the (sequence,
 * split, KV head) items that hold tokens, longest first (up to 64
 * sequences) or in sequence order, so the work spreads evenly over the CUs
 * whatever the mix of context lengths.
 *
 *   q             device [B, Hq, d], dtype q_dtype (KV8_F32 or KV8_BF16)
 *   block_table   device int32 [B, max_blocks_per_seq]
 *   context_lens  device int32 [B]; ctx_b == 0 gives out[b] = 0
 *   max_context_len  host-side upper bound of context_lens (sizes the
 *                 split grid; larger device values are clamped to it)
 *   sm_scale      softmax scale, normally 1/sqrt(d)
 *   out           device fp32 [B, Hq, d]
 *   workspace     device scratch of at least kv8_decode_workspace_size()
 *                 bytes (16-byte aligned).  It must be zero-filled once
 *                 before its first use; every completed call leaves it
 *                 ready for the next call of any shape (layout above).
 *                 Calls sharing one workspace must not overlap in time
 *                 (use one stream, or one workspace per stream).
 *   tokens_per_split  as for kv8_decode_workspace_size (same value!); the
 *                 per-form limits are listed with the kernel forms above
 *   kernel_form   KV8_DECODE_AUTO or a kernel form (see above)
 * Same inputs, tokens_per_split and kernel_form give bitwise-identical
 * output.  batch * num_kv_heads > KV8_DECODE_MAX_PAIRS returns
 * KV8_ERR_SHAPE.
 */
int paged_decode_attn_kv8(const void* q, int q_dtype,
                          const int8_t* k_cache, const int8_t* v_cache,
                          const uint16_t* k_scale, const uint16_t* v_scale,
                          int64_t num_blocks,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* context_lens, int max_context_len,
                          int batch, int num_q_heads, int num_kv_heads,
                          int head_dim, int block_size, float sm_scale,
                          float* out, void* workspace, size_t workspace_bytes,
                          int tokens_per_split, int kernel_form, void* stream);

/*
 * paged_decode_attn_kv8_noalloc - paged_decode_attn_kv8 for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same computation,
 * kernels and results (bitwise those of paged_decode_attn_kv8 with the
 * same tokens_per_split and kernel_form), with no workspace argument.  The
 * split counters and partial results live in a fixed scratch array of
 * KV8_DECODE_NOALLOC_SCRATCH_BYTES that the library holds on every device
 * it runs on until the process ends; the call allocates and frees nothing.
 * The first call on a device resolves that device's scratch address and
 * clears its counters with a kernel on `stream`.
 *   arguments     as for paged_decode_attn_kv8, without workspace and
 *                 workspace_bytes
 * Returns as paged_decode_attn_kv8, and KV8_ERR_WORKSPACE when the call
 * needs more than KV8_DECODE_NOALLOC_SCRATCH_BYTES (the size
 * kv8_decode_workspace_size reports for the same sizes, tokens_per_split
 * and kernel form), before any HIP call.  Every call on a device shares
 * that device's scratch: calls that overlap in time on one device (several
 * streams or host threads) race and give undefined results.
 */
#define KV8_DECODE_NOALLOC_SCRATCH_BYTES 33554432
int paged_decode_attn_kv8_noalloc(const void* q, int q_dtype,
                                  const int8_t* k_cache, const int8_t* v_cache,
                                  const uint16_t* k_scale, const uint16_t* v_scale,
                                  int64_t num_blocks,
                                  const int32_t* block_table, int max_blocks_per_seq,
                                  const int32_t* context_lens, int max_context_len,
                                  int batch, int num_q_heads, int num_kv_heads,
                                  int head_dim, int block_size, float sm_scale,
                                  float* out, int tokens_per_split, int kernel_form,
                                  void* stream);

/*
 * paged_decode_attn_kv8_append - one decode step in one launch: append the
 * newest token of every sequence, then paged_decode_attn_kv8.  The result
 * (cache contents and output) is that of kv8_quant_append on the new
 * tokens followed by paged_decode_attn_kv8 ("KV-Cache 全栈优化系统" README,
 * section 主要特性: K/V quantised as they are written, restored inside
 * attention).  The token of sequence b goes to position context_lens[b] - 1
 * (context_lens already count it; values above max_context_len are clamped
 * first, as in paged_decode_attn_kv8), i.e. to slot
 * block_table[b][p / 16] * 16 + p % 16; sequences with an empty context
 * append nothing, and a block id outside [0, num_blocks) stores nothing
 * (as kv8_quant_append skips such a slot).  The workgroup that attends over a sequence's last split
 * quantises the row and stores it before reading it back, so no separate
 * append kernel and no grid-wide synchronisation is needed.
 *
 *   k_new, v_new  device bf16 [B, Hkv, d], 16-byte aligned
 *   k_cache, v_cache, k_scale, v_scale  as for kv8_quant_append (written)
 *   all other arguments as for paged_decode_attn_kv8
 * Returns as paged_decode_attn_kv8, and KV8_ERR_NULL / KV8_ERR_ALIGN for
 * k_new or v_new.
 */
int paged_decode_attn_kv8_append(const void* q, int q_dtype,
                                 const uint16_t* k_new, const uint16_t* v_new,
                                 int8_t* k_cache, int8_t* v_cache,
                                 uint16_t* k_scale, uint16_t* v_scale,
                                 int64_t num_blocks,
                                 const int32_t* block_table, int max_blocks_per_seq,
                                 const int32_t* context_lens, int max_context_len,
                                 int batch, int num_q_heads, int num_kv_heads,
                                 int head_dim, int block_size, float sm_scale,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 int tokens_per_split, int kernel_form, void* stream);

/*
 * paged_decode_attn_bf16kv - the same decode attention over a paged cache
 * that holds K and V unquantised, as bf16: the 16-bit reference point that
 * the KV8 method is compared with at an equal memory budget ("KV-Cache
 * 全栈优化系统" README, section 实验效果（摘要）, which compares KV8
 * attention with FlashAttention-2 over the unquantised cache).  For every
 * sequence b and query head hq:  out[b,hq] = sum_t softmax_t(<q[b,hq],
 * k[b,g,t]> * sm_scale) v[b,g,t], g = hq / G ("KV Cache 优化全景解析",
 * sections 2.1, 3.3 and 4.2), softmax and accumulation in fp32.  Same
 * split-K scheme, item order and in-launch merge as paged_decode_attn_kv8.
 *
 *   k_cache, v_cache  device bf16 bit patterns [num_blocks, Hkv, 16, d]
 *   all other arguments as for paged_decode_attn_kv8 (there is one kernel
 *   form, so no kernel_form argument); the workspace is sized by
 *   kv8_decode_workspace_size() with the same sizes and tokens_per_split,
 *   zero-filled once, and may be shared with paged_decode_attn_kv8 calls
 *   that do not overlap in time.
 * Slots past a sequence's context are never used, whatever they hold.
 * Returns KV8_OK or a negative kv8_status as paged_decode_attn_kv8 does.
 */
int paged_decode_attn_bf16kv(const void* q, int q_dtype,
                             const uint16_t* k_cache, const uint16_t* v_cache,
                             int64_t num_blocks,
                             const int32_t* block_table, int max_blocks_per_seq,
                             const int32_t* context_lens, int max_context_len,
                             int batch, int num_q_heads, int num_kv_heads,
                             int head_dim, int block_size, float sm_scale,
                             float* out, void* workspace, size_t workspace_bytes,
                             int tokens_per_split, void* stream);

/*
 * paged_prefill_chunk_attn_kv8 - causal attention of a chunk of query rows
 * per sequence over the paged INT8 cache that already holds the chunk's own
 * K/V (append first with kv8_quant_append).  Chunked prefill as in the
 * vLLM chunked-prefill option ("KV Cache 优化全景解析", section 11.2) with
 * the attention of section 2.1 and the KV8 cache of the "KV-Cache 全栈优化
 * 系统" README.  Row i of sequence b's chunk (Lc_b = q_start_loc[b+1] -
 * q_start_loc[b] rows) sits at absolute position p = ctx_b - Lc_b + i and
 * attends to keys 0 .. p inclusive.  QK^T and PV run on the matrix cores.
 *
 *   q             device bf16 [total_q, Hq, d]
 *   q_start_loc   device int32 [B + 1], q_start_loc[0] == 0, non-decreasing,
 *                 q_start_loc[B] == total_q
 *   max_q_len     host-side upper bound of every Lc_b (sizes the grid)
 *   context_lens  device int32 [B], counts the chunk's tokens too; must be
 *                 >= Lc_b (rows of a sequence violating this are undefined)
 *   out           device fp32 [total_q, Hq, d]
 *   workspace     may be NULL when kv8_prefill_workspace_size() returns 0,
 *                 which it does for every shape: the prefill kernels keep
 *                 all their state on chip.  The argument stays in the ABI so
 *                 that a kernel needing one can be added without changing
 *                 the signature.
 */
size_t kv8_prefill_workspace_size(int batch, int num_q_heads, int head_dim,
                                  int max_q_len, int max_context_len);

int paged_prefill_chunk_attn_kv8(const uint16_t* q, const int32_t* q_start_loc,
                                 int64_t total_q, int max_q_len,
                                 const int8_t* k_cache, const int8_t* v_cache,
                                 const uint16_t* k_scale, const uint16_t* v_scale,
                                 int64_t num_blocks,
                                 const int32_t* block_table, int max_blocks_per_seq,
                                 const int32_t* context_lens, int max_context_len,
                                 int batch, int num_q_heads, int num_kv_heads,
                                 int head_dim, int block_size, float sm_scale,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * FP8 (e4m3) cache.  The KV cache kept as FP8 e4m3 with quantisation
 * scales ("KV Cache 优化全景解析", section 7.4; about half the bytes of a
 * 16-bit cache, section 11.3).  Same layout as the INT8 cache: one byte per
 * element, codes [num_blocks, Hkv, 16, d] and one fp16 scale per (token
 * slot, KV head) for K and for V.  Codes are OCP e4m3 (bias 7, subnormals,
 * largest finite 448, no infinity):
 *   s    = fp16_rne(fp32_rne(absmax / 448)), saturated to 65504;
 *   code = e4m3 round-to-nearest-even of the fp32 quotient x / s, saturated
 *          to +-448 (never NaN), the sign of a zero kept; all-zero codes
 *          when s == 0;
 *   x_hat = e4m3 value(code) * s.
 * kv8_quant_append_fp8, paged_decode_attn_fp8kv and
 * paged_prefill_chunk_attn_fp8kv take the same arguments, with the same
 * meaning, ownership and errors, as their INT8 counterparts above (the
 * decode workspace is sized by kv8_decode_workspace_size); only the code
 * format of the cache differs.
 */
int kv8_quant_append_fp8(const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* slot_mapping, int64_t n_tokens,
                         int num_kv_heads, int head_dim, int block_size,
                         int64_t num_blocks,
                         uint8_t* k_cache, uint8_t* v_cache,
                         uint16_t* k_scale, uint16_t* v_scale,
                         void* stream);

int paged_decode_attn_fp8kv(const void* q, int q_dtype,
                            const uint8_t* k_cache, const uint8_t* v_cache,
                            const uint16_t* k_scale, const uint16_t* v_scale,
                            int64_t num_blocks,
                            const int32_t* block_table, int max_blocks_per_seq,
                            const int32_t* context_lens, int max_context_len,
                            int batch, int num_q_heads, int num_kv_heads,
                            int head_dim, int block_size, float sm_scale,
                            float* out, void* workspace, size_t workspace_bytes,
                            int tokens_per_split, int kernel_form, void* stream);

int paged_prefill_chunk_attn_fp8kv(const uint16_t* q, const int32_t* q_start_loc,
                                   int64_t total_q, int max_q_len,
                                   const uint8_t* k_cache, const uint8_t* v_cache,
                                   const uint16_t* k_scale, const uint16_t* v_scale,
                                   int64_t num_blocks,
                                   const int32_t* block_table, int max_blocks_per_seq,
                                   const int32_t* context_lens, int max_context_len,
                                   int batch, int num_q_heads, int num_kv_heads,
                                   int head_dim, int block_size, float sm_scale,
                                   float* out, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * INT4 cache.  "KV Cache 优化全景解析" counts INT4 at 0.5 byte per element in
 * its KV-size formula (section 2.3), and the KV-cache optimisation page of
 * garden.houmin.site (section 2.2.2) lists compressing the cache from FP16
 * to INT8 or INT4.  Same recipe as INT8 with 7 in place of 127:
 *   s    = fp16_rne(fp32_rne(absmax / 7)), saturated to 65504;
 *   code = clamp(round_half_even(fp32(x / s)), -7, 7); all zero if s == 0;
 *   x_hat = code * s.
 * Two codes per byte as 4-bit two's complement, element 2i in the low
 * nibble of byte i: codes [num_blocks, Hkv, 16, d/2] bytes; one fp16 scale
 * per (token slot, KV head) for K and for V as in the INT8 cache.
 * kv8_quant_append_int4, paged_decode_attn_int4kv and
 * paged_prefill_chunk_attn_int4kv take the same arguments, with the same
 * meaning, ownership and errors, as kv8_quant_append, paged_decode_attn_kv8
 * and paged_prefill_chunk_attn_kv8 (the decode workspace is sized by
 * kv8_decode_workspace_size).
 */
int kv8_quant_append_int4(const uint16_t* k_new, const uint16_t* v_new,
                          const int32_t* slot_mapping, int64_t n_tokens,
                          int num_kv_heads, int head_dim, int block_size,
                          int64_t num_blocks,
                          uint8_t* k_cache, uint8_t* v_cache,
                          uint16_t* k_scale, uint16_t* v_scale,
                          void* stream);

int paged_decode_attn_int4kv(const void* q, int q_dtype,
                             const uint8_t* k_cache, const uint8_t* v_cache,
                             const uint16_t* k_scale, const uint16_t* v_scale,
                             int64_t num_blocks,
                             const int32_t* block_table, int max_blocks_per_seq,
                             const int32_t* context_lens, int max_context_len,
                             int batch, int num_q_heads, int num_kv_heads,
                             int head_dim, int block_size, float sm_scale,
                             float* out, void* workspace, size_t workspace_bytes,
                             int tokens_per_split, int kernel_form, void* stream);

int paged_prefill_chunk_attn_int4kv(const uint16_t* q, const int32_t* q_start_loc,
                                    int64_t total_q, int max_q_len,
                                    const uint8_t* k_cache, const uint8_t* v_cache,
                                    const uint16_t* k_scale, const uint16_t* v_scale,
                                    int64_t num_blocks,
                                    const int32_t* block_table, int max_blocks_per_seq,
                                    const int32_t* context_lens, int max_context_len,
                                    int batch, int num_q_heads, int num_kv_heads,
                                    int head_dim, int block_size, float sm_scale,
                                    float* out, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * Read ceilings - measurement utilities, not part of the attention method:
 * HBM read rates of this device against which the decode kernels' achieved
 * bandwidth is reported (the memory-bound decode argument of the
 * garden.houmin.site KV-cache optimisation page, section 1.3).  Both are
 * read-only, persistent (`workgroups` workgroups of 256 threads; a few per
 * compute unit, e.g. 4 x 256 on MI355X, give the highest rate) and write
 * one xor per thread of the 16-byte units the thread read to `out` (device
 * uint32 [workgroups * 256]).  Make buf far larger than the last-level
 * cache.  Both return KV8_OK, KV8_ERR_NULL, KV8_ERR_SHAPE (sizes out of
 * range), KV8_ERR_ALIGN (buf not 16-byte aligned) or KV8_ERR_HIP,
 * asynchronously on `stream`.
 *
 * kv8_stream_read - plain streaming read of n_bytes (a positive multiple
 *   of kv8_read_probe_chunk_bytes(), 32 KB): workgroup w reads chunks w,
 *   w + workgroups, ... (chunk c is bytes [c * chunk, (c + 1) * chunk) of
 *   buf) with nontemporal 16-byte loads, 8 per lane in flight; thread t of
 *   a workgroup reads units t, t + 256, ... of each of its chunks.
 * kv8_read_probe - the access pattern of the paged decode: n_bytes / tile_bytes
 *   random tiles, tile i being bytes [tiles[i] * tile_bytes, (tiles[i] + 1) *
 *   tile_bytes) of buf.  tiles: device int32 [n_bytes / tile_bytes], each in
 *   [0, n_tiles) for a buf of n_tiles * tile_bytes bytes (not checked on the
 *   device: an index outside the buffer is undefined); tile_bytes a multiple
 *   of 1024 up to 32768; n_bytes a positive multiple of tile_bytes.  Wave v
 *   (v = 4 * workgroup + wave) of the nw = 4 * workgroups waves reads tiles
 *   v, v + nw, v + 2 nw, ... in order as 1 KB rows, lane l reading unit l of
 *   each row, 4 rows in flight, ordinary loads.
 */
int64_t kv8_read_probe_chunk_bytes(void);
int kv8_stream_read(const void* buf, int64_t n_bytes, int64_t workgroups, uint32_t* out,
                    void* stream);
int kv8_read_probe(const void* buf, const int32_t* tiles, int tile_bytes, int64_t n_bytes,
                   int64_t workgroups, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KV8_H */
