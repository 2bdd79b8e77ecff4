// Internal launchers of libkv8: called by the C ABI layer (kv8_api.cpp)
// after host validation.  `fmt` selects the code format of the cache
// (kFmtInt8, kFmtFp8 = e4m3, kFmtInt4 = packed nibbles); caches are passed
// as bytes either way.  A non-null k_new/v_new makes launch_decode append
// each sequence's newest token (position context_lens[b] - 1) before
// attending.  Each returns 0 on success and -1 when the HIP runtime reports
// a launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kv8 {

enum : int { kFmtInt8 = 0, kFmtFp8 = 1, kFmtInt4 = 2 };

int launch_quant_append(const uint16_t* k_new, const uint16_t* v_new,
                        const int32_t* slot_mapping, int64_t n_tokens, int num_kv_heads,
                        int head_dim, int64_t num_blocks, int8_t* k_cache, int8_t* v_cache,
                        uint16_t* k_scale, uint16_t* v_scale, int fmt, hipStream_t stream);

int launch_rope_quant_append(const uint16_t* k_new, const uint16_t* v_new,
                             const int32_t* slot_mapping, const int32_t* positions,
                             const float* cos_sin, int max_position, int64_t n_tokens,
                             int num_kv_heads, int head_dim, int64_t num_blocks, int8_t* k_cache,
                             int8_t* v_cache, uint16_t* k_scale, uint16_t* v_scale,
                             hipStream_t stream);

// Which form of the INT8 / FP8 / INT4 decode kernel a call launches:
// automatic (by group size and size), the v_dot2 kernel, or the two-pass,
// one-pass or stream-K matrix-core kernel.  A per-call choice (the library
// keeps no setting).  decode_form: the form a launch of this code format,
// group size, grid bound (workgroups with every sequence at the longest
// context and 1024-token splits), longest context and head dim takes when
// `requested` is asked for.
enum : int {
  kDecodeKernelAuto = 0, kDecodeKernelDot = 1, kDecodeKernelMfma = 2, kDecodeKernelMfmaOnePass = 3,
  kDecodeKernelStreamK = 4
};

// The stream-K form launches one workgroup per compute unit (at most
// kSkMaxWorkgroups); its workspace holds two partial states per workgroup
// after the counters.  decode_sk_workgroups: the workgroups of a launch on
// the current device.
constexpr int kSkMaxWorkgroups = 1024;
int decode_sk_workgroups();
int decode_form(int requested, int fmt, int G, long long grid_bound, int max_context_len,
                int head_dim);

// The decode workspace starts with a fixed region of per-(sequence, KV
// head) split counters, one uint32 per pair at index b * Hkv + g, for up to
// kMaxDecodePairs pairs; the partial results follow it.  Because the
// counters never move with the shape, a workspace zero-filled once stays
// ready for every later call of any shape (the counters reset themselves).
constexpr int64_t kMaxDecodePairs = 65536;
constexpr size_t kCounterBytes = (size_t)kMaxDecodePairs * sizeof(unsigned);

// Fixed scratch of the allocation-free decode entry: its bytes, and this
// device's address of it (resolved once per device; on the first call the
// counter prefix is cleared by a kernel on `stream`).  nullptr on a HIP
// error.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
void* decode_scratch(hipStream_t stream);

struct DecodePlan {
  int form;              // kDecodeKernelDot / Mfma / MfmaOnePass / StreamK
  int split_tokens;      // tokens per workgroup (multiple of 64)
  int n_split;           // workgroups per (sequence, KV head)
  size_t counter_bytes;  // kCounterBytes: uint32 finished-split counters (self-resetting)
  size_t o_bytes;        // partial outputs  fp32 [B, Hq, n_split, d]
  size_t lse_bytes;      // partial log2-sum-exp fp32 [B, Hq, n_split]
  size_t total_bytes;
};

// Split plan shared by the workspace query and the launch.
bool plan_decode(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                 int max_context_len, int tokens_per_split, int form, DecodePlan* plan);

int launch_decode(const void* q, bool q_f32, const int8_t* k_cache, const int8_t* v_cache,
                  const uint16_t* k_scale, const uint16_t* v_scale, int64_t num_blocks,
                  const int32_t* block_table, int max_blocks_per_seq,
                  const int32_t* context_lens, int ctx_cap, int batch, int num_q_heads,
                  int num_kv_heads, int head_dim, float sm_scale, float* out,
                  void* workspace, const DecodePlan& plan, int fmt, const uint16_t* k_new,
                  const uint16_t* v_new, hipStream_t stream);

int launch_decode_bf16kv(const void* q, bool q_f32, const uint16_t* k_cache,
                         const uint16_t* v_cache, int64_t num_blocks,
                         const int32_t* block_table, int max_blocks_per_seq,
                         const int32_t* context_lens, int ctx_cap, int batch, int num_q_heads,
                         int num_kv_heads, int head_dim, float sm_scale, float* out,
                         void* workspace, const DecodePlan& plan, hipStream_t stream);

int launch_prefill(const uint16_t* q, const int32_t* q_start_loc, int64_t total_q, int max_q_len,
                   const int8_t* k_cache, const int8_t* v_cache, const uint16_t* k_scale,
                   const uint16_t* v_scale, int64_t num_blocks, const int32_t* block_table,
                   int max_blocks_per_seq, const int32_t* context_lens, int ctx_cap, int batch,
                   int num_q_heads, int num_kv_heads, int head_dim, float sm_scale, float* out,
                   int fmt, hipStream_t stream);

// The read-only kernels behind kv8_read_probe (tiles given: n_bytes /
// tile_bytes random tiles, streamed per wave) and kv8_stream_read (tiles
// null: contiguous n_bytes, a multiple of read_probe_chunk_bytes, in
// chunks), in kv8_probe.hip, on `workgroups` persistent workgroups.
int64_t read_probe_chunk_bytes();
int launch_read_probe(const void* buf, const int32_t* tiles, int tile_bytes, int64_t n_bytes,
                      int64_t workgroups, uint32_t* out, hipStream_t stream);

}  // namespace kv8
