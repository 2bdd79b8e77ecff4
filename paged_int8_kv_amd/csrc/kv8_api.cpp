// C ABI of libkv8 (declared in include/kv8.h): host-side validation, split
// planning and launch.  Validation runs before any HIP call, so a bad
// argument returns an error code without touching the device.
#include "kv8.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kv8_launch.h"

static_assert(kv8::kDecodeScratchBytes == KV8_DECODE_NOALLOC_SCRATCH_BYTES,
              "the header states the allocation-free decode's scratch size");

namespace {

constexpr int kVersion = 200;   // 0.2.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_dim(int d) { return d == 64 || d == 128; }

bool supported_group(int hq, int hkv) {
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return false;
  const int g = hq / hkv;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

int check_cache(const int8_t* kc, const int8_t* vc, const uint16_t* ks, const uint16_t* vs,
                int64_t num_blocks, int block_size) {
  if (!kc || !vc || !ks || !vs) return KV8_ERR_NULL;
  if (num_blocks <= 0) return KV8_ERR_SHAPE;
  if (block_size != KV8_BLOCK_SIZE) return KV8_ERR_UNSUPPORTED;
  if (!aligned16(kc) || !aligned16(vc) || !aligned16(ks) || !aligned16(vs)) return KV8_ERR_ALIGN;
  return KV8_OK;
}

int append_impl(const uint16_t* k_new, const uint16_t* v_new, const int32_t* slot_mapping,
                 int64_t n_tokens, int num_kv_heads,
                     int head_dim, int block_size, int64_t num_blocks, int8_t* k_cache,
                     int8_t* v_cache, uint16_t* k_scale, uint16_t* v_scale, int fmt, void* stream) {
  if (n_tokens < 0 || num_kv_heads <= 0) return KV8_ERR_SHAPE;
  if (!supported_dim(head_dim)) return KV8_ERR_UNSUPPORTED;
  const int rc = check_cache(k_cache, v_cache, k_scale, v_scale, num_blocks, block_size);
  if (rc != KV8_OK) return rc;
  if (n_tokens == 0) return KV8_OK;
  if (!k_new || !v_new || !slot_mapping) return KV8_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return KV8_ERR_ALIGN;
  if (n_tokens * num_kv_heads >= (int64_t)0x7FFFFFFF) return KV8_ERR_SHAPE;   // rows fit 31 bits
  const int r = kv8::launch_quant_append(k_new, v_new, slot_mapping, n_tokens, num_kv_heads,
                                         head_dim, num_blocks, k_cache, v_cache, k_scale,
                                         v_scale, fmt, static_cast<hipStream_t>(stream));
  return r == 0 ? KV8_OK : KV8_ERR_HIP;
}

int decode_impl(const void* q, int q_dtype, const int8_t* k_cache,
                          const int8_t* v_cache, const uint16_t* k_scale,
                          const uint16_t* v_scale, int64_t num_blocks,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* context_lens, int max_context_len, int batch,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                          int tokens_per_split, int kernel_form, int fmt, const uint16_t* k_new,
                          const uint16_t* v_new, void* stream, bool use_scratch = false) {
  if (!q || !block_table || !context_lens || !out) return KV8_ERR_NULL;
  const int rc = check_cache(k_cache, v_cache, k_scale, v_scale, num_blocks, block_size);
  if (rc != KV8_OK) return rc;
  if (batch <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0) return KV8_ERR_SHAPE;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return KV8_ERR_SHAPE;
  if (batch > 65535 || num_kv_heads > 65535) return KV8_ERR_SHAPE;
  if ((int64_t)batch * num_kv_heads > kv8::kMaxDecodePairs) return KV8_ERR_SHAPE;
  if (q_dtype != KV8_F32 && q_dtype != KV8_BF16) return KV8_ERR_UNSUPPORTED;
  if (!supported_dim(head_dim) || !supported_group(num_q_heads, num_kv_heads))
    return KV8_ERR_UNSUPPORTED;
  if (kernel_form < KV8_DECODE_AUTO || kernel_form > KV8_DECODE_STREAMK)
    return KV8_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(out)) return KV8_ERR_ALIGN;
  if (tokens_per_split > 0 && (tokens_per_split % 64 != 0 || tokens_per_split > 2048))
    return KV8_ERR_UNSUPPORTED;
  kv8::DecodePlan plan;
  if (!kv8::plan_decode(batch, num_q_heads, num_kv_heads, head_dim, max_context_len,
                        tokens_per_split,
                        kv8::decode_form(kernel_form, fmt, num_q_heads / num_kv_heads,
                                         (long long)batch * num_kv_heads *
                                             ((max_context_len + 1023) / 1024),
                                         max_context_len, head_dim),
                        &plan))
    return KV8_ERR_UNSUPPORTED;
  if (use_scratch) {
    // allocation-free entry: the library's fixed scratch stands in for the
    // workspace; a call that needs more is rejected before any HIP call
    if (plan.total_bytes > kv8::kDecodeScratchBytes) return KV8_ERR_WORKSPACE;
    workspace = kv8::decode_scratch(static_cast<hipStream_t>(stream));
    if (!workspace) return KV8_ERR_HIP;
  } else {
    if (!workspace || workspace_bytes < plan.total_bytes) return KV8_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KV8_ERR_ALIGN;
  }
  const long long cap_blocks = (long long)max_blocks_per_seq * KV8_BLOCK_SIZE;
  const int ctx_cap = (int)(cap_blocks < max_context_len ? cap_blocks : max_context_len);
  const int r = kv8::launch_decode(q, q_dtype == KV8_F32, k_cache, v_cache, k_scale, v_scale,
                                   num_blocks, block_table, max_blocks_per_seq, context_lens,
                                   ctx_cap, batch, num_q_heads, num_kv_heads, head_dim,
                                   sm_scale, out, workspace, plan, fmt, k_new, v_new,
                                   static_cast<hipStream_t>(stream));
  if (r == -2) return KV8_ERR_UNSUPPORTED;
  return r == 0 ? KV8_OK : KV8_ERR_HIP;
}

int prefill_impl(const uint16_t* q, const int32_t* q_start_loc,
                                 int64_t total_q, int max_q_len, const int8_t* k_cache,
                                 const int8_t* v_cache, const uint16_t* k_scale,
                                 const uint16_t* v_scale, int64_t num_blocks,
                                 const int32_t* block_table, int max_blocks_per_seq,
                                 const int32_t* context_lens, int max_context_len, int batch,
                                 int num_q_heads, int num_kv_heads, int head_dim,
                                 int block_size, float sm_scale, float* out, void* workspace,
                                 size_t workspace_bytes, int fmt, void* stream) {
  (void)workspace; (void)workspace_bytes;
  if (!q_start_loc || !block_table || !context_lens) return KV8_ERR_NULL;
  const int rc = check_cache(k_cache, v_cache, k_scale, v_scale, num_blocks, block_size);
  if (rc != KV8_OK) return rc;
  if (batch <= 0 || total_q < 0 || max_q_len < 0 || max_blocks_per_seq <= 0 ||
      max_context_len < 0)
    return KV8_ERR_SHAPE;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return KV8_ERR_SHAPE;
  if (batch > 65535 || num_q_heads > 65535) return KV8_ERR_SHAPE;
  if (!supported_dim(head_dim) || !supported_group(num_q_heads, num_kv_heads))
    return KV8_ERR_UNSUPPORTED;
  if (total_q == 0 || max_q_len == 0) return KV8_OK;
  if (!q || !out) return KV8_ERR_NULL;
  if (!aligned16(q) || !aligned16(out)) return KV8_ERR_ALIGN;
  const long long cap_blocks = (long long)max_blocks_per_seq * KV8_BLOCK_SIZE;
  const int ctx_cap = (int)(cap_blocks < max_context_len ? cap_blocks : max_context_len);
  const int r = kv8::launch_prefill(q, q_start_loc, total_q, max_q_len, k_cache, v_cache,
                                    k_scale, v_scale, num_blocks, block_table,
                                    max_blocks_per_seq, context_lens, ctx_cap, batch,
                                    num_q_heads, num_kv_heads, head_dim, sm_scale, out, fmt,
                                    static_cast<hipStream_t>(stream));
  if (r == -2) return KV8_ERR_UNSUPPORTED;
  return r == 0 ? KV8_OK : KV8_ERR_HIP;
}

}  // namespace

extern "C" {

const char* kv8_status_string(int status) {
  switch (status) {
    case KV8_OK: return "KV8_OK";
    case KV8_ERR_NULL: return "KV8_ERR_NULL: a required pointer is NULL";
    case KV8_ERR_SHAPE: return "KV8_ERR_SHAPE: invalid or inconsistent size";
    case KV8_ERR_UNSUPPORTED: return "KV8_ERR_UNSUPPORTED: unsupported shape or dtype";
    case KV8_ERR_ALIGN: return "KV8_ERR_ALIGN: pointer not 16-byte aligned";
    case KV8_ERR_WORKSPACE: return "KV8_ERR_WORKSPACE: workspace missing or too small";
    case KV8_ERR_HIP: return "KV8_ERR_HIP: HIP launch error";
    default: return "unknown kv8 status";
  }
}

int kv8_version(void) { return kVersion; }

int kv8_quant_append(const uint16_t* k_new, const uint16_t* v_new,
                     const int32_t* slot_mapping, int64_t n_tokens, int num_kv_heads,
                     int head_dim, int block_size, int64_t num_blocks, int8_t* k_cache,
                     int8_t* v_cache, uint16_t* k_scale, uint16_t* v_scale, void* stream) {
  return append_impl(k_new, v_new, slot_mapping, n_tokens, num_kv_heads, head_dim, block_size,
                     num_blocks, k_cache, v_cache, k_scale, v_scale, kv8::kFmtInt8, stream);
}

int kv8_quant_append_fp8(const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* slot_mapping, int64_t n_tokens, int num_kv_heads,
                         int head_dim, int block_size, int64_t num_blocks, uint8_t* k_cache,
                         uint8_t* v_cache, uint16_t* k_scale, uint16_t* v_scale, void* stream) {
  return append_impl(k_new, v_new, slot_mapping, n_tokens, num_kv_heads, head_dim, block_size,
                     num_blocks, reinterpret_cast<int8_t*>(k_cache),
                     reinterpret_cast<int8_t*>(v_cache), k_scale, v_scale, kv8::kFmtFp8, stream);
}

int kv8_rope_quant_append(const uint16_t* k_new, const uint16_t* v_new,
                          const int32_t* slot_mapping, const int32_t* positions,
                          const float* cos_sin, int max_position, int64_t n_tokens,
                          int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                          int8_t* k_cache, int8_t* v_cache, uint16_t* k_scale,
                          uint16_t* v_scale, void* stream) {
  if (n_tokens < 0 || num_kv_heads <= 0) return KV8_ERR_SHAPE;
  if (!supported_dim(head_dim)) return KV8_ERR_UNSUPPORTED;
  const int rc = check_cache(k_cache, v_cache, k_scale, v_scale, num_blocks, block_size);
  if (rc != KV8_OK) return rc;
  if (n_tokens == 0) return KV8_OK;
  if (!k_new || !v_new || !slot_mapping || !positions || !cos_sin) return KV8_ERR_NULL;
  if (max_position <= 0) return KV8_ERR_SHAPE;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(cos_sin)) return KV8_ERR_ALIGN;
  if (n_tokens * num_kv_heads >= (int64_t)0x7FFFFFFF) return KV8_ERR_SHAPE;   // rows fit 31 bits
  const int r = kv8::launch_rope_quant_append(k_new, v_new, slot_mapping, positions, cos_sin,
                                              max_position, n_tokens, num_kv_heads, head_dim,
                                              num_blocks, k_cache, v_cache, k_scale, v_scale,
                                              static_cast<hipStream_t>(stream));
  return r == 0 ? KV8_OK : KV8_ERR_HIP;
}

int kv8_quant_append_int4(const uint16_t* k_new, const uint16_t* v_new,
                          const int32_t* slot_mapping, int64_t n_tokens, int num_kv_heads,
                          int head_dim, int block_size, int64_t num_blocks, uint8_t* k_cache,
                          uint8_t* v_cache, uint16_t* k_scale, uint16_t* v_scale, void* stream) {
  return append_impl(k_new, v_new, slot_mapping, n_tokens, num_kv_heads, head_dim, block_size,
                     num_blocks, reinterpret_cast<int8_t*>(k_cache),
                     reinterpret_cast<int8_t*>(v_cache), k_scale, v_scale, kv8::kFmtInt4, stream);
}

size_t kv8_decode_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                 int max_context_len, int tokens_per_split) {
  if (!supported_dim(head_dim) || !supported_group(num_q_heads, num_kv_heads)) return 0;
  // enough for every kernel form (a call may ask for any of them)
  size_t need = 0;
  for (int form : {kv8::kDecodeKernelDot, kv8::kDecodeKernelMfma, kv8::kDecodeKernelMfmaOnePass,
                   kv8::kDecodeKernelStreamK}) {
    kv8::DecodePlan plan;
    if (kv8::plan_decode(batch, num_q_heads, num_kv_heads, head_dim, max_context_len,
                         tokens_per_split, form, &plan) && plan.total_bytes > need)
      need = plan.total_bytes;
  }
  return need;
}

int paged_decode_attn_kv8(const void* q, int q_dtype, const int8_t* k_cache,
                          const int8_t* v_cache, const uint16_t* k_scale,
                          const uint16_t* v_scale, int64_t num_blocks,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* context_lens, int max_context_len, int batch,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                          int tokens_per_split, int kernel_form, void* stream) {
  return decode_impl(q, q_dtype, k_cache, v_cache, k_scale, v_scale, num_blocks, block_table,
                     max_blocks_per_seq, context_lens, max_context_len, batch, num_q_heads,
                     num_kv_heads, head_dim, block_size, sm_scale, out, workspace,
                     workspace_bytes, tokens_per_split, kernel_form, kv8::kFmtInt8, nullptr,
                     nullptr, stream);
}

int paged_decode_attn_kv8_noalloc(const void* q, int q_dtype, const int8_t* k_cache,
                                  const int8_t* v_cache, const uint16_t* k_scale,
                                  const uint16_t* v_scale, int64_t num_blocks,
                                  const int32_t* block_table, int max_blocks_per_seq,
                                  const int32_t* context_lens, int max_context_len, int batch,
                                  int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, float sm_scale, float* out,
                                  int tokens_per_split, int kernel_form, void* stream) {
  return decode_impl(q, q_dtype, k_cache, v_cache, k_scale, v_scale, num_blocks, block_table,
                     max_blocks_per_seq, context_lens, max_context_len, batch, num_q_heads,
                     num_kv_heads, head_dim, block_size, sm_scale, out, nullptr, 0,
                     tokens_per_split, kernel_form, kv8::kFmtInt8, nullptr, nullptr, stream,
                     /*use_scratch=*/true);
}

int paged_decode_attn_fp8kv(const void* q, int q_dtype, const uint8_t* k_cache,
                            const uint8_t* v_cache, const uint16_t* k_scale,
                            const uint16_t* v_scale, int64_t num_blocks,
                            const int32_t* block_table, int max_blocks_per_seq,
                            const int32_t* context_lens, int max_context_len, int batch,
                            int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                            float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                            int tokens_per_split, int kernel_form, void* stream) {
  return decode_impl(q, q_dtype, reinterpret_cast<const int8_t*>(k_cache),
                     reinterpret_cast<const int8_t*>(v_cache), k_scale, v_scale, num_blocks,
                     block_table, max_blocks_per_seq, context_lens, max_context_len, batch,
                     num_q_heads, num_kv_heads, head_dim, block_size, sm_scale, out, workspace,
                     workspace_bytes, tokens_per_split, kernel_form, kv8::kFmtFp8, nullptr,
                     nullptr, stream);
}

int paged_decode_attn_kv8_append(const void* q, int q_dtype, const uint16_t* k_new,
                                 const uint16_t* v_new, int8_t* k_cache, int8_t* v_cache,
                                 uint16_t* k_scale, uint16_t* v_scale, int64_t num_blocks,
                                 const int32_t* block_table, int max_blocks_per_seq,
                                 const int32_t* context_lens, int max_context_len, int batch,
                                 int num_q_heads, int num_kv_heads, int head_dim,
                                 int block_size, float sm_scale, float* out, void* workspace,
                                 size_t workspace_bytes, int tokens_per_split, int kernel_form,
                                 void* stream) {
  if (!k_new || !v_new) return KV8_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return KV8_ERR_ALIGN;
  return decode_impl(q, q_dtype, k_cache, v_cache, k_scale, v_scale, num_blocks, block_table,
                     max_blocks_per_seq, context_lens, max_context_len, batch, num_q_heads,
                     num_kv_heads, head_dim, block_size, sm_scale, out, workspace,
                     workspace_bytes, tokens_per_split, kernel_form, kv8::kFmtInt8, k_new, v_new,
                     stream);
}

int paged_decode_attn_int4kv(const void* q, int q_dtype, const uint8_t* k_cache,
                             const uint8_t* v_cache, const uint16_t* k_scale,
                             const uint16_t* v_scale, int64_t num_blocks,
                             const int32_t* block_table, int max_blocks_per_seq,
                             const int32_t* context_lens, int max_context_len, int batch,
                             int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                             float sm_scale, float* out, void* workspace,
                             size_t workspace_bytes, int tokens_per_split, int kernel_form,
                             void* stream) {
  return decode_impl(q, q_dtype, reinterpret_cast<const int8_t*>(k_cache),
                     reinterpret_cast<const int8_t*>(v_cache), k_scale, v_scale, num_blocks,
                     block_table, max_blocks_per_seq, context_lens, max_context_len, batch,
                     num_q_heads, num_kv_heads, head_dim, block_size, sm_scale, out, workspace,
                     workspace_bytes, tokens_per_split, kernel_form, kv8::kFmtInt4, nullptr,
                     nullptr, stream);
}

int paged_decode_attn_bf16kv(const void* q, int q_dtype, const uint16_t* k_cache,
                             const uint16_t* v_cache, int64_t num_blocks,
                             const int32_t* block_table, int max_blocks_per_seq,
                             const int32_t* context_lens, int max_context_len, int batch,
                             int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                             float sm_scale, float* out, void* workspace,
                             size_t workspace_bytes, int tokens_per_split, void* stream) {
  if (!q || !block_table || !context_lens || !out || !k_cache || !v_cache) return KV8_ERR_NULL;
  if (num_blocks <= 0) return KV8_ERR_SHAPE;
  if (block_size != KV8_BLOCK_SIZE) return KV8_ERR_UNSUPPORTED;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return KV8_ERR_ALIGN;
  if (batch <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0) return KV8_ERR_SHAPE;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return KV8_ERR_SHAPE;
  if (batch > 65535 || num_kv_heads > 65535) return KV8_ERR_SHAPE;
  if ((int64_t)batch * num_kv_heads > kv8::kMaxDecodePairs) return KV8_ERR_SHAPE;
  if (q_dtype != KV8_F32 && q_dtype != KV8_BF16) return KV8_ERR_UNSUPPORTED;
  if (!supported_dim(head_dim) || !supported_group(num_q_heads, num_kv_heads))
    return KV8_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(out)) return KV8_ERR_ALIGN;
  if (tokens_per_split > 0 && (tokens_per_split % 64 != 0 || tokens_per_split > 2048))
    return KV8_ERR_UNSUPPORTED;
  kv8::DecodePlan plan;
  if (!kv8::plan_decode(batch, num_q_heads, num_kv_heads, head_dim, max_context_len,
                        tokens_per_split, kv8::kDecodeKernelDot, &plan))
    return KV8_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < plan.total_bytes) return KV8_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KV8_ERR_ALIGN;
  const long long cap_blocks = (long long)max_blocks_per_seq * KV8_BLOCK_SIZE;
  const int ctx_cap = (int)(cap_blocks < max_context_len ? cap_blocks : max_context_len);
  const int r = kv8::launch_decode_bf16kv(q, q_dtype == KV8_F32, k_cache, v_cache, num_blocks,
                                          block_table, max_blocks_per_seq, context_lens,
                                          ctx_cap, batch, num_q_heads, num_kv_heads, head_dim,
                                          sm_scale, out, workspace, plan,
                                          static_cast<hipStream_t>(stream));
  if (r == -2) return KV8_ERR_UNSUPPORTED;
  return r == 0 ? KV8_OK : KV8_ERR_HIP;
}

size_t kv8_prefill_workspace_size(int batch, int num_q_heads, int head_dim, int max_q_len,
                                  int max_context_len) {
  (void)batch; (void)num_q_heads; (void)head_dim; (void)max_q_len; (void)max_context_len;
  return 0;
}

int paged_prefill_chunk_attn_kv8(const uint16_t* q, const int32_t* q_start_loc,
                                 int64_t total_q, int max_q_len, const int8_t* k_cache,
                                 const int8_t* v_cache, const uint16_t* k_scale,
                                 const uint16_t* v_scale, int64_t num_blocks,
                                 const int32_t* block_table, int max_blocks_per_seq,
                                 const int32_t* context_lens, int max_context_len, int batch,
                                 int num_q_heads, int num_kv_heads, int head_dim,
                                 int block_size, float sm_scale, float* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return prefill_impl(q, q_start_loc, total_q, max_q_len, k_cache, v_cache, k_scale, v_scale,
                      num_blocks, block_table, max_blocks_per_seq, context_lens,
                      max_context_len, batch, num_q_heads, num_kv_heads, head_dim, block_size,
                      sm_scale, out, workspace, workspace_bytes, kv8::kFmtInt8, stream);
}

int paged_prefill_chunk_attn_fp8kv(const uint16_t* q, const int32_t* q_start_loc,
                                   int64_t total_q, int max_q_len, const uint8_t* k_cache,
                                   const uint8_t* v_cache, const uint16_t* k_scale,
                                   const uint16_t* v_scale, int64_t num_blocks,
                                   const int32_t* block_table, int max_blocks_per_seq,
                                   const int32_t* context_lens, int max_context_len, int batch,
                                   int num_q_heads, int num_kv_heads, int head_dim,
                                   int block_size, float sm_scale, float* out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return prefill_impl(q, q_start_loc, total_q, max_q_len,
                      reinterpret_cast<const int8_t*>(k_cache),
                      reinterpret_cast<const int8_t*>(v_cache), k_scale, v_scale, num_blocks,
                      block_table, max_blocks_per_seq, context_lens, max_context_len, batch,
                      num_q_heads, num_kv_heads, head_dim, block_size, sm_scale, out, workspace,
                      workspace_bytes, kv8::kFmtFp8, stream);
}

int paged_prefill_chunk_attn_int4kv(const uint16_t* q, const int32_t* q_start_loc,
                                    int64_t total_q, int max_q_len, const uint8_t* k_cache,
                                    const uint8_t* v_cache, const uint16_t* k_scale,
                                    const uint16_t* v_scale, int64_t num_blocks,
                                    const int32_t* block_table, int max_blocks_per_seq,
                                    const int32_t* context_lens, int max_context_len, int batch,
                                    int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, float sm_scale, float* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return prefill_impl(q, q_start_loc, total_q, max_q_len,
                      reinterpret_cast<const int8_t*>(k_cache),
                      reinterpret_cast<const int8_t*>(v_cache), k_scale, v_scale, num_blocks,
                      block_table, max_blocks_per_seq, context_lens, max_context_len, batch,
                      num_q_heads, num_kv_heads, head_dim, block_size, sm_scale, out, workspace,
                      workspace_bytes, kv8::kFmtInt4, stream);
}

int64_t kv8_read_probe_chunk_bytes(void) { return kv8::read_probe_chunk_bytes(); }

int kv8_read_probe(const void* buf, const int32_t* tiles, int tile_bytes, int64_t n_bytes,
                   int64_t workgroups, uint32_t* out, void* stream) {
  if (!buf || !tiles || !out) return KV8_ERR_NULL;
  if (tile_bytes < 1024 || tile_bytes > 32768 || tile_bytes % 1024 != 0) return KV8_ERR_SHAPE;
  if (n_bytes <= 0 || n_bytes % tile_bytes != 0) return KV8_ERR_SHAPE;
  if (workgroups <= 0 || workgroups > 0x7FFFFFFF) return KV8_ERR_SHAPE;
  if (!aligned16(buf)) return KV8_ERR_ALIGN;
  return kv8::launch_read_probe(buf, tiles, tile_bytes, n_bytes, workgroups, out,
                                static_cast<hipStream_t>(stream)) == 0
             ? KV8_OK
             : KV8_ERR_HIP;
}

int kv8_stream_read(const void* buf, int64_t n_bytes, int64_t workgroups, uint32_t* out,
                    void* stream) {
  if (!buf || !out) return KV8_ERR_NULL;
  const int64_t chunk = kv8::read_probe_chunk_bytes();
  if (n_bytes <= 0 || n_bytes % chunk != 0) return KV8_ERR_SHAPE;
  if (workgroups <= 0 || workgroups > 0x7FFFFFFF) return KV8_ERR_SHAPE;
  if (!aligned16(buf)) return KV8_ERR_ALIGN;
  return kv8::launch_read_probe(buf, nullptr, 0, n_bytes, workgroups, out,
                                static_cast<hipStream_t>(stream)) == 0
             ? KV8_OK
             : KV8_ERR_HIP;
}

}  // extern "C"
