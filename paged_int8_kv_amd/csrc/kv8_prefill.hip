// paged_prefill_chunk_attn_kv8 kernel (MFMA chunked prefill) - not built yet.
#include "kv8_device.h"
#include "kv8_launch.h"

namespace kv8 {

int launch_prefill(const uint16_t*, const int32_t*, int64_t, int, const int8_t*, const int8_t*,
                   const uint16_t*, const uint16_t*, int64_t, const int32_t*, int,
                   const int32_t*, int, int, int, int, int, float, float*, hipStream_t) {
  return -2;
}

}  // namespace kv8
