// Chunked-prefill attention (MFMA) mixed with decode rows: placeholder until
// the matrix-core kernel lands.
#include "device_common.h"

extern "C" size_t pkv_prefill_workspace_size(const pkv_cache* cache, int32_t num_rows, int32_t total_q,
                                             int32_t max_q_per_row, int32_t max_context_len) {
  (void)cache; (void)num_rows; (void)total_q; (void)max_q_per_row; (void)max_context_len;
  return 0;
}

extern "C" int pkv_chunked_prefill_attention(const pkv_cache*, int32_t, void*, const void*, const int32_t*,
                                             const int32_t*, int32_t, const int32_t*, int32_t, int32_t, int32_t,
                                             int32_t, float, void*, size_t, void*) {
  return pkv::fail(PKV_ERR_UNSUPPORTED, "chunked prefill is not built yet");
}
