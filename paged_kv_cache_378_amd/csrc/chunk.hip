// Chunked-query paged attention (MFMA).  Placeholder until the kernel lands.
#include "device_common.h"

extern "C" pa_status pa_chunk_attend(void* out, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     const int32_t* ctx_lens, int32_t S, int32_t C, int32_t Hq,
                                     int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
                                     int32_t max_blocks, float scale, int32_t dtype, void* stream) {
  (void)out; (void)q; (void)k_cache; (void)v_cache; (void)block_tables; (void)ctx_lens; (void)S;
  (void)C; (void)Hq; (void)Hkv; (void)D; (void)B; (void)num_blocks; (void)max_blocks;
  (void)scale; (void)dtype; (void)stream;
  return pa::fail(PA_ERR_UNSUPPORTED, "pa_chunk_attend: not built yet");
}
