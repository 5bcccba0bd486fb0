// decode_attn_latent.hip — latent-cache decode attention (one kv head whose
// first Dv dims double as the value vector, per-token scales, >= 16 query
// rows per kv head) on MFMA. Not built yet: the entry points report the
// shape as unsupported.
#include "pda_internal.h"

namespace pda {

bool latent_supported(const pda_attn_shape& sh) {
  (void)sh;
  return false;
}

size_t latent_workspace_bytes(const pda_attn_shape& sh, int32_t max_seq_len) {
  (void)sh;
  (void)max_seq_len;
  return 0;
}

int latent_launch(const pda_attn_shape& sh, const void* q, const void* k_cache,
                  const float* token_scale, const int32_t* block_table, const int32_t* seq_lens,
                  int32_t max_seq_len, const int32_t* verdict, void* workspace,
                  size_t workspace_bytes, float* out, hipStream_t stream) {
  (void)sh; (void)q; (void)k_cache; (void)token_scale; (void)block_table; (void)seq_lens;
  (void)max_seq_len; (void)verdict; (void)workspace; (void)workspace_bytes; (void)out;
  (void)stream;
  return PDA_ERR_UNSUPPORTED;
}

}  // namespace pda
