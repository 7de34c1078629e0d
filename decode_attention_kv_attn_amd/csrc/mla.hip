// Absorbed MLA decode: host entry points (matrix-core kernel pending).
#include <math.h>

#include "../../include/attn_decode.h"
#include "internal.h"

namespace {

int check_mla(int B, int H, int T_cap, int d_c, int d_rope) {
  if (B < 0 || H <= 0 || T_cap <= 0) return ATTN_ERR_SHAPE;
  if (d_c != 512 || d_rope != 64) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_mla_splits(int B, int H, int T_cap, int d_c, int d_rope,
                           int num_splits) {
  const int st = check_mla(B, H, T_cap, d_c, d_rope);
  if (st != ATTN_OK) return st;
  if (num_splits < 0 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_ARG;
  return ATTN_ERR_UNSUPPORTED;
}

size_t attn_decode_mla_workspace_bytes(int B, int H, int T_cap, int d_c,
                                       int d_rope, int num_splits) {
  (void)B; (void)H; (void)T_cap; (void)d_c; (void)d_rope; (void)num_splits;
  return (size_t)-1;
}

int attn_decode_mla(const void* q, const void* latent, float* out,
                    float* lse_out, const int32_t* seq_lens, int B, int H,
                    int T_cap, int d_c, int d_rope, float scale,
                    int num_splits, void* workspace, size_t workspace_bytes,
                    void* stream) {
  (void)lse_out; (void)seq_lens; (void)workspace; (void)workspace_bytes;
  (void)stream;
  if (!q || !latent || !out) return ATTN_ERR_NULL;
  int st = check_mla(B, H, T_cap, d_c, d_rope);
  if (st != ATTN_OK) return st;
  if (!(scale > 0.f) || isinf(scale)) return ATTN_ERR_ARG;
  if (num_splits < 0 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_ARG;
  return ATTN_ERR_UNSUPPORTED;
}

}  // extern "C"
