// Block attention entry point (MFMA kernels land in this file).
#include "kvq_internal.h"

using namespace kvq;

extern "C" kvq_status kvq_block_attn(const kvq_config* cfg, const kvq_state* st, const kvq_cache* cache,
                                     const void* q, const void* k_blk, const void* v_blk, int32_t tq,
                                     int32_t q_heads, float softmax_scale, int32_t num_splits,
                                     float* out, void* workspace, size_t workspace_bytes, void* stream) {
  (void)cfg; (void)st; (void)cache; (void)q; (void)k_blk; (void)v_blk; (void)tq; (void)q_heads;
  (void)softmax_scale; (void)num_splits; (void)out; (void)workspace; (void)workspace_bytes; (void)stream;
  return KVQ_EINVAL;
}
