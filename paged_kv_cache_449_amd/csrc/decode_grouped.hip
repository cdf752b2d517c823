// Host entry points of prefix-grouped decode: argument checks, workspace
// and dispatch to the kernel instantiations.
#include "decode_grouped.h"

using namespace pkv;

extern "C" kv_status_t paged_attention_decode_grouped_workspace_size(const kv_pool_t* pool, int32_t num_seqs,
                                                                     int32_t num_q_heads, size_t* bytes) {
  if (!pool || !bytes || num_seqs < 0 || num_q_heads <= 0) return KV_ERR_INVALID_ARG;
  // the counter header of paged_attention_decode / _prefill is skipped and
  // left untouched, so one workspace serves all three calls
  *bytes = (size_t)kCounterSlots * sizeof(int32_t) +
           (size_t)num_seqs * num_q_heads * (pool->head_dim + 4) * sizeof(float);
  return KV_OK;
}

extern "C" kv_status_t paged_attention_decode_grouped(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype,
                                                      void* out, const int32_t* block_tables, int32_t max_blocks,
                                                      const int32_t* context_lens, int32_t num_seqs,
                                                      int32_t num_q_heads, float scale, const int32_t* group_start,
                                                      const int32_t* group_shared, int32_t num_groups,
                                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!pool || num_seqs < 0 || num_q_heads <= 0 || max_blocks <= 0 || num_groups < 0 || !valid_dtype(q_dtype))
    return KV_ERR_INVALID_ARG;
  if (num_q_heads % pool->num_kv_heads) return KV_ERR_INVALID_ARG;
  const int G = num_q_heads / pool->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return KV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return KV_OK;
  if (!q || !out || !block_tables || !context_lens) return KV_ERR_INVALID_ARG;
  if (num_groups > 0 && (!group_start || !group_shared)) return KV_ERR_INVALID_ARG;
  if ((((uintptr_t)q) | ((uintptr_t)out)) & 15) return KV_ERR_INVALID_ARG;
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return KV_ERR_INVALID_ARG;
  if (pool->log2_block_size < 4) return KV_ERR_UNSUPPORTED;   // matrix-core tiles of 16 tokens within one block
  if ((int64_t)max_blocks * pool->block_size > (1LL << 30)) return KV_ERR_INVALID_ARG;
  if ((int64_t)num_seqs * pool->num_kv_heads > (1LL << 31) - 1 ||
      (int64_t)num_groups * pool->num_kv_heads > (1LL << 31) - 1)
    return KV_ERR_INVALID_ARG;
  size_t need;
  paged_attention_decode_grouped_workspace_size(pool, num_seqs, num_q_heads, &need);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255)) return KV_ERR_WORKSPACE;

  DecodeParams p{};
  p.k_pool = (const uint8_t*)pool->k;
  p.v_pool = (const uint8_t*)pool->v;
  p.q = (const uint8_t*)q;
  p.out = (uint8_t*)out;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start = nullptr;
  p.counters = nullptr;
  p.partials = (float*)((uint8_t*)workspace + (size_t)kCounterSlots * sizeof(int32_t));
  p.num_seqs = num_seqs;
  p.total_q = 0;
  p.num_kv_heads = pool->num_kv_heads;
  p.max_blocks = max_blocks;
  p.num_blocks = pool->num_blocks;
  p.log2_bs = pool->log2_block_size;
  p.chunk = 0;
  p.num_workers = 0;
  const bool fp8 = pool->dtype == KV_FP8_E4M3FN;
  p.q_scale = scale * kLog2e * (fp8 ? pool->k_scale : 1.0f);
  p.v_scale = fp8 ? pool->v_scale : 1.0f;
  p.qk_scale = scale * kLog2e;
  p.head_scales = fp8 && pool->per_head ? pool->head_scales : nullptr;

  const int D = pool->head_dim;
  hipStream_t s = (hipStream_t)stream;
  if (pool->dtype == KV_BF16 && q_dtype == KV_BF16)
    return launch_grouped_bf16_bf16(p, D, G, group_start, group_shared, num_groups, s);
  if (pool->dtype == KV_F16 && q_dtype == KV_F16)
    return launch_grouped_f16_f16(p, D, G, group_start, group_shared, num_groups, s);
  if (fp8 && q_dtype == KV_BF16) return launch_grouped_fp8_bf16(p, D, G, group_start, group_shared, num_groups, s);
  if (fp8 && q_dtype == KV_F16) return launch_grouped_fp8_f16(p, D, G, group_start, group_shared, num_groups, s);
  return KV_ERR_UNSUPPORTED;
}
