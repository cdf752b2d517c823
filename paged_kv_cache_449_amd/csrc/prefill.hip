// Host entry points of multi-token paged attention: argument checks,
// workspace layout and dispatch to the kernel instantiations.
#include <algorithm>

#include "prefill_kernel.h"

namespace {

using namespace pkv;

// One-wave workers (16-row tiles) and multi-wave work-groups (128- or
// 64-row blocks).
constexpr int kPrefillWavesPerCu = 8;
constexpr int kPrefillGroupsPerCu = 1;
// Rows per (sequence, kv head), on average, from which the work-groups pay
// off: below it most of a row block would be empty.
constexpr int kGroupMinRows = 96;
// Row blocks per CU from which one work-group per row block balances well.
constexpr int kUnitsPerCu = 4;

int64_t round_workers(int64_t w) {
  w = (w + 7) & ~7LL;
  if (w < 8) w = 8;
  return w > kCounterSlots ? kCounterSlots : w;
}

// Launch shape of either path; the workspace fits both.
kv_status_t prefill_plan(const kv_pool_t* pool, int32_t num_q_heads, bool wg, int32_t* workers,
                         size_t* counters_bytes, size_t* bytes) {
  if (!pool || num_q_heads <= 0 || num_q_heads % pool->num_kv_heads) return KV_ERR_INVALID_ARG;
  const int G = num_q_heads / pool->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return KV_ERR_UNSUPPORTED;
  const int64_t w_wave = round_workers((int64_t)pool->num_cus * kPrefillWavesPerCu);
  const int64_t w_wg = round_workers((int64_t)pool->num_cus * kPrefillGroupsPerCu);
  *workers = (int32_t)(wg ? w_wg : w_wave);
  *counters_bytes = (size_t)kCounterSlots * sizeof(int32_t);
  const size_t rec = (size_t)(pool->head_dim + 4) * sizeof(float);
  const size_t wave_recs = (size_t)2 * w_wave * 16 * rec, wg_recs = (size_t)2 * w_wg * kMaxWgRows * rec;
  *bytes = *counters_bytes + (wave_recs > wg_recs ? wave_recs : wg_recs);
  return KV_OK;
}

// Launch shape: 0 one-wave tiles, 1 split work-groups, 2 one work-group per
// row block.  A pool made with PAGEDKV_PREFILL_PATH=wave / group / unit
// forces one (tests); otherwise the average rows per (sequence, kv head)
// picks the work-groups, and units when there are enough row blocks to fill
// the chip several times.
int prefill_mode(int forced, int64_t total_q, int G, int num_seqs, int num_kv_heads, int D, int num_cus) {
  if (forced >= 0) return forced;
  if (total_q * G < (int64_t)kGroupMinRows * num_seqs) return 0;
  const int64_t rows = 16LL * (D <= 128 ? 8 : 4);
  const int64_t units = total_q * G / rows * num_kv_heads;
  return units >= (int64_t)kUnitsPerCu * num_cus ? 2 : 1;
}

}  // namespace

extern "C" kv_status_t paged_attention_prefill_workspace_size(const kv_pool_t* pool, int32_t num_q_heads,
                                                              size_t* bytes) {
  if (!bytes) return KV_ERR_INVALID_ARG;
  int32_t workers;
  size_t counters;
  return prefill_plan(pool, num_q_heads, false, &workers, &counters, bytes);
}

extern "C" kv_status_t paged_attention_prefill(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype, void* out,
                                               const int32_t* block_tables, int32_t max_blocks,
                                               const int32_t* context_lens, const int32_t* query_start,
                                               int32_t num_seqs, int32_t total_q, int32_t num_q_heads, float scale,
                                               void* workspace, size_t workspace_bytes, void* stream) {
  int32_t workers;
  size_t counters_bytes, need;
  const int mode = pool && num_q_heads > 0 && num_q_heads % pool->num_kv_heads == 0
                       ? prefill_mode(pool->prefill_shape, total_q, num_q_heads / pool->num_kv_heads,
                                      num_seqs > 0 ? num_seqs : 1,
                                      pool->num_kv_heads, pool->head_dim, pool->num_cus)
                       : 0;
  kv_status_t st = prefill_plan(pool, num_q_heads, mode == 1, &workers, &counters_bytes, &need);
  if (st != KV_OK) return st;
  if (num_seqs < 0 || total_q < 0 || max_blocks <= 0 || !valid_dtype(q_dtype)) return KV_ERR_INVALID_ARG;
  if (num_seqs == 0 || total_q == 0) return KV_OK;
  if (!q || !out || !block_tables || !context_lens || !query_start) return KV_ERR_INVALID_ARG;
  if ((((uintptr_t)q) | ((uintptr_t)out)) & 15) return KV_ERR_INVALID_ARG;
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return KV_ERR_INVALID_ARG;
  if (pool->log2_block_size < 4) return KV_ERR_UNSUPPORTED;   // tiles of 16 tokens within one block
  const int G = num_q_heads / pool->num_kv_heads;
  // stream length bound: tiles * blocks per tile * kv heads must fit in int32
  const int64_t tiles = ((int64_t)total_q * G + 15) / 16 + num_seqs;
  if (tiles * max_blocks * pool->num_kv_heads > (1LL << 30) || (int64_t)max_blocks * pool->block_size > (1LL << 30))
    return KV_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255)) return KV_ERR_WORKSPACE;
  int32_t unit_run = 0;
  if (mode == 2) {
    // at most total_q * G / rows + num_seqs row blocks per kv head when
    // query_start is consistent (the tiles bound above keeps this far below
    // 2^31); units past the grid of an inconsistent one are left undone
    const int64_t rows = 16LL * (pool->head_dim <= 128 ? 8 : 4);
    const int64_t units = ((int64_t)total_q * G / rows + num_seqs + 1) * pool->num_kv_heads;
    workers = (int32_t)((units + 7) & ~7LL);
    if (num_seqs <= kUnitRankSeqs) {
      // ranked order dealt to the XCDs in runs of about one (sequence, kv
      // head) pair's row blocks; each XCD gets ceil(units / 8c) runs at most
      const int64_t c = std::min<int64_t>(16, std::max<int64_t>(1, ((int64_t)total_q * G + rows * num_seqs - 1) /
                                                                       (rows * num_seqs)));
      unit_run = (int32_t)c;
      workers = (int32_t)(8 * ((units + 8 * c - 1) / (8 * c)) * c);
    }
  }

  DecodeParams p{};
  p.k_pool = (const uint8_t*)pool->k;
  p.v_pool = (const uint8_t*)pool->v;
  p.q = (const uint8_t*)q;
  p.out = (uint8_t*)out;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start = query_start;
  p.counters = (int32_t*)workspace;
  p.partials = (float*)((uint8_t*)workspace + counters_bytes);
  p.num_seqs = num_seqs;
  p.total_q = total_q;
  p.num_kv_heads = pool->num_kv_heads;
  p.max_blocks = max_blocks;
  p.num_blocks = pool->num_blocks;
  p.log2_bs = pool->log2_block_size;
  p.chunk = unit_run;   // unit mode: the run length of the XCD deal
  p.num_workers = workers;
  const bool fp8 = pool->dtype == KV_FP8_E4M3FN;
  p.q_scale = scale * kLog2e * (fp8 ? pool->k_scale : 1.0f);
  p.v_scale = fp8 ? pool->v_scale : 1.0f;
  p.qk_scale = scale * kLog2e;
  p.head_scales = fp8 && pool->per_head ? pool->head_scales : nullptr;

  const int D = pool->head_dim;
  hipStream_t s = (hipStream_t)stream;
  if (pool->dtype == KV_BF16 && q_dtype == KV_BF16) return launch_prefill_bf16_bf16(p, D, G, mode, s);
  if (pool->dtype == KV_F16 && q_dtype == KV_F16) return launch_prefill_f16_f16(p, D, G, mode, s);
  if (fp8 && q_dtype == KV_BF16) return launch_prefill_fp8_bf16(p, D, G, mode, s);
  if (fp8 && q_dtype == KV_F16) return launch_prefill_fp8_f16(p, D, G, mode, s);
  return KV_ERR_UNSUPPORTED;
}
