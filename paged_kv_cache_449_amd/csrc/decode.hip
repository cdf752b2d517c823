// Host entry points of paged decode attention: argument checks, work split,
// workspace layout and dispatch to the kernel instantiations.
#include <mutex>

#include "decode_kernel.h"

namespace {

using namespace pkv;

struct Plan {
  int32_t chunk;        // 0 = derived in the kernel
  int32_t num_workers;  // multiple of 8
  size_t counters_bytes;
  size_t bytes;
};

kv_status_t make_plan(const kv_pool_t* pool, int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks,
                      int32_t partition_tokens, Plan* plan) {
  if (!pool || num_seqs < 0 || num_q_heads <= 0 || max_blocks <= 0 || partition_tokens < 0) return KV_ERR_INVALID_ARG;
  if (num_q_heads % pool->num_kv_heads) return KV_ERR_INVALID_ARG;
  const int G = num_q_heads / pool->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return KV_ERR_UNSUPPORTED;
  const int64_t units = (int64_t)num_seqs * pool->num_kv_heads * max_blocks;  // upper bound of blocks
  if (units > (1LL << 30) || (int64_t)max_blocks * pool->block_size > (1LL << 30)) return KV_ERR_INVALID_ARG;
  int64_t workers;
  if (partition_tokens > 0) {
    if (partition_tokens % pool->block_size) return KV_ERR_INVALID_ARG;
    int64_t chunk = partition_tokens / pool->block_size;
    // longer runs when the batch would need more runs than counter slots
    const int64_t min_chunk = (units + kCounterSlots - 9) / (kCounterSlots - 8);
    if (chunk < min_chunk) chunk = min_chunk;
    plan->chunk = (int32_t)chunk;
    workers = (units + chunk - 1) / chunk;
  } else {
    plan->chunk = 0;
    workers = (int64_t)pool->num_cus * pool->decode_waves_per_cu;
    if (workers > units) workers = units;
  }
  if (workers < 1) workers = 1;
  workers = (workers + 7) & ~7LL;
  // chunks (virtual workers): the library-sized split may cut the stream
  // kSharedSplit times finer when sequences share blocks
  const int64_t chunks = partition_tokens > 0 ? workers : workers * kSharedSplit;
  if (chunks > kCounterSlots) return KV_ERR_INVALID_ARG;
  plan->num_workers = (int32_t)workers;
  plan->counters_bytes = (size_t)kCounterSlots * sizeof(int32_t);
  plan->bytes = plan->counters_bytes + (size_t)2 * chunks * G * (pool->head_dim + 4) * sizeof(float);
  return KV_OK;
}

}  // namespace

extern "C" kv_status_t paged_attention_workspace_size(const kv_pool_t* pool, int32_t num_seqs, int32_t num_q_heads,
                                                      int32_t max_blocks, int32_t partition_tokens, size_t* bytes) {
  if (!bytes) return KV_ERR_INVALID_ARG;
  Plan plan;
  kv_status_t st = make_plan(pool, num_seqs, num_q_heads, max_blocks, partition_tokens, &plan);
  if (st != KV_OK) return st;
  *bytes = plan.bytes;
  return KV_OK;
}

namespace {

kv_status_t decode(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype, void* out, const int32_t* block_tables,
                   int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                   float scale, int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  Plan plan;
  kv_status_t st = make_plan(pool, num_seqs, num_q_heads, max_blocks, partition_tokens, &plan);
  if (st != KV_OK) return st;
  if (!valid_dtype(q_dtype)) return KV_ERR_INVALID_ARG;
  if (num_seqs == 0) return KV_OK;
  if (!q || !out || !block_tables || !context_lens) return KV_ERR_INVALID_ARG;
  if ((((uintptr_t)q) | ((uintptr_t)out)) & 15) return KV_ERR_INVALID_ARG;
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return KV_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < plan.bytes || ((uintptr_t)workspace & 255)) return KV_ERR_WORKSPACE;

  const int D = pool->head_dim;
  const int G = num_q_heads / pool->num_kv_heads;
  DecodeParams p;
  p.k_pool = (const uint8_t*)pool->k;
  p.v_pool = (const uint8_t*)pool->v;
  p.q = (const uint8_t*)q;
  p.out = (uint8_t*)out;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start = nullptr;
  p.total_q = 0;
  p.counters = (int32_t*)workspace;
  p.partials = (float*)((uint8_t*)workspace + plan.counters_bytes);
  p.num_seqs = num_seqs;
  p.num_kv_heads = pool->num_kv_heads;
  p.max_blocks = max_blocks;
  p.num_blocks = pool->num_blocks;
  p.log2_bs = pool->log2_block_size;
  p.chunk = plan.chunk;
  p.num_workers = plan.num_workers;
  const bool fp8 = pool->dtype == KV_FP8_E4M3FN;
  p.q_scale = scale * kLog2e * (fp8 ? pool->k_scale : 1.0f);
  p.v_scale = fp8 ? pool->v_scale : 1.0f;
  p.qk_scale = scale * kLog2e;
  p.head_scales = fp8 && pool->per_head ? pool->head_scales : nullptr;

  // a wave load covers 64 / (lanes per token row) tokens of one block
  const int lanes_per_row = D * (int)elem_bytes(pool->dtype) / 16;
  if (64 / lanes_per_row > pool->block_size) return KV_ERR_UNSUPPORTED;

  hipStream_t s = (hipStream_t)stream;
  // Query groups (G > 1) run on the matrix cores where the dtype pair has a
  // 16-bit operand type and blocks hold whole 16-token tiles, unless the
  // pool was made with PAGEDKV_DECODE_MFMA=0.
  const bool mfma = G > 1 && pool->decode_mfma;
  if (!fp8) {
    if (q_dtype != pool->dtype) return KV_ERR_UNSUPPORTED;
    switch (pool->dtype) {
      case KV_F32: return launch_decode_f32_f32(p, D, G, mfma, s);
      case KV_F16: return launch_decode_f16_f16(p, D, G, mfma, s);
      case KV_BF16: return launch_decode_bf16_bf16(p, D, G, mfma, s);
      default: return KV_ERR_UNSUPPORTED;
    }
  }
  switch (q_dtype) {
    case KV_F32: return launch_decode_fp8_f32(p, D, G, mfma, s);
    case KV_F16: return launch_decode_fp8_f16(p, D, G, mfma, s);
    case KV_BF16: return launch_decode_fp8_bf16(p, D, G, mfma, s);
    default: return KV_ERR_UNSUPPORTED;
  }
}

}  // namespace

extern "C" kv_status_t paged_attention_decode(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype, void* out,
                                              const int32_t* block_tables, int32_t max_blocks,
                                              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                              float scale, int32_t partition_tokens, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  return decode(pool, q, q_dtype, out, block_tables, max_blocks, context_lens, num_seqs, num_q_heads, scale,
                partition_tokens, workspace, workspace_bytes, stream);
}

// ------------------------------------------------- allocation-free variant
//
// paged_attention_decode_noalloc runs the same kernels with the workspace in
// this file-scope device array instead of a caller's buffer, for callers that
// cannot allocate (code under graph capture, tight serving loops).  Every
// device the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// the device address is fetched once per device with hipGetSymbolAddress and
// only that address is passed on.
static __device__ __align__(256) uint8_t scratch[PAGEDKV_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device (null: not set up)

__global__ void clear_words_kernel(uint32_t* p, int words) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < words; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The device address of the pool's device's scratch, set up on first use:
// the address is looked up with that device current, and the arrival
// counters at its start are cleared on `stream` (a kernel, not a memset, so
// a captured first call records no memset).
kv_status_t device_scratch(const kv_pool_t* pool, hipStream_t stream, void** out) {
  if (pool->device < 0 || pool->device >= kMaxDevices) return KV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[pool->device]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return KV_ERR_HIP;
    if (cur != pool->device && hipSetDevice(pool->device) != hipSuccess) return KV_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    kv_status_t st = KV_OK;
    if (e != hipSuccess || !ptr) {
      st = KV_ERR_HIP;
    } else {
      const int words = (int)(kCounterSlots);
      hipLaunchKernelGGL(clear_words_kernel, dim3(64), dim3(256), 0, stream, (uint32_t*)ptr, words);
      st = launch_status();
    }
    if (cur != pool->device) (void)hipSetDevice(cur);
    if (st != KV_OK) return st;
    g_scratch[pool->device] = ptr;
  }
  *out = g_scratch[pool->device];
  return KV_OK;
}

}  // namespace

extern "C" kv_status_t paged_attention_decode_noalloc(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype,
                                                      void* out, const int32_t* block_tables, int32_t max_blocks,
                                                      const int32_t* context_lens, int32_t num_seqs,
                                                      int32_t num_q_heads, float scale, int32_t partition_tokens,
                                                      void* stream) {
  Plan plan;
  kv_status_t st = make_plan(pool, num_seqs, num_q_heads, max_blocks, partition_tokens, &plan);
  if (st != KV_OK) return st;
  if (plan.bytes > (size_t)PAGEDKV_DECODE_SCRATCH_BYTES) return KV_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = device_scratch(pool, (hipStream_t)stream, &ws)) != KV_OK) return st;
  return decode(pool, q, q_dtype, out, block_tables, max_blocks, context_lens, num_seqs, num_q_heads, scale,
                partition_tokens, ws, PAGEDKV_DECODE_SCRATCH_BYTES, stream);
}
