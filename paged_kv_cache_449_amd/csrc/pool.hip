// Pool descriptor management and status strings of the C ABI.
//
// The pool is one preallocated region per tensor (K and V), carved into equal
// blocks once ("vLLM KV Cache 实现机制" §4.1 pool diagram; "vLLM — 把操作系统的
// 分页搬进 GPU KV cache", case 1).  One hipMalloc per pool keeps the blocks in
// a few large physically contiguous fragments, which keeps address
// translation cheap for the scattered block reads of decode.
#include <stdlib.h>
#include <string.h>

#include <new>

#include "common.h"

namespace {

kv_status_t check_shape(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                        kv_dtype_t dtype, size_t* bytes) {
  if (num_blocks <= 0 || num_kv_heads <= 0 || !pkv::valid_dtype(dtype)) return KV_ERR_INVALID_ARG;
  if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64) return KV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return KV_ERR_UNSUPPORTED;
  unsigned __int128 b = (unsigned __int128)num_blocks * num_kv_heads * block_size * head_dim * pkv::elem_bytes(dtype);
  if (b > ((unsigned __int128)1 << 46)) return KV_ERR_INVALID_ARG;
  *bytes = (size_t)b;
  return KV_OK;
}

kv_status_t fill(kv_pool_t* p, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                 kv_dtype_t dtype) {
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->log2_block_size = pkv::ilog2_exact(block_size);
  p->num_kv_heads = num_kv_heads;
  p->head_dim = head_dim;
  p->dtype = dtype;
  p->k_scale = 1.0f;
  p->v_scale = 1.0f;
  p->head_scales = nullptr;
  p->per_head = false;
  if (hipGetDevice(&p->device) != hipSuccess) return KV_ERR_HIP;
  if (hipDeviceGetAttribute(&p->num_cus, hipDeviceAttributeMultiprocessorCount, p->device) != hipSuccess)
    return KV_ERR_HIP;
  // tuning and test overrides of the launch shape, fixed for the pool's life
  const char* e = getenv("PAGEDKV_DECODE_WAVES_PER_CU");
  const int w = e ? atoi(e) : 0;
  p->decode_waves_per_cu = (w >= 1 && w <= 64) ? w : 8;
  e = getenv("PAGEDKV_DECODE_MFMA");
  p->decode_mfma = !(e && e[0] == '0');
  e = getenv("PAGEDKV_PREFILL_PATH");
  p->prefill_shape = !e                          ? -1
                     : strcmp(e, "wave") == 0   ? 0
                     : strcmp(e, "group") == 0  ? 1
                     : strcmp(e, "unit") == 0   ? 2
                                                : -1;
  // fp8 pools: the per-kv-head scale table, so that setting scales later
  // allocates nothing
  if (dtype == KV_FP8_E4M3FN) {
    if (hipMalloc(&p->head_scales, 2 * (size_t)num_kv_heads * sizeof(float)) != hipSuccess) {
      p->head_scales = nullptr;
      return KV_ERR_OOM;
    }
  }
  return KV_OK;
}

}  // namespace

extern "C" kv_status_t kv_pool_create(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                      kv_dtype_t dtype, kv_pool_t** out) {
  if (!out) return KV_ERR_INVALID_ARG;
  *out = nullptr;
  size_t bytes = 0;
  kv_status_t st = check_shape(num_blocks, block_size, num_kv_heads, head_dim, dtype, &bytes);
  if (st != KV_OK) return st;
  kv_pool_t* p = new (std::nothrow) kv_pool_t();
  if (!p) return KV_ERR_OOM;
  if ((st = fill(p, num_blocks, block_size, num_kv_heads, head_dim, dtype)) != KV_OK) {
    if (p->head_scales) (void)hipFree(p->head_scales);
    delete p;
    return st;
  }
  if (hipMalloc(&p->k, bytes) != hipSuccess) {
    if (p->head_scales) (void)hipFree(p->head_scales);
    delete p;
    return KV_ERR_OOM;
  }
  if (hipMalloc(&p->v, bytes) != hipSuccess) {
    (void)hipFree(p->k);
    if (p->head_scales) (void)hipFree(p->head_scales);
    delete p;
    return KV_ERR_OOM;
  }
  p->bytes_each = bytes;
  p->owned = true;
  *out = p;
  return KV_OK;
}

extern "C" kv_status_t kv_pool_create_from(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                                           int32_t head_dim, kv_dtype_t dtype, void* k_buf, void* v_buf,
                                           size_t bytes_each, kv_pool_t** out) {
  if (!out) return KV_ERR_INVALID_ARG;
  *out = nullptr;
  size_t bytes = 0;
  kv_status_t st = check_shape(num_blocks, block_size, num_kv_heads, head_dim, dtype, &bytes);
  if (st != KV_OK) return st;
  if (!k_buf || !v_buf || bytes_each < bytes) return KV_ERR_INVALID_ARG;
  if (((uintptr_t)k_buf | (uintptr_t)v_buf) & 15) return KV_ERR_INVALID_ARG;
  kv_pool_t* p = new (std::nothrow) kv_pool_t();
  if (!p) return KV_ERR_OOM;
  if ((st = fill(p, num_blocks, block_size, num_kv_heads, head_dim, dtype)) != KV_OK) {
    if (p->head_scales) (void)hipFree(p->head_scales);
    delete p;
    return st;
  }
  p->k = k_buf;
  p->v = v_buf;
  p->bytes_each = bytes;
  p->owned = false;
  *out = p;
  return KV_OK;
}

extern "C" kv_status_t kv_pool_destroy(kv_pool_t* pool) {
  if (!pool) return KV_OK;
  kv_status_t st = KV_OK;
  if (pool->owned) {
    if (hipFree(pool->k) != hipSuccess) st = KV_ERR_HIP;
    if (hipFree(pool->v) != hipSuccess) st = KV_ERR_HIP;
  }
  if (pool->head_scales && hipFree(pool->head_scales) != hipSuccess) st = KV_ERR_HIP;
  delete pool;
  return st;
}

extern "C" kv_status_t kv_pool_info(const kv_pool_t* pool, void** k, void** v, size_t* bytes_each,
                                    int64_t strides[4]) {
  if (!pool) return KV_ERR_INVALID_ARG;
  if (k) *k = pool->k;
  if (v) *v = pool->v;
  if (bytes_each) *bytes_each = pool->bytes_each;
  if (strides) {
    strides[3] = 1;
    strides[2] = pool->head_dim;
    strides[1] = (int64_t)pool->block_size * pool->head_dim;
    strides[0] = (int64_t)pool->num_kv_heads * pool->block_size * pool->head_dim;
  }
  return KV_OK;
}

extern "C" kv_status_t kv_pool_set_scales(kv_pool_t* pool, float k_scale, float v_scale) {
  if (!pool || pool->dtype != KV_FP8_E4M3FN) return KV_ERR_INVALID_ARG;
  if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || k_scale > 3.0e38f || v_scale > 3.0e38f) return KV_ERR_INVALID_ARG;
  pool->k_scale = k_scale;
  pool->v_scale = v_scale;
  pool->per_head = false;
  return KV_OK;
}

extern "C" kv_status_t kv_pool_set_head_scales(kv_pool_t* pool, const float* k_scales, const float* v_scales,
                                               void* stream) {
  if (!pool || pool->dtype != KV_FP8_E4M3FN || (!k_scales) != (!v_scales)) return KV_ERR_INVALID_ARG;
  if (!k_scales) {
    pool->per_head = false;
    return KV_OK;
  }
  if (!pool->head_scales) return KV_ERR_INVALID_ARG;
  const size_t n = (size_t)pool->num_kv_heads * sizeof(float);
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(pool->head_scales, k_scales, n, hipMemcpyDeviceToDevice, s) != hipSuccess ||
      hipMemcpyAsync(pool->head_scales + pool->num_kv_heads, v_scales, n, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return KV_ERR_HIP;
  pool->per_head = true;
  return KV_OK;
}

extern "C" const char* kv_status_string(kv_status_t status) {
  switch (status) {
    case KV_OK: return "ok";
    case KV_ERR_INVALID_ARG: return "invalid argument";
    case KV_ERR_UNSUPPORTED: return "unsupported dtype/shape combination";
    case KV_ERR_OOM: return "device allocation failed";
    case KV_ERR_HIP: return "HIP runtime or launch error";
    case KV_ERR_WORKSPACE: return "workspace missing or too small";
    case KV_ERR_NO_BLOCKS: return "no free or evictable block left";
  }
  return "unknown status";
}
