// Cache writes (reshape_and_cache) and copy-on-write block copies
// (copy_blocks).
//
// Both are plain HBM streams: each lane moves 16-byte pieces, consecutive
// lanes cover consecutive bytes of one token row (write) or one block
// (copy), so every wave touches whole 1 KiB runs.
#include "common.h"

namespace {

using namespace pkv;

struct CacheWriteParams {
  uint8_t* k_pool;
  uint8_t* v_pool;
  const uint8_t* k_new;
  const uint8_t* v_new;
  const int64_t* slots;
  int64_t num_slots;       // num_blocks * block_size
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t log2_bs;
  float k_scale;
  float v_scale;
  const float* head_scales;  // [2][num_kv_heads] per-head scales (k then v), or null
};

// One lane per 16 bytes of destination row.  Rows are (token, kv head) pairs
// of head_dim elements; K rows come first, then V rows.
template <typename SRC, typename DST, int D>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteParams p) {
  constexpr int DE = elem_size<DST>::value;
  constexpr int SE = elem_size<SRC>::value;
  constexpr int VEC = 16 / DE;            // destination elements per lane
  constexpr int LPR = D * DE / 16;        // lanes per row
  const int64_t rows = (int64_t)p.num_tokens * p.num_kv_heads;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row2 = gid / LPR;
  if (row2 >= 2 * rows) return;
  const int col = (int)(gid % LPR);
  const bool is_v = row2 >= rows;
  const int64_t row = is_v ? row2 - rows : row2;
  const int64_t tok = row / p.num_kv_heads;
  const int h = (int)(row % p.num_kv_heads);
  const int64_t slot = p.slots[tok];
  if (slot < 0 || slot >= p.num_slots) return;
  const int64_t blk = slot >> p.log2_bs;
  const int64_t off = slot & ((1 << p.log2_bs) - 1);
  const int64_t dst_elem = ((blk * p.num_kv_heads + h) * (1 << p.log2_bs) + off) * D + (int64_t)col * VEC;
  const int64_t src_elem = row * D + (int64_t)col * VEC;
  uint8_t* dst = (is_v ? p.v_pool : p.k_pool) + dst_elem * DE;
  const uint8_t* src = (is_v ? p.v_new : p.k_new) + src_elem * SE;
  if constexpr (SE == DE) {
    *(uint4*)dst = *(const uint4*)src;
  } else {
    // fp8 destination: VEC = 16 codes from 16 source elements.
    static_assert(DE == 1, "only fp8 pools quantise");
    const float scale = p.head_scales ? p.head_scales[(is_v ? p.num_kv_heads : 0) + h] : (is_v ? p.v_scale : p.k_scale);
    constexpr int SW = 16 * SE / 4;  // source 32-bit words
    uint32_t w[SW];
#pragma unroll
    for (int i = 0; i < SW / 4; ++i) {
      uint4 t = ((const uint4*)src)[i];
      w[4 * i + 0] = t.x;
      w[4 * i + 1] = t.y;
      w[4 * i + 2] = t.z;
      w[4 * i + 3] = t.w;
    }
    float x[16];
#pragma unroll
    for (int i = 0; i < SW; ++i) unpack<SRC>::run(w[i], x + i * unpack<SRC>::per_word);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = f32_to_e4m3(x[4 * i + 0] / scale) | (f32_to_e4m3(x[4 * i + 1] / scale) << 8) |
             (f32_to_e4m3(x[4 * i + 2] / scale) << 16) | (f32_to_e4m3(x[4 * i + 3] / scale) << 24);
    }
    *(uint4*)dst = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

template <typename SRC, typename DST>
kv_status_t launch_write(const CacheWriteParams& p, int D, hipStream_t st) {
  const int lpr = D * elem_size<DST>::value / 16;
  const int64_t lanes = 2LL * p.num_tokens * p.num_kv_heads * lpr;
  const int64_t grid = (lanes + 255) / 256;
  if (grid > 0x7fffffff) return KV_ERR_INVALID_ARG;
  switch (D) {
    case 64: hipLaunchKernelGGL((cache_write_kernel<SRC, DST, 64>), dim3(grid), dim3(256), 0, st, p); break;
    case 128: hipLaunchKernelGGL((cache_write_kernel<SRC, DST, 128>), dim3(grid), dim3(256), 0, st, p); break;
    case 256: hipLaunchKernelGGL((cache_write_kernel<SRC, DST, 256>), dim3(grid), dim3(256), 0, st, p); break;
    default: return KV_ERR_UNSUPPORTED;
  }
  return launch_status();
}

// ------------------------------------------------------------- block copies

struct CopyParams {
  uint8_t* k_pool;
  uint8_t* v_pool;
  const int32_t* pairs;
  int32_t num_pairs;
  int32_t num_blocks;
  int64_t block_bytes;   // bytes of one block in one pool
  int32_t parts;         // work-groups per (pair, pool)
};

constexpr int kCopyUnroll = 4;  // 16-byte pieces in flight per lane
constexpr int kBufWord3 = 0x00020000;
constexpr int kNonTemporal = 2;  // cache policy: each byte is moved once
typedef unsigned u32x4 __attribute__((__vector_size__(16)));

// grid.x = num_pairs * 2 * parts: each work-group copies a contiguous share of
// one block of one pool.  Buffer descriptors bound both sides to the share,
// so the tail needs no per-lane branches (out-of-range loads read zero and
// out-of-range stores are dropped).
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyParams p) {
  const int part = blockIdx.x % p.parts;
  const int rest = blockIdx.x / p.parts;
  const int pool = rest & 1;
  const int pair = rest >> 1;
  const int32_t src = p.pairs[2 * pair];
  const int32_t dst = p.pairs[2 * pair + 1];
  if ((uint32_t)src >= (uint32_t)p.num_blocks || (uint32_t)dst >= (uint32_t)p.num_blocks) return;
  uint8_t* base = pool ? p.v_pool : p.k_pool;
  const int64_t share = ((p.block_bytes / 16 + p.parts - 1) / p.parts) * 16;
  const int64_t lo = (int64_t)part * share;
  if (lo >= p.block_bytes) return;
  const int n = (int)(lo + share < p.block_bytes ? share : p.block_bytes - lo);
  __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)src * p.block_bytes + lo), (short)0, n, kBufWord3);
  __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)dst * p.block_bytes + lo), (short)0, n, kBufWord3);
  for (int i = threadIdx.x * 16; i < n; i += 256 * 16 * kCopyUnroll) {
    u32x4 t[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      t[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, i + u * 256 * 16, 0, kNonTemporal);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(t[u], rd, i + u * 256 * 16, 0, kNonTemporal);
  }
}

// ------------------------------------------------------------ swap copies

struct SwapParams {
  uint8_t* dev_k;
  uint8_t* dev_v;
  uint8_t* host_k;        // device-accessible addresses of the host buffers
  uint8_t* host_v;
  const int32_t* pairs;
  int32_t num_pairs;
  int32_t dev_blocks;
  int64_t host_blocks;
  int64_t block_bytes;
  int32_t parts;
  int32_t out;            // 1: device -> host, 0: host -> device
};

// Same shape as copy_blocks_kernel; one side of every copy is host memory the
// device reads or writes over the host link.
__global__ __launch_bounds__(256) void swap_blocks_kernel(SwapParams p) {
  const int part = blockIdx.x % p.parts;
  const int rest = blockIdx.x / p.parts;
  const int pool = rest & 1;
  const int pair = rest >> 1;
  const int32_t src = p.pairs[2 * pair];
  const int32_t dst = p.pairs[2 * pair + 1];
  const int64_t src_n = p.out ? p.dev_blocks : p.host_blocks;
  const int64_t dst_n = p.out ? p.host_blocks : p.dev_blocks;
  if (src < 0 || src >= src_n || dst < 0 || dst >= dst_n) return;
  uint8_t* dev = pool ? p.dev_v : p.dev_k;
  uint8_t* host = pool ? p.host_v : p.host_k;
  uint8_t* sbase = p.out ? dev : host;
  uint8_t* dbase = p.out ? host : dev;
  const int64_t share = ((p.block_bytes / 16 + p.parts - 1) / p.parts) * 16;
  const int64_t lo = (int64_t)part * share;
  if (lo >= p.block_bytes) return;
  const int n = (int)(lo + share < p.block_bytes ? share : p.block_bytes - lo);
  __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(sbase + (int64_t)src * p.block_bytes + lo), (short)0, n, kBufWord3);
  __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc((void*)(dbase + (int64_t)dst * p.block_bytes + lo), (short)0, n, kBufWord3);
  for (int i = threadIdx.x * 16; i < n; i += 256 * 16 * kCopyUnroll) {
    u32x4 t[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      t[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, i + u * 256 * 16, 0, kNonTemporal);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(t[u], rd, i + u * 256 * 16, 0, kNonTemporal);
  }
}

}  // namespace

extern "C" kv_status_t swap_blocks(kv_pool_t* pool, void* host_k, void* host_v, int64_t num_host_blocks,
                                   const int32_t* pairs, int32_t num_pairs, kv_swap_dir_t direction, void* stream) {
  if (!pool || num_pairs < 0 || num_host_blocks < 0) return KV_ERR_INVALID_ARG;
  if (direction != KV_SWAP_OUT && direction != KV_SWAP_IN) return KV_ERR_INVALID_ARG;
  if (num_pairs == 0) return KV_OK;
  if (!pairs || !host_k || !host_v || num_host_blocks == 0) return KV_ERR_INVALID_ARG;
  if (((uintptr_t)host_k | (uintptr_t)host_v) & 15) return KV_ERR_INVALID_ARG;
  SwapParams p;
  p.block_bytes = (int64_t)pool->num_kv_heads * pool->block_size * pool->head_dim * elem_bytes(pool->dtype);
  if (p.block_bytes % 16 || p.block_bytes >= (1LL << 31)) return KV_ERR_UNSUPPORTED;
  if (num_host_blocks > (INT64_MAX / p.block_bytes)) return KV_ERR_INVALID_ARG;
  // the host buffers must be pinned memory mapped for this device (a failed
  // lookup's error is cleared so it does not surface at a later launch)
  void* hk = nullptr;
  void* hv = nullptr;
  if (hipHostGetDevicePointer(&hk, host_k, 0) != hipSuccess || !hk ||
      hipHostGetDevicePointer(&hv, host_v, 0) != hipSuccess || !hv) {
    (void)hipGetLastError();
    return KV_ERR_INVALID_ARG;
  }
  p.dev_k = (uint8_t*)pool->k;
  p.dev_v = (uint8_t*)pool->v;
  p.host_k = (uint8_t*)hk;
  p.host_v = (uint8_t*)hv;
  p.pairs = pairs;
  p.num_pairs = num_pairs;
  p.dev_blocks = pool->num_blocks;
  p.host_blocks = num_host_blocks;
  p.out = direction == KV_SWAP_OUT ? 1 : 0;
  int64_t parts = (p.block_bytes + 16383) / 16384;
  p.parts = (int32_t)(parts < 1 ? 1 : parts);
  const int64_t grid = (int64_t)num_pairs * 2 * p.parts;
  if (grid > 0x7fffffff) return KV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, p);
  return launch_status();
}

extern "C" kv_status_t reshape_and_cache(kv_pool_t* pool, const void* k_new, const void* v_new, kv_dtype_t src_dtype,
                                         const int64_t* slot_mapping, int32_t num_tokens, void* stream) {
  if (!pool || num_tokens < 0 || !valid_dtype(src_dtype)) return KV_ERR_INVALID_ARG;
  if (num_tokens == 0) return KV_OK;
  if (!k_new || !v_new || !slot_mapping) return KV_ERR_INVALID_ARG;
  if (((uintptr_t)k_new | (uintptr_t)v_new) & 15) return KV_ERR_INVALID_ARG;
  CacheWriteParams p;
  p.k_pool = (uint8_t*)pool->k;
  p.v_pool = (uint8_t*)pool->v;
  p.k_new = (const uint8_t*)k_new;
  p.v_new = (const uint8_t*)v_new;
  p.slots = slot_mapping;
  p.num_slots = (int64_t)pool->num_blocks * pool->block_size;
  p.num_tokens = num_tokens;
  p.num_kv_heads = pool->num_kv_heads;
  p.log2_bs = pool->log2_block_size;
  p.k_scale = pool->k_scale;
  p.v_scale = pool->v_scale;
  p.head_scales = pool->per_head ? pool->head_scales : nullptr;
  hipStream_t st = (hipStream_t)stream;
  const int D = pool->head_dim;
  if (src_dtype == pool->dtype) {
    switch (pool->dtype) {
      case KV_F32: return launch_write<f32_t, f32_t>(p, D, st);
      case KV_F16: return launch_write<f16_t, f16_t>(p, D, st);
      case KV_BF16: return launch_write<bf16_t, bf16_t>(p, D, st);
      case KV_FP8_E4M3FN: return launch_write<fp8_t, fp8_t>(p, D, st);
    }
  } else if (pool->dtype == KV_FP8_E4M3FN) {
    switch (src_dtype) {
      case KV_F32: return launch_write<f32_t, fp8_t>(p, D, st);
      case KV_F16: return launch_write<f16_t, fp8_t>(p, D, st);
      case KV_BF16: return launch_write<bf16_t, fp8_t>(p, D, st);
      default: break;
    }
  }
  return KV_ERR_UNSUPPORTED;
}

extern "C" kv_status_t copy_blocks(kv_pool_t* pool, const int32_t* pairs, int32_t num_pairs, void* stream) {
  if (!pool || num_pairs < 0) return KV_ERR_INVALID_ARG;
  if (num_pairs == 0) return KV_OK;
  if (!pairs) return KV_ERR_INVALID_ARG;
  CopyParams p;
  p.k_pool = (uint8_t*)pool->k;
  p.v_pool = (uint8_t*)pool->v;
  p.pairs = pairs;
  p.num_pairs = num_pairs;
  p.num_blocks = pool->num_blocks;
  p.block_bytes = (int64_t)pool->num_kv_heads * pool->block_size * pool->head_dim * elem_bytes(pool->dtype);
  // about 16 KiB per work-group (one round of 4 x 16 bytes per lane); a
  // buffer descriptor spans at most 2 GiB
  if (p.block_bytes % 16 || p.block_bytes >= (1LL << 31)) return KV_ERR_UNSUPPORTED;
  int64_t parts = (p.block_bytes + 16383) / 16384;
  p.parts = (int32_t)(parts < 1 ? 1 : parts);
  const int64_t grid = (int64_t)num_pairs * 2 * p.parts;
  if (grid > 0x7fffffff) return KV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, p);
  return launch_status();
}
