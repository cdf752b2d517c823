// Internal declarations shared by the HIP translation units of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

struct kv_pool {
  int32_t num_blocks;
  int32_t block_size;
  int32_t log2_block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  kv_dtype_t dtype;
  void* k;
  void* v;
  size_t bytes_each;
  bool owned;
  float k_scale;
  float v_scale;
  float* head_scales;   // device [2][num_kv_heads] (k then v) fp8 per-head scales, allocated with the pool
  bool per_head;        // head_scales in use
  int device;
  int num_cus;
  // dispatch settings, read from the environment once when the pool is made
  int decode_waves_per_cu;  // PAGEDKV_DECODE_WAVES_PER_CU (default 8)
  bool decode_mfma;         // PAGEDKV_DECODE_MFMA=0 keeps query groups on the vector ALUs
  int prefill_shape;        // PAGEDKV_PREFILL_PATH: -1 auto, 0 wave, 1 group, 2 unit
};

namespace pkv {

inline size_t elem_bytes(kv_dtype_t dt) {
  switch (dt) {
    case KV_F32: return 4;
    case KV_F16: return 2;
    case KV_BF16: return 2;
    case KV_FP8_E4M3FN: return 1;
  }
  return 0;
}

inline bool valid_dtype(int dt) { return dt >= KV_F32 && dt <= KV_FP8_E4M3FN; }

inline int ilog2_exact(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return (1 << r) == x ? r : -1;
}

inline kv_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

// ------------------------------------------------------------ device helpers

// Element storage types: the kernels move raw bits and convert in registers.
struct f32_t { using bits = uint32_t; };
struct f16_t { using bits = uint16_t; };
struct bf16_t { using bits = uint16_t; };
struct fp8_t { using bits = uint8_t; };

template <typename T> struct elem_size;
template <> struct elem_size<f32_t> { static constexpr int value = 4; };
template <> struct elem_size<f16_t> { static constexpr int value = 2; };
template <> struct elem_size<bf16_t> { static constexpr int value = 2; };
template <> struct elem_size<fp8_t> { static constexpr int value = 1; };

typedef float float2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Widen the elements packed in one 32-bit word to fp32 (exact for all types).
template <typename T> struct unpack;
template <> struct unpack<f32_t> {
  static constexpr int per_word = 1;
  __device__ static inline void run(uint32_t w, float* o) { o[0] = __uint_as_float(w); }
};
template <> struct unpack<f16_t> {
  static constexpr int per_word = 2;
  __device__ static inline void run(uint32_t w, float* o) {
    half2v h = __builtin_bit_cast(half2v, w);
    o[0] = (float)h.x;
    o[1] = (float)h.y;
  }
};
template <> struct unpack<bf16_t> {
  static constexpr int per_word = 2;
  __device__ static inline void run(uint32_t w, float* o) {
    o[0] = __uint_as_float(w << 16);
    o[1] = __uint_as_float(w & 0xffff0000u);
  }
};
template <> struct unpack<fp8_t> {
  static constexpr int per_word = 4;
  __device__ static inline void run(uint32_t w, float* o) {
    // gfx950 converts OCP E4M3FN codes exactly (bytes 0,1 then 2,3).
    float2v a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    float2v b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    o[0] = a.x;
    o[1] = a.y;
    o[2] = b.x;
    o[3] = b.y;
  }
};

// Scalar element load/store in fp32 (used outside the streaming loops).
template <typename T> __device__ inline float load_f32(const void* base, int64_t i);
template <> __device__ inline float load_f32<f32_t>(const void* base, int64_t i) {
  return ((const float*)base)[i];
}
template <> __device__ inline float load_f32<f16_t>(const void* base, int64_t i) {
  return (float)((const _Float16*)base)[i];
}
template <> __device__ inline float load_f32<bf16_t>(const void* base, int64_t i) {
  return __uint_as_float((uint32_t)((const uint16_t*)base)[i] << 16);
}

// fp32 -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ inline uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct pack_out;
template <> struct pack_out<f32_t> {
  static constexpr int per_word = 1;
  __device__ static inline uint32_t run(const float* v) { return __float_as_uint(v[0]); }
};
template <> struct pack_out<f16_t> {
  static constexpr int per_word = 2;
  __device__ static inline uint32_t run(const float* v) {
    half2v h;
    h.x = (_Float16)v[0];
    h.y = (_Float16)v[1];
    return __builtin_bit_cast(uint32_t, h);
  }
};
template <> struct pack_out<bf16_t> {
  static constexpr int per_word = 2;
  __device__ static inline uint32_t run(const float* v) {
    return (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
  }
};

// fp32 -> OCP E4M3FN code, round to nearest even, saturating to +-448.
// NaN -> 0x7F.  Built from the format's definition: below 2^-6 the code is
// the integer nearest to |x| * 2^9; above, the exponent is taken from the
// fp32 exponent and the 3-bit fraction is the nearest integer to
// |x| * 2^(3-e) - 8, with a carry into the exponent when it rounds up to 8.
__device__ inline uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fu;
  float a = __uint_as_float(u & 0x7fffffffu);
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) {  // below the smallest normal, 2^-6
    int r = (int)__builtin_rintf(a * 512.0f);
    return sign | (uint32_t)r;
  }
  int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;  // -6 .. 8
  int r = (int)__builtin_rintf(__builtin_ldexpf(a, 3 - e)); // 8 .. 16
  if (r == 16) {
    r = 8;
    e += 1;
  }
  return sign | (uint32_t)((e + 7) << 3) | (uint32_t)(r - 8);
}

// Sum over aligned groups of N lanes (N = 1..64); every lane of a group gets
// the group's sum.  Within a 16-lane row the butterfly uses DPP (quad
// permutes, then half-row and row mirrors); across rows it uses lane permutes.
template <int N> __device__ inline float group_sum(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  if constexpr (N >= 2)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  if constexpr (N >= 4)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  if constexpr (N >= 8)  // row_half_mirror: lane i <-> 7-i within 8 lanes
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  if constexpr (N >= 16)  // row_mirror: lane i <-> 15-i within 16 lanes
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

__device__ inline int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ inline int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ inline int wave_inclusive_scan_i32(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

}  // namespace pkv
