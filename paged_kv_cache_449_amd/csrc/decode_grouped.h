// Prefix-grouped decode: sequences forked from one prompt (parallel
// sampling) share the prompt's blocks, so their decode attention reads the
// same K/V.  Grouped, the shared prefix is read once per group: the group's
// candidates (times the query heads of a kv head) are the rows of one
// matrix-core run, and only each candidate's own suffix is read per
// sequence.
//
// Two launches on the caller's stream:
//   1. shared kernel: one wave per (kv head, group) runs the shared prefix
//      (the group's first shared_len tokens) for all members and leaves each
//      row's unnormalised state (acc, reference max, sum) in the workspace;
//   2. suffix kernel: one wave per (sequence, kv head) starts from that
//      state, streams the sequence's remaining tokens on the vector ALUs and
//      writes the output.
// The result is the decode attention of every sequence over its whole
// context, as paged_attention_decode computes it.
#pragma once

#include "decode_kernel.h"

namespace pkv {

// Group g of sequences [gs, ge) and its shared token count: whole blocks,
// clamped so that it never passes a member's context, and only members that
// fit the matrix-core rows (16 / G) take part.  Both kernels compute it the
// same way; members left out stream their whole context in the suffix
// kernel.
struct GroupInfo {
  int gs, ge;      // members taking part: [gs, ge)
  int shared;      // tokens of the shared prefix (0: none)
};

__device__ inline GroupInfo group_info(const DecodeParams& p, const int32_t* group_start, const int32_t* group_shared,
                                       int g, int max_members) {
  const int S = p.num_seqs;
  const int max_len = p.max_blocks << p.log2_bs;
  GroupInfo gi;
  gi.gs = min(max(group_start[g], 0), S);
  const int end = min(max(group_start[g + 1], gi.gs), S);
  gi.ge = min(end, gi.gs + max_members);
  int shared = min(max(group_shared[g], 0), p.max_blocks) << p.log2_bs;
  for (int s = gi.gs; s < gi.ge; ++s) shared = min(shared, clamp_len(p.context_lens[s], max_len));
  // whole blocks only: each member's own tokens start at a block boundary
  gi.shared = gi.ge > gi.gs ? (shared >> p.log2_bs) << p.log2_bs : 0;
  return gi;
}

template <typename KV, typename QT, int D, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void paged_decode_shared_kernel(const DecodeParams p, const int32_t* group_start, const int32_t* group_shared,
                                int num_groups) {
  const int u = (int)blockIdx.x;
  const int h = u / num_groups;
  const int g = u - h * num_groups;
  if (h >= p.num_kv_heads) return;
  const GroupInfo gi = group_info(p, group_start, group_shared, g, 16 / G);
  const int members = gi.ge - gi.gs;
  const int j16 = threadIdx.x & 15;
  const int Hq = p.num_kv_heads * G;
  const int mem = j16 / G;                     // member of row j16
  MfmaRow row;
  row.valid = mem < members;
  const int64_t qrow = (int64_t)(gi.gs + mem) * Hq + (int64_t)h * G + j16 % G;
  row.qoff = qrow * D;
  row.part = qrow;
  row.limit = gi.shared;
  row.min_limit = gi.shared;
  if (gi.shared == 0) return;   // nothing shared: the suffix kernel reads the whole context
  const int nb = gi.shared >> p.log2_bs;
  mfma_rows_run<KV, QT, D, 16, kStreamPolicy, ContiguousRows, true>(p, 0, uniform_grid(1), 0, 0, gi.gs, h, 0, nb,
                                                                   gi.shared, nb, row, ContiguousRows{0, D});
}

template <typename KV, typename QT, int D, int G>
__global__ __launch_bounds__(64) void paged_decode_suffix_kernel(const DecodeParams p, const int32_t* group_start,
                                                                 const int32_t* group_shared, int num_groups) {
  using Sh = DecodeShape<KV, D>;
  constexpr int VEC = Sh::VEC, L = Sh::L;
  constexpr int QE = elem_size<QT>::value;
  const int S = p.num_seqs;
  const int s = (int)blockIdx.x / p.num_kv_heads;
  const int h = (int)blockIdx.x - s * p.num_kv_heads;
  if (s >= S) return;
  const int lane = threadIdx.x;
  const int row = lane / L;
  const int col = lane % L;
  const int Hq = p.num_kv_heads * G;
  const int max_len = p.max_blocks << p.log2_bs;
  const int n = clamp_len(p.context_lens[s], max_len);

  // the group of s (group_start ascending: the last start <= s)
  int lo = 0, hi = num_groups;   // search [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (group_start[mid] <= s) lo = mid; else hi = mid;
  }
  int shared = 0;
  if (num_groups > 0) {
    const GroupInfo gi = group_info(p, group_start, group_shared, lo, 16 / G);
    if (s >= gi.gs && s < gi.ge) shared = gi.shared;
  }

  const int bs = 1 << p.log2_bs;
  const int off = shared >> p.log2_bs;   // shared is a whole number of blocks, at most n
  const int nb = (n + bs - 1) >> p.log2_bs;
  const int tab = nb > off ? load_table_window(p, run_table(p, s, off), 0, nb - off) : -1;
  const float qs = run_q_scale(p, h), vs = run_v_scale(p, h);
  float qv[G][VEC];
  {
    const int64_t qe = ((int64_t)s * Hq + (int64_t)h * G) * D + (int64_t)col * VEC;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      load_row_f32<QT, VEC>(p.q + (qe + (int64_t)g * D) * QE, qv[g]);
#pragma unroll
      for (int i = 0; i < VEC; ++i) qv[g][i] *= qs;
    }
  }
  // start from the shared prefix's state in row group 0; the other row
  // groups start empty and are merged below
  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[g][i] = 0.0f;
    if (shared > 0 && row == 0) {
      const float* rec = p.partials + ((int64_t)s * Hq + (int64_t)h * G + g) * (D + 4);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[g][i] = rec[col * VEC + i];
      m[g] = rec[D];
      l[g] = rec[D + 1];
    }
  }
  if (shared < n && nb > off) valu_stream<KV, D, G, kStreamPolicy>(p, s, h, off, nb - off, n, tab, qv, m, l, acc);

#pragma unroll
  for (int o = L; o < 64; o <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], o);
      const float lo2 = __shfl_xor(l[g], o);
      const float mn = fmaxf(m[g], mo);
      const float mu = mn == -INFINITY ? 0.0f : mn;
      const float a = fexp2(m[g] - mu), b = fexp2(mo - mu);
      l[g] = l[g] * a + lo2 * b;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[g][i] = acc[g][i] * a + __shfl_xor(acc[g][i], o) * b;
      m[g] = mn;
    }
  }
  if (row == 0) {
    const int64_t oe = ((int64_t)s * Hq + (int64_t)h * G) * D + (int64_t)col * VEC;
#pragma unroll
    for (int g = 0; g < G; ++g)
      store_row<QT, VEC>(p.out + (oe + (int64_t)g * D) * QE, acc[g], l[g] > 0.0f ? vs / l[g] : 0.0f);
  }
}

template <typename KV, typename QT>
kv_status_t launch_grouped(const DecodeParams& p, int D, int G, const int32_t* group_start,
                           const int32_t* group_shared, int num_groups, hipStream_t stream) {
#define PKV_GCASE(DD, GG)                                                                                          \
  if (D == DD && G == GG) {                                                                                        \
    if (num_groups > 0) {                                                                                          \
      hipLaunchKernelGGL((paged_decode_shared_kernel<KV, QT, DD, GG>), dim3(p.num_kv_heads * num_groups), dim3(64), \
                         0, stream, p, group_start, group_shared, num_groups);                                     \
      const kv_status_t st = launch_status();                                                                      \
      if (st != KV_OK) return st;                                                                                  \
    }                                                                                                              \
    hipLaunchKernelGGL((paged_decode_suffix_kernel<KV, QT, DD, GG>), dim3(p.num_seqs * p.num_kv_heads), dim3(64), 0, \
                       stream, p, group_start, group_shared, num_groups);                                          \
    return launch_status();                                                                                        \
  }
#define PKV_GCASES(DD) PKV_GCASE(DD, 1) PKV_GCASE(DD, 2) PKV_GCASE(DD, 4) PKV_GCASE(DD, 8) PKV_GCASE(DD, 16)
  PKV_GCASES(64)
  PKV_GCASES(128)
  PKV_GCASES(256)
#undef PKV_GCASES
#undef PKV_GCASE
  return KV_ERR_UNSUPPORTED;
}

kv_status_t launch_grouped_bf16_bf16(const DecodeParams& p, int D, int G, const int32_t* gs, const int32_t* gsh,
                                     int ng, hipStream_t s);
kv_status_t launch_grouped_f16_f16(const DecodeParams& p, int D, int G, const int32_t* gs, const int32_t* gsh,
                                   int ng, hipStream_t s);
kv_status_t launch_grouped_fp8_bf16(const DecodeParams& p, int D, int G, const int32_t* gs, const int32_t* gsh,
                                    int ng, hipStream_t s);
kv_status_t launch_grouped_fp8_f16(const DecodeParams& p, int D, int G, const int32_t* gs, const int32_t* gsh,
                                   int ng, hipStream_t s);

}  // namespace pkv
