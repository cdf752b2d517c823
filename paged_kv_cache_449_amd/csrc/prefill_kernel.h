// Paged attention for several new query tokens per sequence (chunked prefill,
// or verifying speculative tokens), on the matrix cores.
//
// What it computes: sequence s owns query rows [query_start[s],
// query_start[s+1]); its m new tokens are the last m of its n cached tokens
// (their K/V written by reshape_and_cache), so query row i sits at position
// n - m + (i - query_start[s]) and attends causally to tokens 0..position,
// read through the block table exactly as in decode.
//
// Row tiles.  The rows of one (sequence, kv head) pair are (new token, query
// head) pairs; 16 of them -- Q = 16 / G consecutive tokens times the G query
// heads of the kv head -- form a row tile, the 16 query rows of one
// matrix-core run.  Row j of tile r is token r*Q + j / G, head j % G; it
// masks tokens past its own position.  A tile reads the blocks up to the
// position of its last token.
//
// Work split.  Tiles are streamed like decode runs: the blocks of all
// (kv head, sequence, tile) runs are laid end to end and cut into equal
// chunks, one per worker wavefront; runs cut between chunks are merged by the
// last-arriving chunk (16-row records).
#pragma once

#include "decode_kernel.h"

namespace pkv {

// Out rows of a tile's records: row j is token q0 + j / G (valid while
// j / G < m_left), query head hG + j % G.
struct TokenRows {
  int64_t q0;
  int m_left;
  int hq;
  int hG;
  int g;
  int d;
  __device__ int64_t operator()(int j) const {
    const int tok = j / g;
    if (tok >= m_left) return -1;
    return ((q0 + tok) * hq + hG + j % g) * (int64_t)d;
  }
};

// Tokens a tile reads: the position of its last token + 1.
__device__ inline int tile_limit(int n, int m, int Q, int r) { return n - m + min((r + 1) * Q, m); }

// Blocks of all row tiles of a sequence with n cached tokens, m of them new
// (at most ceil(total_q / Q) tiles of at most max_blocks blocks: the host
// bounds that product by 2^30).
__device__ inline int sequence_tile_blocks(int n, int m, int Q, int log2_bs) {
  const int bs = 1 << log2_bs;
  int tot = 0;
  for (int r = 0; r * Q < m; ++r) tot += (tile_limit(n, m, Q, r) + bs - 1) >> log2_bs;
  return tot;
}

// Context length n, new-token count m and first query row q0 of sequence s,
// clamped so that 0 <= m <= n and rows q0 .. q0 + m - 1 lie in [0, total_q):
// an inconsistent query_start yields wrong rows, never an access outside q
// or out.
__device__ inline void prefill_lengths(const DecodeParams& p, int s, int max_len, int& n, int& m, int& q0) {
  n = clamp_len(p.context_lens[s], max_len);
  const int a = min(max(p.query_start[s], 0), p.total_q);
  const int b = min(max(p.query_start[s + 1], a), p.total_q);
  q0 = a;
  m = min(b - a, n);
}

template <typename KV, typename QT, int D, int G>
__device__ inline void prefill_run(const DecodeParams& p, int w, int chunk, int wstart, int pos, int s, int h, int r,
                                   int off, int len, int n, int m, int qs) {
  constexpr int Q = 16 / G;
  const int Hq = p.num_kv_heads * G;
  const int j16 = threadIdx.x & 15;
  const int q0 = qs + r * Q;
  const int tok = j16 / G;              // token within the tile
  const int lim = tile_limit(n, m, Q, r);
  const int nb = (lim + (1 << p.log2_bs) - 1) >> p.log2_bs;
  MfmaRow row;
  row.valid = r * Q + tok < m;
  row.qoff = ((int64_t)(q0 + tok) * Hq + (int64_t)h * G + j16 % G) * D;
  row.limit = n - m + r * Q + tok + 1;
  const TokenRows rows{q0, m - r * Q, Hq, h * G, G, D};
  mfma_rows_run<KV, QT, D, 16, kStreamPolicy>(p, w, chunk, wstart, pos, s, h, off, len, lim, nb, row, rows);
}

// Chunk v of the (kv head, sequence, tile, block) stream, `total` blocks per
// kv head and T in all.
template <typename KV, typename QT, int D, int G>
__device__ inline void prefill_chunk(const DecodeParams& p, int v, int chunk, int T, int total) {
  constexpr int Q = 16 / G;
  const int lane = threadIdx.x;
  const int S = p.num_seqs;
  const int max_len = p.max_blocks << p.log2_bs;
  const int start = v * chunk;
  if (start >= T) return;
  const int end = min(start + chunk, T);
  int h = start / total;
  const int rr = start - h * total;

  // the sequence whose tiles contain block rr of kv head h
  int s = 0, pre = 0;
  bool found = false;
  {
    int carry = 0;
    for (int base = 0; base < S; base += 64) {
      const int sl = base + lane;
      int nb = 0;
      if (sl < S) {
        int n, m, q0;
        prefill_lengths(p, sl, max_len, n, m, q0);
        nb = sequence_tile_blocks(n, m, Q, p.log2_bs);
      }
      const int incl = wave_inclusive_scan_i32(nb, lane);
      const int excl = carry + incl - nb;
      const unsigned long long hit = __ballot(nb > 0 && excl <= rr && rr < excl + nb);
      if (hit) {
        const int src = __builtin_ctzll(hit);
        s = base + src;
        pre = __shfl(excl, src);
        found = true;
        break;
      }
      carry += __shfl(incl, 63);
    }
  }
  if (!found) return;  // lengths changed under the launch: nothing consistent to do
  s = uniform(s);
  int n, m, qs;
  prefill_lengths(p, s, max_len, n, m, qs);
  n = uniform(n);
  m = uniform(m);
  qs = uniform(qs);
  // the tile of s holding offset rr - pre
  int r = 0, off = uniform(rr - pre);
  for (;;) {
    const int nb = (tile_limit(n, m, Q, r) + (1 << p.log2_bs) - 1) >> p.log2_bs;
    if (off < nb) break;
    off -= nb;
    ++r;
  }
  int pos = start;
  while (true) {
    const int nb = (tile_limit(n, m, Q, r) + (1 << p.log2_bs) - 1) >> p.log2_bs;
    const int len = min(nb - off, end - pos);
    prefill_run<KV, QT, D, G>(p, v, chunk, start, pos, s, h, r, off, len, n, m, qs);
    pos += len;
    if (pos >= end) break;
    off = 0;
    if ((++r) * Q < m) continue;
    r = 0;
    do {
      if (++s == S) {
        s = 0;
        if (++h == p.num_kv_heads) return;
      }
      prefill_lengths(p, s, max_len, n, m, qs);
      n = uniform(n);
      m = uniform(m);
      qs = uniform(qs);
    } while (m == 0);
  }
}

template <typename KV, typename QT, int D, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void paged_prefill_kernel(const DecodeParams p) {
  constexpr int Q = 16 / G;
  const int lane = threadIdx.x;
  const int S = p.num_seqs;
  const int max_len = p.max_blocks << p.log2_bs;
  // Host checks bound the stream of a consistent query_start by 2^30 blocks;
  // an inconsistent one can exceed that, and then nothing is computed.
  int64_t total64 = 0;
  for (int base = 0; base < S; base += 64) {
    const int s = base + lane;
    int nb = 0;
    if (s < S) {
      int n, m, q0;
      prefill_lengths(p, s, max_len, n, m, q0);
      nb = sequence_tile_blocks(n, m, Q, p.log2_bs);
    }
    total64 += wave_sum_i64(nb);   // the same in every lane
    if (total64 * p.num_kv_heads > (1LL << 30)) return;
  }
  const int total = uniform((int)total64);
  const int T = total * p.num_kv_heads;
  if (T == 0) return;
  // chunks spread over the 8 XCDs as in decode (one round)
  const int chunk = max(1, (T + p.num_workers - 1) / p.num_workers);
  const int nv = (T + chunk - 1) / chunk;
  const int per_round = (nv + 7) & ~7;   // <= num_workers
  if ((int)blockIdx.x >= per_round) return;
  const int v = (int)(blockIdx.x & 7) * (per_round >> 3) + (int)(blockIdx.x >> 3);
  if (v >= nv) return;
  prefill_chunk<KV, QT, D, G>(p, v, chunk, T, total);
}

template <typename KV, typename QT>
kv_status_t launch_prefill(const DecodeParams& p, int D, int G, hipStream_t stream) {
#define PKV_PCASE(DD, GG)                                                                                     \
  if (D == DD && G == GG) {                                                                                   \
    hipLaunchKernelGGL((paged_prefill_kernel<KV, QT, DD, GG>), dim3(p.num_workers), dim3(64), 0, stream, p); \
    return launch_status();                                                                                   \
  }
#define PKV_PCASES(DD) PKV_PCASE(DD, 1) PKV_PCASE(DD, 2) PKV_PCASE(DD, 4) PKV_PCASE(DD, 8) PKV_PCASE(DD, 16)
  PKV_PCASES(64)
  PKV_PCASES(128)
  PKV_PCASES(256)
#undef PKV_PCASES
#undef PKV_PCASE
  return KV_ERR_UNSUPPORTED;
}

kv_status_t launch_prefill_bf16_bf16(const DecodeParams& p, int D, int G, hipStream_t s);
kv_status_t launch_prefill_f16_f16(const DecodeParams& p, int D, int G, hipStream_t s);
kv_status_t launch_prefill_fp8_bf16(const DecodeParams& p, int D, int G, hipStream_t s);
kv_status_t launch_prefill_fp8_f16(const DecodeParams& p, int D, int G, hipStream_t s);

}  // namespace pkv
