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

// Per-lane sequence tile blocks of the four 64-sequence slices from base
// (0 past S), with every length load issued before any is used: the scans
// below take one memory round trip per 256 sequences.
__device__ inline void slice_tile_blocks4(const DecodeParams& p, int base, int max_len, int Q, int (&nb)[4]) {
  const int lane = (int)(threadIdx.x & 63);
  const int S = p.num_seqs;
  int cl[4], qa[4], qb[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int sc = min(base + 64 * k + lane, S - 1);
    cl[k] = p.context_lens[sc];
    qa[k] = p.query_start[sc];
    qb[k] = p.query_start[sc + 1];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int n = clamp_len(cl[k], max_len);
    const int a = min(max(qa[k], 0), p.total_q);
    const int b = min(max(qb[k], a), p.total_q);
    nb[k] = base + 64 * k + lane < S ? sequence_tile_blocks(n, min(b - a, n), Q, p.log2_bs) : 0;
  }
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
  row.min_limit = n - m + r * Q + 1;   // the tile's first row
  const TokenRows rows{q0, m - r * Q, Hq, h * G, G, D};
  mfma_rows_run<KV, QT, D, 16, kStreamPolicy>(p, w, uniform_grid(chunk), wstart, pos, s, h, off, len, lim, nb, row,
                                              rows);
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
    for (int base = 0; base < S && !found; base += 4 * 64) {
      int nbs[4];
      slice_tile_blocks4(p, base, max_len, Q, nbs);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (found) break;
        const int nb = nbs[k];
        const int incl = wave_inclusive_scan_i32(nb, lane);
        const int excl = carry + incl - nb;
        const unsigned long long hit = __ballot(nb > 0 && excl <= rr && rr < excl + nb);
        if (hit) {
          const int src = __builtin_ctzll(hit);
          s = base + 64 * k + src;
          pre = __shfl(excl, src);
          found = true;
        }
        carry += __shfl(incl, 63);
      }
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
  const int S = p.num_seqs;
  const int max_len = p.max_blocks << p.log2_bs;
  // Host checks bound the stream of a consistent query_start by 2^30 blocks;
  // an inconsistent one can exceed that, and then nothing is computed.
  int64_t total64 = 0;
  for (int base = 0; base < S; base += 4 * 64) {
    int nbs[4];
    slice_tile_blocks4(p, base, max_len, Q, nbs);
#pragma unroll
    for (int k = 0; k < 4; ++k) total64 += wave_sum_i64(nbs[k]);   // the same in every lane
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

// ------------------------------------------------------------------------
// Work-group variant for long chunks.  Four waves share one (sequence, kv
// head) row block of 4 row tiles (64 rows): each 64-token step, wave w loads
// tile w of the step into its own LDS slot, and after one barrier every wave
// runs its 16 rows against all four tiles.  A block of K/V is then read once
// per 64 rows instead of once per 16, and each wave issues a quarter of the
// loads.  The stream is the (kv head, sequence, row block, block) sequence;
// split row blocks leave 64-row records that the last-arriving work-group
// merges with all its threads.

// Waves per work-group and 16-row tiles per wave of the split work-groups:
// 8 x 1 (128-row blocks) for head dim up to 128, 4 x 1 (64-row blocks) for
// head dim 256, whose two LDS buffers of 8 tiles would not fit.
template <int D>
constexpr int wg_waves() { return D <= 128 ? 8 : 4; }
template <int D>
constexpr int wg_row_tiles() { return 1; }
// rows per block
template <int D>
constexpr int wg_rows() { return 16 * wg_waves<D>() * wg_row_tiles<D>(); }
constexpr int kMaxWgRows = 128;   // records are sized for the largest block
constexpr int kTileGroup = 4;     // tiles a wave computes together

// The one-work-group-per-block kernel takes the same 128-row blocks as
// 4 waves x 2 row tiles for head dim up to 128: every K and V word a wave
// reads from LDS then feeds 32 rows, and two work-groups share a CU (two
// waves per SIMD, 240-248 VGPRs).  On MI355X that took the chunked-prefill
// workload from 770 to 702 us and the fp8 GQA chunks from 427 to 373 us.
// Every pool computes 4 tiles together (one group per 64-token step):
// with one f16 P operand and the row sums on the matrix cores the 16-bit
// loop fits the 256-VGPR cap at 4 as well, and ran 2-3% faster than 2 on
// the chunked-prefill batch.  The split work-groups keep 8 x 1: their
// merge code would spill at that cap.
template <int D>
constexpr int unit_waves() { return D <= 128 ? 4 : wg_waves<D>(); }
template <int D>
constexpr int unit_row_tiles() { return D <= 128 ? 2 : 1; }
template <typename KV, int D>
constexpr int unit_tile_group() { return 4; }

// Out rows of a row block's records: row j is row tile waves * rb + j / 16
// (waves: row tiles per block), slot j % 16 of it.
struct BlockRows {
  int64_t qs;      // the sequence's first query row
  int waves;       // row tiles per block
  int rb;
  int m;
  int q;           // tokens per row tile (16 / G)
  int hq;
  int hG;
  int g;
  int d;
  __device__ int64_t operator()(int j) const {
    const int r = waves * rb + j / 16;
    const int tok = r * q + (j % 16) / g;
    if (tok >= m) return -1;
    return ((qs + tok) * hq + hG + (j % 16) % g) * (int64_t)d;
  }
};

// Blocks of all row blocks of a sequence with n cached tokens, m of them new.
__device__ inline int sequence_rowblock_blocks(int n, int m, int QB, int log2_bs) {
  const int bs = 1 << log2_bs;
  int tot = 0;
  for (int rb = 0; rb * QB < m; ++rb) tot += (tile_limit(n, m, QB, rb) + bs - 1) >> log2_bs;
  return tot;
}

// LDS of a work-group's two staging buffers (V then K).
template <int VSLOTS, int KSLOTS>
__device__ inline uint8_t* wg_stage_lds() {
  __shared__ __attribute__((aligned(16))) uint8_t buf[2 * (VSLOTS + KSLOTS)];
  return buf;
}

// W waves of RT 16-row tiles each; TG tiles computed together.
//
// F16V (bf16 pools): V is staged in LDS as f16 and P is one f16 operand, as
// for fp8 and f16 pools.  bf16 -> f16 is exact for every |v| below 65520
// except in f16's subnormal range (|v| < 2^-14, absolute error at most
// 2^-25); a wave that stages a value of magnitude 65536 or more (or a NaN)
// flags it, and then the work-group returns false before storing anything,
// for the caller to run the block again with F16V off (bf16 V, split P).
template <typename KV, typename QT, int D, int G, int W, int RT, int TG, bool F16V = false>
__device__ inline bool prefill_wg_run(const DecodeParams& p, int w, int chunk, int wstart, int pos, int s, int h,
                                      int rb, int off, int len, int n, int m, int qs) {
  using MT = typename mfma_operand<KV, QT>::type;
  using Ops = mfma_ops<MT>;
  static_assert(!F16V || std::is_same<KV, bf16_t>::value, "f16 staging converts bf16 pools");
  using PT = typename std::conditional<F16V, f16_t, typename pv_operand<KV, MT>::type>::type;
  using PVOps = mfma_ops<PT>;
  constexpr bool kSplitP = !F16V && pv_operand<KV, MT>::split;
  using Sh = MfmaShape<KV, D>;
  constexpr int kTileGroup = TG;
  static_assert(TG == 2 || TG == 4, "tiles computed together");
  constexpr int TB = W * RT;              // row tiles per block
  constexpr int Q = 16 / G;
  constexpr int KS = Sh::KS, DT = Sh::DT, LSTRIDE = Sh::LSTRIDE, KSTRIDE = Sh::KSTRIDE;
  constexpr int QE = elem_size<QT>::value;
  constexpr int VBYTES = 16 * LSTRIDE, KBYTES = 16 * KSTRIDE;
  // two buffers of W tile slots: step st computes from buffer st & 1
  // while the waves stage step st + 1 into the other (shared by both F16V
  // forms of a block: V elements are two bytes either way)
  uint8_t* const vbuf = wg_stage_lds<W * VBYTES, W * KBYTES>();
  uint8_t* const kbuf = vbuf + 2 * W * VBYTES;
  __shared__ int last_flag;

  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // uniform: scalar LDS slot bases
  const int lane = (int)(threadIdx.x & 63);
  const int j16 = lane & 15;
  const int kg = lane >> 4;
  const int Hq = p.num_kv_heads * G;
  const float qsc = run_q_scale(p, h), vsc = run_v_scale(p, h);
  // Scores are scaled inside the exponent, exp2(sc * qabs - mu), and their
  // max is taken before scaling, which needs a positive scale: a negative
  // one flips the sign of the q operand instead (exact).  A zero scale
  // becomes 1e-30, under which every score still rounds to exp2(0) = 1 and
  // masked ones stay -inf.
  const float qabs = fmaxf(fabsf(qsc), 1e-30f);
  const uint32_t qflip = qsc < 0.0f ? 0x80008000u : 0u;

  // this wave's rows: row tiles TB rb + RT wave + t, t < RT
  int tok[RT], limit[RT];
  bool valid[RT];
  int64_t qoff[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int r = TB * rb + RT * wave + t;
    tok[t] = r * Q + j16 / G;
    valid[t] = tok[t] < m;
    qoff[t] = ((int64_t)(qs + tok[t]) * Hq + (int64_t)h * G + j16 % G) * D;
    limit[t] = n - m + tok[t] + 1;
  }
  const int lim_blk = tile_limit(n, m, TB * Q, rb);   // tokens the row block reads
  const int first_limit = n - m + TB * rb * Q + 1;     // smallest causal limit of the block's rows
  const int nb = (lim_blk + (1 << p.log2_bs) - 1) >> p.log2_bs;

  uint4 qop[RT][KS];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int k = 0; k < KS; ++k) qop[t][k] = make_uint4(0u, 0u, 0u, 0u);
    if (valid[t]) {
      const int64_t qe = qoff[t] + kg * (D / 4);
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const uint4 w4 = *(const uint4*)(p.q + (qe + k * 8) * QE);
        qop[t][k] = make_uint4(w4.x ^ qflip, w4.y ^ qflip, w4.z ^ qflip, w4.w ^ qflip);
      }
    }
  }

  f32x4 acc[RT][DT];
  float mx_run[RT], mu[RT];   // reference max, the same as an exponent offset (0 while -inf)
  // Row sums on the matrix cores: P times a tile of ones, alongside PV, so
  // the sum is of the very weights PV used and needs no cross-lane
  // reduction (every element of lsum[t] holds the row's whole sum).
  f32x4 lsum[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[t][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    mx_run[t] = -INFINITY;
    mu[t] = 0.0f;
    lsum[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  RunCtx c;
  const int64_t tile = (int64_t)Sh::ROW << p.log2_bs;
  c.k_head = p.k_pool + tile * h;
  c.v_head = p.v_pool + tile * h;
  c.blk_stride = tile * p.num_kv_heads;
  c.tile_bytes = (uint32_t)tile;
  c.lane_off = 0;
  c.row_bytes = Sh::ROW;
  c.log2_bs = p.log2_bs;
  c.bs_mask = (1 << p.log2_bs) - 1;
  const int32_t* trow = p.block_tables + (int64_t)s * p.max_blocks + off;

  // this wave's tile of a step, into slot `wave` of buffer `buf`
  float big = 0.0f;   // F16V: max |v| staged (NaN if a NaN was)
  auto stage = [&](const MfmaTileRegs<KV, D>& t, int buf) {
    const int slot = __builtin_amdgcn_readfirstlane(buf * W + wave);   // scalar slot bases
    uint8_t* vb = vbuf + slot * VBYTES;
    uint8_t* kb = kbuf + slot * KBYTES;
#pragma unroll
    for (int u = 0; u < Sh::VL; ++u) {
      const int byte = (u * 64 + lane) * 16;
      const int vr = byte / Sh::ROW, ve = (byte % Sh::ROW) / Sh::EB;
      uint8_t* dst = vb + vr * LSTRIDE + ve * 2;
      if constexpr (F16V) {
        const uint32_t wv[4] = {t.v[u].x, t.v[u].y, t.v[u].z, t.v[u].w};
        uint32_t hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = __uint_as_float(wv[i] << 16), hi = __uint_as_float(wv[i] & 0xffff0000u);
          big = __builtin_elementwise_maximum(__builtin_elementwise_maximum(big, fabsf(lo)), fabsf(hi));
          hv[i] = PVOps::pack(lo, hi);
        }
        *(uint4*)dst = make_uint4(hv[0], hv[1], hv[2], hv[3]);
      } else if constexpr (Sh::EB == 2) {
        *(uint4*)dst = t.v[u];
      } else {
        const uint4 w4 = t.v[u];
        *(uint4*)dst = make_uint4(PVOps::template from_fp8<false>(w4.x), PVOps::template from_fp8<true>(w4.x),
                                  PVOps::template from_fp8<false>(w4.y), PVOps::template from_fp8<true>(w4.y));
        *(uint4*)(dst + 16) = make_uint4(PVOps::template from_fp8<false>(w4.z), PVOps::template from_fp8<true>(w4.z),
                                         PVOps::template from_fp8<false>(w4.w), PVOps::template from_fp8<true>(w4.w));
      }
      *(uint4*)(kb + vr * KSTRIDE + (byte % Sh::ROW)) = t.k[u];
    }
  };

  // this wave's RT row tiles against tiles g0 .. g0+3 of step st (LDS slots
  // g0.., tiles st*W + g0 .. of the window): every K word and V^T read from
  // LDS feeds all RT row tiles.  Per row tile: QK of the four tiles
  // interleaved, one online-softmax update for their 64 tokens, then PV on
  // 16x16x32 steps that pair tiles (0, 1) and (2, 3).  In a paired step the
  // contraction index 8kg + e stands for token 4kg + e of the first tile
  // (e < 4) and token 4kg + e - 4 of the second, on both operands: two
  // transposing reads give the V^T words, the two tiles' score words the P
  // words.
  // QK of the group's tiles (scores in sc) ...
  auto qk_group = [&](int st, int g0, f32x4 (&sc)[RT][kTileGroup]) {
    const uint8_t* klds = kbuf + ((st & 1) * W + g0) * KBYTES;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < kTileGroup; ++t) sc[rt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < Sh::KL; ++q) {
      uint4 kq[kTileGroup];
#pragma unroll
      for (int t = 0; t < kTileGroup; ++t)
        kq[t] = *(const uint4*)(klds + t * KBYTES + j16 * KSTRIDE + kg * (Sh::ROW / 4) + q * 16);
      // the QK steps this quarter-row word feeds: one (16-bit K) or two (fp8 K)
#pragma unroll
      for (int k = 0; k < KS / Sh::KL; ++k) {
        const int kst = q * (KS / Sh::KL) + k;
#pragma unroll
        for (int t = 0; t < kTileGroup; ++t) {
          uint4 kw[Sh::KL];
          kw[q] = kq[t];
          const uint4 ka = mfma_k_operand<KV, MT, D>(kw, kst);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) sc[rt][t] = Ops::qk(ka, qop[rt][kst], sc[rt][t]);
        }
      }
    }
  };
  // ... then the online softmax and PV.  Every row tile's max is taken
  // before one rescale check for all of them, so the rare rescale is the
  // only branch between the group's max and its exponentials.
  auto softmax_pv_group = [&](int tab, int tlo, int thi, int st, int g0, int unmasked_end,
                              const f32x4 (&sc)[RT][kTileGroup]) {
    const uint8_t* vlds = vbuf + ((st & 1) * W + g0) * VBYTES;
    const int j0 = st * W + g0;   // window tile index of slot g0
    const bool masked = tlo + (j0 + kTileGroup) * 16 > unmasked_end;
    uint32_t ph[RT][kTileGroup][2], pr[RT][kTileGroup][2];
    float x[RT][kTileGroup][4], mx[RT];
    // Raw scores; qabs * score is in log2 units.  Masking (causal limits, the
    // window's end, table entries outside the pool) is needed only where a
    // group reaches past the block's smallest limit or the window holds an
    // invalid entry.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < kTileGroup; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[rt][t][i] = sc[rt][t][i];
    if (masked) {
#pragma unroll
      for (int t = 0; t < kTileGroup; ++t) {
        const int j = j0 + t;
        const bool bvalid = __builtin_amdgcn_readlane(tab, min((j * 16) >> p.log2_bs, 63)) >= 0;
        const int t0 = tlo + j * 16 + 4 * kg;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int lim = min(thi, limit[rt]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!(bvalid && t0 + i < lim)) x[rt][t][i] = -INFINITY;
        }
      }
    }
    // each row's max over the group: the lane's values, then the four lane
    // groups kg of the row (lanes j16 + 16 kg) by two half swaps.  NaN
    // propagates, as it would through the exponentials.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float m = max_of<kTileGroup * 4>(&x[rt][0][0]);
      mx[rt] = lane_max_xor32_xor16(m) * qabs;
    }
    // Lazy rescaling: the reference max moves only when a row's max passes
    // it by more than kRescaleSlack (log2 units); all row tiles move together.
    bool grow = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) grow = grow || mx[rt] > mx_run[rt] + kRescaleSlack;
    if (__ballot(grow)) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float mn = fmaxf(mx_run[rt], mx[rt]);
        const float alpha = mx_run[rt] == -INFINITY ? 0.0f : fexp2(mx_run[rt] - mn);
        mx_run[rt] = mn;
        mu[rt] = mn == -INFINITY ? 0.0f : mn;
        lsum[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[rt][dt] *= alpha;
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int t = 0; t < kTileGroup; ++t) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = fexp2(__builtin_fmaf(x[rt][t][i], qabs, -mu[rt]));
        ph[rt][t][0] = PVOps::pack(e[0], e[1]);
        ph[rt][t][1] = PVOps::pack(e[2], e[3]);
        if constexpr (kSplitP) {
          pr[rt][t][0] = PVOps::pack(e[0] - PVOps::lo(ph[rt][t][0]), e[1] - PVOps::hi(ph[rt][t][0]));
          pr[rt][t][1] = PVOps::pack(e[2] - PVOps::lo(ph[rt][t][1]), e[3] - PVOps::hi(ph[rt][t][1]));
        }
      }
    }
    const int tro = (4 * kg + (j16 >> 2)) * LSTRIDE + (lane & 3) * 8;
#pragma unroll
    for (int pair = 0; pair < kTileGroup / 2; ++pair) {
      const int ta = 2 * pair, tb = 2 * pair + 1;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint2 va = PVOps::read_tr(vlds + ta * VBYTES + tro + dt * 32);
        const uint2 vb = PVOps::read_tr(vlds + tb * VBYTES + tro + dt * 32);
        const uint4 a = make_uint4(va.x, va.y, vb.x, vb.y);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const uint4 bh = make_uint4(ph[rt][ta][0], ph[rt][ta][1], ph[rt][tb][0], ph[rt][tb][1]);
          acc[rt][dt] = PVOps::qk(a, bh, acc[rt][dt]);
          if constexpr (kSplitP) {
            const uint4 br = make_uint4(pr[rt][ta][0], pr[rt][ta][1], pr[rt][tb][0], pr[rt][tb][1]);
            acc[rt][dt] = PVOps::qk(a, br, acc[rt][dt]);
          }
        }
      }
      const uint32_t one2 = PVOps::pack(1.0f, 1.0f);
      const uint4 ones = make_uint4(one2, one2, one2, one2);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        lsum[rt] = PVOps::qk(ones, make_uint4(ph[rt][ta][0], ph[rt][ta][1], ph[rt][tb][0], ph[rt][tb][1]), lsum[rt]);
        if constexpr (kSplitP)
          lsum[rt] = PVOps::qk(ones, make_uint4(pr[rt][ta][0], pr[rt][ta][1], pr[rt][tb][0], pr[rt][tb][1]), lsum[rt]);
      }
    }
  };

  int tab = load_table_window(p, trow, 0, len);
  for (int wb = 0; wb < len; wb += 64) {
    const int cnt = min(64, len - wb);
    const int tab_next = wb + 64 < len ? load_table_window(p, trow, wb + 64, len) : -1;
    const int tlo = (off + wb) << p.log2_bs;
    const int thi = min((off + wb + cnt) << p.log2_bs, n);
    const int tiles = (thi - tlo + 15) >> 4;
    const int steps = (tiles + W - 1) / W;
    // tokens below this need no mask: the block's first row sees up to
    // first_limit - 1, and every table entry of the window is in the pool
    const bool all_in_pool = __ballot(lane < cnt && tab < 0) == 0;
    const int unmasked_end = all_in_pool ? min(thi, first_limit) : tlo;
    // One register set: the tile of step st + 1 is loaded while step st
    // computes, then staged into the other buffer; one barrier per step.
    // Issues are unconditional (tiles past the window read zeros, masked).
    // The row blocks of a (sequence, kv head) pair read the same prefix, so
    // the loads keep the default cache policy: with the non-temporal one the
    // chunked-prefill batch read 1.9x its K/V bytes from HBM, with the
    // default about 1.0x (MI355X counters; the time is the same).
    MfmaTileRegs<KV, D> rt;
    mfma_issue<KV, D, kSharedPolicy>(c, tab, tlo, thi, wave, rt);
    stage(rt, 0);
    mfma_issue<KV, D, kSharedPolicy>(c, tab, tlo, thi, W + wave, rt);
    __syncthreads();
    for (int st = 0; st < steps; ++st) {
      if constexpr (W == 2 * kTileGroup) {
        // both groups' QK first: the second group's runs on the matrix
        // cores while the first group's softmax runs on the vector ALUs
        f32x4 sa[RT][kTileGroup], sb[RT][kTileGroup];
        qk_group(st, 0, sa);
        qk_group(st, kTileGroup, sb);
        softmax_pv_group(tab, tlo, thi, st, 0, unmasked_end, sa);
        softmax_pv_group(tab, tlo, thi, st, kTileGroup, unmasked_end, sb);
      } else {
#pragma unroll
        for (int g0 = 0; g0 < W; g0 += kTileGroup) {
          f32x4 sg[RT][kTileGroup];
          qk_group(st, g0, sg);
          softmax_pv_group(tab, tlo, thi, st, g0, unmasked_end, sg);
        }
      }
      if (st + 1 < steps) {
        stage(rt, (st + 1) & 1);
        mfma_issue<KV, D, kSharedPolicy>(c, tab, tlo, thi, (st + 2) * W + wave, rt);
      }
      __syncthreads();
    }
    tab = tab_next;
  }
  if constexpr (F16V) {
    // the bf16 values next to f16's largest (65504) are 65280 and 65536:
    // 65536 or more (inf included) or NaN is out of range
    if (__syncthreads_or(!(big < 65536.0f))) return false;
  }

  float l[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) l[t] = lsum[t][0];

  if (off == 0 && off + len == nb) {   // the whole row block is ours
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      if (valid[t]) {
        const float mul = l[t] > 0.0f ? vsc / l[t] : 0.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const float v4[4] = {acc[t][dt][0], acc[t][dt][1], acc[t][dt][2], acc[t][dt][3]};
          store_row<QT, 4>(p.out + (qoff[t] + dt * 16 + 4 * kg) * QE, v4, mul);
        }
      }
    }
    return true;
  }

  // publish this wave's rows of the block's record, then one arrival for
  // the work-group
  const RecordRef rec = record_ref<D, 16 * TB>(partial_record<D, 16 * TB>(p, w, wstart, pos));
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    if (valid[t]) {
      const int rg = ((RT * wave + t) * 16 + j16) * (D + 4);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        record_store4(rec, rg + dt * 16 + 4 * kg, acc[t][dt][0], acc[t][dt][1], acc[t][dt][2], acc[t][dt][3]);
      if (kg == 0) record_store4(rec, rg + D, mx_run[t], l[t], 0.0f, 0.0f);
    }
  }
  const int seg_start = pos - off;
  const int first_w = seg_start / chunk;
  const int last_w = (seg_start + nb - 1) / chunk;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();   // every wave's record stores have completed
  if (threadIdx.x == 0) {
    const int done = __hip_atomic_fetch_add(p.counters + first_w, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = done == last_w - first_w;
  }
  __syncthreads();
  if (last_flag)
    merge_records<QT, D, 16 * TB, BlockRows, 64 * W>(
        p, first_w, last_w, seg_start, uniform_grid(chunk), BlockRows{qs, TB, rb, m, Q, Hq, h * G, G, D}, vsc);
  return true;
}

template <typename KV, typename QT, int D, int G>
__device__ inline void prefill_wg_chunk(const DecodeParams& p, int v, int chunk, int T, int total) {
  constexpr int QB = wg_rows<D>() / G;   // tokens per row block
  const int lane = (int)(threadIdx.x & 63);
  const int S = p.num_seqs;
  const int max_len = p.max_blocks << p.log2_bs;
  const int start = v * chunk;
  if (start >= T) return;
  const int end = min(start + chunk, T);
  int h = start / total;
  const int rr = start - h * total;

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
        nb = sequence_rowblock_blocks(n, m, QB, p.log2_bs);
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
  if (!found) return;
  s = uniform(s);
  int n, m, qs;
  prefill_lengths(p, s, max_len, n, m, qs);
  n = uniform(n);
  m = uniform(m);
  qs = uniform(qs);
  int rb = 0, off = uniform(rr - pre);
  for (;;) {
    const int nb = (tile_limit(n, m, QB, rb) + (1 << p.log2_bs) - 1) >> p.log2_bs;
    if (off < nb) break;
    off -= nb;
    ++rb;
  }
  int pos = start;
  while (true) {
    const int nb = (tile_limit(n, m, QB, rb) + (1 << p.log2_bs) - 1) >> p.log2_bs;
    const int len = min(nb - off, end - pos);
    prefill_wg_run<KV, QT, D, G, wg_waves<D>(), wg_row_tiles<D>(), kTileGroup>(p, v, chunk, start, pos, s, h, rb,
                                                                              off, len, n, m, qs);
    pos += len;
    if (pos >= end) break;
    off = 0;
    if ((++rb) * QB < m) continue;
    rb = 0;
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
__global__ __launch_bounds__(64 * wg_waves<D>()) void paged_prefill_wg_kernel(const DecodeParams p) {
  constexpr int QB = wg_rows<D>() / G;
  const int lane = (int)(threadIdx.x & 63);
  const int S = p.num_seqs;
  const int max_len = p.max_blocks << p.log2_bs;
  int64_t total64 = 0;
  for (int base = 0; base < S; base += 64) {
    const int s = base + lane;
    int nb = 0;
    if (s < S) {
      int n, m, q0;
      prefill_lengths(p, s, max_len, n, m, q0);
      nb = sequence_rowblock_blocks(n, m, QB, p.log2_bs);
    }
    total64 += wave_sum_i64(nb);
    if (total64 * p.num_kv_heads > (1LL << 30)) return;   // the same in every wave: no barrier is left waiting
  }
  const int total = uniform((int)total64);
  const int T = total * p.num_kv_heads;
  if (T == 0) return;
  const int chunk = max(1, (T + p.num_workers - 1) / p.num_workers);
  const int nv = (T + chunk - 1) / chunk;
  const int per_round = (nv + 7) & ~7;
  if ((int)blockIdx.x >= per_round) return;
  const int v = (int)(blockIdx.x & 7) * (per_round >> 3) + (int)(blockIdx.x >> 3);
  if (v >= nv) return;
  prefill_wg_chunk<KV, QT, D, G>(p, v, chunk, T, total);
}

// Unit mode: one work-group per whole row block; no run is split (no
// records).
//
// Order.  Row blocks differ in length by the cached prefix and by their
// causal limit, and only a handful of work-groups per CU run them, so a long
// row block dispatched last sets the launch's end: in (kv head, sequence,
// row block) order the CUs' slots sat idle for about a quarter of the
// chunked-prefill launches (per-work-group timestamps on MI355X, and a
// simulation of the dispatch).  Up to kUnitRankSeqs sequences every
// work-group therefore ranks the sequences by context length (longest first,
// those without new rows last) and takes its unit from the list (rank, kv
// head, row block last-first).  The list is dealt to the XCDs in runs of
// p.chunk units (run j to XCD j % 8; a work-group's XCD is its index mod 8,
// the order in which its units are dispatched there is its index / 8).  A
// run is sized to a (sequence, kv head) pair's row blocks, which then run
// side by side on one XCD and stream the shared prefix through its L2; the
// XCDs see the ranks in the same order, longest first.  Above kUnitRankSeqs
// sequences the units keep (kv head, sequence, row block) order, in
// contiguous ranges per XCD.
constexpr int kUnitRankSeqs = 256;

// Unit u = (i-th of the list) of the ranked order: its sequence, kv head and
// row block, and that sequence's lengths and first query row (kept from the
// ranking, so the unit needs no second round trip for them), or false past
// the list.
template <int QB, int NT>
__device__ inline bool ranked_unit(const DecodeParams& p, int i, int& s, int& h, int& rb, int& n, int& m, int& qs) {
  __shared__ int key[kUnitRankSeqs];         // context length, -1 without new rows
  __shared__ int new_of[kUnitRankSeqs];      // new rows of sequence j
  __shared__ int q0_of[kUnitRankSeqs];       // its first query row
  __shared__ int rows_of[kUnitRankSeqs];     // row blocks of sequence j
  __shared__ int rank_seq[kUnitRankSeqs];    // the sequence of rank r
  __shared__ int rank_rows[kUnitRankSeqs];   // its row blocks
  const int tid = (int)threadIdx.x, lane = tid & 63;
  const int S = p.num_seqs, H = p.num_kv_heads;
  const int max_len = p.max_blocks << p.log2_bs;
  for (int j = tid; j < S; j += NT) {
    int nj, mj, q0;
    prefill_lengths(p, j, max_len, nj, mj, q0);
    key[j] = mj > 0 ? nj : -1;
    new_of[j] = mj;
    q0_of[j] = q0;
    rows_of[j] = (mj + QB - 1) / QB;
  }
  __syncthreads();
  for (int j = tid; j < S; j += NT) {
    const int kj = key[j];
    int r = 0;
    for (int o = 0; o < S; ++o) {
      const int ko = key[o];
      r += (ko > kj || (ko == kj && o < j)) ? 1 : 0;
    }
    rank_seq[r] = j;
    rank_rows[r] = rows_of[j];
  }
  __syncthreads();
  // the rank holding list entry i: rank r owns H * rank_rows[r] entries
  int carry = 0;
  for (int base = 0; base < S; base += 64) {
    const int c = base + lane < S ? H * rank_rows[base + lane] : 0;
    const int incl = wave_inclusive_scan_i32(c, lane);
    const int excl = carry + incl - c;
    const unsigned long long hit = __ballot(c > 0 && excl <= i && i < excl + c);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      const int r = base + src;
      const int R = uniform(rank_rows[r]);
      const int off = i - uniform(__shfl(excl, src));
      s = uniform(rank_seq[r]);
      h = off / R;
      rb = R - 1 - (off - h * R);
      n = uniform(key[s]);
      m = uniform(new_of[s]);
      qs = uniform(q0_of[s]);
      return true;
    }
    carry += __shfl(incl, 63);
  }
  return false;
}

template <typename KV, typename QT, int D, int G>
__global__ __launch_bounds__(64 * unit_waves<D>()) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void paged_prefill_unit_kernel(const DecodeParams p) {
  static_assert(16 * unit_waves<D>() * unit_row_tiles<D>() == wg_rows<D>(), "the split work-groups' blocks");
  constexpr int QB = wg_rows<D>() / G;
  const int lane = (int)(threadIdx.x & 63);
  const int S = p.num_seqs;
  const int max_len = p.max_blocks << p.log2_bs;
  int s = 0, h = 0, rb = 0, n, m, qs;
  if (S <= kUnitRankSeqs) {
    // work-group k of XCD x: entry (k / c) 8c + x c + k % c of the list
    const int c = p.chunk, x = (int)(blockIdx.x & 7), k = (int)(blockIdx.x >> 3);
    if (!ranked_unit<QB, 64 * unit_waves<D>()>(p, (k / c) * 8 * c + x * c + k % c, s, h, rb, n, m, qs)) return;
  } else {
    int64_t per_head64 = 0;
    for (int base = 0; base < S; base += 64) {
      const int sl = base + lane;
      int cnt = 0;
      if (sl < S) {
        int n, m, q0;
        prefill_lengths(p, sl, max_len, n, m, q0);
        cnt = (m + QB - 1) / QB;
      }
      per_head64 += wave_sum_i64(cnt);
    }
    if (per_head64 == 0 || per_head64 * p.num_kv_heads > (1LL << 30)) return;
    const int per_head = uniform((int)per_head64);
    const int U = per_head * p.num_kv_heads;
    const int per_xcd = (U + 7) >> 3;
    const int k = (int)(blockIdx.x >> 3);
    const int u = (int)(blockIdx.x & 7) * per_xcd + k;
    if (k >= per_xcd || u >= U) return;
    h = u / per_head;
    const int r = u - h * per_head;
    // the sequence holding unit r of kv head h
    int pre = 0;
    bool found = false;
    int carry = 0;
    for (int base = 0; base < S; base += 64) {
      const int sl = base + lane;
      int cnt = 0;
      if (sl < S) {
        int n, m, q0;
        prefill_lengths(p, sl, max_len, n, m, q0);
        cnt = (m + QB - 1) / QB;
      }
      const int incl = wave_inclusive_scan_i32(cnt, lane);
      const int excl = carry + incl - cnt;
      const unsigned long long hit = __ballot(cnt > 0 && excl <= r && r < excl + cnt);
      if (hit) {
        const int src = __builtin_ctzll(hit);
        s = base + src;
        pre = __shfl(excl, src);
        found = true;
        break;
      }
      carry += __shfl(incl, 63);
    }
    if (!found) return;
    s = uniform(s);
    rb = uniform(r - pre);
    prefill_lengths(p, s, max_len, n, m, qs);
    n = uniform(n);
    m = uniform(m);
    qs = uniform(qs);
  }
  const int nb = (tile_limit(n, m, QB, rb) + (1 << p.log2_bs) - 1) >> p.log2_bs;
  // the whole row block: stored directly, no record; bf16 pools stage V as
  // f16 and run again with bf16 V if it holds a value out of f16's range
  constexpr int UW = unit_waves<D>(), URT = unit_row_tiles<D>(), UTG = unit_tile_group<KV, D>();
  if constexpr (std::is_same<KV, bf16_t>::value) {
    if (prefill_wg_run<KV, QT, D, G, UW, URT, UTG, true>(p, 0, 1, 0, 0, s, h, rb, 0, nb, n, m, qs)) return;
  }
  prefill_wg_run<KV, QT, D, G, UW, URT, UTG>(p, 0, 1, 0, 0, s, h, rb, 0, nb, n, m, qs);
}

// Prefill launch shape: 0 one-wave tiles, 1 split work-groups, 2 units.
template <typename KV, typename QT>
kv_status_t launch_prefill(const DecodeParams& p, int D, int G, int mode, hipStream_t stream) {
#define PKV_PCASE(DD, GG)                                                                                         \
  if (D == DD && G == GG) {                                                                                       \
    if (mode == 2)                                                                                                \
      hipLaunchKernelGGL((paged_prefill_unit_kernel<KV, QT, DD, GG>), dim3(p.num_workers),                       \
                         dim3(64 * unit_waves<DD>()), 0, stream, p);                                              \
    else if (mode == 1)                                                                                           \
      hipLaunchKernelGGL((paged_prefill_wg_kernel<KV, QT, DD, GG>), dim3(p.num_workers), dim3(64 * wg_waves<DD>()), 0, \
                         stream, p);                                                                              \
    else                                                                                                          \
      hipLaunchKernelGGL((paged_prefill_kernel<KV, QT, DD, GG>), dim3(p.num_workers), dim3(64), 0, stream, p);   \
    return launch_status();                                                                                       \
  }
#define PKV_PCASES(DD) PKV_PCASE(DD, 1) PKV_PCASE(DD, 2) PKV_PCASE(DD, 4) PKV_PCASE(DD, 8) PKV_PCASE(DD, 16)
  PKV_PCASES(64)
  PKV_PCASES(128)
  PKV_PCASES(256)
#undef PKV_PCASES
#undef PKV_PCASE
  return KV_ERR_UNSUPPORTED;
}

kv_status_t launch_prefill_bf16_bf16(const DecodeParams& p, int D, int G, int mode, hipStream_t s);
kv_status_t launch_prefill_f16_f16(const DecodeParams& p, int D, int G, int mode, hipStream_t s);
kv_status_t launch_prefill_fp8_bf16(const DecodeParams& p, int D, int G, int mode, hipStream_t s);
kv_status_t launch_prefill_fp8_f16(const DecodeParams& p, int D, int G, int mode, hipStream_t s);

}  // namespace pkv
