// Grouped decode plans: the pieces of G-items (a group's shared prefix, read
// once for every member's query rows) and S-items (one sequence's own
// blocks) that a worker streams, and the merge of each output from its
// partial records.
//
// An output -- the G query rows of sequence s served by kv head h -- gets one
// contribution per piece of its group's G-item and one per piece of its own
// S-item (a piece is the part of an item inside one worker's chunk).  A
// sequence outside any group with a single piece writes its rows directly.
// Otherwise every piece leaves a partial record (unnormalised accumulator,
// reference max, running sum) and counts itself in on the output's arrival
// counter; the piece that completes the count merges the records, G-item
// pieces first, then S-item pieces, each in stream order, so results do not
// depend on which worker finishes last.  Shared prefixes are read once per
// group ("vLLM — 把操作系统的分页搬进 GPU KV cache": core mechanism 3 and case
// 2: forked candidates share the prompt's blocks).
#pragma once

namespace pkv {

// Pieces of an item of kv head h that starts at block `ipos` of the head's
// stream and holds `ilen` blocks: the chunks it spans.
__device__ inline int item_first_chunk(const ChunkCtx& d, int h, int ipos) { return d.grid().of(h * d.TB + ipos); }
__device__ inline int item_pieces(const ChunkCtx& d, int h, int ipos, int ilen) {
  const int a = h * d.TB + ipos;
  const ChunkGrid g = d.grid();
  return g.of(a + ilen - 1) - g.of(a) + 1;
}

// First float of piece k of an item (kv head h, first record row rbase)
// whose records hold `rows` rows of [D + 4] floats.
template <int D>
__device__ inline float* item_record(const DecodeParams& p, const ChunkCtx& d, int h, int rbase, int k, int rows) {
  return p.partials + ((int64_t)h * d.RH + rbase + (int64_t)k * rows) * (D + 4);
}

__device__ inline int32_t* output_counter(const DecodeParams& p, int h, int s) {
  return p.counters + (int64_t)h * p.num_seqs + s;
}

// Count one contribution in on an output that takes `expected`; true in the
// contribution that completes the count.  The caller's record stores are
// written through to the device coherence point first (see arrive()).
__device__ inline bool arrive_output(int32_t* ctr, int expected) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int done = 0;
  if (threadIdx.x == 0) done = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  done = uniform(__shfl(done, 0));
  return done == expected - 1;
}

// Merge the pg pieces of the group's G-item (rows mem*G .. mem*G + G - 1 of
// each g_rows-row record) and then the ps pieces of the output's S-item.
template <typename QT, int D, int G>
__device__ inline void merge_output(const DecodeParams& p, const ChunkCtx& d, int h, int s, int mem, int g_rbase,
                                    int g_rows, int pg, int s_rbase, int ps) {
  const float* gb = item_record<D>(p, d, h, g_rbase, 0, g_rows) + (int64_t)mem * G * (D + 4);
  const float* sb = item_record<D>(p, d, h, s_rbase, 0, G);
  auto rec_at = [&](int c) {
    return c < pg ? gb + (int64_t)c * g_rows * (D + 4) : sb + (int64_t)(c - pg) * G * (D + 4);
  };
  const int Hq = p.num_kv_heads * G;
  merge_list<QT, D, G>(p, pg + ps, rec_at, ContiguousRows{((int64_t)s * Hq + (int64_t)h * G) * D, D},
                       run_v_scale(p, h), output_counter(p, h, s));
}

// Matrix-core run state -> the rows' output, or a record of the valid rows.
template <typename KV, typename QT, int D>
__device__ inline void mfma_store_out(const DecodeParams& p, const MfmaRow& row, float vs,
                                      const f32x4 (&acc)[MfmaShape<KV, D>::DT], float l) {
  constexpr int DT = MfmaShape<KV, D>::DT;
  constexpr int QE = elem_size<QT>::value;
  const int kg = threadIdx.x >> 4;
  if (row.valid) {
    const float mul = l > 0.0f ? vs / l : 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const float v4[4] = {acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]};
      store_row<QT, 4>(p.out + (row.qoff + dt * 16 + 4 * kg) * QE, v4, mul);
    }
  }
}
// A piece of an S-item: blocks [off, off + len) of the item (sequence it.s).
template <typename KV, typename QT, int D, int G, bool MFMA>
__device__ inline void seq_piece(const DecodeParams& p, const ChunkCtx& d, int h, const PlanItem& it, int off,
                                 int len) {
  const int s = it.s;
  const int Hq = p.num_kv_heads * G;
  const int ps = item_pieces(d, h, it.pos, it.len);
  const int pg = it.g_len > 0 ? item_pieces(d, h, it.g_pos, it.g_len) : 0;
  const int k = d.v - item_first_chunk(d, h, it.pos);
  if constexpr (MFMA) {
    constexpr int DT = MfmaShape<KV, D>::DT;
    const int j16 = threadIdx.x & 15;
    MfmaRow row;
    row.valid = j16 < G;
    row.qoff = ((int64_t)s * Hq + (int64_t)h * G + j16) * D;
    row.limit = it.n;
    row.min_limit = it.n;
    row.part = 0;
    f32x4 acc[DT];
    float m, l;
    mfma_rows_core<KV, QT, D, kStreamPolicy>(p, s, h, it.off + off, len, it.n, row, acc, m, l);
    if (ps + pg == 1) {
      mfma_store_out<KV, QT, D>(p, row, run_v_scale(p, h), acc, l);
      return;
    }
    mfma_store_record<KV, D>(record_ref<D, G>(item_record<D>(p, d, h, it.rbase, k, G)), row.valid, acc, m, l);
  } else {
    constexpr int VEC = DecodeShape<KV, D>::VEC;
    float m[G], l[G], acc[G][VEC];
    valu_core<KV, QT, D, G, kStreamPolicy>(p, s, h, it.off + off, len, it.n, m, l, acc);
    if (ps + pg == 1) {
      valu_store_out<KV, QT, D, G>(p, s, h, run_v_scale(p, h), l, acc);
      return;
    }
    valu_store_record<KV, D, G>(record_ref<D, G>(item_record<D>(p, d, h, it.rbase, k, G)), m, l, acc);
  }
  if (arrive_output(output_counter(p, h, s), ps + pg))
    merge_output<QT, D, G>(p, d, h, s, it.member, it.g_rbase, it.g_m * G, pg, it.rbase, ps);
}

// A piece of a G-item: blocks [off, off + len) of the group's shared prefix,
// for the query rows of its it.m members (row j: member j / G, query head
// j % G of kv head h).
template <typename KV, typename QT, int D, int G>
__device__ inline void group_piece(const DecodeParams& p, const ChunkCtx& d, int h, const PlanItem& it, int off,
                                   int len) {
  constexpr int DT = MfmaShape<KV, D>::DT;
  const int lane = threadIdx.x;
  const int j16 = lane & 15;
  const int members = it.m, rows = it.m * G;
  const int Hq = p.num_kv_heads * G;
  MfmaRow row;
  row.valid = j16 < rows;
  row.qoff = ((int64_t)(it.s + j16 / G) * Hq + (int64_t)h * G + j16 % G) * D;
  row.limit = it.n;
  row.min_limit = it.n;
  row.part = 0;
  f32x4 acc[DT];
  float m, l;
  mfma_rows_core<KV, QT, D, kStreamPolicy>(p, it.s, h, it.off + off, len, it.n, row, acc, m, l);
  const int pg = item_pieces(d, h, it.pos, it.len);
  const int k = d.v - item_first_chunk(d, h, it.pos);
  // member `lane`'s own blocks, for its contribution count: loaded with the
  // record stores, which are waited for before the arrival anyway
  int4 own = make_int4(-1, 0, 0, 0);
  if (lane < members) own = *(const int4*)(p.pseqs + it.s + lane);
  mfma_store_record<KV, D>(record_ref_rows<D>(item_record<D>(p, d, h, it.rbase, k, rows), rows), row.valid, acc, m,
                           l);
  // per-lane values of member `lane`: s_item, s_pos, s_len, s_rbase
  const int s_rbase = own.w;
  const int ps = (lane < members && own.x >= 0) ? item_pieces(d, h, own.y, own.z) : 0;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int done = -1;
  if (lane < members)
    done = __hip_atomic_fetch_add(output_counter(p, h, it.s + lane), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t last = __ballot(lane < members && done == pg + ps - 1);
  while (last) {
    const int j = __builtin_ctzll(last);
    last &= last - 1;
    merge_output<QT, D, G>(p, d, h, it.s + j, j, it.rbase, rows, pg, __builtin_amdgcn_readlane(s_rbase, j),
                           __builtin_amdgcn_readlane(ps, j));
  }
}

// Stream chunk d.v of a grouped plan.
template <typename KV, typename QT, int D, int G, bool MFMA>
__device__ inline void grouped_chunk(const DecodeParams& p, const ChunkCtx& d) {
  const int start = d.grid().start(d.v);
  const int end = d.grid().end(d.v, d.T);
  int h = d.h, i = d.i, off = d.off, pos = start;
  PlanItem it = load_item(p.items + i);
  while (true) {
    const int len = min(it.len - off, end - pos);
    int ni = i + 1, nh = h;
    if (ni == d.NI) {
      ni = 0;
      ++nh;
    }
    const bool more = pos + len < end;
    const PlanItem nx = load_item(p.items + ni);   // in flight during the run
    if (it.m > 0)
      group_piece<KV, QT, D, G>(p, d, h, it, off, len);
    else
      seq_piece<KV, QT, D, G, MFMA>(p, d, h, it, off, len);
    pos += len;
    if (!more) return;
    i = ni;
    h = nh;
    it = nx;
    off = 0;
  }
}

}  // namespace pkv
