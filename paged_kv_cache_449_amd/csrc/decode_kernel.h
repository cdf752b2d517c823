// Paged decode attention kernel (wave-per-worker, balanced split-KV).
//
// What it computes: for every sequence s and query head hq,
//   out[s][hq] = sum_t softmax_t(scale * q[s][hq] . K_t) * V_t,  t < len[s],
// where K_t/V_t are read through the block table: physical block
// block_tables[s][t / bs], slot t % bs, kv head hq / G.  The table lookup is
// one integer load per block followed by an offset computation ("vLLM — 把操作
// 系统的分页搬进 GPU KV cache": core mechanisms, kernel paragraph).  Decode is
// bound by the KV read bandwidth (same page, lessons), so the kernel is built
// as an HBM stream on the vector ALUs; there is no dense contraction for the
// matrix cores when each kv head serves one query row.
//
// Work split.  The blocks of all (kv head, sequence) pairs are laid end to end
// in (kv head, sequence, block) order -- T blocks in all -- and worker w (one
// 64-lane wavefront) takes blocks [w*chunk, (w+1)*chunk).  Every worker
// streams the same number of bytes however the context lengths are spread.
// A run of one (kv head, sequence) that lies inside one worker is finished by
// it; a run cut between workers leaves one partial (running max m, sum l,
// unnormalised accumulator) per worker, and the worker that finishes last
// (an atomic counter per run) merges them in worker order.
//
// Worker ids are assigned so that consecutive ids run on the same XCD (the
// dispatcher deals work-groups round robin over the 8 XCDs) and every XCD
// gets an equal share of the workers that have blocks: neighbouring runs --
// e.g. candidates sharing a prompt's blocks -- then share that XCD's L2.
//
// Lane layout.  A token row of head_dim elements is read by L lanes with one
// 16-byte load each; a wave load covers TPL = 64/L consecutive tokens of one
// block tile (a tile [bs][head_dim] of one kv head is contiguous in the pool).
// The L lanes of a row reduce their partial dot products with DPP; each row
// keeps its own online-softmax state over the tokens it sees, and the TPL
// rows are merged once at the end of a run.
#pragma once

#include <type_traits>

#include "common.h"
#include "decode_plan.h"

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;
// Wave loads of K (and of V) issued together per step of a vector-ALU run:
// four when blocks are shared, so reads served by the L2 have a deep
// pipeline; one when every byte streams from HBM once, which measured 1-3%
// faster than four on MI355X (the other waves of a CU keep HBM busy, and
// shorter steps leave less masked issue at the end of each window).
constexpr int kLoadsPerStep = 4;
constexpr int kStreamLoadsPerStep = 1;
// Arrival counters of split runs, indexed by the run's first worker (a worker
// starts at most one run that continues past its end).  The region has a
// fixed size and sits at the start of the workspace, so calls with different
// batch shapes can share one workspace: each call leaves it zero.
constexpr int kCounterSlots = 65536;
// When sequences share blocks (copy-on-write candidates of one prompt), the
// library-sized split cuts the stream kSharedSplit times finer and each
// worker takes kSharedSplit chunks, one per round: the candidates' runs then
// sit in neighbouring chunks that run at the same time on one XCD and meet
// in its L2.
constexpr int kSharedSplit = 4;

struct DecodeParams {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const uint8_t* q;
  uint8_t* out;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;  // multi-token attention: [num_seqs + 1] query row offsets
  int32_t* counters;     // [kCounterSlots], zero between calls
  float* partials;       // [2 * chunk ids][rows][head_dim + 4] (grouped plans: per item)
  int32_t num_seqs;
  int32_t total_q;       // multi-token attention: rows of q and out
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t log2_bs;
  int32_t chunk;         // blocks per worker; 0 = ceil(T / num_workers)
  int32_t num_workers;   // multiple of 8
  float q_scale;         // softmax scale * log2(e) * k_scale
  float v_scale;
  const float* head_scales;  // fp8 per-kv-head scales [2][num_kv_heads] (k then v), or null
  float qk_scale;            // softmax scale * log2(e) (per-head scales multiply it)
  // decode: the launch's work plan (written by paged_decode_plan_kernel)
  const PlanHeader* header;  // what every worker of the launch shares
  const PlanDesc* desc;      // [rounds][num_workers]
  const PlanItem* items;     // items of a kv head's stream
  const PlanSeq* pseqs;      // [num_seqs], grouped mode
};

// Scales a run of kv head h uses: the per-tensor ones, or head h's.
__device__ inline float run_q_scale(const DecodeParams& p, int h) {
  return p.head_scales ? p.qk_scale * p.head_scales[h] : p.q_scale;
}
__device__ inline float run_v_scale(const DecodeParams& p, int h) {
  return p.head_scales ? p.head_scales[p.num_kv_heads + h] : p.v_scale;
}

template <typename KV, int D>
struct DecodeShape {
  static constexpr int EB = elem_size<KV>::value;
  static constexpr int VEC = 16 / EB;   // elements per lane per load
  static constexpr int L = D / VEC;     // lanes per token row
  static constexpr int TPL = 64 / L;    // tokens per wave load
  static constexpr int REC = D + 4;     // floats per partial record: acc[D], m, l, pad
  static_assert(L >= 1 && L <= 64 && (64 % L) == 0, "row layout");
};

__device__ inline int clamp_len(int n, int max_len) { return n < 0 ? 0 : (n > max_len ? max_len : n); }

__device__ inline float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Load VEC elements of type T (4-byte aligned) and widen them to fp32.
template <typename T, int VEC>
__device__ inline void load_row_f32(const uint8_t* p, float* o) {
  constexpr int PW = unpack<T>::per_word;
  constexpr int NW = VEC / PW;
  const uint32_t* w = (const uint32_t*)p;
#pragma unroll
  for (int i = 0; i < NW; ++i) unpack<T>::run(w[i], o + i * PW);
}

// Store VEC fp32 values * mul as type T (4-byte aligned destination).
template <typename T, int VEC>
__device__ inline void store_row(uint8_t* p, const float* v, float mul) {
  constexpr int PW = pack_out<T>::per_word;
  constexpr int NW = VEC / PW;
  uint32_t* w = (uint32_t*)p;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    float t[PW];
#pragma unroll
    for (int j = 0; j < PW; ++j) t[j] = v[i * PW + j] * mul;
    w[i] = pack_out<T>::run(t);
  }
}

// Online-softmax update of one state (m, l, acc) with NS new scores whose
// exponentials are returned in pw (scores are already in log2 units).
template <int NS>
__device__ inline float softmax_step(float& m, float& l, const float* sc, float* pw) {
  float mx = sc[0];
#pragma unroll
  for (int u = 1; u < NS; ++u) mx = fmaxf(mx, sc[u]);
  const float mn = fmaxf(m, mx);
  const float mu = mn == -INFINITY ? 0.0f : mn;
  const float alpha = fexp2(m - mu);
  float ps = 0.0f;
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    pw[u] = fexp2(sc[u] - mu);
    ps += pw[u];
  }
  l = l * alpha + ps;
  m = mn;
  return alpha;
}

// Buffer resource word 3 for raw (untyped) buffer loads on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;
// Lane offset that lies outside every tile: the load returns zeros.
constexpr uint32_t kMaskedOffset = 0x80000000u;
// Cache policy of the K/V stream loads: non-temporal when each byte is used
// once per launch (on MI355X this lifts a random-4-KiB-tile read stream from
// about 6.1 to about 6.8 TB/s); the default policy when sequences share
// blocks, so a block read for one candidate can serve the others from L2.
constexpr int kStreamPolicy = 2;
constexpr int kSharedPolicy = 0;

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Registers of one step: U wave loads of K and of V.
template <int U>
struct StepRegs {
  uint4 k[U];
  uint4 v[U];
};

// Per-run constants shared by the load and compute phases.
struct RunCtx {
  const uint8_t* k_head;   // pool base + kv head offset (uniform)
  const uint8_t* v_head;
  int64_t blk_stride;      // bytes between consecutive physical blocks
  uint32_t tile_bytes;     // bytes of one (block, head) tile
  uint32_t lane_off;       // col * 16
  int row_bytes;
  int log2_bs;
  int bs_mask;
};

// Issue the U K and V loads of step `step` of the current table window.
// Tokens at or past `thi`, and blocks whose table entry is out of range,
// read as zeros (offset outside the tile, or an empty tile).
template <int U, int TPL, int POL>
__device__ inline void issue_step(const RunCtx& c, int tab, int tlo, int thi, int step, int row,
                                  StepRegs<U>& r) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = step * U + u;                    // wave load index in the window
    const int bi = min((j * TPL) >> c.log2_bs, 63);
    const int phys = __builtin_amdgcn_readlane(tab, bi);
    // an invalid entry (-1) gives an empty descriptor at the head's base
    const int64_t boff = c.blk_stride * max(phys, 0);
    const uint32_t nrec = c.tile_bytes & (uint32_t)~(phys >> 31);
    __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(c.k_head + boff), (short)0, (int)nrec,
                                                                  kBufferWord3);
    __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(c.v_head + boff), (short)0, (int)nrec,
                                                                  kBufferWord3);
    const int t = tlo + j * TPL + row;
    const uint32_t off = t < thi ? (uint32_t)((t & c.bs_mask) * c.row_bytes) + c.lane_off : kMaskedOffset;
    r.k[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, POL));
    r.v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, POL));
  }
}

// Scores, online-softmax update and V accumulation for one step.
template <typename KV, int VEC, int L, int TPL, int G, int U>
__device__ inline void compute_step(const StepRegs<U>& r, const float (&qv)[G][VEC], float (&m)[G], float (&l)[G],
                                    float (&acc)[G][VEC], int tab, int tlo, int thi, int step, int row,
                                    int log2_bs) {
  float sc[G][U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = step * U + u;
    const int bi = min((j * TPL) >> log2_bs, 63);
    const bool ok = (tlo + j * TPL + row < thi) && (__builtin_amdgcn_readlane(tab, bi) >= 0);
    float kf[VEC];
    const uint32_t kw[4] = {r.k[u].x, r.k[u].y, r.k[u].z, r.k[u].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) unpack<KV>::run(kw[i], kf + i * unpack<KV>::per_word);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d = 0.0f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) d = fmaf(qv[g][i], kf[i], d);
      d = group_sum<L>(d);
      sc[g][u] = ok ? d : -INFINITY;
    }
  }
  float pw[G][U];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float alpha = softmax_step<U>(m[g], l[g], sc[g], pw[g]);
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[g][i] *= alpha;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float vf[VEC];
    const uint32_t vw[4] = {r.v[u].x, r.v[u].y, r.v[u].z, r.v[u].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) unpack<KV>::run(vw[i], vf + i * unpack<KV>::per_word);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[g][i] = fmaf(pw[g][u], vf[i], acc[g][i]);
  }
}

// Device-scope coherent record traffic.  Cache policy sc1 is what the
// compiler emits for relaxed agent-scope atomic loads and stores on gfx950
// (stores write through to the device coherence point, loads do not return
// stale cache lines); here it is applied to 16-byte buffer accesses so a
// record moves in whole 16-byte pieces rather than 4-byte stores, each of
// which costs a full memory write when it is written through.
constexpr int kCoherentPolicy = 16;
typedef unsigned u32x4 __attribute__((__vector_size__(16)));

struct RecordRef {
  __amdgpu_buffer_rsrc_t rsrc;
};

template <int D, int G>
__device__ inline RecordRef record_ref(const float* rec) {
  return {__builtin_amdgcn_make_buffer_rsrc((void*)rec, (short)0, G * (D + 4) * 4, kBufferWord3)};
}
// a record of `rows` rows (rows known at run time)
template <int D>
__device__ inline RecordRef record_ref_rows(const float* rec, int rows) {
  return {__builtin_amdgcn_make_buffer_rsrc((void*)rec, (short)0, rows * (D + 4) * 4, kBufferWord3)};
}
// store floats [i, i+4) of the record (i a multiple of 4)
__device__ inline void record_store4(const RecordRef& r, int i, float a, float b, float c, float d) {
  const uint4 v = make_uint4(__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r.rsrc, i * 4, 0, kCoherentPolicy);
}
__device__ inline float4 record_load4(const RecordRef& r, int i) {
  const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r.rsrc, i * 4, 0, kCoherentPolicy));
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// ------------------------------------------------------ split-run bookkeeping
//
// A run cut between workers leaves one partial record per worker:
// [G][D + 4] floats holding the unnormalised accumulator acc[g][0..D), the
// running max (log2 units) at [g][D] and the running sum at [g][D + 1].  A
// worker has at most two partial runs: the one it starts with (slot 0) and
// the one it ends with (slot 1).

// Record of this worker for the run that reaches position `pos`.
template <int D, int G>
__device__ inline float* partial_record(const DecodeParams& p, int w, int wstart, int pos) {
  const int k = pos == wstart ? 0 : 1;
  return p.partials + (int64_t)(2 * w + k) * G * (D + 4);
}

// Publish-side half of the hand-over: the caller has stored its record with
// record_store4 (written through to the device coherence point).  Wait for
// those stores to complete, then count this worker in.  Returns true in the
// worker that completes the count, which then merges.  Its loads of the
// records are coherent loads, so no cache-wide writeback or invalidate is
// needed on either side.
// `pieces` counts in that many records of the run at once (a run that
// crosses chunk boundaries leaves one per chunk).
__device__ inline bool arrive(const DecodeParams& p, int first_w, int last_w, int pieces = 1) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int done = 0;
  if (threadIdx.x == 0)
    done = __hip_atomic_fetch_add(p.counters + first_w, pieces, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  done = uniform(__shfl(done, 0));
  return done + pieces == last_w - first_w + 1;
}

// Output rows of a run's records: record row j -> element offset of its out
// row (-1: the row holds no query).
struct ContiguousRows {   // G query heads of one sequence: rows orow + j*D
  int64_t orow;
  int d;
  __device__ int64_t operator()(int j) const { return orow + (int64_t)j * d; }
};

// Merge `count` partial records -- record c starts at rec_at(c) and holds
// G rows of [D + 4] floats -- in the order c = 0, 1, ... (results are
// reproducible) into the out rows that `rows` names, then clear the
// arrival counter `ctr` for the next call.  Each of the NT threads owns 4
// consecutive elements of [G][D] per pass.
//
// The records are read through the coherence point, a full memory round
// trip each, so they are fetched in batches of B records with every load of
// a batch (all passes) issued before any is used: up to B records cost one
// round trip.  Within a batch the weights are taken against the batch's
// maximum; a later batch with a larger maximum rescales what is summed so
// far.
template <typename QT, int D, int G, typename RecAt, typename Rows, int NT = 64>
__device__ inline void merge_list(const DecodeParams& p, int count, const RecAt& rec_at, const Rows& rows,
                                  float v_scale, int32_t* ctr) {
  constexpr int REC = D + 4;
  constexpr int QE = elem_size<QT>::value;
  static_assert(D % 4 == 0, "record layout");
  constexpr int PASSES = (G * D + 4 * NT - 1) / (4 * NT);
  constexpr int B = PASSES >= 8 ? 1 : 8 / PASSES;   // about 64 registers of loads in flight
  float M[PASSES], lsum[PASSES], o[PASSES][4];
#pragma unroll
  for (int q = 0; q < PASSES; ++q) {
    M[q] = -INFINITY;
    lsum[q] = 0.0f;
    o[q][0] = o[q][1] = o[q][2] = o[q][3] = 0.0f;
  }
  for (int c0 = 0; c0 < count; c0 += B) {
    float4 ml[B][PASSES], a[B][PASSES];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int c = min(c0 + b, count - 1);   // past the list: a repeat, not used
      const RecordRef r = record_ref<D, G>(rec_at(c));
#pragma unroll
      for (int q = 0; q < PASSES; ++q) {
        const int e0 = min((int)threadIdx.x * 4 + q * 4 * NT, G * D - 4);
        const int g = e0 / D, d = e0 % D;
        ml[b][q] = record_load4(r, g * REC + D);
        a[b][q] = record_load4(r, g * REC + d);
      }
    }
#pragma unroll
    for (int q = 0; q < PASSES; ++q) {
      float mb = -INFINITY;
#pragma unroll
      for (int b = 0; b < B; ++b)
        if (c0 + b < count) mb = fmaxf(mb, ml[b][q].x);
      const float mn = fmaxf(M[q], mb);
      if (mn > M[q] && M[q] != -INFINITY) {   // rescale the earlier batches
        const float r = fexp2(M[q] - mn);
        lsum[q] *= r;
        o[q][0] *= r; o[q][1] *= r; o[q][2] *= r; o[q][3] *= r;
      }
      M[q] = mn;
      const float mu = mn == -INFINITY ? 0.0f : mn;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (c0 + b >= count) continue;
        const float f = fexp2(ml[b][q].x - mu);
        lsum[q] = fmaf(f, ml[b][q].y, lsum[q]);
        o[q][0] = fmaf(f, a[b][q].x, o[q][0]);
        o[q][1] = fmaf(f, a[b][q].y, o[q][1]);
        o[q][2] = fmaf(f, a[b][q].z, o[q][2]);
        o[q][3] = fmaf(f, a[b][q].w, o[q][3]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < PASSES; ++q) {
    const int e0 = (int)threadIdx.x * 4 + q * 4 * NT;
    if (e0 >= G * D) continue;
    const int g = e0 / D, d = e0 % D;
    const int64_t orow = rows(g);
    if (orow < 0) continue;
    store_row<QT, 4>(p.out + (orow + d) * QE, o[q], lsum[q] > 0.0f ? v_scale / lsum[q] : 0.0f);
  }
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the records of workers first_w..last_w (in worker order) of a run
// whose first position in the flattened stream is seg_start.
template <typename QT, int D, int G, typename Rows, int NT = 64>
__device__ inline void merge_records(const DecodeParams& p, int first_w, int last_w, int seg_start,
                                     const ChunkGrid& grid, const Rows& rows, float v_scale) {
  auto rec_at = [&](int c) {
    const int v = first_w + c;
    return (const float*)p.partials + (int64_t)(2 * v + (grid.start(v) >= seg_start ? 0 : 1)) * G * (D + 4);
  };
  merge_list<QT, D, G, decltype(rec_at), Rows, NT>(p, last_w - first_w + 1, rec_at, rows, v_scale,
                                                   p.counters + first_w);
}

// Table window: lane i holds the physical block of logical block wb + i of
// the run (-1 past the run or for an id outside the pool).
__device__ inline int load_table_window(const DecodeParams& p, const int32_t* trow, int wb, int len) {
  const int cnt = min(64, len - wb);
  const int lane = (int)(threadIdx.x & 63);
  int e = -1;
  if (lane < cnt) e = trow[wb + lane];
  return (uint32_t)e < (uint32_t)p.num_blocks ? e : -1;
}

// The run's table row from logical block off on.
__device__ inline const int32_t* run_table(const DecodeParams& p, int s, int off) {
  return p.block_tables + (int64_t)s * p.max_blocks + off;
}

// Stream blocks [off, off+len) of the (kv head h, sequence s) context of n
// tokens through one wave's online-softmax state (per-row-group m, l, acc of
// the G query rows, qv pre-scaled into log2 units).  tab is the run's first
// table window, load_table_window(p, run_table(p, s, off), 0, len), which the
// caller loads before its query rows so the two loads overlap.
template <typename KV, int D, int G, int POL>
__device__ inline void valu_stream(const DecodeParams& p, int s, int h, int off, int len, int n, int tab,
                                   const float (&qv)[G][DecodeShape<KV, D>::VEC], float (&m)[G], float (&l)[G],
                                   float (&acc)[G][DecodeShape<KV, D>::VEC]) {
  using Sh = DecodeShape<KV, D>;
  constexpr int VEC = Sh::VEC, L = Sh::L, TPL = Sh::TPL;
  constexpr int U = POL == kStreamPolicy ? kStreamLoadsPerStep : kLoadsPerStep;
  const int lane = threadIdx.x & 63;
  const int row = lane / L;
  const int col = lane % L;
  RunCtx c;
  const int64_t tile = ((int64_t)D * Sh::EB) << p.log2_bs;
  c.k_head = p.k_pool + tile * h;
  c.v_head = p.v_pool + tile * h;
  c.blk_stride = tile * p.num_kv_heads;
  c.tile_bytes = (uint32_t)tile;
  c.lane_off = (uint32_t)col * 16u;
  c.row_bytes = D * Sh::EB;
  c.log2_bs = p.log2_bs;
  c.bs_mask = (1 << p.log2_bs) - 1;
  const int32_t* trow = run_table(p, s, off);

  for (int wb = 0; wb < len; wb += 64) {
    const int cnt = min(64, len - wb);
    // the next window's table entries load while this window streams
    const int tab_next = wb + 64 < len ? load_table_window(p, trow, wb + 64, len) : -1;
    const int tlo = (off + wb) << p.log2_bs;
    const int thi = min((off + wb + cnt) << p.log2_bs, n);
    const int steps = (thi - tlo + U * TPL - 1) / (U * TPL);
    // Two register sets in flight.  Issues are unconditional so the wait
    // counts stay exact: a step past the window reads zeros (its offsets lie
    // outside the tile) and computes nothing (every score is masked).
    StepRegs<U> a, b;
    issue_step<U, TPL, POL>(c, tab, tlo, thi, 0, row, a);
    for (int st = 0; st < steps; st += 2) {
      issue_step<U, TPL, POL>(c, tab, tlo, thi, st + 1, row, b);
      compute_step<KV, VEC, L, TPL, G, U>(a, qv, m, l, acc, tab, tlo, thi, st, row, p.log2_bs);
      issue_step<U, TPL, POL>(c, tab, tlo, thi, st + 2, row, a);
      compute_step<KV, VEC, L, TPL, G, U>(b, qv, m, l, acc, tab, tlo, thi, st + 1, row, p.log2_bs);
    }
    tab = tab_next;
  }

}

// The state of one run on the vector ALUs: the G query rows of sequence s
// served by kv head h, over blocks [off, off+len) of its n tokens.  On return
// every row group of the wave holds the merged (m, l, acc) of the run, in
// log2 units, lane col holding elements [col*VEC, (col+1)*VEC).  All scalars
// are uniform.
template <typename KV, typename QT, int D, int G, int POL>
__device__ inline void valu_core(const DecodeParams& p, int s, int h, int off, int len, int n, float (&m)[G],
                                 float (&l)[G], float (&acc)[G][DecodeShape<KV, D>::VEC]) {
  using Sh = DecodeShape<KV, D>;
  constexpr int VEC = Sh::VEC, L = Sh::L;
  constexpr int QE = elem_size<QT>::value;
  const int lane = threadIdx.x;
  const int col = lane % L;
  const int Hq = p.num_kv_heads * G;
  const float qs = run_q_scale(p, h);
  const int tab = load_table_window(p, run_table(p, s, off), 0, len);

  // query rows of the G heads served by kv head h, pre-scaled into log2 units
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

#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[g][i] = 0.0f;
  }

  valu_stream<KV, D, G, POL>(p, s, h, off, len, n, tab, qv, m, l, acc);

  // merge the TPL row states (rows hold the same columns)
#pragma unroll
  for (int o = L; o < 64; o <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], o);
      const float lo = __shfl_xor(l[g], o);
      const float mn = fmaxf(m[g], mo);
      const float mu = mn == -INFINITY ? 0.0f : mn;
      const float a = fexp2(m[g] - mu), b = fexp2(mo - mu);
      l[g] = l[g] * a + lo * b;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[g][i] = acc[g][i] * a + __shfl_xor(acc[g][i], o) * b;
      m[g] = mn;
    }
  }
}

// Store a vector-ALU run's state as a partial record (row group 0 writes).
template <typename KV, int D, int G>
__device__ inline void valu_store_record(const RecordRef& rec, const float (&m)[G], const float (&l)[G],
                                         const float (&acc)[G][DecodeShape<KV, D>::VEC]) {
  using Sh = DecodeShape<KV, D>;
  constexpr int VEC = Sh::VEC, L = Sh::L, REC = Sh::REC;
  const int lane = threadIdx.x;
  const int row = lane / L;
  const int col = lane % L;
  if (row == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i = 0; i < VEC; i += 4)
        record_store4(rec, g * REC + col * VEC + i, acc[g][i], acc[g][i + 1], acc[g][i + 2], acc[g][i + 3]);
      if (col == 0) record_store4(rec, g * REC + D, m[g], l[g], 0.0f, 0.0f);
    }
  }
}

// Write a vector-ALU run's state as the output rows of sequence s (row
// group 0 writes).
template <typename KV, typename QT, int D, int G>
__device__ inline void valu_store_out(const DecodeParams& p, int s, int h, float vs, const float (&l)[G],
                                      const float (&acc)[G][DecodeShape<KV, D>::VEC]) {
  using Sh = DecodeShape<KV, D>;
  constexpr int VEC = Sh::VEC, L = Sh::L;
  constexpr int QE = elem_size<QT>::value;
  const int lane = threadIdx.x;
  const int row = lane / L;
  const int col = lane % L;
  const int Hq = p.num_kv_heads * G;
  const int64_t oe = ((int64_t)s * Hq + (int64_t)h * G) * D + (int64_t)col * VEC;
  if (row == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      store_row<QT, VEC>(p.out + (oe + (int64_t)g * D) * QE, acc[g], l[g] > 0.0f ? vs / l[g] : 0.0f);
  }
}

// One run on the vector ALUs: blocks [off, off+len) of the (kv head h,
// sequence s) stream, which has nb blocks and n tokens.  pos is the run's
// place in the flattened stream and wstart the worker's first block.  All
// scalars are uniform.
template <typename KV, typename QT, int D, int G, int POL>
__device__ inline void valu_run(const DecodeParams& p, int w, const ChunkGrid& grid, int wstart, int pos, int s,
                                int h, int off, int len, int n, int nb) {
  using Sh = DecodeShape<KV, D>;
  constexpr int VEC = Sh::VEC;
  const int Hq = p.num_kv_heads * G;
  // the chunks the whole run spans (worked out before the run, while few
  // registers are live)
  const int seg_start = pos - off;
  const int first_w = grid.of(seg_start);
  const int last_w = grid.of(seg_start + nb - 1);
  float m[G], l[G], acc[G][VEC];
  valu_core<KV, QT, D, G, POL>(p, s, h, off, len, n, m, l, acc);
  const float vs = run_v_scale(p, h);

  if (off == 0 && off + len == nb) {   // the whole run is ours
    valu_store_out<KV, QT, D, G>(p, s, h, vs, l, acc);
    return;
  }

  // Partial: publish (acc, m, l) through the device coherence point; the
  // worker that completes the run's count merges.
  valu_store_record<KV, D, G>(record_ref<D, G>(partial_record<D, G>(p, w, wstart, pos)), m, l, acc);
  if (arrive(p, first_w, last_w))
    merge_records<QT, D, G>(p, first_w, last_w, seg_start, grid,
                            ContiguousRows{((int64_t)s * Hq + (int64_t)h * G) * D, D}, vs);
}

}  // namespace pkv

#include "decode_mfma.h"
#include "decode_items.h"

namespace pkv {

// Stream chunk d.v of a flat plan, whose items are the non-empty sequences;
// the descriptor names the chunk's first item.  SPAN (matrix-core runs over
// partitions): stream the chunk's whole span, the runs leaving a record at
// every chunk boundary they cross.
template <typename KV, typename QT, int D, int G, bool MFMA, int POL, bool SPAN = false>
__device__ inline void decode_chunk(const DecodeParams& p, const ChunkCtx& d) {
  static_assert(!SPAN || MFMA, "span runs are matrix-core runs");
  const ChunkGrid grid = d.grid();
  const int start = grid.start(d.v);
  const int end = SPAN ? grid.span_end(d.v, d.T) : grid.end(d.v, d.T);
  int h = d.h, i = d.i, off = d.off, pos = start;
  FlatItem it{d.s, d.len, d.n};
  while (true) {
    const int len = min(it.len - off, end - pos);
    // the next run's item loads while this run streams
    int ni = i + 1, nh = h;
    if (ni == d.NI) {
      ni = 0;
      ++nh;
    }
    const bool more = pos + len < end;
    const FlatItem nx = load_flat_item(p.items + ni);
    // the chunk where the run starts, and that chunk's first block
    const int w = SPAN ? grid.of(pos) : d.v;
    const int wstart = SPAN ? grid.start(w) : start;
    if constexpr (MFMA)
      mfma_run<KV, QT, D, G, POL>(p, w, grid, wstart, pos, it.s, h, off, len, it.n, it.len);
    else
      valu_run<KV, QT, D, G, POL>(p, w, grid, wstart, pos, it.s, h, off, len, it.n, it.len);
    pos += len;
    if (!more) return;
    i = ni;
    h = nh;
    it = nx;
    off = 0;
  }
}

// A worker's chunks, one per round; the next round's descriptor loads as the
// current chunk starts.
template <typename Chunk>
__device__ inline void run_rounds(const DecodeParams& p, const PlanHeader& H, int rounds, Chunk chunk) {
  const PlanDesc* dp = p.desc + blockIdx.x;
  PlanDesc cur = load_desc(dp);
  for (int rd = 0; rd < rounds; ++rd) {
    const PlanDesc nxt = load_desc(dp + (int64_t)min(rd + 1, rounds - 1) * p.num_workers);
    if (cur.v >= 0) chunk(chunk_ctx(H, cur));
    cur = nxt;
  }
}

// Empty contexts attend to nothing: their output rows are zero.  The first
// worker checks 64 lengths per load and clears the rows of the empty ones.
template <typename QT, int D, int G>
__device__ inline void zero_empty_rows(const DecodeParams& p) {
  constexpr int QE = elem_size<QT>::value;
  const int lane = threadIdx.x;
  const int words = p.num_kv_heads * G * D * QE / 4;
  for (int base = 0; base < p.num_seqs; base += 64) {
    const int s = base + lane;
    const bool empty = s < p.num_seqs && p.context_lens[s] <= 0;
    unsigned long long mask = __ballot(empty);
    while (mask) {
      const int e = base + __builtin_ctzll(mask);
      mask &= mask - 1;
      uint32_t* o = (uint32_t*)(p.out + (int64_t)e * words * 4);
      for (int w = lane; w < words; w += 64) o[w] = 0u;
    }
  }
}

// One worker wavefront per work-group.  MFMA selects the matrix-core run
// (query groups with a 16-bit operand type) over the vector-ALU run.  The
// grid is 8 workers per CU, two per SIMD, so the matrix-core runs may take
// up to 256 VGPRs: with the earlier cap of 168 (three waves per SIMD, which
// only short-lived partition work-groups could use) the fp8 GQA workloads
// ran about 2% slower on MI355X.
//
// The plan kernel, run just before on the same stream, gives each worker
// one descriptor per round: the chunk it streams and where that chunk
// starts.  Grouped plans (shared prefixes read once per group) run where the
// dtype pair has a matrix-core operand type.
template <typename KV, typename QT, int D, int G, bool MFMA>
__global__ __launch_bounds__(64)
__attribute__((amdgpu_waves_per_eu(MFMA && D <= 128 ? 2 : 1)))
void paged_decode_kernel(const DecodeParams p) {
  constexpr bool kGroupable = !std::is_void<typename mfma_operand<KV, QT>::type>::value && G <= 8;
  const PlanHeader H = load_header(p.header);
  if ((H.flags & kPlanEmpty) && blockIdx.x == 0) zero_empty_rows<QT, D, G>(p);
  if (H.rounds == 0) return;
  if (H.flags & kPlanGrouped) {
    if constexpr (kGroupable)
      run_rounds(p, H, H.rounds, [&](const ChunkCtx& d) { grouped_chunk<KV, QT, D, G, MFMA>(p, d); });
    return;
  }
  if constexpr (MFMA) {
    // partitions: a matrix-core worker streams its span in one pass (the
    // span's first chunk, its one descriptor, opens it), leaving a record per
    // partition
    if (H.q > 1) {
      if (H.flags & kPlanShared)
        run_rounds(p, H, 1,
                   [&](const ChunkCtx& d) { decode_chunk<KV, QT, D, G, MFMA, kSharedPolicy, true>(p, d); });
      else
        run_rounds(p, H, 1,
                   [&](const ChunkCtx& d) { decode_chunk<KV, QT, D, G, MFMA, kStreamPolicy, true>(p, d); });
      return;
    }
  }
  if (H.flags & kPlanShared)
    run_rounds(p, H, H.rounds, [&](const ChunkCtx& d) { decode_chunk<KV, QT, D, G, MFMA, kSharedPolicy>(p, d); });
  else
    run_rounds(p, H, H.rounds, [&](const ChunkCtx& d) { decode_chunk<KV, QT, D, G, MFMA, kStreamPolicy>(p, d); });
}

// Launch one instantiation; defined per KV/Q dtype pair in decode_*.hip.
// use_mfma asks for the matrix-core run; it is honoured where the dtype pair
// has an operand type and blocks hold whole 16-token tiles.
template <typename KV, typename QT>
kv_status_t launch_decode(const DecodeParams& p, int D, int G, bool use_mfma, hipStream_t stream) {
  constexpr bool kHasMfma = !std::is_void<typename mfma_operand<KV, QT>::type>::value;
  const bool mfma = kHasMfma && use_mfma && p.log2_bs >= 4;
#define PKV_CASE(DD, GG)                                                                                   \
  if (D == DD && G == GG) {                                                                                \
    if constexpr (kHasMfma && GG > 1) {                                                                    \
      if (mfma) {                                                                                          \
        hipLaunchKernelGGL((paged_decode_kernel<KV, QT, DD, GG, true>), dim3(p.num_workers), dim3(64), 0, \
                           stream, p);                                                                     \
        return launch_status();                                                                            \
      }                                                                                                    \
    }                                                                                                      \
    hipLaunchKernelGGL((paged_decode_kernel<KV, QT, DD, GG, false>), dim3(p.num_workers), dim3(64), 0,    \
                       stream, p);                                                                         \
    return launch_status();                                                                                \
  }
  // 16 query heads per kv head fill the matrix-core tile's 16 rows; the
  // vector-ALU run does not hold that many query rows in registers
#define PKV_CASE16(DD)                                                                                     \
  if (D == DD && G == 16) {                                                                                \
    if constexpr (kHasMfma) {                                                                              \
      if (mfma) {                                                                                          \
        hipLaunchKernelGGL((paged_decode_kernel<KV, QT, DD, 16, true>), dim3(p.num_workers), dim3(64), 0,  \
                           stream, p);                                                                     \
        return launch_status();                                                                            \
      }                                                                                                    \
    }                                                                                                      \
    return KV_ERR_UNSUPPORTED;                                                                             \
  }
#define PKV_CASES(DD) PKV_CASE(DD, 1) PKV_CASE(DD, 2) PKV_CASE(DD, 4) PKV_CASE(DD, 8) PKV_CASE16(DD)
  PKV_CASES(64)
  PKV_CASES(128)
  PKV_CASES(256)
#undef PKV_CASES
#undef PKV_CASE16
#undef PKV_CASE
  return KV_ERR_UNSUPPORTED;
}

kv_status_t launch_decode_f32_f32(const DecodeParams& p, int D, int G, bool mfma, hipStream_t s);
kv_status_t launch_decode_f16_f16(const DecodeParams& p, int D, int G, bool mfma, hipStream_t s);
kv_status_t launch_decode_bf16_bf16(const DecodeParams& p, int D, int G, bool mfma, hipStream_t s);
kv_status_t launch_decode_fp8_f32(const DecodeParams& p, int D, int G, bool mfma, hipStream_t s);
kv_status_t launch_decode_fp8_f16(const DecodeParams& p, int D, int G, bool mfma, hipStream_t s);
kv_status_t launch_decode_fp8_bf16(const DecodeParams& p, int D, int G, bool mfma, hipStream_t s);

}  // namespace pkv
