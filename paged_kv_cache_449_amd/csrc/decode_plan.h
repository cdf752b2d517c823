// Work plan of one decode launch.
//
// Before the decode kernel runs, one work-group reads every sequence's
// context length and the heads of the block tables once, and writes to the
// workspace everything the decode workers would otherwise each work out for
// themselves: the runs ("items") the block stream is made of, and where each
// worker's share of that stream starts.  A worker then finds its start with
// one load, however many sequences the batch holds.
//
// The planner also finds sequences that share the blocks of a common prefix:
// the n candidates forked from one prompt read the prompt's blocks through
// their own tables, with reference count n ("vLLM — 把操作系统的分页搬进 GPU KV
// cache": core mechanism 3 and case 2).  Consecutive sequences linked by a
// shared first block form a run, cut into groups of at most 16 query rows
// (16/G members).  A group's shared length is the number of leading table
// entries all its members hold in common, counted only over blocks every
// member fills completely.  Groups are found by comparing the table entries
// themselves, so any prefix the tables share is read once, and nothing else
// is merged.
//
// Items.  Each (kv head, item) is a run of whole blocks:
//   - a G-item: a group's shared prefix, read once for every member's query
//     rows (members x query heads, at most 16 matrix-core rows);
//   - an S-item: one sequence's own blocks (all of them, or those after its
//     group's shared prefix).
// Items are laid out in sequence order per kv head (a group's G-item, then
// each member's S-item), and the kv heads one after another: the stream of T
// blocks that the workers cut into equal chunks.  Without groups every item
// is a whole sequence, and the stream is the flat (kv head, sequence, block)
// stream.
#pragma once

#include "common.h"

namespace pkv {

// One item (48 bytes).
struct PlanItem {
  int32_t s;        // sequence (G-item: the group's first member)
  int32_t off;      // first block of the item in the sequence's table
  int32_t len;      // blocks (>= 1)
  int32_t n;        // token limit: the sequence's context length (G-item: len * block_size)
  int32_t pos;      // first block of the item in a kv head's stream
  int32_t m;        // G-item: members (>= 2); S-item: 0
  int32_t rbase;    // grouped mode: first record row of the item in a kv head's record rows
  // S-items of group members (grouped mode): the group's G-item, for the merge
  int32_t member;   // index of the sequence in its group
  int32_t g_pos;    // the G-item's first block in a kv head's stream
  int32_t g_len;    // its blocks (0: the sequence is in no group)
  int32_t g_rbase;  // its first record row
  int32_t g_m;      // the group's members
};

// Per sequence, grouped mode (16 bytes): its S-item, for the merge a G-item
// piece may run for it.
struct PlanSeq {
  int32_t s_item;   // -1: all of its blocks are shared
  int32_t s_pos;
  int32_t s_len;
  int32_t s_rbase;
};

// Start of one worker's chunk in one round (32 bytes).
struct PlanDesc {
  int32_t v;       // chunk id; -1: no chunk for this worker in this round
  int32_t h;       // kv head of the chunk's first block
  int32_t i;       // item of the chunk's first block
  int32_t off;     // block of the chunk's start within that item
  int32_t s;       // that item's sequence, blocks and token limit (flat
  int32_t len;     // plans; a grouped chunk loads its item)
  int32_t n;
  int32_t pad;
};

// How the stream of T blocks is cut into chunks: spans of `span` blocks,
// each cut into q chunks of `chunk` blocks (the last chunk of a span may be
// shorter, and the last span).  Chunk ids follow stream order.  With q = 1
// (span = chunk) the cut is uniform.
struct ChunkGrid {
  int32_t chunk, span, q;
  // chunk holding stream block x
  __device__ int of(int x) const {
    if (q == 1) return x / chunk;
    const int u = x / span;
    return u * q + (x - u * span) / chunk;
  }
  // first block of chunk v
  __device__ int start(int v) const {
    if (q == 1) return v * chunk;
    const int u = v / q;
    return u * span + (v - u * q) * chunk;
  }
  // one past its last block
  __device__ int end(int v, int T) const {
    if (q == 1) return min((v + 1) * chunk, T);
    const int u = v / q;
    return min(min(u * span + (v - u * q + 1) * chunk, (u + 1) * span), T);
  }
  // one past the last block of its span
  __device__ int span_end(int v, int T) const { return min((v / q + 1) * span, T); }
};
__device__ inline ChunkGrid uniform_grid(int chunk) { return ChunkGrid{chunk, chunk, 1}; }

// What every worker of a launch shares (48 bytes).
struct PlanHeader {
  int32_t chunk;   // blocks per chunk
  int32_t T;       // blocks in the stream (all kv heads)
  int32_t TB;      // blocks per kv head
  int32_t NI;      // items per kv head
  int32_t flags;   // kPlanShared | kPlanGrouped | kPlanEmpty
  int32_t rounds;  // chunks per worker
  int32_t RH;      // grouped mode: record rows per kv head
  int32_t span;    // blocks per span (the chunk grid)
  int32_t q;       // chunks per span
  int32_t pad[3];
};

// A worker's view of one chunk: the launch's header and the chunk's start.
struct ChunkCtx {
  int32_t chunk, T, TB, NI, flags, rounds, RH, span, q;
  int32_t v, h, i, off, s, len, n;
  __device__ ChunkGrid grid() const { return ChunkGrid{chunk, span, q}; }
};

// Flat mode in which some sequence starts on its predecessor's first block
// (sharing that is not grouped): the stream is cut kSharedSplit times finer
// and read with the default cache policy, so candidates meet in the L2.
constexpr int kPlanShared = 1;
// Grouped mode: G-items read shared prefixes once per group.
constexpr int kPlanGrouped = 2;
// Some context is empty: the decode kernel zeroes those output rows.
constexpr int kPlanEmpty = 4;

// Per-sequence state of the planner (32 bytes).
struct PlanScratch {
  int32_t n;        // context length, clamped to [0, max_blocks * bs]
  int32_t eq;       // starts on its predecessor's first block (both non-empty)
  int32_t c;        // leading full blocks shared with the predecessor
  int32_t gid;      // group
  int32_t s_item;   // its S-item (-1: none), then that item's position,
  int32_t s_pos;    // blocks and first record row
  int32_t s_len;
  int32_t s_rbase;
};

// Per group (24 bytes).
struct PlanGroup {
  int32_t k;        // shared blocks: the least c over the non-first members
  int32_t m;        // members
  int32_t first;    // its first member
  int32_t item;     // real groups: its G-item, with that item's position and
  int32_t pos;      // first record row
  int32_t rbase;
};

struct PlanParams {
  const int32_t* block_tables;
  const int32_t* context_lens;
  PlanScratch* scr;          // [num_seqs] (batches past the LDS capacity)
  PlanGroup* groups;         // [num_seqs] (same)
  PlanItem* items;           // [3 * num_seqs / 2 + 1]
  PlanSeq* seqs;             // [num_seqs]
  PlanDesc* desc;            // [desc_rounds][num_workers]
  PlanHeader* header;
  int64_t grec_rows;         // record rows the workspace holds for grouped mode
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t log2_bs;
  int32_t G;                 // query heads per kv head
  int32_t chunk;             // blocks per chunk; 0 = sized from num_workers
  int32_t num_workers;       // decode work-groups launched (multiple of 8)
  int32_t desc_rounds;       // rounds the descriptor table holds
  int32_t max_members;       // sequences per group; < 2 = no grouping
  int32_t shared_split;      // rounds of the shared mode (kSharedSplit)
  int32_t counter_slots;     // arrival counters (grouped mode uses one per (kv head, sequence))
  int32_t span_runs;         // the decode kernel streams a span of partitions in one pass
};

// Sequences whose planner state fits the work-group's LDS; larger batches
// keep it in the workspace.
constexpr int kPlanLdsSeqs = 1024;
constexpr int kPlanLdsItems = kPlanLdsSeqs + kPlanLdsSeqs / 2;

// Plan entries are stored 16 bytes at a time (all are 16-byte aligned).
__device__ inline void put_item(PlanItem* dst, const PlanItem& v) {
  int4* d = (int4*)dst;
  d[0] = make_int4(v.s, v.off, v.len, v.n);
  d[1] = make_int4(v.pos, v.m, v.rbase, v.member);
  d[2] = make_int4(v.g_pos, v.g_len, v.g_rbase, v.g_m);
}
__device__ inline void put_desc(PlanDesc* dst, const PlanDesc& v) {
  int4* d = (int4*)dst;
  d[0] = make_int4(v.v, v.h, v.i, v.off);
  d[1] = make_int4(v.s, v.len, v.n, 0);
}

// The decode kernel reads the plan with scalar loads: the addresses are
// uniform, and the data was written by the planner before the launch started
// and is only read during it, so it can go through the scalar cache into
// scalar registers, where an item load issued before a run stays in flight
// while the run streams without taking vector registers.
typedef const __attribute__((address_space(4))) int32_t* const_words;
__device__ inline PlanItem load_item(const PlanItem* it) {
  const const_words w = (const_words)it;
  return PlanItem{w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7], w[8], w[9], w[10], w[11]};
}
// What a flat plan's chunks read of an item: its sequence, blocks and token
// limit.
struct FlatItem {
  int32_t s, len, n;
};
__device__ inline FlatItem load_flat_item(const PlanItem* it) {
  const const_words w = (const_words)it;
  return FlatItem{w[0], w[2], w[3]};
}
__device__ inline PlanHeader load_header(const PlanHeader* h) {
  const const_words w = (const_words)h;
  return PlanHeader{w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7], w[8], {0, 0, 0}};
}
__device__ inline PlanDesc load_desc(const PlanDesc* d) {
  const const_words w = (const_words)d;
  return PlanDesc{w[0], w[1], w[2], w[3], w[4], w[5], w[6], 0};
}
__device__ inline ChunkCtx chunk_ctx(const PlanHeader& H, const PlanDesc& d) {
  return ChunkCtx{H.chunk, H.T, H.TB, H.NI, H.flags, H.rounds, H.RH, H.span, H.q,
                  d.v, d.h, d.i, d.off, d.s, d.len, d.n};
}

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

// Exclusive prefix sum of v over the work-group's threads in thread order;
// *total receives the sum of all.  lds: kPlanWaves ints.
__device__ inline int plan_scan_sum(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_inclusive_scan_i32(v, lane);
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    const int x = lds[w];
    before += w < wave ? x : 0;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Exclusive prefix sums of three values at once (one pair of barriers).
// lds: 3 * kPlanWaves ints.
__device__ inline int3 plan_scan_sum3(int3 v, int* lds, int3* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ia = wave_inclusive_scan_i32(v.x, lane);
  const int ib = wave_inclusive_scan_i32(v.y, lane);
  const int ic = wave_inclusive_scan_i32(v.z, lane);
  if (lane == 63) {
    lds[wave] = ia;
    lds[kPlanWaves + wave] = ib;
    lds[2 * kPlanWaves + wave] = ic;
  }
  __syncthreads();
  int3 before = make_int3(0, 0, 0), all = make_int3(0, 0, 0);
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    const int x = lds[w], y = lds[kPlanWaves + w], z = lds[2 * kPlanWaves + w];
    if (w < wave) {
      before.x += x;
      before.y += y;
      before.z += z;
    }
    all.x += x;
    all.y += y;
    all.z += z;
  }
  __syncthreads();
  *total = all;
  return make_int3(before.x + ia - v.x, before.y + ib - v.y, before.z + ic - v.z);
}

// Inclusive prefix max of v over the work-group's threads; *total receives
// the maximum of all.
__device__ inline int plan_scan_max(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl = max(incl, t);
  }
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  int before = INT32_MIN, all = INT32_MIN;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    const int x = lds[w];
    before = w < wave ? max(before, x) : before;
    all = max(all, x);
  }
  __syncthreads();
  *total = all;
  return max(before, incl);
}

// Items of one sequence.
struct SeqItems {
  bool lead;     // it writes its group's G-item
  int k;         // blocks of its group's shared prefix (0: none)
  int suffix;    // blocks of its S-item (0: none)
  int m;         // members of its group (real groups)
};

__device__ inline bool real_group(const PlanGroup& g) { return g.m >= 2 && g.k >= 1; }

__device__ inline int plan_clamp(int n, int max_len) { return n < 0 ? 0 : (n > max_len ? max_len : n); }

__device__ inline SeqItems seq_items(const PlanScratch* scr, const PlanGroup* grp, int log2_bs, int s,
                                     bool grouped) {
  SeqItems r{false, 0, 0, 0};
  const int n = scr[s].n;
  if (n == 0) return r;
  const int nb = (n + (1 << log2_bs) - 1) >> log2_bs;
  if (grouped) {
    const PlanGroup g = grp[scr[s].gid];
    if (real_group(g)) {
      r.k = g.k;
      r.m = g.m;
      r.lead = g.first == s;
    }
  }
  r.suffix = nb - r.k;
  return r;
}

}  // namespace pkv
