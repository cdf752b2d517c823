// Work plan of one decode launch.
//
// Before the decode kernel runs, one work-group reads every sequence's
// context length and the heads of the block tables once, and writes to the
// workspace everything the decode workers would otherwise each work out for
// themselves: where each worker's share of the block stream starts, and the
// runs ("items") the stream is made of.  A worker then finds its start with
// one load, however many sequences the batch holds.
//
// The planner also finds sequences that share the blocks of a common prefix
// -- the n candidates forked from one prompt read the prompt's blocks through
// their own tables, with reference count n ("vLLM — 把操作系统的分页搬进 GPU KV
// cache": core mechanism 3 and case 2).  Consecutive sequences whose tables
// start with the same physical block are a group (at most 16 query rows: 16/G
// members); the group's shared length is the number of leading table entries
// all members hold in common, cut to whole blocks inside every member's
// context.  Groups are found by comparing the table entries themselves, so any
// table that shares a prefix is read once for it, and nothing else is.
//
// Items.  Each (kv head, item) is a run of whole blocks:
//   - a G-item: a group's shared prefix, read once for every member's query
//     rows (members x query heads, at most 16 matrix-core rows);
//   - an S-item: one sequence's own blocks (all of them, or those after its
//     group's shared prefix).
// Items are laid out in sequence order per kv head (a group's G-item, then
// the members' S-items), and the kv heads one after another: the stream of
// T blocks the workers split into equal chunks.  Without groups every item
// is a whole sequence and the stream is the flat (kv head, sequence, block)
// stream of the decode kernel.
#pragma once

#include "common.h"

namespace pkv {

// One item (32 bytes).
struct PlanItem {
  int32_t s;      // sequence (G-item: the group's first member)
  int32_t off;    // first block of the item in the sequence's table
  int32_t len;    // blocks (>= 1)
  int32_t n;      // token limit: the sequence's context length (G-item: len * block_size)
  int32_t pos;    // first block of the item in a kv head's stream
  int32_t m;      // G-item: members (>= 2); S-item: 0
  int32_t rbase;  // grouped mode: first record row of the item in a kv head's record rows
  int32_t pad;
};

// Per sequence, grouped mode (16 bytes).
struct PlanSeq {
  int32_t g_item;  // item of its group's shared prefix, -1 if it has none
  int32_t member;  // its index in the group
  int32_t s_item;  // item of its own blocks, -1 if they are all shared
  int32_t pad;
};

// Start of one worker's chunk for one round (48 bytes).  Every field but v,
// h, i and off is the same in all descriptors of a launch.
struct PlanDesc {
  int32_t v;       // chunk id; -1: this worker has no chunk in this round
  int32_t h;       // kv head of the chunk's first block
  int32_t i;       // item of the chunk's first block
  int32_t off;     // block of the chunk's start within that item
  int32_t chunk;   // blocks per chunk
  int32_t T;       // blocks in the stream (all kv heads)
  int32_t TB;      // blocks per kv head
  int32_t NI;      // items per kv head
  int32_t flags;   // kPlanShared | kPlanGrouped
  int32_t rounds;  // chunks per worker (1, or kSharedSplit in shared mode)
  int32_t RH;      // grouped mode: record rows per kv head
  int32_t pad;
};

// Flat mode with some sequence starting on its predecessor's first block
// (sharing that could not be grouped): the stream is cut finer and read with
// the default cache policy, so candidates meet in the L2.
constexpr int kPlanShared = 1;
// Grouped mode: G-items read shared prefixes once per group.
constexpr int kPlanGrouped = 2;

// Per-sequence scratch of the planner (16 bytes).
struct PlanScratch {
  int32_t n;      // context length, clamped to [0, max_blocks * bs]
  int32_t c;      // table entries shared with the previous sequence (0: none)
  int32_t gid;    // group of the sequence
  int32_t pad;
};

struct PlanGroup {
  int32_t k;      // shared blocks (min over the non-first members' c)
  int32_t m;      // members
};

struct PlanParams {
  const int32_t* block_tables;
  const int32_t* context_lens;
  uint8_t* out;              // rows of empty contexts are zeroed here
  PlanScratch* scr;          // [num_seqs]
  PlanGroup* groups;         // [num_seqs]
  PlanItem* items;           // [max_items]
  PlanSeq* seqs;             // [num_seqs]
  PlanDesc* desc;            // [desc_rounds * num_workers]
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t log2_bs;
  int32_t G;                 // query heads per kv head
  int32_t out_row_bytes;     // bytes of one sequence's output rows (all query heads)
  int32_t chunk;             // blocks per chunk; 0 = sized from num_workers
  int32_t num_workers;       // decode work-groups launched (multiple of 8)
  int32_t desc_rounds;       // rounds the descriptor table holds
  int32_t max_members;       // sequences per group; < 2 = no grouping
  int32_t shared_split;      // rounds of the shared mode
  int64_t grec_rows;         // record rows the workspace holds for grouped mode
  int32_t counter_slots;     // arrival counters (grouped mode needs one per (kv head, sequence))
};

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

__device__ inline int plan_clamp_len(int n, int max_len) { return n < 0 ? 0 : (n > max_len ? max_len : n); }

// Items of sequence s (n > 0): its group's G-item if it leads a real group,
// then its S-item if any of its blocks are its own.  Returns the number of
// items and, in *blocks, the stream blocks they hold.
struct SeqItems {
  bool lead;     // writes its group's G-item
  int k;         // blocks of its group's shared prefix (0: none)
  int suffix;    // blocks of its S-item (0: none)
};

__device__ inline SeqItems seq_items(const PlanParams& pp, int s, bool grouped) {
  SeqItems r{false, 0, 0};
  const PlanScratch sc = pp.scr[s];
  if (sc.n == 0) return r;
  const int nb = (sc.n + (1 << pp.log2_bs) - 1) >> pp.log2_bs;
  if (grouped) {
    const PlanGroup g = pp.groups[sc.gid];
    if (g.m >= 2 && g.k >= 1) {
      r.k = g.k;
      r.lead = s == 0 || pp.scr[s - 1].gid != sc.gid;
    }
  }
  r.suffix = nb - r.k;
  return r;
}

// Lay out the items of every sequence (grouped or flat), then, once the
// chunk size is known, their record rows.  Returns per-kv-head item and
// block counts through the LDS scalars.
__device__ inline void plan_items(const PlanParams& pp, bool grouped, int* lds, int* NI_out, int* TB_out) {
  const int S = pp.num_seqs;
  int icarry = 0, bcarry = 0;
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + (int)threadIdx.x;
    SeqItems it{false, 0, 0};
    if (s < S) it = seq_items(pp, s, grouped);
    const int ni = (it.lead ? 1 : 0) + (it.suffix > 0 ? 1 : 0);
    const int nbk = (it.lead ? it.k : 0) + it.suffix;
    int itot, btot;
    const int ib = icarry + plan_scan_sum(ni, lds, &itot);
    const int bb = bcarry + plan_scan_sum(nbk, lds, &btot);
    if (s < S) {
      const PlanScratch sc = pp.scr[s];
      int i = ib, pos = bb;
      PlanSeq ps{-1, 0, -1, 0};
      if (it.lead) {
        PlanItem g{s, 0, it.k, it.k << pp.log2_bs, pos, pp.groups[sc.gid].m, 0, 0};
        pp.items[i] = g;
        ++i;
        pos += it.k;
      }
      if (it.suffix > 0) {
        PlanItem q{s, it.k, it.suffix, sc.n, pos, 0, 0, 0};
        pp.items[i] = q;
        ps.s_item = i;
      }
      pp.seqs[s] = ps;   // g_item and member are filled in by plan_members
    }
    icarry += itot;
    bcarry += btot;
  }
  *NI_out = icarry;
  *TB_out = bcarry;
}

// Grouped mode: each sequence's group item and member index (the group's
// G-item sits at the first member's item index).
__device__ inline void plan_members(const PlanParams& pp) {
  const int S = pp.num_seqs;
  for (int s = threadIdx.x; s < S; s += kPlanThreads) {
    const PlanScratch sc = pp.scr[s];
    if (sc.n == 0) continue;
    const PlanGroup g = pp.groups[sc.gid];
    if (!(g.m >= 2 && g.k >= 1)) continue;
    // the group's first member: walk back over the members (at most 15)
    int f = s;
    while (f > 0 && pp.scr[f - 1].gid == sc.gid) --f;
    // the first member's items start with the G-item: its index is the one
    // before the first member's S-item, or the item right after the previous
    // sequence's items
    const PlanSeq pf = pp.seqs[f];
    int gi;
    if (pf.s_item >= 0) {
      gi = pf.s_item - 1;
    } else {
      // the first member has no blocks of its own: find the G-item by
      // scanning back from the next item of a later member or sequence
      int t = f + 1;
      while (t < S && pp.seqs[t].s_item < 0) ++t;
      gi = -1;
      // items between the first member and sequence t: the G-item, then the
      // S-items of members f+1..t-1 (none, since their s_item < 0)
      gi = (t < S) ? pp.seqs[t].s_item - 1 - (pp.scr[t].gid == sc.gid ? 0 : 0) : -2;
    }
    PlanSeq ps = pp.seqs[s];
    ps.g_item = gi;
    ps.member = s - f;
    pp.seqs[s] = ps;
  }
}

}  // namespace pkv
