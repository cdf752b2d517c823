// Host entry points of paged decode attention: argument checks, work split,
// workspace layout and dispatch to the kernel instantiations.
#include <algorithm>
#include <mutex>

#include "decode_kernel.h"

namespace pkv {

// Lay out the items of every sequence, grouped or flat, and the chunk size;
// in grouped mode also every item's record rows.  Only the planner's state
// is written here (each sequence's S-item, each group's G-item, and, when it
// is in LDS, every item's first block and sequence in item_ls); returns
// ok = false when a grouped layout's records would not fit the workspace.
struct Layout {
  int NI, TB, chunk, span, q, rounds, flags;
  int64_t RH;
  bool ok;
};

// Most pieces (parts inside one chunk) a run of len blocks can be cut into.
__device__ inline int max_pieces(int len, int chunk, int span, int q) {
  return (len + chunk - 1) / chunk + 1 + (q > 1 ? (len + span - 1) / span : 0);
}

__device__ __attribute__((always_inline)) inline Layout plan_layout(const PlanParams& pp, PlanScratch* scr,
                                                                    PlanGroup* grp, int2* item_ls, bool grouped,
                                                                    bool has_eq, int* lds) {
  const int S = pp.num_seqs;
  const int tid = threadIdx.x;
  // blocks per kv head first: they fix the chunk size, which the record
  // rows depend on
  int TB = 0;
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + tid;
    int nbk = 0;
    if (s < S) {
      const SeqItems it = seq_items(scr, grp, pp.log2_bs, s, grouped);
      nbk = (it.lead ? it.k : 0) + it.suffix;
    }
    int tot;
    plan_scan_sum(nbk, lds, &tot);
    TB += tot;
  }
  const int flags = grouped ? kPlanGrouped : (has_eq ? kPlanShared : 0);
  const int64_t T64 = (int64_t)TB * pp.num_kv_heads;
  int rounds, chunk, span, q;
  if (pp.chunk > 0) {
    // caller-sized partitions: every worker takes an equal span of the
    // stream and runs it as q chunks of at most pp.chunk blocks, one per
    // round
    span = (int)max((int64_t)1, (T64 + pp.num_workers - 1) / pp.num_workers);
    chunk = min(pp.chunk, span);
    q = (span + chunk - 1) / chunk;
    rounds = q;
  } else {
    rounds = (flags & kPlanShared) ? pp.shared_split : 1;
    const int64_t w = (int64_t)pp.num_workers * rounds;
    chunk = (int)max((int64_t)1, (T64 + w - 1) / w);
    span = chunk;
    q = 1;
  }

  int icarry = 0, bcarry = 0;
  int64_t rcarry = 0;
  for (int base = 0; base < S; base += kPlanThreads) {
    const int s = base + tid;
    SeqItems it{false, 0, 0, 0};
    if (s < S) it = seq_items(scr, grp, pp.log2_bs, s, grouped);
    // record rows: at most ceil(len / chunk) + 1 pieces, each with the
    // item's rows (G-item: members x query heads)
    const int gp = (grouped && it.lead) ? max_pieces(it.k, chunk, span, q) * it.m * pp.G : 0;
    const int sp = (grouped && it.suffix > 0) ? max_pieces(it.suffix, chunk, span, q) * pp.G : 0;
    int3 tot;
    const int3 ex = plan_scan_sum3(make_int3((it.lead ? 1 : 0) + (it.suffix > 0 ? 1 : 0),
                                             (it.lead ? it.k : 0) + it.suffix, gp + sp), lds, &tot);
    const int ib = icarry + ex.x, bb = bcarry + ex.y;
    const int64_t rb = rcarry + ex.z;
    if (s < S) {
      PlanScratch* sc = scr + s;
      if (it.lead) {
        PlanGroup* g = grp + sc->gid;
        g->item = ib;
        g->pos = bb;
        g->rbase = (int32_t)rb;
        if (item_ls) item_ls[ib] = make_int2(bb, s);
      }
      sc->s_item = it.suffix > 0 ? ib + (it.lead ? 1 : 0) : -1;
      sc->s_pos = bb + (it.lead ? it.k : 0);
      sc->s_len = it.suffix;
      sc->s_rbase = (int32_t)(rb + gp);
      if (item_ls && it.suffix > 0) item_ls[sc->s_item] = make_int2(sc->s_pos, s);
    }
    icarry += tot.x;
    bcarry += tot.y;
    rcarry += tot.z;
    if (rcarry > ((int64_t)1 << 30)) return Layout{0, 0, 0, 0, 0, 0, 0, 0, false};   // past any workspace
  }
  if (grouped && rcarry * pp.num_kv_heads > pp.grec_rows) return Layout{0, 0, 0, 0, 0, 0, 0, 0, false};
  return Layout{icarry, bcarry, chunk, span, q, rounds, flags, rcarry, true};
}

// The items and each sequence's entry, from the planner's state.
__device__ __attribute__((always_inline)) inline void plan_write_items(const PlanParams& pp, const PlanScratch* scr,
                                                                       const PlanGroup* grp, bool grouped) {
  for (int s = threadIdx.x; s < pp.num_seqs; s += kPlanThreads) {
    const PlanScratch sc = scr[s];
    PlanGroup g{0, 0, 0, 0, 0, 0};
    if (grouped && sc.n > 0) g = grp[sc.gid];
    const bool member = grouped && sc.n > 0 && real_group(g);
    if (member && g.first == s)
      put_item(pp.items + g.item, PlanItem{s, 0, g.k, g.k << pp.log2_bs, g.pos, g.m, g.rbase, 0, 0, 0, 0, 0});
    if (sc.s_item >= 0) {
      PlanItem q{s, 0, sc.s_len, sc.n, sc.s_pos, 0, sc.s_rbase, 0, 0, 0, 0, 0};
      if (member) {
        q.off = g.k;
        q.member = s - g.first;
        q.g_pos = g.pos;
        q.g_len = g.k;
        q.g_rbase = g.rbase;
        q.g_m = g.m;
      }
      put_item(pp.items + sc.s_item, q);
    }
    *(int4*)(pp.seqs + s) = make_int4(sc.s_item, sc.s_pos, sc.s_len, sc.s_rbase);
  }
}

// The descriptors, one worker slot per thread, so the stores of a wave fill
// whole cache lines.  Where a chunk runs:
//   - uniform cut (q = 1): chunk v in round v / per_round, with id
//     v % per_round;
//   - partitions (q > 1): chunk v, the (v % q)-th of span v / q, in round
//     v % q, with id v / q, so a worker runs its span's chunks in order;
// slot b runs on XCD b % 8 and takes id (b % 8) * (per_round / 8) + b / 8.
// A slot finds its chunk's first item by binary search over the items'
// first blocks.  A descriptor also carries the sequence, blocks and token
// limit of that item (flat plans start from them without an item load).
// Slots without a chunk are marked empty.  item_at(i) gives item i's first
// block, sequence, blocks and token limit.
template <typename ItemAt>
__device__ __attribute__((always_inline)) inline void plan_write_descs(const PlanParams& pp, const Layout& L,
                                                                       const ItemAt& item_at) {
  const int tid = threadIdx.x;
  const int TB = L.TB, W = pp.num_workers, C = L.chunk, SP = L.span, Q = L.q;
  const int T = TB * pp.num_kv_heads;
  const int spans = (T + SP - 1) / SP;
  // chunk ids; those of the last span that start past the stream's end hold
  // no chunk
  const int nid = spans * Q;
  int per_round, rounds;
  if (Q > 1) {
    per_round = (spans + 7) & ~7;   // spans <= W, a multiple of 8
    rounds = Q;
  } else {
    // spread evenly over the rounds: a multiple of 8, at most W
    per_round = min(W, ((nid + L.rounds - 1) / L.rounds + 7) & ~7);
    rounds = nid > 0 ? (nid + per_round - 1) / per_round : 0;   // rounds that hold a chunk
  }
  const int q8 = per_round >> 3;
  // one pass per span (flat plans): only the first chunk of each span has a
  // descriptor (round 0, id = span)
  const bool one_pass = Q > 1 && pp.span_runs && !(L.flags & kPlanGrouped);
  auto find = [&](int r) {   // the last item whose first block is <= r
    int lo = 0, hi = L.NI;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (item_at(mid).x <= r) lo = mid; else hi = mid;
    }
    return lo;
  };
  // the first round's descriptors are written even when no chunk exists
  const int n_slots = one_pass ? W : max(rounds, 1) * W;
  int b = tid % W, rd = tid / W;
  const int db = kPlanThreads % W, drd = kPlanThreads / W;
  for (int k = tid; k < n_slots; k += kPlanThreads) {
    const int u = (b & 7) * q8 + (b >> 3);
    const int v = Q > 1 ? u * Q + rd : rd * per_round + u;
    const int st = Q > 1 ? u * SP + rd * C : v * C;
    PlanDesc d{-1, 0, 0, 0, 0, 0, 0, 0};
    if (b < per_round && v < nid && st < T) {
      const int h = st / TB, r = st - h * TB;
      const int i = find(r);
      const int4 it = item_at(i);
      d = PlanDesc{v, h, i, r - it.x, it.y, it.z, it.w, 0};
    }
    put_desc(pp.desc + k, d);
    b += db;
    rd += drd;
    if (b >= W) {
      b -= W;
      ++rd;
    }
  }
  if (tid == 0)
    *pp.header = PlanHeader{L.chunk, T, TB, L.NI, L.flags, one_pass ? 1 : rounds, (int32_t)L.RH, L.span, L.q,
                            {0, 0, 0}};
}

template <bool IN_LDS>
__device__ __attribute__((always_inline)) inline void plan_body(const PlanParams& pp, PlanScratch* scr,
                                                                PlanGroup* grp, int2* item_ls, int* lds, int* any) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int S = pp.num_seqs;
  const int max_len = pp.max_blocks << pp.log2_bs;

  // A. Lengths, and whether a sequence starts on its predecessor's first
  //    block (both sequences' lengths and first entries loaded together).
  bool eq_any = false, empty_any = false;
  for (int s = tid; s < S; s += kPlanThreads) {
    const int sp = max(s - 1, 0);
    const int n = plan_clamp(pp.context_lens[s], max_len);
    const int np = plan_clamp(pp.context_lens[sp], max_len);
    const int b0 = pp.block_tables[(int64_t)s * pp.max_blocks];
    const int bp = pp.block_tables[(int64_t)sp * pp.max_blocks];
    const bool eq = s > 0 && n > 0 && np > 0 && (uint32_t)b0 < (uint32_t)pp.num_blocks && b0 == bp;
    scr[s] = PlanScratch{n, eq ? 1 : 0, 0, s, -1, 0, 0, 0};
    eq_any |= eq;
    empty_any |= n == 0;
  }
  if (eq_any) atomicOr(&any[0], 1);
  if (empty_any) atomicOr(&any[1], 1);
  __syncthreads();
  const bool has_eq = any[0] != 0, has_empty = any[1] != 0;
  bool grouped = has_eq && pp.max_members >= 2 && (int64_t)pp.num_kv_heads * S <= (int64_t)pp.counter_slots;

  if (grouped) {
    // B. Leading full blocks shared with the predecessor.  A wave compares
    //    the two table rows of up to 16 of its sequences at a time, 64
    //    consecutive entries per row per load (all loads issued together).
    constexpr int K = 16;
    for (int s0 = wave; s0 < S; s0 += kPlanWaves * K) {
      int cap[K], c[K];
      bool open[K];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int s = s0 + j * kPlanWaves;
        const bool e = s < S && scr[s].eq;
        cap[j] = e ? min(scr[s].n, scr[s - 1].n) >> pp.log2_bs : 0;
        c[j] = 0;
        open[j] = cap[j] > 0;
      }
      for (int base = 0;; base += 64) {
        bool any_open = false;
#pragma unroll
        for (int j = 0; j < K; ++j) any_open |= open[j];
        if (!any_open) break;
        int x[K], y[K];
        const int e = base + lane;
        // (loading every row unconditionally, to keep all 2K loads in flight,
        // measured 6 us slower on the parallel-sampling batch)
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const int s = s0 + j * kPlanWaves;
          const int32_t* a = pp.block_tables + (int64_t)s * pp.max_blocks;
          const bool ld = open[j] && e < cap[j];
          x[j] = ld ? a[e] : 0;
          y[j] = ld ? a[e - pp.max_blocks] : 0;
        }
#pragma unroll
        for (int j = 0; j < K; ++j) {
          if (!open[j]) continue;
          const unsigned long long mism = __ballot(e < cap[j] && x[j] != y[j]);
          if (mism) {
            c[j] = base + __builtin_ctzll(mism);
            open[j] = false;
          } else if (base + 64 >= cap[j]) {
            c[j] = cap[j];
            open[j] = false;
          }
        }
      }
      if (lane == 0) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const int s = s0 + j * kPlanWaves;
          if (s < S) scr[s].c = c[j];
        }
      }
    }
    __syncthreads();

    // C. Groups: runs of sequences linked to their predecessor by a shared
    //    full block, cut every max_members sequences.
    int run_carry = 0, gid_carry = 0;
    for (int base = 0; base < S; base += kPlanThreads) {
      const int s = base + tid;
      const bool link = s < S && scr[s].c >= 1;
      int mx;
      const int run_start = max(run_carry, plan_scan_max(link ? -1 : s, lds, &mx));
      const bool lead = s < S && ((s - run_start) % pp.max_members) == 0;
      int nl;
      const int excl = plan_scan_sum(lead ? 1 : 0, lds, &nl);
      if (s < S) scr[s].gid = gid_carry + excl - (lead ? 0 : 1);
      run_carry = max(run_carry, mx);
      gid_carry += nl;
    }
    __syncthreads();
    // each group's first member gathers its members (at most 15 more)
    bool real_any = false;
    for (int s = tid; s < S; s += kPlanThreads) {
      const int gid = scr[s].gid;
      if (s > 0 && scr[s - 1].gid == gid) continue;
      int k = INT32_MAX, m = 1;
      for (int j = 1; j < pp.max_members && s + j < S; ++j) {
        const PlanScratch t = scr[s + j];
        if (t.gid != gid) break;
        k = min(k, t.c);
        ++m;
      }
      const PlanGroup g{k, m, s, -1, 0, 0};
      grp[gid] = g;
      real_any |= real_group(g);
    }
    if (tid == 0) any[0] = 0;
    __syncthreads();
    if (real_any) atomicOr(&any[0], 1);
    __syncthreads();
    grouped = any[0] != 0;   // no group shares a whole block: the flat shared mode
  }

  // D. Items and the chunk size (grouped records that would not fit the
  //    workspace: laid out again without groups).
  Layout L = plan_layout(pp, scr, grp, item_ls, grouped, has_eq, lds);
  if (!L.ok) {
    __syncthreads();
    L = plan_layout(pp, scr, grp, item_ls, false, has_eq, lds);
  }
  if (!(L.flags & kPlanGrouped)) L.RH = 0;
  if (has_empty) L.flags |= kPlanEmpty;
  __syncthreads();   // the planner's state is complete

  // E. The plan itself: items, per-sequence entries, worker descriptors and
  //    the header.  With the state in LDS nothing written here is read back,
  //    so no barrier waits for these stores; in the workspace the descriptor
  //    search reads the items' first blocks from the items.
  plan_write_items(pp, scr, grp, (L.flags & kPlanGrouped) != 0);
  if constexpr (IN_LDS) {
    // flat items are whole sequences: blocks and token limit from the length
    plan_write_descs(pp, L, [&](int i) {
      const int2 e = item_ls[i];
      const int n = scr[e.y].n;
      return make_int4(e.x, e.y, (n + (1 << pp.log2_bs) - 1) >> pp.log2_bs, n);
    });
  } else {
    __syncthreads();
    plan_write_descs(pp, L, [&](int i) {
      const PlanItem* it = pp.items + i;
      return make_int4(it->pos, it->s, it->len, it->n);
    });
  }

}

// One work-group of kPlanThreads threads.  For batches of up to
// kPlanLdsSeqs sequences the planner's state stays in LDS, so the plan costs
// one round of length and table-head loads (and, when tables share blocks,
// one coalesced wave load per 64 table entries compared).
__global__ __launch_bounds__(kPlanThreads) void paged_decode_plan_kernel(const PlanParams pp) {
  __shared__ int lds[3 * kPlanWaves];
  __shared__ int any[2];
  __shared__ PlanScratch scr_lds[kPlanLdsSeqs];
  __shared__ PlanGroup grp_lds[kPlanLdsSeqs];
  __shared__ int2 item_lds[kPlanLdsItems];
  if (threadIdx.x < 2) any[threadIdx.x] = 0;
  __syncthreads();
  if (pp.num_seqs <= kPlanLdsSeqs)
    plan_body<true>(pp, scr_lds, grp_lds, item_lds, lds, any);
  else
    plan_body<false>(pp, pp.scr, pp.groups, nullptr, lds, any);
}

}  // namespace pkv

namespace {

using namespace pkv;

// Workspace layout of one call: the arrival counters, the launch's plan
// (worker descriptors, items, per-sequence entries and the planner's
// scratch), then the partial records.  Flat and grouped plans share the
// record area; it is sized for the larger.
struct Plan {
  int32_t chunk;        // 0 = derived in the planner
  int32_t num_workers;  // multiple of 8
  int32_t desc_rounds;  // rounds the descriptor table holds
  int32_t max_members;  // sequences per group (< 2: no grouping)
  size_t header_off, desc_off, items_off, seqs_off, scr_off, groups_off, recs_off;
  int64_t grec_rows;    // record rows a grouped plan may use
  size_t bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Query groups up to 8 per kv head with a matrix-core operand type can read a
// shared prefix once for all members of a group (16 query rows per group).
bool groupable(const kv_pool_t* pool, int G) {
  return pool->dtype != KV_F32 && pool->log2_block_size >= 4 && pool->decode_mfma && G <= 8;
}

kv_status_t make_plan(const kv_pool_t* pool, int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks,
                      int32_t partition_tokens, Plan* plan) {
  if (!pool || num_seqs < 0 || num_q_heads <= 0 || max_blocks <= 0 || partition_tokens < 0) return KV_ERR_INVALID_ARG;
  if (num_q_heads % pool->num_kv_heads) return KV_ERR_INVALID_ARG;
  const int G = num_q_heads / pool->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return KV_ERR_UNSUPPORTED;
  const int64_t units = (int64_t)num_seqs * pool->num_kv_heads * max_blocks;  // upper bound of blocks
  if (units > (1LL << 30) || (int64_t)max_blocks * pool->block_size > (1LL << 30)) return KV_ERR_INVALID_ARG;
  // The decode grid is resident: num_cus x decode_waves_per_cu one-wave
  // workers, each taking one chunk per round.  With caller-sized partitions
  // every worker gets an equal span of the stream, cut into partitions of
  // at most partition_tokens tokens; the library-sized split makes one chunk
  // per worker, or kSharedSplit finer ones when sequences share blocks.
  int64_t workers = (int64_t)pool->num_cus * pool->decode_waves_per_cu;
  int64_t chunks;   // chunk ids the descriptor table and the records cover
  if (partition_tokens > 0) {
    if (partition_tokens % pool->block_size) return KV_ERR_INVALID_ARG;
    if (workers > units) workers = units;
    if (workers < 1) workers = 1;
    workers = (workers + 7) & ~7LL;
    // each worker's span of the stream is cut into partitions; longer ones
    // when the batch would need more chunk ids than counter slots
    int64_t chunk = partition_tokens / pool->block_size;
    const int64_t span_max = (units + workers - 1) / workers;
    const int64_t max_q = kCounterSlots / workers;
    if ((span_max + chunk - 1) / chunk > max_q) chunk = (span_max + max_q - 1) / max_q;
    plan->chunk = (int32_t)chunk;
    plan->desc_rounds = (int32_t)std::max<int64_t>(1, (span_max + chunk - 1) / chunk);
    chunks = workers * plan->desc_rounds;
  } else {
    plan->chunk = 0;
    if (workers > units) workers = units;
    if (workers < 1) workers = 1;
    workers = (workers + 7) & ~7LL;
    plan->desc_rounds = kSharedSplit;
    chunks = workers * kSharedSplit;
  }
  // arrival counters are indexed by chunk id
  if (chunks > kCounterSlots) return KV_ERR_INVALID_ARG;
  const int64_t descs = workers * plan->desc_rounds;
  plan->num_workers = (int32_t)workers;
  const bool grouping = groupable(pool, G) && (int64_t)pool->num_kv_heads * num_seqs <= kCounterSlots;
  plan->max_members = grouping ? 16 / G : 0;
  const size_t S = (size_t)num_seqs;
  size_t off = (size_t)kCounterSlots * sizeof(int32_t);
  plan->header_off = off;
  off = align256(off + sizeof(PlanHeader));
  plan->desc_off = off;
  off = align256(off + (size_t)descs * sizeof(PlanDesc));
  plan->items_off = off;
  off = align256(off + (S + S / 2 + 1) * sizeof(PlanItem));
  plan->seqs_off = off;
  off = align256(off + (S + 1) * sizeof(PlanSeq));
  plan->scr_off = off;
  off = align256(off + (S + 1) * sizeof(PlanScratch));
  plan->groups_off = off;
  off = align256(off + (S + 1) * sizeof(PlanGroup));
  plan->recs_off = off;
  const size_t row = (size_t)(pool->head_dim + 4) * sizeof(float);
  const size_t flat = (size_t)2 * chunks * G * row;
  // record rows of a grouped plan: at most 2 pieces plus one per chunk of
  // every item, so 4 * Hkv * S * G rows plus 16 per chunk boundary (grouped
  // plans of the library split have one chunk per worker; with partitions,
  // up to `chunks`); past 8192 chunks a grouped plan that does not fit falls
  // back to a flat one
  const int64_t grouped_chunks = partition_tokens > 0 ? chunks : workers;
  plan->grec_rows =
      grouping ? 4LL * pool->num_kv_heads * num_seqs * G + 16LL * std::min<int64_t>(grouped_chunks, 8192) : 0;
  const size_t grouped = (size_t)plan->grec_rows * row;
  plan->bytes = off + std::max(flat, grouped);
  if (!grouping) plan->grec_rows = 0;
  return KV_OK;
}

}  // namespace

extern "C" kv_status_t paged_attention_workspace_size(const kv_pool_t* pool, int32_t num_seqs, int32_t num_q_heads,
                                                      int32_t max_blocks, int32_t partition_tokens, size_t* bytes) {
  if (!bytes) return KV_ERR_INVALID_ARG;
  Plan plan;
  kv_status_t st = make_plan(pool, num_seqs, num_q_heads, max_blocks, partition_tokens, &plan);
  if (st != KV_OK) return st;
  *bytes = plan.bytes;
  return KV_OK;
}

namespace {

// Which kernels a call enqueues: the planner, the decode kernel, or both.
enum Stage { kPlanAndRun, kPlanOnly, kRunOnly };

kv_status_t decode(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype, void* out, const int32_t* block_tables,
                   int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                   float scale, int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* stream,
                   Stage stage) {
  Plan plan;
  kv_status_t st = make_plan(pool, num_seqs, num_q_heads, max_blocks, partition_tokens, &plan);
  if (st != KV_OK) return st;
  if (!valid_dtype(q_dtype)) return KV_ERR_INVALID_ARG;
  if (num_seqs == 0) return KV_OK;
  if (!block_tables || !context_lens) return KV_ERR_INVALID_ARG;
  if (stage != kPlanOnly) {
    if (!q || !out) return KV_ERR_INVALID_ARG;
    if ((((uintptr_t)q) | ((uintptr_t)out)) & 15) return KV_ERR_INVALID_ARG;
    if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return KV_ERR_INVALID_ARG;
  }
  if (!workspace || workspace_bytes < plan.bytes || ((uintptr_t)workspace & 255)) return KV_ERR_WORKSPACE;

  const int D = pool->head_dim;
  const int G = num_q_heads / pool->num_kv_heads;
  const bool fp8 = pool->dtype == KV_FP8_E4M3FN;
  // dtype pairs: q in the pool dtype, or f32/f16/bf16 q over an fp8 pool
  if (fp8 ? q_dtype == KV_FP8_E4M3FN : q_dtype != pool->dtype) return KV_ERR_UNSUPPORTED;
  // pairs with a 16-bit matrix-core operand type
  const bool pair_mfma = (pool->dtype == KV_BF16 && q_dtype == KV_BF16) ||
                         (pool->dtype == KV_F16 && q_dtype == KV_F16) ||
                         (fp8 && (q_dtype == KV_BF16 || q_dtype == KV_F16));
  // Query groups (G > 1) run on the matrix cores where the dtype pair has a
  // 16-bit operand type and blocks hold whole 16-token tiles, unless the
  // pool was made with PAGEDKV_DECODE_MFMA=0.
  const bool mfma = G > 1 && pool->decode_mfma;
  // 16 query rows per kv head only on the matrix cores
  if (G == 16 && !(mfma && pair_mfma && pool->log2_block_size >= 4)) return KV_ERR_UNSUPPORTED;
  // a wave load covers 64 / (lanes per token row) tokens of one block
  const int lanes_per_row = D * (int)elem_bytes(pool->dtype) / 16;
  if (64 / lanes_per_row > pool->block_size) return KV_ERR_UNSUPPORTED;

  DecodeParams p{};
  p.k_pool = (const uint8_t*)pool->k;
  p.v_pool = (const uint8_t*)pool->v;
  p.q = (const uint8_t*)q;
  p.out = (uint8_t*)out;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start = nullptr;
  p.total_q = 0;
  uint8_t* ws = (uint8_t*)workspace;
  p.counters = (int32_t*)ws;
  p.partials = (float*)(ws + plan.recs_off);
  p.header = (const PlanHeader*)(ws + plan.header_off);
  p.desc = (const PlanDesc*)(ws + plan.desc_off);
  p.items = (const PlanItem*)(ws + plan.items_off);
  p.pseqs = (const PlanSeq*)(ws + plan.seqs_off);
  p.num_seqs = num_seqs;
  p.num_kv_heads = pool->num_kv_heads;
  p.max_blocks = max_blocks;
  p.num_blocks = pool->num_blocks;
  p.log2_bs = pool->log2_block_size;
  p.chunk = plan.chunk;
  p.num_workers = plan.num_workers;
  p.q_scale = scale * kLog2e * (fp8 ? pool->k_scale : 1.0f);
  p.v_scale = fp8 ? pool->v_scale : 1.0f;
  p.qk_scale = scale * kLog2e;
  p.head_scales = fp8 && pool->per_head ? pool->head_scales : nullptr;

  hipStream_t s = (hipStream_t)stream;
  if (stage != kRunOnly) {
    PlanParams pp;
    pp.block_tables = block_tables;
    pp.context_lens = context_lens;
    pp.scr = (PlanScratch*)(ws + plan.scr_off);
    pp.groups = (PlanGroup*)(ws + plan.groups_off);
    pp.items = (PlanItem*)(ws + plan.items_off);
    pp.seqs = (PlanSeq*)(ws + plan.seqs_off);
    pp.desc = (PlanDesc*)(ws + plan.desc_off);
    pp.header = (PlanHeader*)(ws + plan.header_off);
    pp.grec_rows = plan.grec_rows;
    pp.num_seqs = num_seqs;
    pp.num_kv_heads = pool->num_kv_heads;
    pp.max_blocks = max_blocks;
    pp.num_blocks = pool->num_blocks;
    pp.log2_bs = pool->log2_block_size;
    pp.G = G;
    pp.chunk = plan.chunk;
    pp.num_workers = plan.num_workers;
    pp.desc_rounds = plan.desc_rounds;
    pp.max_members = pair_mfma ? plan.max_members : 0;   // groups run on the matrix cores
    // matrix-core runs stream a span of partitions in one pass
    pp.span_runs = mfma && pair_mfma && pool->log2_block_size >= 4 ? 1 : 0;
    pp.shared_split = kSharedSplit;
    pp.counter_slots = kCounterSlots;
    hipLaunchKernelGGL(paged_decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, pp);
    if (launch_status() != KV_OK) return KV_ERR_HIP;
  }
  if (stage == kPlanOnly) return KV_OK;
  if (!fp8) {
    if (q_dtype != pool->dtype) return KV_ERR_UNSUPPORTED;
    switch (pool->dtype) {
      case KV_F32: return launch_decode_f32_f32(p, D, G, mfma, s);
      case KV_F16: return launch_decode_f16_f16(p, D, G, mfma, s);
      case KV_BF16: return launch_decode_bf16_bf16(p, D, G, mfma, s);
      default: return KV_ERR_UNSUPPORTED;
    }
  }
  switch (q_dtype) {
    case KV_F32: return launch_decode_fp8_f32(p, D, G, mfma, s);
    case KV_F16: return launch_decode_fp8_f16(p, D, G, mfma, s);
    case KV_BF16: return launch_decode_fp8_bf16(p, D, G, mfma, s);
    default: return KV_ERR_UNSUPPORTED;
  }
}

}  // namespace

extern "C" kv_status_t paged_attention_decode(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype, void* out,
                                              const int32_t* block_tables, int32_t max_blocks,
                                              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                              float scale, int32_t partition_tokens, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  return decode(pool, q, q_dtype, out, block_tables, max_blocks, context_lens, num_seqs, num_q_heads, scale,
                partition_tokens, workspace, workspace_bytes, stream, kPlanAndRun);
}

extern "C" kv_status_t paged_attention_plan(const kv_pool_t* pool, kv_dtype_t q_dtype, const int32_t* block_tables,
                                            int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs,
                                            int32_t num_q_heads, int32_t partition_tokens, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  return decode(pool, nullptr, q_dtype, nullptr, block_tables, max_blocks, context_lens, num_seqs, num_q_heads, 1.0f,
                partition_tokens, workspace, workspace_bytes, stream, kPlanOnly);
}

extern "C" kv_status_t paged_attention_decode_planned(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype,
                                                      void* out, const int32_t* block_tables, int32_t max_blocks,
                                                      const int32_t* context_lens, int32_t num_seqs,
                                                      int32_t num_q_heads, float scale, int32_t partition_tokens,
                                                      void* workspace, size_t workspace_bytes, void* stream) {
  return decode(pool, q, q_dtype, out, block_tables, max_blocks, context_lens, num_seqs, num_q_heads, scale,
                partition_tokens, workspace, workspace_bytes, stream, kRunOnly);
}

// ------------------------------------------------- allocation-free variant
//
// paged_attention_decode_noalloc runs the same kernels with the workspace in
// this file-scope device array instead of a caller's buffer, for callers that
// cannot allocate (code under graph capture, tight serving loops).  Every
// device the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// the device address is fetched once per device with hipGetSymbolAddress and
// only that address is passed on.
static __device__ __align__(256) uint8_t scratch[PAGEDKV_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device (null: not set up)

__global__ void clear_words_kernel(uint32_t* p, int words) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < words; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The device address of the pool's device's scratch, set up on first use:
// the address is looked up with that device current, and the arrival
// counters at its start are cleared on `stream` (a kernel, not a memset, so
// a captured first call records no memset).
kv_status_t device_scratch(const kv_pool_t* pool, hipStream_t stream, void** out) {
  if (pool->device < 0 || pool->device >= kMaxDevices) return KV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[pool->device]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return KV_ERR_HIP;
    if (cur != pool->device && hipSetDevice(pool->device) != hipSuccess) return KV_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    kv_status_t st = KV_OK;
    if (e != hipSuccess || !ptr) {
      st = KV_ERR_HIP;
    } else {
      const int words = (int)(kCounterSlots);
      hipLaunchKernelGGL(clear_words_kernel, dim3(64), dim3(256), 0, stream, (uint32_t*)ptr, words);
      st = launch_status();
    }
    if (cur != pool->device) (void)hipSetDevice(cur);
    if (st != KV_OK) return st;
    g_scratch[pool->device] = ptr;
  }
  *out = g_scratch[pool->device];
  return KV_OK;
}

}  // namespace

extern "C" kv_status_t paged_attention_decode_noalloc(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype,
                                                      void* out, const int32_t* block_tables, int32_t max_blocks,
                                                      const int32_t* context_lens, int32_t num_seqs,
                                                      int32_t num_q_heads, float scale, int32_t partition_tokens,
                                                      void* stream) {
  Plan plan;
  kv_status_t st = make_plan(pool, num_seqs, num_q_heads, max_blocks, partition_tokens, &plan);
  if (st != KV_OK) return st;
  if (plan.bytes > (size_t)PAGEDKV_DECODE_SCRATCH_BYTES) return KV_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = device_scratch(pool, (hipStream_t)stream, &ws)) != KV_OK) return st;
  return decode(pool, q, q_dtype, out, block_tables, max_blocks, context_lens, num_seqs, num_q_heads, scale,
                partition_tokens, ws, PAGEDKV_DECODE_SCRATCH_BYTES, stream, kPlanAndRun);
}
