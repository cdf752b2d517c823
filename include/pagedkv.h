/*
 * pagedkv.h -- C ABI of libpagedkv.so: a paged KV-cache pool and decode
 * attention over it, for AMD Instinct MI355X (gfx950).
 *
 * The method (the pages cited are "vLLM 与 KV Cache" (jeffliulab.github.io),
 * "vLLM KV Cache 实现机制" (devpress.csdn.net) and "vLLM — 把操作系统的分页搬进
 * GPU KV cache" (estelledc.github.io)):
 *   - Each sequence's K/V cache is cut into fixed-size blocks of block_size
 *     tokens (16 by default) that live anywhere in one preallocated pool;
 *     a per-sequence block table maps logical block i to its physical block.
 *     ("vLLM 与 KV Cache": virtual-memory table, how-it-works points 1-3;
 *     "vLLM KV Cache 实现机制": §1.2 diagram, §4.1 pool diagram.)
 *   - Decode attention reads K/V through that table: look up the physical
 *     block, then offset into it. ("vLLM — 把操作系统的分页搬进 GPU KV cache":
 *     core mechanisms, kernel paragraph.)
 *   - Blocks shared by several sequences are copied before the first write
 *     into them (copy-on-write). (Same page: core mechanism 3, case 2,
 *     pitfalls.)
 * Block allocation, reference counts and the copy-on-write plan belong to
 * the caller's block manager; this library only moves and reads bytes.
 *
 * Conventions for every call:
 *   - Device pointers are plain device memory on the device that was current
 *     when the pool was created; the caller owns them and keeps them alive
 *     until the stream work that uses them has finished.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued: no call synchronises the device, and only the two pool
 *     constructors allocate device memory (kv_pool_create: the pools and,
 *     for fp8, the per-head scale table; kv_pool_create_from: that table).
 *   - Launch-shape overrides are read from the environment once, when a pool
 *     is made, and hold for its life: PAGEDKV_DECODE_WAVES_PER_CU (worker
 *     wavefronts per compute unit of the library-sized decode split, 1..64,
 *     default 8), PAGEDKV_DECODE_MFMA=0 (query groups of decode on the
 *     vector ALUs instead of the matrix cores) and PAGEDKV_PREFILL_PATH=
 *     wave|group|unit (the launch shape of paged_attention_prefill).  They
 *     exist for tuning and tests; results agree within the tolerances
 *     whatever they say.
 *   - Host-side arguments are checked before anything is enqueued; a failed
 *     check returns an error status and enqueues nothing.
 *   - Device-side data (lengths, table entries, slots, pairs) are
 *     preconditions, not checked for meaning.  The kernels never access
 *     memory outside the pool, the table rows or the outputs for any values
 *     of them: an out-of-range block id or slot is skipped, a context length
 *     above max_blocks * block_size is clamped to it, and a length <= 0
 *     yields a zero output row.
 *   - Calls are reentrant; a pool has no lock, so the caller orders work on
 *     streams that touch the same pool.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KV_OK = 0,
  KV_ERR_INVALID_ARG = 1,  /* null pointer, bad size, inconsistent shapes */
  KV_ERR_UNSUPPORTED = 2,  /* dtype / head_dim / block_size combination not built */
  KV_ERR_OOM = 3,          /* kv_pool_create could not allocate */
  KV_ERR_HIP = 4,          /* a HIP runtime call or kernel launch failed */
  KV_ERR_WORKSPACE = 5,    /* workspace missing or smaller than required */
  KV_ERR_NO_BLOCKS = 6     /* block manager: no free or evictable block left */
} kv_status_t;

typedef enum {
  KV_F32 = 0,
  KV_F16 = 1,
  KV_BF16 = 2,
  KV_FP8_E4M3FN = 3        /* OCP E4M3FN: bias 7, no infinities, max 448 */
} kv_dtype_t;

typedef struct kv_pool kv_pool_t;  /* opaque pool descriptor (host memory) */

/*
 * kv_pool_create -- allocate a K pool and a V pool of num_blocks blocks on
 * the current device; the library owns the memory and kv_pool_destroy frees
 * it.  The pool is preallocated once and carved into equal blocks ("vLLM KV
 * Cache 实现机制" §4.1; "vLLM — 把操作系统的分页搬进 GPU KV cache", case 1).
 *
 * Layout of each pool: [num_blocks][num_kv_heads][block_size][head_dim] of
 * `dtype`, row-major, so element (b, h, o, j) is at element offset
 * ((b*num_kv_heads + h)*block_size + o)*head_dim + j.  One (block, head)
 * tile of block_size*head_dim elements is contiguous.
 *
 * Supported: block_size in {8, 16, 32, 64}; head_dim in {64, 128, 256};
 * dtype any kv_dtype_t.  num_blocks * num_kv_heads * block_size * head_dim
 * must fit in int64 and every block id must fit in int32.
 * The memory is not initialised.  Returns KV_ERR_OOM if hipMalloc fails.
 */
kv_status_t kv_pool_create(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                           kv_dtype_t dtype, kv_pool_t** out);

/*
 * kv_pool_create_from -- describe caller-owned buffers (e.g. framework
 * tensors) as a pool with the layout above.  bytes_each is the size of each
 * of k_buf and v_buf and must be at least the pool size; both must be
 * 16-byte aligned.  kv_pool_destroy does not free them.
 */
kv_status_t kv_pool_create_from(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                kv_dtype_t dtype, void* k_buf, void* v_buf, size_t bytes_each, kv_pool_t** out);

/* kv_pool_destroy -- free the descriptor (and the memory, if the library
 * allocated it).  NULL is accepted.  The caller ensures no enqueued work
 * still uses the pool. */
kv_status_t kv_pool_destroy(kv_pool_t* pool);

/*
 * kv_pool_info -- device addresses of the K and V pools, bytes of each, and
 * element strides of the four layout dimensions (block, head, token slot,
 * dim).  Any output pointer may be NULL.
 */
kv_status_t kv_pool_info(const kv_pool_t* pool, void** k, void** v, size_t* bytes_each, int64_t strides[4]);

/*
 * kv_pool_set_scales -- per-tensor fp32 scales of an fp8 pool: a stored code
 * c stands for decode(c) * scale.  Default 1.  Must be finite and > 0.
 * KV_ERR_INVALID_ARG for non-fp8 pools.  ("vLLM KV Cache 实现机制" §2.3 table
 * and §5.1 flags name fp8 as a KV cache dtype; the scale convention is this
 * library's.)
 */
kv_status_t kv_pool_set_scales(kv_pool_t* pool, float k_scale, float v_scale);

/*
 * kv_pool_set_head_scales -- fp8 pools: one k and one v scale per kv head
 * instead of one per tensor, for heads whose value ranges differ (a variant
 * of the fp8 KV cache option, "vLLM KV Cache 实现机制" §2.3 table).
 * k_scales and v_scales are DEVICE arrays of num_kv_heads fp32 values, each
 * finite and > 0 (a precondition, like other device data: a bad value gives
 * wrong numbers, never an access outside any buffer).  They are copied, in
 * stream order on `stream`, into the pool's scale table (allocated when the
 * pool was made, so nothing is allocated here).  Work enqueued on `stream`
 * after this call encodes (reshape_and_cache) and decodes (the attention
 * calls) head h with its own scales; work enqueued before it sees the
 * previous table.  Both NULL returns to the per-tensor scales (so does
 * kv_pool_set_scales), for calls made from then on.  The source arrays must
 * stay alive until the copy has run.  KV_ERR_INVALID_ARG: not an fp8 pool or
 * exactly one array NULL; KV_ERR_HIP if the copy cannot be enqueued.
 */
kv_status_t kv_pool_set_head_scales(kv_pool_t* pool, const float* k_scales, const float* v_scales, void* stream);

/*
 * reshape_and_cache -- store the K and V of num_tokens new tokens into their
 * slots ("vLLM 与 KV Cache": why a KV cache -- only the new token's K/V is
 * computed and appended; how-it-works points 2-3).
 *
 *   k_new, v_new  device, [num_tokens][num_kv_heads][head_dim] of src_dtype,
 *                 contiguous, 16-byte aligned.
 *   slot_mapping  device int64 [num_tokens]: slot s names token offset
 *                 s % block_size of physical block s / block_size, i.e. the
 *                 caller computes block_table[pos / bs] * bs + pos % bs.
 *                 A negative slot skips the token; so does a slot at or above
 *                 num_blocks * block_size.
 * Same src and pool dtype: the bytes are copied.  fp8 pool with src f32, f16
 * or bf16: each element becomes E4M3FN(fp32(x) / k_scale) (v_scale for V),
 * rounded to nearest even and saturated to +-448.  Other dtype pairs:
 * KV_ERR_UNSUPPORTED.  Two tokens with the same slot race (precondition:
 * slots unique).  num_tokens == 0 enqueues nothing.
 */
kv_status_t reshape_and_cache(kv_pool_t* pool, const void* k_new, const void* v_new, kv_dtype_t src_dtype,
                              const int64_t* slot_mapping, int32_t num_tokens, void* stream);

/*
 * paged_attention_decode -- one query token per sequence attends to its whole
 * cached context through the block table ("vLLM — 把操作系统的分页搬进 GPU KV
 * cache": core mechanisms and kernel paragraph; lessons: decode is bound by
 * KV read bandwidth).
 *
 *   q             device [num_seqs][num_q_heads][head_dim] of q_dtype.
 *   out           device [num_seqs][num_q_heads][head_dim] of q_dtype.
 *   block_tables  device int32 [num_seqs][max_blocks]; entry i of row s is the
 *                 physical block of logical block i of sequence s.  Entries
 *                 at or beyond ceil(context_len / block_size) are not read.
 *   context_lens  device int32 [num_seqs]: tokens in each sequence's cache,
 *                 including the one appended this step.
 *   scale         softmax scale (typically 1/sqrt(head_dim)).
 * out[s][h] = sum_t softmax_t(scale * q[s][h] . K_t) V_t over t < context_len,
 * with K_t/V_t of kv head h / (num_q_heads / num_kv_heads).  Accumulation is
 * fp32; the result is rounded to nearest even into q_dtype.  For fp8 pools K
 * and V are decoded exactly and multiplied by their scales.
 *
 * q_dtype must equal the pool dtype, except fp8 pools, which take f32, f16
 * or bf16 queries.  num_q_heads must be num_kv_heads times 1, 2, 4, 8 or 16.
 * 16 query heads per kv head run only on the matrix cores (bf16 or f16
 * queries, block_size >= 16, matrix cores not switched off):
 * KV_ERR_UNSUPPORTED otherwise.
 *
 * Two kernels run on `stream`: a one-work-group plan kernel
 * (paged_attention_plan below) and the decode kernel.
 *
 * Work split: the cached tokens of all (kv head, sequence) pairs are laid end
 * to end and cut into equal spans of whole blocks, one per resident worker
 * wavefront, so long and short sequences cost the same per token.
 * partition_tokens == 0 makes each span one run; otherwise (a multiple of
 * block_size) each span is cut into partitions of partition_tokens tokens,
 * the last of a span shorter, and every partition leaves its partial result.
 * A sequence cut into several runs or partitions is merged in the same
 * launch by the worker that finishes last (log-sum-exp merge of the partial
 * results, in a fixed order, so results are bitwise reproducible).
 *
 * Shared prefixes: consecutive sequences whose table rows start with the
 * same whole blocks (candidates forked from one prompt, "vLLM — 把操作系统的
 * 分页搬进 GPU KV cache": core mechanism 3 and case 2) form groups of up to 16
 * query rows (16 / (num_q_heads / num_kv_heads) sequences); each group's
 * common full blocks are read once, on the matrix cores, for every member,
 * and each member's own blocks separately.  This needs a 16-bit operand type
 * (bf16 or f16 queries), block_size >= 16, at most 8 query heads per kv head
 * and num_kv_heads * num_seqs <= 65536; otherwise, or when no group holds a
 * whole shared block, the blocks are read per sequence with the default
 * cache policy and a four times finer split, so candidates meet in the L2.
 * Query groups
 * (num_q_heads > num_kv_heads) with a 16-bit operand type (bf16 or f16
 * queries) and block_size >= 16 run on the matrix cores (unless the pool
 * was made with PAGEDKV_DECODE_MFMA=0).
 *
 * When partition_tokens is given and the batch would need more than 65536
 * partitions in all, they are lengthened to the smallest whole number of
 * blocks that fits.
 *
 * workspace: device memory of at least paged_attention_workspace_size()
 * bytes, 256-byte aligned.  Its first 256 KiB hold arrival counters and must
 * be zero before the first use; every completed call leaves them zero again,
 * so one workspace serves calls of any shape without clearing.  The rest holds
 * the launch plan and partial results.  Calls sharing a workspace must not
 * overlap.
 */
kv_status_t paged_attention_decode(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype, void* out,
                                   const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                                   int32_t num_seqs, int32_t num_q_heads, float scale, int32_t partition_tokens,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attention_plan, paged_attention_decode_planned -- the two halves of
 * paged_attention_decode, for callers that decode many times over the same
 * tables: every layer of a model in one serving step reads its own pool
 * through the same block tables and context lengths ("vLLM KV Cache 实现机制"
 * §1.2: one block table per sequence, shared by all layers' caches).
 *
 * paged_attention_plan enqueues the plan kernel: one work-group reads the
 * lengths and table heads (and compares the rows of sequences that start on
 * the same block), and writes the launch plan into `workspace` -- the runs of
 * blocks the stream is made of, where every worker's share starts, and the
 * groups of sequences whose shared prefix is read once.  It depends only on
 * the tables, the lengths, the shapes and q_dtype; no q, out or scale.
 *
 * paged_attention_decode_planned enqueues the decode kernel alone, using the
 * plan in `workspace`.  Preconditions (not checked): a paged_attention_plan
 * call made earlier on the same stream (or ordered before this one) wrote it
 * with the same block_tables, max_blocks, context_lens, num_seqs,
 * num_q_heads, partition_tokens and q_dtype, for a pool of the same shape
 * (num_blocks, block_size, num_kv_heads, head_dim, dtype, matrix-core
 * setting); the tables and lengths have not changed since; and no other call
 * has used the workspace in between.  Any number of planned decodes may
 * follow one plan, on different pools of that shape and different q, out
 * and scale.  Same workspace size and arguments as paged_attention_decode;
 * the result is bitwise the same.
 */
kv_status_t paged_attention_plan(const kv_pool_t* pool, kv_dtype_t q_dtype, const int32_t* block_tables,
                                 int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t partition_tokens, void* workspace,
                                 size_t workspace_bytes, void* stream);
kv_status_t paged_attention_decode_planned(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype, void* out,
                                           const int32_t* block_tables, int32_t max_blocks,
                                           const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                           float scale, int32_t partition_tokens, void* workspace,
                                           size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode_noalloc -- paged_attention_decode for callers that
 * cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, result and kernels as paged_attention_decode, without
 * workspace/workspace_bytes: the call uses a fixed scratch area of
 * PAGEDKV_DECODE_SCRATCH_BYTES (64 MiB) that the library holds in device
 * memory on every device it runs on, until the process ends.  It allocates
 * nothing.  The first call on a device looks the area up and clears its
 * arrival counters on `stream` (one small kernel); every call leaves them
 * zero again.  All calls on one device share the area: two calls that
 * overlap in time on one device (different streams, or threads without
 * ordering) race and give wrong results.  KV_ERR_WORKSPACE: the shape needs
 * more than PAGEDKV_DECODE_SCRATCH_BYTES of workspace
 * (paged_attention_workspace_size tells how much); other errors as
 * paged_attention_decode.
 */
#define PAGEDKV_DECODE_SCRATCH_BYTES (64u << 20)
kv_status_t paged_attention_decode_noalloc(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype, void* out,
                                           const int32_t* block_tables, int32_t max_blocks,
                                           const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                           float scale, int32_t partition_tokens, void* stream);

/* paged_attention_workspace_size -- bytes of workspace paged_attention_decode needs
 * for these arguments (depends on the pool's device, not on lengths). */
kv_status_t paged_attention_workspace_size(const kv_pool_t* pool, int32_t num_seqs, int32_t num_q_heads,
                                           int32_t max_blocks, int32_t partition_tokens, size_t* bytes);

/*
 * paged_attention_decode_grouped -- the same result as paged_attention_decode,
 * for batches in which groups of sequences share the blocks of a common
 * prefix (parallel sampling: n candidates forked from one prompt share its
 * blocks with ref_count n, "vLLM — 把操作系统的分页搬进 GPU KV cache", core
 * mechanism 3 and case 2).  The shared prefix is read once per group: its
 * members' query rows (members x query heads of a kv head, at most 16) are
 * the rows of one matrix-core pass; each member's remaining blocks are read
 * per sequence.
 *
 * group_start: device int32 [num_groups + 1], ascending; group g is
 *   sequences group_start[g] .. group_start[g+1]-1 (groups need not cover
 *   every sequence: the others are decoded on their own).
 * group_shared: device int32 [num_groups]; the first group_shared[g] table
 *   entries are identical in every member's table (caller's contract).
 * Members beyond 16 / (num_q_heads / num_kv_heads) in a group, and tokens
 * past a member's context, are handled without sharing, and the shared part
 * is cut to whole blocks.  Inconsistent groups (overlapping, unsorted, or
 * sharing that the tables do not have) give wrong rows but stay inside every
 * buffer.  The other arguments are paged_attention_decode's; workspace:
 * paged_attention_decode_grouped_workspace_size() bytes, 256-byte aligned.
 * Its first 256 KiB are the arrival-counter header of paged_attention_decode
 * and paged_attention_prefill: this call neither reads nor writes them, so
 * one workspace serves all three calls.  The rest holds per-row records and
 * keeps no state across calls.
 * Supported: bf16/bf16, f16/f16, fp8 with bf16 or f16 queries; block_size
 * >= 16 (KV_ERR_UNSUPPORTED otherwise: call paged_attention_decode).
 * Two kernels run on `stream`.
 */
kv_status_t paged_attention_decode_grouped(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype, void* out,
                                           const int32_t* block_tables, int32_t max_blocks,
                                           const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                           float scale, const int32_t* group_start, const int32_t* group_shared,
                                           int32_t num_groups, void* workspace, size_t workspace_bytes,
                                           void* stream);

/* paged_attention_decode_grouped_workspace_size -- bytes of workspace the
 * call above needs: the 256 KiB counter header it leaves alone, then one
 * partial record per (sequence, query head). */
kv_status_t paged_attention_decode_grouped_workspace_size(const kv_pool_t* pool, int32_t num_seqs,
                                                          int32_t num_q_heads, size_t* bytes);

/*
 * paged_attention_prefill -- several new query tokens per sequence attend
 * causally to the cached context through the block table: a chunk of a
 * prompt being prefilled into the pool, or speculative tokens being verified
 * ("vLLM — 把操作系统的分页搬进 GPU KV cache": related work (FlashAttention is
 * the prefill twin of PagedAttention) and fit (speculative decoding on top);
 * the paged read path is the decode one above).
 *
 *   q, out        device [total_q][num_q_heads][head_dim] of q_dtype.
 *   query_start   device int32 [num_seqs + 1], nondecreasing, query_start[0]
 *                 = 0: sequence s owns query rows [query_start[s],
 *                 query_start[s+1]).  Its m_s new tokens are the last m_s of
 *                 its context_lens[s] cached tokens (their K/V already stored
 *                 with reshape_and_cache), so row i sits at position
 *                 context_lens[s] - m_s + (i - query_start[s]).
 * out[i][h] = sum_t softmax_t(scale * q[i][h] . K_t) V_t over t <= position
 * of row i, kv head h / (num_q_heads / num_kv_heads); fp32 accumulation, the
 * result rounded to nearest even into q_dtype.  Rows not owned by any
 * sequence are not written; m_s is clamped to [0, context_lens[s]].
 *
 * Runs on the matrix cores: q_dtype bf16 with bf16 or fp8 pools, f16 with f16
 * or fp8 pools; block_size >= 16; num_q_heads / num_kv_heads in {1, 2, 4, 8,
 * 16} (other combinations: KV_ERR_UNSUPPORTED).  Work split as in decode: the
 * (kv head, sequence, 16-row tile) runs are laid end to end and cut into
 * equal chunks; cut runs are merged in the same launch.
 *
 * workspace: at least paged_attention_prefill_workspace_size() bytes,
 * 256-byte aligned, with the same counter convention as decode (first 256 KiB
 * zero before first use, left zero by every call); calls sharing a workspace
 * must not overlap.
 */
kv_status_t paged_attention_prefill(const kv_pool_t* pool, const void* q, kv_dtype_t q_dtype, void* out,
                                    const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                                    const int32_t* query_start, int32_t num_seqs, int32_t total_q,
                                    int32_t num_q_heads, float scale, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* paged_attention_prefill_workspace_size -- bytes of workspace the call above
 * needs (depends on the pool's device and head_dim only). */
kv_status_t paged_attention_prefill_workspace_size(const kv_pool_t* pool, int32_t num_q_heads, size_t* bytes);

/*
 * copy_blocks -- copy-on-write support: for each pair (src, dst) copy the
 * whole physical block src onto dst in both pools (every head, every token
 * slot).  ("vLLM — 把操作系统的分页搬进 GPU KV cache": core mechanism 3, case 2
 * and pitfalls -- n candidates sharing a prompt copy n-1 blocks on their first
 * step.)  All pairs are copied by one launch.
 *
 *   pairs  device int32 [num_pairs][2].  Preconditions: dst ids distinct and
 *          not also used as src.  Pairs with an id outside [0, num_blocks)
 *          are skipped.
 * num_pairs == 0 enqueues nothing.
 */
kv_status_t copy_blocks(kv_pool_t* pool, const int32_t* pairs, int32_t num_pairs, void* stream);

typedef enum {
  KV_SWAP_OUT = 0,  /* pool block src -> host block dst */
  KV_SWAP_IN = 1    /* host block src -> pool block dst */
} kv_swap_dir_t;

/*
 * swap_blocks -- move whole blocks between the pool and a host swap area, for
 * offloading a preempted sequence's KV to CPU memory and bringing it back
 * ("vLLM KV Cache 实现机制" §2.1 storage tiers and §3.3 RECOMPUTE vs offload
 * table; "vLLM — 把操作系统的分页搬进 GPU KV cache", case 3: SWAP copies
 * blocks to CPU memory and back over the host link).  All pairs move in one
 * launch: the device reads and writes the host memory directly.
 *
 *   host_k, host_v   host memory the device can access: pinned memory from
 *                    hipHostMalloc (or a framework's pinned allocator); each
 *                    holds num_host_blocks blocks in the pool's layout
 *                    ([num_host_blocks][num_kv_heads][block_size][head_dim] of
 *                    the pool dtype, 16-byte aligned).  Memory that is not
 *                    pinned or not mapped for the pool's device is rejected
 *                    with KV_ERR_INVALID_ARG.
 *   pairs            device int32 [num_pairs][2] (src, dst).  KV_SWAP_OUT
 *                    copies pool block src to host block dst; KV_SWAP_IN
 *                    copies host block src to pool block dst.  Pairs with an
 *                    id outside its side's range are skipped.  Preconditions:
 *                    destinations distinct.
 * num_pairs == 0 enqueues nothing.  The host memory must stay alive and
 * untouched by the CPU until the stream work has finished.
 */
kv_status_t swap_blocks(kv_pool_t* pool, void* host_k, void* host_v, int64_t num_host_blocks, const int32_t* pairs,
                        int32_t num_pairs, kv_swap_dir_t direction, void* stream);

/*
 * kv_stream_read -- measurement primitive, not part of the pages' method: read
 * whole tiles of a device buffer with the load form of the decode kernel
 * (16-byte non-temporal buffer loads; 256 lanes per work-group, 32 KiB in
 * flight per work-group, 8 work-groups per compute unit) and compute
 * nothing.  Timed over a random tile order, it gives the HBM read rate a
 * streaming kernel reaches on the part, which the decode kernel's achieved
 * rate is set against.  Decode is bound by that read rate ("vLLM — 把操作系统
 * 的分页搬进 GPU KV cache": lessons).
 *
 *   buf, bytes   device buffer (16-byte aligned); tile i covers bytes
 *                [i * tile_bytes, (i + 1) * tile_bytes)
 *   tile_bytes   a positive multiple of 4096, at most bytes
 *   tiles        device int32 [num_tiles]: tile ids in the order read; an id
 *                outside [0, bytes / tile_bytes) reads nothing
 *   sink         device uint32 [1]: written only if the data read hash to one
 *                fixed value (this keeps the loads); its content has no meaning
 * Runs on the current device.  num_tiles == 0 enqueues nothing.  Errors:
 * KV_ERR_INVALID_ARG for a null pointer, a misaligned buffer or a bad tile
 * size; KV_ERR_HIP if the device cannot be queried or the launch fails.
 */
kv_status_t kv_stream_read(const void* buf, size_t bytes, int32_t tile_bytes, const int32_t* tiles, int32_t num_tiles,
                           uint32_t* sink, void* stream);

/* kv_status_string -- static description of a status code. */
const char* kv_status_string(kv_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
