/*
 * pa.h -- C ABI of libpa, a paged KV-cache attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * What it computes.  The KV cache of every sequence is split into logical
 * blocks of block_size tokens; each logical block lives in a physical block
 * of a shared pool, and a per-sequence block table maps logical to physical
 * block indices (page "vLLM PagedAttention chuyên sâu: Phân mảnh bộ nhớ KV
 * Cache, Prefill theo khối & Prefix Caching", locionic.com -- "the deep-dive
 * page" below -- section "Tương tự phân trang bộ nhớ ảo").  Attention looks
 * up each token's physical block in the table, gathers K and V from those
 * scattered blocks and runs ordinary softmax(q K^T * scale) V on them (same
 * page, section "Cơ chế PagedAttention").
 *
 * Conventions shared by every entry point:
 *  - Every function returns a pa_status (0 = success, < 0 = error).
 *  - Kernel entry points take device pointers owned by the caller and a
 *    hipStream_t passed as void*; they only enqueue work on that stream, never
 *    synchronise and never allocate device memory.  Host-side argument checks
 *    run before anything is enqueued; a failed check enqueues nothing.  A
 *    launch failure is reported as PA_ERR_DEVICE.
 *  - Values that live in device memory (block-table entries, context
 *    lengths, slots, query offsets) are preconditions and are not checked:
 *    every table entry of a logical block below ceil(context_len/block_size)
 *    lies in [0, num_blocks), 0 <= context_len <= max_blocks_per_seq *
 *    block_size, slots are < num_blocks * block_size and distinct within one
 *    call.  Violating them is undefined behaviour (out-of-bounds access).
 *  - dtype: PA_F32 (float) or PA_BF16 (bfloat16 stored as raw 16-bit).
 *    Outputs have the dtype of the inputs; accumulation is fp32 and the final
 *    bf16 rounding is round-to-nearest-even.
 *  - block_size is 16, the value every example on the deep-dive page uses;
 *    pa_reshape_and_cache, pa_copy_blocks and pa_decode also take 8, 32 and
 *    64 (the page's block_size trade-off).  head_dim is 64 or 128.  Anything
 *    else returns PA_ERR_UNSUPPORTED.
 *
 * Cache layout (the pages leave it open).  X = 16 / sizeof(element)
 * (8 for bf16, 4 for fp32):
 *    k_cache[num_blocks][num_kv_heads][head_dim / X][block_size][X]
 *    v_cache[num_blocks][num_kv_heads][head_dim][block_size]
 * Key element (block b, kv head g, offset o, dim d) is
 * k_cache[b][g][d / X][o][d % X]; the value element is v_cache[b][g][d][o].
 * A slot is a flat token position in the pool: block * block_size + offset.
 *
 * Grouped-query attention: query head h reads KV head h / (num_heads /
 * num_kv_heads); num_heads must be a multiple of num_kv_heads.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,    /* null pointer, negative size, inconsistent shapes */
  PA_ERR_NO_FREE_BLOCKS = -2, /* allocator: the pool cannot satisfy the request */
  PA_ERR_UNKNOWN_SEQ = -3,    /* allocator: no sequence with that id */
  PA_ERR_SEQ_EXISTS = -4,     /* allocator: the id is already in use */
  PA_ERR_UNSUPPORTED = -5,    /* a shape/dtype this build has no kernel for */
  PA_ERR_WORKSPACE = -6,      /* workspace missing or smaller than required */
  PA_ERR_DEVICE = -7          /* a HIP call or kernel launch failed */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/*
 * Flags of the decode entry points (pa_decode, pa_decode_no_alloc,
 * pa_decode_shared_prefix, pa_mixed_step).  PA_DECODE_STREAM_KV: read the K/V pages with the
 * non-temporal hint.  Pass it when no physical block is read by more than one
 * sequence of the call (the allocator's reference counts tell the caller):
 * each page is then read once per call, and the hint keeps those reads from
 * displacing cached data; on one MI355X it made the decode 8-11% faster.
 * Leave it out when sequences of the call share blocks (forked samples,
 * matched prompt prefixes read through pa_decode): their repeat reads of a
 * shared page are served from the caches only without it (measured 42% slower
 * with it on 8 samples per prompt).  Results are the same either way.
 *
 * PA_DECODE_FIND_SHARED (pa_decode and pa_decode_no_alloc only; bf16,
 * head_dim 128, block_size 16, else PA_ERR_UNSUPPORTED): the call finds
 * shared prefixes itself, on the device, and reads their pages once per group
 * as pa_decode_shared_prefix does (deep-dive page, section "Cơ chế APC", item
 * 2: requests with a matching prefix link the same physical blocks; the
 * skymod.tech overview on vLLM: the samples of a prompt share its blocks).
 * The batch is cut into aligned runs of PA_PREFIX_MAX_MEMBERS sequences; in
 * each run, the first sequence leads a group that the following sequences
 * join, in order, by the rule of pa_prefix_plan with min_prefix =
 * PA_FIND_SHARED_MIN_PREFIX tokens (leading block ids in common with the
 * leader, within both contexts' whole blocks, the page reads saved not
 * falling).  Sharing that crosses a run boundary is read once per run.  The
 * workspace must hold pa_decode_workspace_bytes_flags(..., flags) bytes.
 * Results are those of pa_decode to fp32 rounding (the shared pages' partials
 * are merged with the rest by the same log-sum-exp weights).  Pass
 * PA_DECODE_STREAM_KV with it when no block is read by two groups or by a
 * group and a sequence outside it.  Other bits are reserved and must be 0
 * (PA_ERR_INVALID_ARG).
 */
#define PA_DECODE_STREAM_KV 1
#define PA_DECODE_FIND_SHARED 2
#define PA_FIND_SHARED_MIN_PREFIX 256

/* Human-readable name of a status code (static storage, never NULL). */
const char* pa_status_str(int status);

/* ABI version of this library; bumped on any incompatible change. */
int pa_version(void);

/* ------------------------------------------------------------------ kernels */

/*
 * pa_reshape_and_cache -- write new tokens' K and V into their cache slots.
 *
 * New tokens of a growing sequence are stored in the physical blocks the
 * allocator mapped for them, without moving earlier tokens (deep-dive page,
 * section "Tương tự phân trang bộ nhớ ảo", dynamic resizing; section "Cơ chế
 * của Chunked Prefill", step 3: a chunk's KV accumulates in blocks the block
 * manager provides).
 *
 *   key, value    device, [num_tokens][num_kv_heads][head_dim], dtype; token i
 *                 starts at element i * key_stride (resp. value_stride), heads
 *                 are contiguous (stride head_dim).  strides >= num_kv_heads *
 *                 head_dim.
 *   k_cache, v_cache  device, the pool in the layout above (num_blocks blocks).
 *   slot_mapping  device int64 [num_tokens]; token i goes to slot
 *                 slot_mapping[i]; a negative slot skips the token.
 * Bit-exact copy: no value is changed.  num_tokens == 0 enqueues nothing.
 */
int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int32_t num_tokens, int64_t key_stride,
                         int64_t value_stride, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, int32_t dtype, void* stream);

/*
 * pa_copy_blocks -- copy-on-write block copies.
 *
 * A sequence about to write into a physical block it shares first gets a
 * private copy of that block (deep-dive page, section "Cơ chế APC", item 3).
 * For each pair p, the whole physical block pairs[2p] (all KV heads, all
 * offsets, K and V) is copied to block pairs[2p+1].
 *   pairs  device int32 [num_pairs][2] (src, dst); no dst may appear twice or
 *          also appear as a src in the same call (the copies run in parallel).
 * Bit-exact.  num_pairs == 0 enqueues nothing.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                   int32_t dtype, void* stream);

/*
 * pa_decode_workspace_bytes -- bytes of device workspace pa_decode needs.
 * Zero when no sequence can span more than one partition.  Partials are fp32:
 * num_seqs * num_heads * ceil(max_context_len / partition) * (head_dim + 2)
 * values, plus alignment.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition);

/*
 * pa_decode_workspace_bytes_flags -- device workspace of pa_decode called
 * with `flags`: pa_decode_workspace_bytes without PA_DECODE_FIND_SHARED; with
 * it, the partials of a prefix of up to max_context_len tokens and of the
 * rest (as pa_decode_shared_prefix_workspace_bytes with max_prefix_len =
 * max_context_len) plus the groups found: 4 bytes per sequence and 12 per run
 * of PA_PREFIX_MAX_MEMBERS sequences, 256-byte aligned.
 */
size_t pa_decode_workspace_bytes_flags(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition,
                                       int32_t flags);

/*
 * pa_decode -- one query token per sequence against its paged context.
 *
 * For sequence s and query head h (kv head g = h / (num_heads/num_kv_heads)),
 * with L = context_lens[s], token t in [0, L) is read from physical block
 * block_tables[s][t / block_size] at offset t % block_size; the output is
 * sum_t softmax_t(scale * <q[s][h], K_t>) V_t (deep-dive page, section "Cơ chế
 * PagedAttention", steps 1-3).  L counts every attended token, including the
 * token written in the same step.  L == 0 gives a zero row.
 *
 *   out, q         device [num_seqs][num_heads][head_dim], dtype.
 *   block_tables   device int32 [num_seqs][max_blocks_per_seq] (row-major,
 *                  entries past a sequence's last block are ignored; -1 is
 *                  the conventional padding).
 *   context_lens   device int32 [num_seqs].
 *   partition      split-context partition size in tokens: 0 = one pass per
 *                  (sequence, kv head); otherwise a positive multiple of 64.
 *                  The result does not depend on the partition size beyond
 *                  fp32 rounding.  A sequence longer than one partition is
 *                  processed by ceil(L/partition) independent workgroups
 *                  whose partial (max, sum, output) triples a second kernel
 *                  merges with log-sum-exp weights.
 *   max_context_len  host upper bound of context_lens (sizes the grid).
 *   workspace      device scratch of at least pa_decode_workspace_bytes(...)
 *                  bytes (pa_decode_workspace_bytes_flags(...) with
 *                  PA_DECODE_FIND_SHARED; may be NULL when that is 0);
 *                  contents on entry are ignored, contents on exit are
 *                  unspecified.  Calls that overlap in time must not share a
 *                  workspace.
 *   flags          0, PA_DECODE_STREAM_KV, PA_DECODE_FIND_SHARED, or both
 *                  (see there).
 * Deterministic: the merge runs in partition order and the reduction order
 * depends only on logical positions, so results do not depend on block
 * placement, on which blocks are shared, or on scheduling.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
              float scale, int32_t partition, int32_t max_context_len, void* workspace,
              size_t workspace_bytes, int32_t dtype, int32_t flags, void* stream);

/*
 * pa_decode_no_alloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same checks, kernels and results as pa_decode with
 * the same arguments, but the split-context partials live in a device array
 * inside the library (PA_NO_ALLOC_SCRATCH_BYTES, one copy per GPU, loaded
 * with the library's code and held until the process ends) instead of a
 * caller workspace.  No allocation or free is made by the call.
 *
 * A call whose partials (pa_decode_workspace_bytes_flags with the same
 * arguments) exceed PA_NO_ALLOC_SCRATCH_BYTES returns PA_ERR_WORKSPACE before any device
 * work.  Nothing in the array needs to start at zero.  Every call on a GPU
 * uses that GPU's one array: calls that may overlap in time on one GPU (two
 * streams, or two threads) race and must be serialized by the caller.
 * Returns PA_ERR_DEVICE if the array's address cannot be looked up.
 */
#define PA_NO_ALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int pa_decode_no_alloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, float scale, int32_t partition,
                       int32_t max_context_len, int32_t dtype, int32_t flags, void* stream);

/*
 * Shared-prefix decode.  Sequences that share the physical blocks of a common
 * prefix -- the samples of one prompt (the skymod.tech overview on vLLM:
 * parallel sampling shares the prompt's memory), or requests whose prompts
 * matched cached blocks (deep-dive page, section "Cơ chế APC", item 2) --
 * hold the same block ids at the start of their tables.  pa_decode reads
 * those pages once per sequence; pa_decode_shared_prefix reads them once per
 * group of up to PA_PREFIX_MAX_MEMBERS neighbouring sequences and attends the
 * rest of every context as pa_decode does.  The result is pa_decode's (same
 * softmax, merged with the same log-sum-exp weights) up to fp32 rounding.
 */
#define PA_PREFIX_MAX_MEMBERS 8

/*
 * pa_prefix_plan -- find prefix groups in a batch's block tables (host
 * memory; no device work).  Greedy in batch order: a group is a run of
 * consecutive sequences starting at its first member; its prefix is the
 * leading whole blocks whose ids all members share, in tokens (a multiple of
 * block_size, at most every member's context).  The next sequence joins while
 * the group has fewer than max_members (1..PA_PREFIX_MAX_MEMBERS) members and
 * the prefix stays at least max(min_prefix, block_size) tokens and keeps the
 * page reads saved (prefix * members) from falling.  Groups of one are
 * dropped.
 *
 *   block_tables     host int32 [num_seqs][max_blocks_per_seq].
 *   context_lens     host int32 [num_seqs], each in [0, max_blocks_per_seq *
 *                    block_size] (else PA_ERR_INVALID_ARG).
 *   groups           host int32 [num_seqs][3] out: per group (first
 *                    sequence, members, prefix tokens); rows past
 *                    *num_groups are untouched.
 *   seq_prefix_lens  host int32 [num_seqs] out: the prefix of the sequence's
 *                    group, 0 for a sequence in no group.
 *   num_groups, max_prefix_len  out.
 */
int pa_prefix_plan(const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                   int32_t max_members, int32_t min_prefix, int32_t* groups,
                   int32_t* seq_prefix_lens, int32_t* num_groups, int32_t* max_prefix_len);

/*
 * pa_decode_shared_prefix_workspace_bytes -- device workspace of
 * pa_decode_shared_prefix: fp32 partials for ceil(max_prefix_len /
 * (2 * partition)) prefix partitions plus ceil(max_context_len / partition)
 * others per (sequence, head); 0 when that is at most one.  partition 0 means
 * one partition covering max_context_len, as in pa_decode.
 */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                               int32_t head_dim, int32_t max_context_len,
                                               int32_t max_prefix_len, int32_t partition);

/*
 * pa_decode_shared_prefix -- pa_decode for a batch with prefix groups.
 *
 * Arguments as for pa_decode, plus (device memory, as pa_prefix_plan returns
 * them, copied to the device):
 *   prefix_groups    device int32 [num_groups][3]: (first sequence, members,
 *                    prefix tokens).  Preconditions: members in
 *                    1..PA_PREFIX_MAX_MEMBERS, groups disjoint, the prefix a
 *                    multiple of block_size, at most every member's context,
 *                    and every member's first prefix / block_size table
 *                    entries equal to the first member's.
 *   seq_prefix_lens  device int32 [num_seqs]: each sequence's group prefix,
 *                    0 outside any group.
 *   max_prefix_len   host: the largest prefix, a multiple of block_size and
 *                    at most max_context_len.
 * With num_groups == 0 or max_prefix_len == 0 the call is pa_decode (the two
 * arrays may then be NULL).  A group's prefix pages are read from its first
 * member's table in partitions of 2 * partition tokens, once for the queries
 * of all members; each member's remaining tokens [prefix, L) are attended per
 * sequence; the partials of both are merged per (sequence, head) in a fixed
 * order (prefix partitions first), so the result is deterministic.  bf16,
 * head_dim 128, num_heads / num_kv_heads in {1, 2, 4, 8}; anything else
 * returns PA_ERR_UNSUPPORTED.  Violated preconditions give wrong results but
 * no access outside the buffers pa_decode may touch.
 */
int pa_decode_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, float scale, int32_t partition,
                            int32_t max_context_len, const int32_t* prefix_groups,
                            int32_t num_groups, const int32_t* seq_prefix_lens,
                            int32_t max_prefix_len, void* workspace, size_t workspace_bytes,
                            int32_t dtype, int32_t flags, void* stream);

/*
 * pa_prefill_chunk -- causal attention of a chunk of query tokens per
 * sequence against that sequence's paged context (chunked prefill: the
 * prompt is processed in chunks whose KV accumulates in the cache, deep-dive
 * page, section "Cơ chế của Chunked Prefill", steps 1-3).
 *
 * Sequence s owns query rows query_start_loc[s] .. query_start_loc[s+1]-1
 * (n_q rows); context_lens[s] = L counts the cached tokens plus this chunk,
 * whose K/V must already be in the cache.  Query i of the chunk sits at
 * position L - n_q + i and attends to positions 0 .. L - n_q + i.
 *
 *   out, q           device [total_query_rows][num_heads][head_dim], bf16.
 *   query_start_loc  device int32 [num_seqs + 1], non-decreasing, [0] = 0.
 *   max_query_len    host upper bound of n_q (sizes the grid).
 * bf16 only (matrix-core path); PA_F32 returns PA_ERR_UNSUPPORTED.
 * num_kv_heads above 2^19 (a cache block of more than 2^31 bytes) returns
 * PA_ERR_INVALID_ARG.
 */
int pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* query_start_loc, const int32_t* context_lens, int32_t num_seqs,
                     int32_t max_query_len, int32_t num_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                     int32_t dtype, void* stream);

/*
 * pa_mixed_step -- one launch for a batch that mixes prefill chunks and
 * single decode tokens (deep-dive page, sections "Chunked Prefill" and "Cơ chế
 * của Chunked Prefill": the scheduler interleaves prefill chunks with other
 * requests' decode steps; the tr.news.hada.io summary page: requests join
 * the batch as they arrive and finished ones leave it).
 *
 * Sequences 0 .. num_prefill_seqs-1 are chunks, exactly as in
 * pa_prefill_chunk (query rows query_start_loc[s] .. query_start_loc[s+1]-1,
 * query_start_loc[num_prefill_seqs] == num_prefill_tokens).  Sequences
 * num_prefill_seqs .. num_prefill_seqs+num_decode_seqs-1 are decode steps, as
 * in pa_decode: decode sequence j has the one query row num_prefill_tokens + j
 * and attends to its whole context.
 *
 *   out, q           device bf16 [num_prefill_tokens + num_decode_seqs]
 *                    [num_heads][head_dim].
 *   block_tables     device int32 [num_prefill_seqs + num_decode_seqs]
 *                    [max_blocks_per_seq]; context_lens likewise [..].
 *   query_start_loc  device int32 [num_prefill_seqs + 1] (may be NULL when
 *                    num_prefill_seqs == 0).
 *   max_query_len    host upper bound of the chunks' n_q.
 *   max_decode_context  host upper bound of the decode sequences' contexts
 *                    (sizes the grid); with partition 0, a decode sequence
 *                    whose context exceeds it gets no output.
 *   partition        decode partition in tokens, as in pa_decode: 0 = one
 *                    partition covering max_decode_context, else a positive
 *                    multiple of 64; decode sequences longer than one
 *                    partition are merged by a second launch.
 *   workspace        device scratch of pa_mixed_step_workspace_bytes(...)
 *                    bytes (NULL when that is 0), as in pa_decode.
 * Prefill rows are computed by the pa_prefill_chunk workgroup (bit-identical
 * to it), decode rows by pa_decode's per-item bodies (bit-identical to
 * pa_decode with the same partition).  bf16,
 * head_dim 128, num_heads / num_kv_heads in {1, 2, 4, 8}.
 */
int pa_mixed_step(void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* query_start_loc, const int32_t* context_lens,
                  int32_t num_prefill_seqs, int32_t num_prefill_tokens, int32_t max_query_len,
                  int32_t num_decode_seqs, int32_t max_decode_context, int32_t num_heads,
                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                  float scale, int32_t partition, void* workspace, size_t workspace_bytes,
                  int32_t dtype, int32_t flags, void* stream);

/* Workspace bytes of pa_mixed_step: the decode partials, as in pa_decode. */
size_t pa_mixed_step_workspace_bytes(int32_t num_decode_seqs, int32_t num_heads,
                                     int32_t head_dim, int32_t max_decode_context,
                                     int32_t partition);

/* ---------------------------------------------------------- block allocator */

/*
 * Host-side block allocator: logical-to-physical block tables, a free list,
 * per-block reference counts for blocks shared between sequences, and
 * copy-on-write (deep-dive page, sections "Tương tự phân trang bộ nhớ ảo" and
 * "Cơ chế APC"; the skymod.tech overview: in parallel sampling the prompt's
 * memory is shared by the output sequences).  It owns host memory only and
 * never touches the device: a copy-on-write it decides is returned to the
 * caller, who enqueues pa_copy_blocks before writing the new tokens.  Not
 * thread-safe: one scheduler thread drives it.  Every call either succeeds
 * completely or changes nothing.
 *
 * Policies: the free list is a LIFO stack, free_order[0] handed out first;
 * released blocks are pushed on top, a sequence's blocks from its last
 * logical block to its first.  fork gives the child the parent's table and
 * length, each block one more reference.  append of n tokens to a sequence of
 * length L: if L % block_size != 0 and the last block has more than one
 * reference, that block is copied first (a fresh block dst replaces src in the
 * table, src loses one reference, (src, dst) is reported); then
 * ceil((L+n)/block_size) - blocks_held blocks are popped in logical order, and
 * the slots of positions L .. L+n-1 are
 *   slot(p) = table[p / block_size] * block_size + p % block_size.
 */
typedef struct pa_allocator pa_allocator;

/* free_order: NULL (identity order) or a permutation of [0, num_blocks). */
int pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                    pa_allocator** out);
void pa_alloc_destroy(pa_allocator* a);

int pa_seq_new(pa_allocator* a, int64_t seq);
int pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child);
/* slots_out: [n] (may be NULL when n == 0); cow_pair_out: [2]; *n_cow_out is
 * 0 or 1. */
int pa_seq_append(pa_allocator* a, int64_t seq, int32_t n, int64_t* slots_out,
                  int32_t* cow_pair_out, int32_t* n_cow_out);
int pa_seq_free(pa_allocator* a, int64_t seq);
int pa_seq_len(const pa_allocator* a, int64_t seq, int32_t* len_out);
/* Copies up to cap entries of the block table; *n_out = the table's length. */
int pa_seq_block_table(const pa_allocator* a, int64_t seq, int32_t* out, int32_t cap,
                       int32_t* n_out);
int pa_block_refcount(const pa_allocator* a, int32_t block, int32_t* rc_out);
int pa_num_free(const pa_allocator* a, int32_t* n_out);
/* Copies the free list, bottom of the stack first; *n_out = its length. */
int pa_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n_out);

/*
 * pa_batch_append -- one decode/prefill step's worth of appends in one call.
 * Appends n[i] tokens to seqs[i] for i = 0 .. num_seqs-1, in order, each as
 * pa_seq_append would.  Stops at the first failing append: *n_done_out tells
 * how many succeeded (those stay applied); the status is that failure's.
 *   slots_out      [sum n] slots, sequence after sequence.
 *   cow_pairs_out  [num_seqs][2]; *n_cow_out pairs are written, in order.
 * Then, on success, exports the batch for the kernels:
 *   block_tables_out [num_seqs][max_blocks_per_seq] (-1 padded), and
 *   context_lens_out [num_seqs] (either may be NULL to skip).
 * A table wider than max_blocks_per_seq returns PA_ERR_INVALID_ARG after the
 * appends are applied.
 */
int pa_batch_append(pa_allocator* a, const int64_t* seqs, int32_t num_seqs, const int32_t* n,
                    int64_t* slots_out, int32_t* cow_pairs_out, int32_t* n_cow_out,
                    int32_t* block_tables_out, int32_t max_blocks_per_seq,
                    int32_t* context_lens_out, int32_t* n_done_out);

/* Block tables and context lengths of seqs[0..num_seqs) as above. */
int pa_export_tables(const pa_allocator* a, const int64_t* seqs, int32_t num_seqs,
                     int32_t* block_tables_out, int32_t max_blocks_per_seq,
                     int32_t* context_lens_out);

/*
 * pa_alloc_stats -- out[0] free blocks (on the free list), out[1] the rest
 * (held by a sequence or kept by the prefix cache), out[2] blocks
 * with more than one reference, out[3] live sequences, out[4] wasted slots
 * (internal fragmentation: sum over sequences of blocks_held * block_size -
 * length; below block_size per sequence).
 */
int pa_alloc_stats(const pa_allocator* a, int64_t out[5]);

/* ------------------------------------------------ automatic prefix caching */

/*
 * Automatic prefix caching (deep-dive page, section "Cơ chế APC", items 1-2:
 * a trie of cached KV blocks; a new request whose prefix matches links the
 * matched physical blocks into its table instead of recomputing them; and
 * its advice to evict blocks not recently used under memory pressure).
 *
 * Granularity is whole blocks: a trie node is one full block's token ids
 * under its parent (the blocks before it).  Rules:
 *  - A block enters the trie when it becomes full through
 *    pa_seq_append_tokens (token ids known for the whole sequence so far) and
 *    no node with the same tokens exists under the same parent; otherwise it
 *    stays private.  Appends without token ids (pa_seq_append,
 *    pa_batch_append) end caching for that sequence.
 *  - pa_seq_new_cached matches the prompt's full blocks from the root,
 *    leaving at least the last prompt token uncached (at most (n - 1) /
 *    block_size blocks), links the matched blocks (one more reference each)
 *    and starts the sequence at the matched length.
 *  - A cached block that no sequence holds any more is kept; the free list is
 *    used first, and only when it is empty is a kept block evicted: least
 *    recently used first (use = matched, registered or released), the deeper
 *    block first among equals, then the lower block id.  Evicting a block
 *    drops its trie node and everything under it; their blocks become
 *    ordinary blocks (to the free list if no sequence holds them).
 *  - Out of blocks means free list plus kept blocks cannot cover a request.
 * The hit rate is hit tokens / prompt tokens over pa_seq_new_cached calls.
 */

/* Turn prefix caching on; only while the allocator holds no sequence. */
int pa_alloc_enable_prefix_cache(pa_allocator* a);

/*
 * pa_seq_new_cached -- new sequence `seq` for a prompt of n tokens (host
 * int32 token ids).  *n_cached_out = tokens found in the cache (a multiple of
 * block_size); the sequence starts with that length, and the caller appends
 * the remaining n - *n_cached_out prompt tokens with pa_seq_append_tokens.
 * PA_ERR_INVALID_ARG if caching is off.
 */
int pa_seq_new_cached(pa_allocator* a, int64_t seq, const int32_t* tokens, int32_t n,
                      int32_t* n_cached_out);

/* pa_seq_append with the appended tokens' ids (host int32 [n]). */
int pa_seq_append_tokens(pa_allocator* a, int64_t seq, const int32_t* tokens, int32_t n,
                         int64_t* slots_out, int32_t* cow_pair_out, int32_t* n_cow_out);

/*
 * pa_prefix_cache_stats -- out[0] hit tokens, out[1] prompt tokens looked up,
 * out[2] blocks in the trie, out[3] of those, blocks no sequence holds,
 * out[4] evictions.
 */
int pa_prefix_cache_stats(const pa_allocator* a, int64_t out[5]);

/*
 * pa_prefix_cache_blocks -- the blocks in the trie, by block id, with their
 * depth (logical block index + 1), and optionally (evictable_out, same cap)
 * the kept blocks in eviction order.  *n_out = number of blocks in the trie.
 */
int pa_prefix_cache_blocks(const pa_allocator* a, int32_t* blocks_out, int32_t* depths_out,
                           int32_t* evictable_out, int32_t cap, int32_t* n_out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
