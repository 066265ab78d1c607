/*
 * pa.h -- C ABI of libpa.so: paged KV-cache decode attention for AMD
 * Instinct MI355X (gfx950).
 *
 * The method (PagedAttention): a sequence's cached keys and values live in
 * fixed-size physical blocks of `block_size` token slots, not in one
 * contiguous slab; a per-sequence block table lists, in logical order, the
 * physical block that holds each run of `block_size` positions.  Zero-based
 * position t lives in logical block t / block_size at slot t % block_size.
 * ("How PagedAttention works", aiinfrainterviews.com, sections "TL;DR" and
 * "A strong answer"; lihaoran.work PagedAttention explainer, section "A block
 * table maps logical order to physical storage".)
 *
 * Common conventions for every entry point below
 * ----------------------------------------------
 * Memory.  Every array argument is DEVICE memory owned by the caller, in the
 * layout stated (C order, densely packed), aligned to 16 bytes, unless its
 * call says otherwise: the group arrays of pa_decode_shared_prefix and every
 * block-manager argument are host memory, and pa_swap_blocks moves blocks to
 * and from pinned host memory.  The library allocates nothing and frees
 * nothing.  Its only state is a cached compute-unit count per device (used
 * to size the shared-prefix split) and, for pa_decode_noalloc only, one
 * static scratch array per device; every call is otherwise independent.
 *
 * One layer's cache.  `k_cache` and `v_cache` are each
 *     [num_blocks][kv_heads][block_size][head_dim]
 * elements of the call's dtype: physical block p holds, for each KV head,
 * block_size consecutive token slots of head_dim elements.
 *
 * dtype.  PA_F32 (IEEE binary32) or PA_BF16 (bfloat16).  q, out, caches and
 * new tokens of one call share the dtype.  Arithmetic is in fp32 either way.
 *
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Calls are
 * asynchronous and ordered on that stream; nothing synchronises the host.
 *
 * Errors.  Host-side arguments are checked before anything is launched:
 *   PA_ERR_INVALID_ARG  a size is negative or zero where it must be positive,
 *                       a pointer is NULL or not 16-byte aligned, head counts
 *                       do not divide, a workspace is too small (the same
 *                       convention as the explainer's block_layout, which
 *                       rejects negative sizes);
 *   PA_ERR_UNSUPPORTED  a shape with no kernel instance (see each call);
 *   PA_ERR_HIP          the HIP runtime reported a launch error;
 *   PA_ERR_NO_SPACE     (block manager) the pool cannot cover the request:
 *                       wait, or preempt a sequence; nothing changed;
 *   PA_ERR_SCRATCH      (pa_decode_noalloc) the call needs more workspace
 *                       than the library's static scratch holds.
 * On an error nothing has been launched (PA_ERR_HIP: possibly part of it).
 * Device-resident contents (table entries, slots, lengths) are read by the
 * kernels, which never access memory outside the arrays described here:
 * see each call for what happens to out-of-range contents.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,
  PA_ERR_UNSUPPORTED = 2,
  PA_ERR_HIP = 3,
  PA_ERR_NO_SPACE = 4,
  PA_ERR_SCRATCH = 5
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* Decode kernel selection for pa_decode_ex. */
typedef enum pa_kernel {
  PA_KERNEL_AUTO = 0,   /* MFMA when it supports the shape, else VALU        */
  PA_KERNEL_VALU = 1,   /* vector-ALU split kernel: fp32 or bf16, G <= 8     */
  PA_KERNEL_MFMA = 2    /* matrix-core split kernel (+ reduce kernel): bf16,
                           head_dim 64/128, block_size 16..256,
                           num_heads/kv_heads <= 16                          */
} pa_kernel;

/* Version of this ABI (increments on any signature change). */
int32_t pa_abi_version(void);

/* Static text for a status code; never NULL. */
const char* pa_status_string(int32_t status);

/*
 * Host helper: blocks an unshared sequence of `tokens` cached positions
 * occupies, and the unused slots in its last block
 * (lihaoran.work explainer, section "How many tail slots remain unused?":
 * blocks = ceil(tokens / block_size), unused = blocks*block_size - tokens,
 * which is in [0, block_size-1] for tokens > 0 and 0 for tokens = 0).
 * `blocks` and `unused` are HOST pointers.  tokens < 0 or block_size <= 0
 * gives PA_ERR_INVALID_ARG and leaves the outputs untouched.
 */
pa_status pa_block_layout(int64_t tokens, int32_t block_size, int64_t* blocks, int64_t* unused);

/*
 * KV append: write the keys and values of `num_tokens` new tokens into the
 * cache slots named by `slot_mapping` ("How PagedAttention works", section
 * "A strong answer": every decode step adds the new token's K/V to the
 * sequence's blocks).
 *
 *   k_new, v_new   [num_tokens][kv_heads][head_dim], dtype
 *   k_cache,       [num_blocks][kv_heads][block_size][head_dim], written in place
 *   v_cache
 *   slot_mapping   int64 [num_tokens]: slot s means physical block
 *                  s / block_size, slot s % block_size.  s < 0 marks a padding
 *                  token and is skipped; s >= num_blocks*block_size is also
 *                  skipped (never written out of bounds).
 *
 * The copy is bit-exact.  Slots must be distinct (two tokens writing one slot
 * race).  num_tokens = 0 launches nothing.  Shapes: head_dim*elem_size a
 * multiple of 16 bytes (head_dim in {64, 128} is instantiated for both
 * dtypes; any multiple of 8 for bf16 / 4 for fp32 works), block_size >= 1.
 */
pa_status pa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                       const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                       int32_t kv_heads, int32_t block_size, int32_t head_dim, int32_t dtype,
                       void* stream);

/*
 * Decode plan: the kernel, partition size, grid and workspace size that
 * pa_decode/pa_decode_ex will use for these host-side sizes.  All outputs
 * are HOST pointers (any may be NULL).
 *
 * Split kernels (VALU, MFMA): each sequence's history is cut into partitions
 * of `partition_size` tokens, one work-group per (sequence, KV head,
 * partition); a sequence spanning several partitions leaves one partial
 * result per partition (running max, running sum, unnormalised output) in the
 * workspace and a reduce kernel merges them.
 *   partition_size > 0 : used as given by VALU; rounded up to a multiple of
 *                        32 tokens by MFMA; in both cases capped at
 *                        max_seq_len (rounded the same way), so any value up
 *                        to INT32_MAX is accepted and a huge one means "do
 *                        not split";
 *   partition_size = 0 : chosen from num_seqs*kv_heads and max_seq_len (no
 *                        split when there are enough (sequence, head) pairs
 *                        to fill the GPU).
 *   workspace = num_seqs*num_heads*num_partitions*(head_dim+2)*4 bytes when
 *   num_partitions > 1, else 0.  More than 16384 partitions per sequence is
 *   PA_ERR_UNSUPPORTED; max_seq_len within 32 of INT32_MAX is
 *   PA_ERR_INVALID_ARG.
 * Two calls in flight at once must not share a workspace.
 */
pa_status pa_decode_plan(int32_t num_seqs, int32_t num_heads, int32_t kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t max_seq_len, int32_t partition_size,
                         int32_t dtype, int32_t kernel, int32_t* kernel_used,
                         int32_t* eff_partition_size, int32_t* num_partitions,
                         size_t* workspace_bytes);

/* Workspace bytes pa_decode needs (0 on invalid arguments). */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                                 int32_t partition_size, int32_t dtype);

/*
 * Paged decode attention for one layer: one query token per sequence attends
 * over all of that sequence's cached positions [0, seq_lens[s]), gathered
 * through its block table (zenaique.com page, conceptual block-lookup code;
 * lihaoran.work explainer, section "A block table maps logical order to
 * physical storage").
 *
 *   out           [num_seqs][num_heads][head_dim], dtype, written
 *   q             [num_seqs][num_heads][head_dim], dtype
 *   k_cache,      [num_blocks][kv_heads][block_size][head_dim], dtype, read only
 *   v_cache
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; entries past a
 *                 sequence's last block are never read
 *   seq_lens      int32 [num_seqs]
 *   max_seq_len   host upper bound of seq_lens (sizes the grid)
 *   scale         multiplies q.k before the softmax (e.g. 1/sqrt(head_dim))
 *   workspace     device scratch of at least pa_decode_workspace_bytes();
 *                 may be NULL when that is 0.  Contents need no initialising;
 *                 calls in flight at the same time need separate workspaces.
 *
 * out[s][h] = sum_t softmax_t(scale * q[s][h] . K[t][h / G]) * V[t][h / G]
 * with G = num_heads / kv_heads (query head h reads KV head h / G), K[t]/V[t]
 * the key/value rows of position t.  seq_lens[s] = 0 gives a zero row.
 * Out-of-range device contents produce NaN rows instead of out-of-bounds
 * reads: a sequence with seq_lens[s] < 0, > max_seq_len or
 * > max_blocks_per_seq*block_size, or whose table names a block outside
 * [0, num_blocks), gets NaN in all of its heads' outputs.
 * `out` must not alias any input.  Shapes: head_dim in {64, 128};
 * block_size a power of two in [1, 256]; num_heads % kv_heads == 0 with
 * G in {1, 2, 4, 8, 16}.
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t max_seq_len, int32_t num_seqs,
                    int32_t num_heads, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, float scale, int32_t partition_size, void* workspace,
                    size_t workspace_bytes, int32_t dtype, void* stream);

/* pa_decode with an explicit kernel choice (pa_kernel).  PA_KERNEL_MFMA on a
 * shape it does not support returns PA_ERR_UNSUPPORTED. */
pa_status pa_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* seq_lens, int32_t max_seq_len, int32_t num_seqs,
                       int32_t num_heads, int32_t kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, float scale,
                       int32_t partition_size, void* workspace, size_t workspace_bytes,
                       int32_t dtype, int32_t kernel, void* stream);

/*
 * pa_decode_ex with the caller's processing order: `order` (device int32
 * [num_seqs]) is a permutation of the sequences, longest first.  The
 * matrix-core kernel otherwise ranks the batch by length inside every
 * work-group (hardware dispatches work-groups in index order, so long
 * sequences first trims the launch's tail); a caller that keeps the order
 * (it changes only when the batch does: every decode step adds one token to
 * every sequence) saves that prologue.  The order affects speed only: any
 * permutation gives the same outputs; the other kernels ignore it.  With the
 * matrix-core kernel an entry outside [0, num_seqs) leaves its work item
 * idle, and a sequence missing from `order` gets an unspecified output (no
 * memory outside the arrays is touched).  NULL order with num_seqs > 0 ->
 * PA_ERR_INVALID_ARG; otherwise as pa_decode_ex.
 */
pa_status pa_decode_ordered(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t max_seq_len, const int32_t* order,
                            int32_t num_seqs, int32_t num_heads, int32_t kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                            int32_t partition_size, void* workspace, size_t workspace_bytes,
                            int32_t dtype, int32_t kernel, void* stream);

/*
 * pa_decode_ex for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as pa_decode_ex, without the workspace: the
 * split kernels' partials go to a static device array of
 * PA_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on every device it
 * runs on until the process ends.  A call whose workspace need
 * (pa_decode_plan's workspace_bytes) exceeds it returns PA_ERR_SCRATCH before
 * anything is launched; 16 MiB covers, e.g., 16 sequences x 64 query heads x
 * 16 partitions at head_dim 128 (8.5 MB).  The call allocates and frees
 * nothing.  The scratch needs no clearing (every partial the merge reads is
 * written by the same call first), and every call on a device shares that
 * device's array: two pa_decode_noalloc calls that can overlap on one device
 * (different streams, no ordering between them) race and give undefined
 * outputs.  The first call on a device looks the array's address up once
 * (hipGetSymbolAddress); a failed lookup returns PA_ERR_HIP.
 */
#define PA_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)
pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t max_seq_len, int32_t num_seqs,
                            int32_t num_heads, int32_t kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, float scale,
                            int32_t partition_size, int32_t dtype, int32_t kernel,
                            void* stream);

/*
 * Fused decode step: the KV append of one new token per sequence and the
 * paged decode, in one launch ("How PagedAttention works", section "A strong
 * answer": each decode step writes the new token's K/V, then attends over the
 * sequence's blocks).  Same result as
 *     pa_kv_append(k_new, v_new, k_cache, v_cache, slot_mapping, num_seqs, ...)
 *     pa_decode(out, q, k_cache, v_cache, block_tables, ..., seq_lens, ...)
 * (bit-identical cache; bit-identical outputs when the decode runs the same
 * kernel shape: pa_decode_plan's choice unless it splits partitions per
 * wave, which the fused call does not), without the second launch.
 *
 *   k_new, v_new   [num_seqs][kv_heads][head_dim], dtype: sequence s's new token
 *   slot_mapping   int64 [num_seqs]: cache slot of sequence s's new token, or
 *                  < 0 when sequence s appends nothing this step
 *   seq_lens       lengths AFTER the append; when slot_mapping[s] >= 0 the new
 *                  token is position seq_lens[s] - 1, and slot_mapping[s] must
 *                  be that position's slot under the sequence's block table
 * The new token's K and V come from k_new/v_new: the work-group whose
 * partition holds the token (the sequence's last one) loads the token's tile
 * from the cache as usual and replaces that row with the new rows in
 * registers before the step's math, then writes the rows to the slot after
 * its last cache read.  No other work-group reads the slot.  The slot's
 * block must not be read by any other sequence in the same call
 * (copy-on-write first).  Other arguments, errors and shapes as
 * pa_decode_ex.
 */
pa_status pa_decode_append(void* out, const void* q, void* k_cache, void* v_cache,
                           const void* k_new, const void* v_new, const int64_t* slot_mapping,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t max_seq_len, int32_t num_seqs,
                           int32_t num_heads, int32_t kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, float scale,
                           int32_t partition_size, void* workspace, size_t workspace_bytes,
                           int32_t dtype, int32_t kernel, void* stream);

/*
 * pa_decode_append with the work-groups dispatched in the caller's order, as
 * pa_decode_ordered does for pa_decode (same `order` argument: a permutation
 * of the batch, longest sequence first for speed; it changes only the
 * dispatch order, never a result).  An entry outside [0, num_seqs) leaves its
 * work-group idle, so a sequence missing from `order` gets neither its
 * output row nor its append.  A null `order` (with num_seqs > 0) ->
 * PA_ERR_INVALID_ARG; everything else as pa_decode_append.  On the 70B-shaped
 * batch this one launch is the decode step (append and decode).
 */
pa_status pa_decode_append_ordered(void* out, const void* q, void* k_cache, void* v_cache,
                                   const void* k_new, const void* v_new,
                                   const int64_t* slot_mapping, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                   int32_t max_seq_len, const int32_t* order, int32_t num_seqs,
                                   int32_t num_heads, int32_t kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks, float scale,
                                   int32_t partition_size, void* workspace,
                                   size_t workspace_bytes, int32_t dtype, int32_t kernel,
                                   void* stream);

/*
 * Shared-prefix decode: the result of pa_decode for a batch in which groups of
 * sequences share the leading blocks of their tables (one prefix, refcounted,
 * N tables pointing at it: "How PagedAttention works", section "A strong
 * answer", the shared system prompt across 200 conversations; lihaoran.work
 * explainer, section "Shared prefixes need matching computation").  Every
 * member's query attends the shared keys in one matrix-core pass per group,
 * which reads each shared K/V tile once per work-group instead of once per
 * sequence; the positions after the prefix run through the decode kernel, and
 * a merge kernel combines the two softmax partials.  Outputs equal pa_decode's
 * up to rounding.
 *
 *   group_start          HOST int32 [num_groups + 1], non-decreasing, in
 *                        [0, num_seqs]: group g is sequences
 *                        group_start[g] .. group_start[g+1]-1 (order the batch
 *                        so that each group's members are adjacent)
 *   group_prefix_blocks  HOST int32 [num_groups]: the number of leading table
 *                        entries every member of group g shares with its
 *                        first member (the leader); whole blocks only, so the
 *                        prefix is group_prefix_blocks[g] * block_size tokens
 *   num_groups           0 .. PA_MAX_PREFIX_GROUPS (0: plain decode)
 *   prefix_partition_size  keys per prefix-kernel partition (rounded up to a
 *                        multiple of 32 and capped at the longest prefix, so
 *                        INT32_MAX means "do not split"); 0 = the library's
 *                        choice (about one work-group per compute unit)
 *   partition_size       tail partitions, as in pa_decode (0 = default)
 *   workspace            device, >= pa_decode_shared_prefix_workspace_bytes()
 *                        with the same arguments, 16-byte aligned
 * Sequences outside every group, and groups with no member or no shared
 * block, decode as in pa_decode.  A member whose table does not start with
 * its leader's group_prefix_blocks entries, or whose length is below the
 * prefix, gets a NaN row (checked on the device); other device contents as in
 * pa_decode.  Requirements: bf16, the matrix-core kernel's shapes
 * (head_dim in {64, 128}, block_size a power of two in [16, 256]) with
 * G = num_heads / kv_heads a power of two <= 16, and scale > 0 (the prefix
 * kernel scales row maxima of raw scores); a group's prefix may not exceed
 * max_blocks_per_seq blocks or max_seq_len tokens.  Errors: bad host
 * arguments -> PA_ERR_INVALID_ARG; more than PA_MAX_PREFIX_GROUPS groups or
 * an unsupported shape -> PA_ERR_UNSUPPORTED.  Two launches on `stream`
 * (the prefix attention and the tail decode in one, then the merge);
 * allocates nothing.
 */
#define PA_MAX_PREFIX_GROUPS 32
pa_status pa_decode_shared_prefix(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                  int32_t max_seq_len, int32_t num_seqs, int32_t num_heads,
                                  int32_t kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, float scale, const int32_t* group_start,
                                  const int32_t* group_prefix_blocks, int32_t num_groups,
                                  int32_t prefix_partition_size, int32_t partition_size,
                                  void* workspace, size_t workspace_bytes, int32_t dtype,
                                  void* stream);

/*
 * pa_decode_shared_prefix with the caller's processing order for the tails
 * (each sequence's positions after its group's prefix): `order` (device int32
 * [num_seqs]) is a permutation of the sequences, longest tail first.  The
 * tail work-groups follow the prefix work-groups in one launch and the
 * hardware dispatches them in index order, so the longest tails first leave
 * only short ones for the end of the launch (measured on the shared-prefix
 * workload: 67.7 us per call against 73.1 us in index order).  The order
 * affects speed only: any permutation gives the same outputs as
 * pa_decode_shared_prefix, bit for bit.  An entry outside [0, num_seqs)
 * leaves its tail work item idle, and a sequence missing from `order` gets an
 * unspecified output row (no memory outside the arrays is touched).  A caller
 * keeps the order while the batch is unchanged (every decode step adds one
 * token to every sequence).  NULL order with num_seqs > 0, or an order not
 * 4-byte aligned -> PA_ERR_INVALID_ARG; otherwise as pa_decode_shared_prefix
 * (with no group, as pa_decode_ordered with the matrix-core kernel).
 */
pa_status pa_decode_shared_prefix_ordered(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
    int32_t max_seq_len, const int32_t* order, int32_t num_seqs, int32_t num_heads,
    int32_t kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    const int32_t* group_start, const int32_t* group_prefix_blocks, int32_t num_groups,
    int32_t prefix_partition_size, int32_t partition_size, void* workspace,
    size_t workspace_bytes, int32_t dtype, void* stream);

/* Workspace bytes pa_decode_shared_prefix needs for these arguments (0 when
 * they are invalid or unsupported, or when nothing is shared and the plain
 * decode needs none). */
size_t pa_decode_shared_prefix_workspace_bytes(
    int32_t num_seqs, int32_t num_heads, int32_t kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_seq_len, int32_t max_blocks_per_seq, const int32_t* group_start,
    const int32_t* group_prefix_blocks, int32_t num_groups, int32_t prefix_partition_size,
    int32_t partition_size, int32_t dtype);

/*
 * Copy-on-write block copy: for each (src, dst) pair, copy every KV head and
 * every slot of physical block src into physical block dst, in both caches
 * ("How PagedAttention works", feature table row on beam search and parallel
 * sampling; zenaique.com follow-up on beam search: a fork shares blocks and
 * copies only the block that diverges, into a freshly allocated block).
 *
 *   k_cache, v_cache  [num_blocks][kv_heads][block_size][head_dim], in place
 *   block_mapping     int64 [num_pairs][2] = (src, dst)
 *
 * Bit-exact.  The dst ids must be distinct and disjoint from the src ids
 * (otherwise the result depends on ordering).  A pair with either id outside
 * [0, num_blocks) is skipped.  num_pairs = 0 launches nothing.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                         int32_t num_pairs, int32_t num_blocks, int32_t kv_heads,
                         int32_t block_size, int32_t head_dim, int32_t dtype, void* stream);

/*
 * Chunked causal prefill over the paged cache: every sequence brings a chunk
 * of queries whose K/V are already in the cache (pa_kv_append), at its last
 * positions, and each query attends every position up to and including its
 * own ("How PagedAttention works", section "A strong answer": the kernel
 * gathers each query's blocks through the table; lihaoran.work explainer, section "A block
 * table maps logical order to physical storage": full causal attention over
 * the visible history).
 *
 *   out, q         [num_queries][num_heads][head_dim], dtype; sequence s owns
 *                  rows [query_start[s], query_start[s+1])
 *   k_cache,       [num_blocks][kv_heads][block_size][head_dim], dtype
 *   v_cache
 *   block_tables   int32 [num_seqs][max_blocks_per_seq]
 *   seq_lens       int32 [num_seqs]: cached positions, chunk included; the
 *                  chunk of n queries sits at positions seq_lens[s]-n .. -1
 *   query_start    int32 [num_seqs + 1], non-decreasing, 0 .. num_queries
 *   max_query_len  host upper bound on every chunk length (sizes the grid)
 *
 * All device pointers are caller-owned; the call is asynchronous on `stream`
 * and allocates nothing.  Rows of a chunk that cannot be served (longer than
 * its sequence or than max_query_len, or a sequence longer than its table)
 * are NaN; a sequence whose offsets fall outside [0, num_queries] or decrease
 * is skipped (its rows are not written); a table entry outside the pool
 * makes the rows that read it NaN.  Host checks: negative sizes, a zero
 * size, num_heads % kv_heads != 0, a scale that is not finite and positive
 * (the kernel takes row maxima of unscaled scores), null or misaligned
 * pointers -> PA_ERR_INVALID_ARG.  Kernels: bf16 with block_size a power of
 * two in [16, 256] and a query group (num_heads / kv_heads) that is a power
 * of two <= 16 runs on the matrix cores; fp32, or bf16 with a smaller power
 * of two block size, runs on the vector ALUs with a query group in
 * {1, 2, 4, 8}; head_dim 64 or 128 for both.  Other shapes ->
 * PA_ERR_UNSUPPORTED.  num_seqs, num_queries or max_query_len of 0 launch
 * nothing.
 */
pa_status pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* seq_lens, const int32_t* query_start, int32_t max_query_len,
                     int32_t num_seqs, int32_t num_queries, int32_t num_heads, int32_t kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                     int32_t dtype, void* stream);

/*
 * Block swap for preemption: move whole blocks between the device pool and a
 * pinned host pool, either way ("How PagedAttention works", section "A strong
 * answer", feature table: preemption swaps blocks to host memory at block
 * granularity; section "What interviewers probe next": over the host link
 * into pinned host memory).  For each (src, dst) pair of block_mapping,
 * block src of the source pool (K and V, every KV head and slot) is copied
 * bit-exactly into block dst of the destination pool.
 *
 *   dst_k, dst_v     destination pool, [dst_num_blocks][kv_heads][block_size][head_dim]
 *   src_k, src_v     source pool, [src_num_blocks][...] with the same block shape
 *   block_mapping    int64 [num_pairs][2] (src, dst), device or pinned host memory
 *
 * Each pool is either device memory or pinned host memory (hipHostMalloc,
 * torch pin_memory); the GPU reaches host memory through its mapping, so the
 * copy is one kernel whatever the pair count.  Device-to-device works too (a
 * move between two device pools).  Host checks, before any launch: every
 * pointer's residency is queried (hipPointerGetAttributes), and pageable or
 * unknown memory, K and V of one pool in different places, misalignment
 * (16 bytes, 8 for the mapping), negative or zero sizes -> PA_ERR_INVALID_ARG;
 * host-to-host, or a block size not a multiple of 16 bytes ->
 * PA_ERR_UNSUPPORTED.  Pairs naming a block outside either pool are skipped.
 * Destination blocks must be distinct and must not be a source of the same
 * call.  Asynchronous on `stream`; num_pairs = 0 launches nothing.
 */
pa_status pa_swap_blocks(void* dst_k, void* dst_v, int64_t dst_num_blocks, const void* src_k,
                         const void* src_v, int64_t src_num_blocks, const int64_t* block_mapping,
                         int32_t num_pairs, int32_t kv_heads, int32_t block_size,
                         int32_t head_dim, int32_t dtype, void* stream);

/*
 * Layered pool: one pool for every layer, [num_blocks][2][num_layers]
 * [kv_heads][block_size][head_dim] -- a block holds the K (index 0) and V
 * (index 1) of all layers for its block_size tokens (zenaique.com code box
 * "Conceptual: PagedAttention block lookup"; "How PagedAttention works",
 * section "A strong answer": a pool for each layer, or one pool holding all
 * layers).  One
 * block table per sequence serves every layer; slots and block ids mean the
 * same as for per-layer pools.  Same element types, shapes, errors and
 * device-content behaviour as the per-layer calls, plus: layer indices out
 * of [0, num_layers) -> PA_ERR_INVALID_ARG.
 *
 * pa_kv_append_layered   pa_kv_append of layer `layer`'s new K/V rows.
 * pa_decode_layered      decode of layers [first_layer, first_layer + layers)
 *                        in ONE launch (grid over layers): q and out are
 *                        [layers][num_seqs][num_heads][head_dim]; every layer
 *                        uses the same tables and lengths.  The kernel is
 *                        pa_decode's automatic choice (matrix cores for
 *                        bf16 at block sizes >= 16, else the vector-ALU
 *                        kernel, fp32 included); the workspace is `layers`
 *                        times pa_decode_plan's for one layer (kernel
 *                        PA_KERNEL_AUTO).  layers <= 65535.
 * pa_copy_blocks_layered copy-on-write of whole blocks (every layer, K and V).
 * pa_swap_blocks_layered pa_swap_blocks of whole layered blocks between a
 *                        device pool and a pinned-host pool (or two device
 *                        pools); the same residency checks.
 */
pa_status pa_kv_append_layered(const void* k_new, const void* v_new, void* kv_pool, int32_t layer,
                               int32_t num_layers, const int64_t* slot_mapping,
                               int32_t num_tokens, int32_t num_blocks, int32_t kv_heads,
                               int32_t block_size, int32_t head_dim, int32_t dtype,
                               void* stream);
pa_status pa_decode_layered(void* out, const void* q, const void* kv_pool, int32_t first_layer,
                            int32_t layers, int32_t num_layers, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            int32_t max_seq_len, int32_t num_seqs, int32_t num_heads,
                            int32_t kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, float scale, int32_t partition_size,
                            void* workspace, size_t workspace_bytes, int32_t dtype,
                            void* stream);
pa_status pa_copy_blocks_layered(void* kv_pool, const int64_t* block_mapping, int32_t num_pairs,
                                 int32_t num_blocks, int32_t num_layers, int32_t kv_heads,
                                 int32_t block_size, int32_t head_dim, int32_t dtype,
                                 void* stream);
pa_status pa_swap_blocks_layered(void* dst_pool, int64_t dst_num_blocks, const void* src_pool,
                                 int64_t src_num_blocks, const int64_t* block_mapping,
                                 int32_t num_pairs, int32_t num_layers, int32_t kv_heads,
                                 int32_t block_size, int32_t head_dim, int32_t dtype,
                                 void* stream);

/*
 * Block manager: the host-side bookkeeping around the kernels (plain C++, no
 * GPU calls).  It owns the free lists and reference counts of a device pool
 * of num_blocks blocks and a pinned-host pool of num_host_blocks, the block
 * table and cached length of every sequence, and hands out what the kernel
 * calls take: slots for pa_kv_append, (src, dst) pairs for pa_copy_blocks
 * and pa_swap_blocks, block-table rows and lengths for pa_decode.
 *
 *   admission   ("How PagedAttention works", section "What interviewers probe
 *               next") a prompt of T tokens is admitted when
 *               free - watermark >= ceil(T / block_size) + 1; it takes
 *               ceil(T / block_size) blocks;
 *   sharing     (same page, "A strong answer" feature table) fork gives the
 *               child every block of the parent (reference counts + 1); an
 *               append into a shared, partly filled last block first takes a
 *               private copy (copy on write: the (shared, copy) pair goes to
 *               pa_copy_blocks and the shared block loses one reference);
 *               release drops one reference per block;
 *   preemption  (same table) swap-out moves a sequence's blocks to host
 *               blocks, swap-in to fresh device blocks; the pairs go to
 *               pa_swap_blocks.
 * Policies: the lowest-numbered free block is taken first; the watermark
 * gates admission only; a batch of appends is all or nothing; a swapped-out
 * sequence cannot grow, fork or be decoded.  Sequence ids are any int64.
 * Errors: unknown or duplicate ids, a swapped-out sequence where a resident
 * one is needed, NULL outputs, too small output capacities ->
 * PA_ERR_INVALID_ARG; too few free blocks -> PA_ERR_NO_SPACE.  On any error
 * the manager is unchanged.  Not thread-safe: serialise calls on one manager.
 */
typedef struct pa_block_manager pa_block_manager;

pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, int64_t watermark_blocks,
                       int64_t num_host_blocks, pa_block_manager** out);
pa_status pa_bm_destroy(pa_block_manager* bm);
/* *ok = 1 when a prompt of prompt_tokens tokens can be admitted now. */
pa_status pa_bm_can_admit(const pa_block_manager* bm, int64_t prompt_tokens, int32_t* ok);
pa_status pa_bm_admit(pa_block_manager* bm, int64_t seq, int64_t prompt_tokens);
pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);
/* Reserve the next token's slot of each of the n (distinct, resident) seqs:
 * slots[i] for pa_kv_append; cow_pairs (capacity n pairs, int64 (src, dst))
 * receives *num_cow copy-on-write pairs for pa_copy_blocks, in batch order. */
pa_status pa_bm_append_slots(pa_block_manager* bm, const int64_t* seqs, int32_t n,
                             int64_t* slots, int64_t* cow_pairs, int32_t* num_cow);
pa_status pa_bm_release(pa_block_manager* bm, int64_t seq);
/* pairs: capacity entries of int64 (device, host) (swap-out) or (host, device)
 * (swap-in), one per block of the sequence, in table order. */
pa_status pa_bm_swap_out(pa_block_manager* bm, int64_t seq, int64_t* pairs, int64_t capacity,
                         int64_t* num_pairs);
pa_status pa_bm_swap_in(pa_block_manager* bm, int64_t seq, int64_t* pairs, int64_t capacity,
                        int64_t* num_pairs);
/* Host buffers: tables [n][max_blocks] (rows padded with pad_block), seq_lens [n]. */
pa_status pa_bm_decode_inputs(const pa_block_manager* bm, const int64_t* seqs, int32_t n,
                              int32_t max_blocks, int32_t pad_block, int32_t* tables,
                              int32_t* seq_lens);
pa_status pa_bm_sequence(const pa_block_manager* bm, int64_t seq, int64_t* len,
                         int64_t* num_blocks, int32_t* swapped);
pa_status pa_bm_stats(const pa_block_manager* bm, int64_t* free_blocks, int64_t* free_host_blocks,
                      int64_t* num_seqs);
/* Reference count of a device (host = 0) or host (host = 1) block. */
pa_status pa_bm_refcount(const pa_block_manager* bm, int64_t block, int32_t host, int32_t* ref);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
