/*
 * pa.h -- C ABI of the MI355X (gfx950) paged decode attention library
 * (libpa_mi355x.so).
 *
 * Two operations, both from the pages on vLLM's PagedAttention:
 *
 *   pa_decode            -- one decode step of attention for a batch of
 *                           sequences whose K/V history is stored in
 *                           fixed-size blocks scattered through a shared pool
 *                           and reached through a per-sequence block table.
 *                           Source: "vLLM 与 PagedAttention"
 *                           (inference.mavenzero.com/case-studies/vllm),
 *                           section 二, sub-sections "PagedAttention 的解法"
 *                           (blocks of usually 16 tokens, logical-to-physical
 *                           block table, shared pool) and "注意力计算改造"
 *                           (K/V read block by block, per-block results
 *                           accumulated; kernel sketch with q, key/value
 *                           caches, block table, context length and block
 *                           size as its arguments).
 *   pa_reshape_and_cache -- append each new token's K and V rows into its
 *                           slot of the pool.  Source: same page, "PagedAttention
 *                           的解法" (a new block is taken only once the last
 *                           one is full), and "指南" (illegalscreed.cn
 *                           .../vllm/guide-line), section "为什么 vLLM 快：
 *                           PagedAttention" (blocks allocated on demand,
 *                           anywhere in the shared pool).
 *
 * Everything below is a plain C interface: device pointers, sizes, enums and
 * an opaque stream.  No function allocates device memory.
 *
 * Common conventions
 *   - Device pointers are owned by the caller and must stay valid until the
 *     work enqueued on `stream` has finished.  The library keeps no pointer
 *     after a call returns; its only global state is a mutex-guarded cache
 *     of occupancy queries per (device, kernel shape), filled on first use.
 *     Calls are re-entrant and may run concurrently on different streams.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work; they never synchronise.  A call's kernels can
 *     therefore be captured in a graph on `stream` and replayed.
 *   - Every argument check runs on the host before any HIP call.  A return
 *     of PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED or PA_ERR_WORKSPACE means
 *     nothing was enqueued.  PA_ERR_HIP reports a failed launch (for
 *     example: no GPU); a call that enqueues several kernels and fails at a
 *     later one leaves the kernels enqueued before it to run.  Device faults
 *     surface at the caller's next synchronisation, as for any HIP kernel.
 *   - Elements are stored as `dtype`; all arithmetic is fp32.
 *   - 16-byte alignment is required for q, out, k, v, k_cache, v_cache and
 *     workspace (the kernels move 16-byte vectors); 4-byte alignment for the
 *     int32 arrays and 8-byte for slot_mapping.
 */
#ifndef PA_MI355X_PA_H_
#define PA_MI355X_PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, negative size, Hq % Hkv != 0,
                                 non-finite scale, partition not a multiple of block_size */
    PA_ERR_UNSUPPORTED = 2,   /* head_dim, block_size, dtype, layout or kernel outside the supported set */
    PA_ERR_WORKSPACE = 3,     /* split-K needs a workspace and the one given is missing or too small */
    PA_ERR_HIP = 4,           /* a HIP launch failed */
    PA_ERR_NO_BLOCKS = 5,     /* pa_blocks.h: not enough free blocks; nothing was changed */
    /* not values: they give the type the range of a 32-bit int, so that any
       int a C caller passes is a valid value of it and reaches the checks */
    PA_STATUS_RANGE_MIN_ = -2147483647 - 1,
    PA_STATUS_RANGE_MAX_ = 2147483647
} pa_status;

typedef enum pa_dtype {
    PA_F32 = 0,
    PA_F16 = 1,
    PA_BF16 = 2,
    /* not values: they give the type the range of a 32-bit int, so that any
       int a C caller passes is a valid value of it and reaches the checks */
    PA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    PA_DTYPE_RANGE_MAX_ = 2147483647
} pa_dtype;

/*
 * Cache layouts.  Both caches (K and V) use the same one.
 *   PA_LAYOUT_BHTD: [num_blocks, num_kv_heads, block_size, head_dim].  Each
 *                   (block, kv head) tile is one contiguous run of
 *                   block_size*head_dim elements.  Default.
 *   PA_LAYOUT_BTHD: [num_blocks, block_size, num_kv_heads, head_dim], the
 *                   layout of the kernel sketch on "vLLM 与 PagedAttention",
 *                   sub-section "注意力计算改造".
 */
typedef enum pa_layout {
    PA_LAYOUT_BHTD = 0,
    PA_LAYOUT_BTHD = 1,
    /* not values: they give the type the range of a 32-bit int, so that any
       int a C caller passes is a valid value of it and reaches the checks */
    PA_LAYOUT_RANGE_MIN_ = -2147483647 - 1,
    PA_LAYOUT_RANGE_MAX_ = 2147483647
} pa_layout;

/*
 * Kernel choice of pa_decode_ex.  Both kernels compute the same function and
 * meet the same accuracy bound; they differ in how the work maps onto the GPU.
 *   PA_KERNEL_AUTO    the library picks: PA_KERNEL_MFMA when its shape
 *                     conditions hold and at least 4 q heads share a kv head,
 *                     else PA_KERNEL_VECTOR.
 *   PA_KERNEL_VECTOR  scores and weighted sums on the vector ALUs; any
 *                     supported shape.
 *   PA_KERNEL_MFMA    the q heads that share one kv head are one small dense
 *                     contraction per 16-token tile, done on the matrix cores;
 *                     needs f16 or bf16, head_dim 128 or 256, and
 *                     num_q_heads/num_kv_heads <= 16 or a multiple of 16
 *                     (PA_ERR_UNSUPPORTED otherwise).
 */
typedef enum pa_kernel {
    PA_KERNEL_AUTO = 0,
    PA_KERNEL_VECTOR = 1,
    PA_KERNEL_MFMA = 2,
    /* not values: they give the type the range of a 32-bit int, so that any
       int a C caller passes is a valid value of it and reaches the checks */
    PA_KERNEL_RANGE_MIN_ = -2147483647 - 1,
    PA_KERNEL_RANGE_MAX_ = 2147483647
} pa_kernel;

/*
 * How the tokens of one sequence are split across workgroups (the
 * partition_tokens argument of pa_decode_ex; a positive value N is a split-K
 * partition of N tokens, see there).
 *
 *   PA_PARTITION_AUTO      the library picks: a single pass when the
 *                          (sequence, kv head) units number at least four per
 *                          compute unit -- the hardware then balances whole
 *                          units over the device -- else the balanced schedule.
 *   PA_PARTITION_SINGLE    one workgroup reads a whole context; no workspace.
 *   PA_PARTITION_BALANCED  every wave of the device reads the same number of
 *                          tokens: contexts are cut wherever the shares end,
 *                          and a reduce kernel merges the cut units' pieces.
 */
typedef enum pa_partition {
    PA_PARTITION_AUTO = 0,
    PA_PARTITION_SINGLE = -1,
    PA_PARTITION_BALANCED = -2
} pa_partition;

/*
 * Flags of pa_decode_ex.
 *
 *   PA_DECODE_SHARED_BLOCKS  some physical blocks are read by more than one
 *                            sequence in this call (a shared prompt prefix,
 *                            parallel sampling, beams).  K and V are then
 *                            loaded with the caches' normal policy, so that
 *                            the later readers of a shared block find it in
 *                            L2.  Without the flag every K/V row is loaded
 *                            as read-once (the non-temporal hint), which
 *                            streams faster from HBM but leaves no cached
 *                            copy behind.  Results are identical either way.
 */
typedef enum pa_decode_flags {
    PA_DECODE_SHARED_BLOCKS = 1
} pa_decode_flags;

/* Supported shapes: head_dim in {32, 64, 128, 256}; block_size in {8, 16, 32};
 * any num_q_heads that is a multiple of num_kv_heads. */

/*
 * pa_decode -- paged decode attention, one query token per sequence.
 *
 *   out[s, h, :] = softmax_t( scale * q[s, h, :] . K[s, t, g, :] ) V[s, t, g, :]
 *
 * over the tokens t = 0 .. context_lens[s]-1 of sequence s, where token t
 * lives in physical block block_tables[s, t / block_size] at offset
 * t % block_size, and q head h reads kv head g = h / (num_q_heads/num_kv_heads).
 *
 *   out            [num_seqs, num_q_heads, head_dim]  dtype, written in full
 *   q              [num_seqs, num_q_heads, head_dim]  dtype
 *   k_cache,
 *   v_cache        pool in PA_LAYOUT_BHTD, dtype, read only
 *   block_tables   [num_seqs, max_blocks_per_seq] int32, row-major; only the
 *                  first ceil(context_lens[s]/block_size) entries of row s are
 *                  read and each must be a valid physical block
 *   context_lens   [num_seqs] int32, every cached token of the sequence (the
 *                  token appended this step included); 0 gives a zero row;
 *                  values above max_blocks_per_seq*block_size are clamped
 *   scale          finite fp32 factor on q.k (usually 1/sqrt(head_dim))
 *   workspace      device scratch of at least pa_decode_workspace_bytes(...)
 *                  bytes for split-K partials (may be NULL when that is 0);
 *                  its content on entry does not matter
 *
 * Equivalent to pa_decode_ex with num_blocks = INT32_MAX (table entries are
 * trusted), layout PA_LAYOUT_BHTD, PA_PARTITION_AUTO, PA_KERNEL_AUTO and no
 * flags (blocks are taken to be private to their sequence).
 */
pa_status pa_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, const int32_t *context_lens,
                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                    int block_size, int max_blocks_per_seq, float scale, pa_dtype dtype,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_decode_noalloc -- pa_decode without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, path and
 * result as pa_decode; the split-K partials live in PA_NOALLOC_SCRATCH_BYTES
 * of device memory the library owns, one copy per GPU, held until the process
 * ends.  The call allocates nothing (no hipMalloc, no hipFree) and needs no
 * zeroed memory: every kernel writes each scratch word it reads first.
 *
 * Every call on one GPU uses that GPU's one scratch array: calls whose work
 * overlaps in time on the same GPU (different streams, or graphs replayed
 * concurrently) race on it and give wrong results.  Serialise them, or use
 * pa_decode with a workspace per stream.
 *
 * PA_ERR_WORKSPACE when the call would need more scratch than
 * PA_NOALLOC_SCRATCH_BYTES (pa_decode_workspace_bytes with PA_PARTITION_AUTO
 * gives the need); nothing is enqueued then.  Other errors as for pa_decode.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pa_status pa_decode_noalloc(void *out, const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, const int32_t *context_lens,
                            int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                            int block_size, int max_blocks_per_seq, float scale, pa_dtype dtype, void *stream);

/*
 * pa_decode_ex -- pa_decode with the pool size, the cache layout, the
 * split-K partition and the kernel made explicit.
 *
 *   num_blocks        blocks in the pool; a table entry outside [0, num_blocks)
 *                     contributes no tokens instead of being read
 *   layout            PA_LAYOUT_BHTD or PA_LAYOUT_BTHD
 *   partition_tokens  PA_PARTITION_AUTO (0), PA_PARTITION_SINGLE (-1),
 *                     PA_PARTITION_BALANCED (-2) (above), or N > 0: each
 *                     workgroup reads at most N tokens of one sequence (N a
 *                     multiple of block_size) and a reduce kernel merges the
 *                     partitions' (max, sum, partial output).
 *   kernel            PA_KERNEL_AUTO, PA_KERNEL_VECTOR or PA_KERNEL_MFMA (above)
 *   flags             0 or PA_DECODE_SHARED_BLOCKS (above); other bits are
 *                     PA_ERR_INVALID_ARG
 *
 * Per-block partial results are combined with a running max and sum
 * ("online softmax"); the combine across partitions is the same operation.
 */
pa_status pa_decode_ex(void *out, const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, const int32_t *context_lens,
                       int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                       int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                       pa_dtype dtype, pa_layout layout, int partition_tokens, pa_kernel kernel,
                       unsigned flags, void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_prefill -- paged attention for several query rows per sequence: a
 * prefill chunk, or drafted tokens to verify ("vLLM 与 PagedAttention"
 * section 六, "关键的工程优化": a long prompt's prefill in chunks next to
 * decode; "指南", "Speculative Decoding" and "Chunked Prefill").  The chunk's
 * own K/V rows are appended first (pa_reshape_and_cache); then query row i of
 * a sequence with n rows and context_lens L sits at position L - n + i and
 * attends tokens 0 .. L - n + i of its history (causal).  A row with no token
 * to attend (n > L) is zero.
 *
 *   out, q          [total_q, num_q_heads, head_dim] dtype: the rows of all
 *                   sequences, back to back
 *   query_start     int32 [num_seqs + 1], device: the rows of sequence s are
 *                   q[query_start[s] .. query_start[s + 1]); query_start[0] = 0,
 *                   query_start[num_seqs] = total_q; rows outside
 *                   [0, total_q) are never read or written
 *   max_query_len   the most rows of any sequence (sizes the grid; rows past
 *                   it are not computed)
 *   other arguments as for pa_decode_ex; flags: 0 or PA_DECODE_SHARED_BLOCKS
 *                   (accepted; prefill always loads K/V with the caches'
 *                   normal policy, since every tile is read for many rows)
 *
 * Runs on the matrix cores: f16 or bf16, head_dim 128 or 256, at most 16 q
 * heads per kv head or a multiple of 16; otherwise PA_ERR_UNSUPPORTED.  No
 * workspace.  Errors as for pa_decode_ex.
 */
pa_status pa_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_tables, const int32_t *context_lens, const int32_t *query_start,
                     int num_seqs, int total_q, int max_query_len, int num_q_heads, int num_kv_heads, int head_dim,
                     int block_size, int max_blocks_per_seq, int num_blocks, float scale, pa_dtype dtype,
                     pa_layout layout, unsigned flags, void *stream);

/*
 * pa_prefill_shared_prefix -- pa_prefill for a batch whose block tables all
 * start with the same prefix_blocks physical blocks: requests admitted with
 * automatic prefix caching, which point at the cached blocks of a shared
 * prompt ("vLLM 与 PagedAttention" section 四, the shared system prompt;
 * "指南", "Copy-on-Write：Prefix Caching 的基础").  The same function: row i of
 * sequence s attends tokens 0 .. L - n + i of its own history.  Each sequence
 * first reads its keys past the prefix; then the prefix's K/V are read once
 * for the whole batch -- the rows of every sequence are the columns of one
 * matrix-core pass over them, each capped at its own causal limit -- which
 * merges the two and writes the rows.
 *
 *   prefix_blocks   0 .. max_blocks_per_seq: row 0 of block_tables lists the
 *                   prefix's blocks in its first prefix_blocks entries (those
 *                   are the ones read, whatever context_lens[0] is); in every
 *                   other row, the entries that are both inside the prefix and
 *                   below the row's own block count must be the same blocks
 *   workspace       device memory, 16-byte aligned, at least
 *                   pa_prefill_shared_prefix_workspace_bytes(total_q,
 *                   num_q_heads, head_dim, block_size, prefix_blocks) bytes
 *                   (content on entry does not matter): the partial result
 *                   past the prefix of every (row, q head), (8 + 4 head_dim)
 *                   bytes each; may be null when that size is 0
 *   other arguments as for pa_prefill (no flags)
 *
 * The keys read once for every row are the whole 64-token steps inside the
 * prefix; the rest of the prefix is read per sequence with its own keys.  With
 * a prefix shorter than 64 tokens, or at head_dim 256, it computes exactly as
 * pa_prefill (no workspace).  Errors as for pa_prefill; PA_ERR_INVALID_ARG for
 * prefix_blocks out of range; PA_ERR_WORKSPACE for a missing, short or
 * misaligned workspace.
 */
pa_status pa_prefill_shared_prefix(void *out, const void *q, const void *k_cache, const void *v_cache,
                                   const int32_t *block_tables, const int32_t *context_lens,
                                   const int32_t *query_start, int num_seqs, int total_q, int max_query_len,
                                   int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                   int max_blocks_per_seq, int num_blocks, int prefix_blocks, float scale,
                                   pa_dtype dtype, pa_layout layout, void *workspace, size_t workspace_bytes,
                                   void *stream);
pa_status pa_prefill_shared_prefix_workspace_bytes(int total_q, int num_q_heads, int head_dim, int block_size,
                                                   int prefix_blocks, size_t *bytes_out);

/*
 * pa_decode_shared_prefix -- pa_decode_ex for a batch whose block tables all
 * start with the same prefix_blocks physical blocks (a shared system prompt;
 * requests that point at the same blocks, "vLLM 与 PagedAttention" section
 * 二 and "指南", "Copy-on-Write：Prefix Caching 的基础").  The same function:
 * each sequence attends its own context_lens[s] tokens.  The prefix's K/V
 * are read once for the whole batch -- the sequences' query rows are the
 * columns of one matrix-core pass over them, each seeing the prefix tokens
 * below its own context -- and each sequence's remaining blocks are read as
 * split-K partitions; a reduce merges the two.
 *
 *   prefix_blocks   0 .. max_blocks_per_seq: row 0 of block_tables lists the
 *                   prefix's blocks in its first prefix_blocks entries (those
 *                   are the ones read, whatever context_lens[0] is); in every
 *                   other row, the entries that are both inside the prefix
 *                   and below the row's own block count must be the same
 *                   blocks (a context shorter than the prefix is fine)
 *   workspace       at least pa_decode_shared_prefix_workspace_bytes(...) bytes
 *                   (content on entry does not matter)
 *   other arguments as for pa_decode_ex (no kernel, partition or flags: the
 *   prefix pass runs on the matrix cores, the rest takes the library's choice)
 *
 * Needs f16 or bf16, head_dim 128 or 256 and at most 16 q heads per kv head
 * or a multiple of 16 (PA_ERR_UNSUPPORTED otherwise).  Errors as for
 * pa_decode_ex; PA_ERR_INVALID_ARG for prefix_blocks out of range.
 */
pa_status pa_decode_shared_prefix(void *out, const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                                  int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                  int max_blocks_per_seq, int num_blocks, int prefix_blocks, float scale,
                                  pa_dtype dtype, pa_layout layout, void *workspace, size_t workspace_bytes,
                                  void *stream);
pa_status pa_decode_shared_prefix_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                                  int block_size, int max_blocks_per_seq, pa_dtype dtype,
                                                  int prefix_blocks, size_t *bytes_out);

/*
 * pa_decode_path -- the path pa_decode_ex takes for these sizes, with the
 * automatic choices resolved: *partition_out receives PA_PARTITION_SINGLE,
 * PA_PARTITION_BALANCED or the partition in tokens, *kernel_out
 * PA_KERNEL_VECTOR or PA_KERNEL_MFMA.  Arguments and errors as for
 * pa_decode_ex (PA_ERR_INVALID_ARG for a null output pointer); the automatic
 * partition and the balanced schedule query the current device.  Nothing is
 * launched.
 */
pa_status pa_decode_path(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                         int max_blocks_per_seq, pa_dtype dtype, int partition_tokens, pa_kernel kernel,
                         int *partition_out, pa_kernel *kernel_out);

/*
 * pa_decode_workspace_bytes -- bytes of workspace pa_decode / pa_decode_ex
 * need for these sizes and this partition_tokens (0, -1, -2 or N, as above).
 * Writes 0 when the call runs single pass.  Returns the same status the
 * decode call would return for these sizes.
 */
pa_status pa_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, int max_blocks_per_seq, pa_dtype dtype,
                                    int partition_tokens, size_t *bytes_out);

/*
 * pa_decode_append -- one decode step in one call: append each sequence's new
 * K/V row, then attend ("vLLM 与 PagedAttention" section 二: a step writes its
 * token into the last block, which is taken only when the previous one is
 * full, and attention then reads the whole block chain).  Same result, bit for
 * bit in the pool and within the decode's bounds in out, as
 * pa_reshape_and_cache(k_new, v_new, ..., slot_mapping, num_seqs, ...)
 * followed by pa_decode_ex(...) with the same arguments.
 *
 *   k_new, v_new   [num_seqs, num_kv_heads, head_dim] dtype, contiguous: the
 *                  new row of sequence s is token s
 *   k_cache,
 *   v_cache        written at the mapped slots, then read
 *   slot_mapping   [num_seqs] int64: sequence s's new row goes to slot
 *                  slot_mapping[s] (skipped when negative or past the pool)
 *   other arguments as for pa_decode_ex; context_lens count the new token
 *
 * The append kernel is enqueued ahead of the decode, with every argument
 * checked before either: an argument error enqueues neither step.  A launch
 * failure of the decode (PA_ERR_HIP) comes after the append was enqueued,
 * so the pool may already hold the new rows then.  (Folding the append into the decode
 * kernel -- the new row taken from registers where the step reads it --
 * measured no faster on MI355X: 189.9 against 190.5 us per 7B-shaped step,
 * 386.3 against 377.1 us on the mixed batch.)
 */
pa_status pa_decode_append(void *out, const void *q, const void *k_new, const void *v_new, void *k_cache,
                           void *v_cache, const int64_t *slot_mapping, const int32_t *block_tables,
                           const int32_t *context_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                           int head_dim, int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                           pa_dtype dtype, pa_layout layout, int partition_tokens, pa_kernel kernel,
                           unsigned flags, void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_reshape_and_cache -- append new K/V rows into the pool.
 *
 *   k, v           [num_tokens, num_kv_heads, head_dim] dtype, contiguous
 *   k_cache,
 *   v_cache        pool in `layout`, [num_blocks, ...] as above
 *   slot_mapping   [num_tokens] int64; token i goes to physical block
 *                  slot / block_size at offset slot % block_size; a negative
 *                  slot skips the token, a slot >= num_blocks*block_size is
 *                  skipped as well (never written)
 *
 * Elements are copied bit for bit.  Two tokens with the same slot: one of
 * them wins, which one is unspecified.
 */
pa_status pa_reshape_and_cache(const void *k, const void *v, void *k_cache, void *v_cache,
                               const int64_t *slot_mapping, int num_tokens, int num_kv_heads,
                               int head_dim, int block_size, int num_blocks, pa_dtype dtype,
                               pa_layout layout, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *pa_status_string(pa_status status);

/* Version of this interface (major * 100 + minor). */
int pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_MI355X_PA_H_ */
