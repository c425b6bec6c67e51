/*
 * pa_blocks.h -- the paging system around the decode kernel: block copies
 * (copy on write, swapping to and from CPU memory) and a host block manager
 * that hands out blocks, keeps reference counts and produces block tables and
 * slots.
 *
 * What these calls implement comes from the pages:
 *   - "vLLM 与 PagedAttention" (inference.mavenzero.com/case-studies/vllm),
 *     section 二 "PagedAttention 的解法": a request's KV sits in fixed-size
 *     blocks of one shared pool, reached through its table; a block is taken
 *     only when the request's last block is full; requests with a common
 *     prefix point at the same physical blocks, copied on write.
 *   - "指南" (illegalscreed.cn .../vllm/guide-line), "Copy-on-Write：Prefix
 *     Caching 的基础": shared blocks are read-only; a request copies one only
 *     when it diverges.
 *   - "4. vLLM初识" (5688vip.com .../04.html) 4.3 and "vLLM 与 PagedAttention"
 *     section 三: under memory pressure a request's KV moves out to CPU memory
 *     and comes back later.
 *   - "vLLM让大模型推理快10倍？PagedAttention原理详解与实战部署" (298.name/post/186.html),
 *     "PagedAttention怎么解决？": one table per request maps logical pages to
 *     physical pages, allocated on demand (50 tokens at 16 per page: 4 pages).
 *
 * A block is the run of block_size * num_kv_heads * head_dim elements that
 * one pool index covers; both cache layouts of pa.h keep a block contiguous,
 * so the copies below do not depend on the layout.
 */
#ifndef PA_BLOCKS_H
#define PA_BLOCKS_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pa_copy_blocks -- copy on write inside one pool pair: for each i, block
 * pairs[2i + 1] of k_cache and of v_cache takes the contents of block
 * pairs[2i] (bit for bit).
 *
 *   k_cache, v_cache  the pools, [num_blocks, ...] in either pa.h layout
 *                     (device memory, 16-byte aligned)
 *   pairs             int32 [num_pairs][2] (source, destination), device-
 *                     accessible memory; a pair with an index outside
 *                     [0, num_blocks) is skipped
 *   num_pairs         0 is a no-op
 *
 * The destinations must be distinct and none may also be a source of the
 * same call (the block manager's copies are: a copy always goes to a freshly
 * taken block).  Enqueued on `stream`; returns before the copy is done.
 * Errors: PA_ERR_INVALID_ARG for a null or misaligned pointer or a negative
 * count, PA_ERR_UNSUPPORTED for a head_dim / block_size / dtype outside the
 * sets of pa.h, PA_ERR_HIP if the launch fails.
 */
pa_status pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs, int num_pairs, int num_blocks,
                         int block_size, int num_kv_heads, int head_dim, pa_dtype dtype, void *stream);

/*
 * pa_swap_blocks -- move blocks between two pool pairs (GPU <-> CPU): for
 * each i, block pairs[2i + 1] of (dst_k, dst_v) takes block pairs[2i] of
 * (src_k, src_v).
 *
 * Either pool pair may be device memory or pinned host memory that the
 * device can address (hipHostMalloc, or torch's pin_memory); one kernel
 * moves every block of the call over the host link.  pairs must be device-
 * accessible too.  Each pointer is looked up first
 * (hipPointerGetAttributes): memory the device cannot reach (pageable host
 * memory) is PA_ERR_INVALID_ARG, before anything is launched.  A pair with
 * an index outside [0, num_src_blocks) or [0, num_dst_blocks) is skipped.
 * Destinations must be distinct.  Sizes, alignment and errors as for
 * pa_copy_blocks.
 */
pa_status pa_swap_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v, const int32_t *pairs,
                         int num_pairs, int num_dst_blocks, int num_src_blocks, int block_size, int num_kv_heads,
                         int head_dim, pa_dtype dtype, void *stream);

/*
 * The host block manager: a GPU pool of num_gpu_blocks blocks and a CPU
 * pool of num_cpu_blocks blocks of block_size tokens, the table and length
 * of every request (identified by any 64-bit id), and a reference count per
 * block.  Host memory only; it launches nothing.  The caller moves the data
 * it asks for: copies with pa_copy_blocks, swaps with pa_swap_blocks, new
 * tokens with pa_reshape_and_cache at the slots it returns.
 *
 * Rules (readings where the pages are silent are marked *):
 *   - a request takes a block only when its last block is full;
 *   - * the lowest-numbered free block is taken first;
 *   - a forked request shares all its parent's blocks; a request that
 *     appends into a shared, partly filled last block first gets a private
 *     copy of it (one (source, destination) pair to copy);
 *   - * a block returns to its pool when no request holds it (a block in
 *     the prefix cache stays cached until it is taken, see below);
 *   - * swapping out gives a request CPU copies of all its blocks (a GPU
 *     block that other requests hold stays on the GPU for them); swapping in
 *     gives it fresh GPU blocks;
 *   - * an operation that needs more free blocks than its pool has changes
 *     nothing and returns PA_ERR_NO_BLOCKS.
 * Other errors: PA_ERR_INVALID_ARG (null handle or output, unknown or
 * duplicate request id, a request in the wrong pool for the operation,
 * negative counts, an output array too small).  One manager may be used
 * from several threads; each call holds the manager's lock.
 */
typedef struct pa_block_manager pa_block_manager;

pa_status pa_bm_create(int num_gpu_blocks, int num_cpu_blocks, int block_size, pa_block_manager **out);
void pa_bm_destroy(pa_block_manager *bm);

/* a new, empty request on the GPU */
pa_status pa_bm_add(pa_block_manager *bm, int64_t seq);
/* child (a new id) reads all of parent's blocks, shared; parent on the GPU */
pa_status pa_bm_fork(pa_block_manager *bm, int64_t parent, int64_t child);
/* free GPU blocks an append of n tokens to seq would take (new blocks plus a copy) */
pa_status pa_bm_blocks_needed(pa_block_manager *bm, int64_t seq, int n, int *out);
/*
 * Grow seq (on the GPU) by n tokens.  slots[n] receives each new token's slot
 * (physical block * block_size + offset) for pa_reshape_and_cache; copies
 * receives up to max_copies (source, destination) int32 pairs to run through
 * pa_copy_blocks before those writes (an append makes at most one), and
 * *num_copies their count.
 */
pa_status pa_bm_append(pa_block_manager *bm, int64_t seq, int n, int64_t *slots, int32_t *copies, int max_copies,
                       int *num_copies);
/* drop a request; its blocks return to their pool when no one else holds them */
pa_status pa_bm_free(pa_block_manager *bm, int64_t seq);
/*
 * Move seq to CPU blocks (pa_bm_swap_out: (gpu block, cpu block) pairs for
 * pa_swap_blocks from the GPU pools to the CPU pools) or back to fresh GPU
 * blocks (pa_bm_swap_in: (cpu block, gpu block) pairs).  pairs holds up to
 * max_pairs pairs; *num_pairs receives the count (the request's block count).
 */
pa_status pa_bm_swap_out(pa_block_manager *bm, int64_t seq, int32_t *pairs, int max_pairs, int *num_pairs);
pa_status pa_bm_swap_in(pa_block_manager *bm, int64_t seq, int32_t *pairs, int max_pairs, int *num_pairs);
/*
 * Block tables and context lengths of n requests (all on the GPU), as
 * pa_decode takes them: tables int32 [n][max_blocks] row-major, -1 past each
 * request's last block; context_lens int32 [n].  Host arrays.
 */
pa_status pa_bm_block_tables(pa_block_manager *bm, const int64_t *seqs, int n, int max_blocks, int32_t *tables,
                             int32_t *context_lens);
/*
 * Automatic prefix caching ("vLLM 与 PagedAttention" section 四, "Prefix
 * Caching：复用 system prompt 的 KV"): the KV of a prompt's prefix stays
 * cached, and a later request whose prompt starts the same way reuses it and
 * computes only the rest.  Readings where the pages are silent:
 *   - the unit is a full block, known by its whole token prefix (a block's
 *     chain hash covers every token before it; a hit also checks the
 *     block's own tokens and its parent's hash); partly filled blocks are
 *     never cached;
 *   - a full block joins the cache as soon as its request has all its tokens
 *     (pa_bm_append_tokens; the caller writes their KV with
 *     pa_reshape_and_cache before another request looks the prompt up); if
 *     that prefix is cached already, the block stays private;
 *   - a cached block that no request holds stays cached and counts as free:
 *     an allocation takes a free block if there is one, else the cached
 *     block released longest ago (ties: lowest index), which leaves the
 *     cache; a request's blocks are released last block first;
 *   - a request whose tokens were not all given (pa_bm_append) adds nothing
 *     to the cache from then on.
 */
/*
 * A new request (a new id) for prompt[n]: its table starts with the cached
 * blocks the prompt begins with -- at most (n - 1) / block_size of them, so at
 * least one prompt token is left to compute -- and *cached_tokens receives
 * how many tokens that covers (a multiple of block_size).  The caller then
 * appends the rest of the prompt with pa_bm_append_tokens and computes it.
 */
pa_status pa_bm_add_cached(pa_block_manager *bm, int64_t seq, const int32_t *prompt, int n, int *cached_tokens);
/* pa_bm_append, with the tokens given (int32 [n], host), so that the blocks they fill can be cached */
pa_status pa_bm_append_tokens(pa_block_manager *bm, int64_t seq, const int32_t *tokens, int n, int64_t *slots,
                              int32_t *copies, int max_copies, int *num_copies);
/* GPU blocks in the prefix cache, and how many of them no request holds */
pa_status pa_bm_cache_stats(pa_block_manager *bm, int *cached_blocks, int *evictable_blocks);

/* blocks an allocation from a pool (0 = GPU, 1 = CPU) can take: free ones and,
 * on the GPU, cached ones no request holds */
pa_status pa_bm_num_free(pa_block_manager *bm, int pool, int *out);
/* requests holding a block of a pool (0 = GPU, 1 = CPU) */
pa_status pa_bm_ref_count(pa_block_manager *bm, int pool, int block, int *out);
/* tokens and blocks of a request, and whether it is on the GPU (1) or the CPU (0) */
pa_status pa_bm_info(pa_block_manager *bm, int64_t seq, int64_t *num_tokens, int *num_blocks, int *on_gpu);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H */
