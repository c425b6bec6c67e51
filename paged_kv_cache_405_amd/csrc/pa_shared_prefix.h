// pa_shared_prefix.h -- the two passes of a shared-prefix decode in one launch.
//
// Method: "vLLM 与 PagedAttention" (inference.mavenzero.com/case-studies/vllm),
// section 二: sequences that share a prompt point at the same physical
// blocks (copy-on-write), and attention reads K/V block by block and merges
// the per-block results; "指南" ("Copy-on-Write：Prefix Caching 的基础").
//
// pa_decode_shared_prefix reads the prefix's K/V once for the whole batch (the
// prefix pass: its chunks become split-K partitions 0 .. n_chunks - 1 of every
// (sequence, q head)) and each sequence's own blocks as the partitions after
// them; the split-K reduce then merges all of them.  The two passes read and
// write disjoint data, so they need no order between them.  Launched one after
// the other, the prefix pass -- a few hundred workgroups doing a short,
// latency-bound walk over the prefix -- leaves most of the chip idle while it
// runs.  Here one grid holds both: its first workgroups run the prefix pass
// (4-wave workgroups of the same staged-tile worker), the rest run the
// own-blocks pass -- of the vector decode kernel, or of the matrix-core grid
// kernel for grouped heads -- and the hardware fills the chip with whichever
// are ready.
#pragma once

#include "pa_decode_mfma.h"
#include "pa_decode_vec.h"
#include "pa_prefill.h"

namespace pa {

constexpr int SHARED_PREFIX_WAVES = 4;   // waves per workgroup, in both passes

// blocks [0, n_prefix_grid): the prefix pass over PX (n_prefix of them real,
// XCD-major as in prefix_kernel); blocks after: the own-blocks pass over P,
// block b - n_prefix_grid being (partition, head group, row) with the
// partition fastest, as in a launch of decode_vec_kernel of its own
template <typename T, int D, int BS, int GT>
__global__ __launch_bounds__(SHARED_PREFIX_WAVES * 64) void shared_prefix_kernel(
    const DecodeParams P, const DecodeParams PX, int n_prefix, int n_prefix_grid, int col_groups, int n_chunks,
    int prefix_tokens, int chunk, int own_x, int own_y)
{
    const int b = blockIdx.x;
    if (b < n_prefix_grid) {
        const int lg_id = (b & 7) * (n_prefix_grid >> 3) + (b >> 3);
        if (lg_id < n_prefix) {
            __shared__ __attribute__((aligned(16)))
            unsigned char lds[prefix_block_lds<T, D, BS, SHARED_PREFIX_WAVES>()];
            prefix_block<T, D, BS, SHARED_PREFIX_WAVES>(PX, lg_id, col_groups, n_chunks, prefix_tokens, chunk,
                                                        (unsigned char PA_LDS *)lds);
        }
        return;
    }
    const int o = b - n_prefix_grid;
    // the sequences' own blocks are private: K/V with the read-once hint
    decode_vec_block<T, D, BS, GT, SHARED_PREFIX_WAVES, true>(P, o % own_x, (o / own_x) % own_y, o / (own_x * own_y));
}

// the same with the own blocks on the matrix cores (grouped-query heads): the
// grid decode kernel's workgroup (pa_decode_mfma.h) instead of the vector one
template <typename T, int D, int BS>
__global__ __launch_bounds__(SHARED_PREFIX_WAVES * 64) void shared_prefix_mfma_kernel(
    const DecodeParams P, const DecodeParams PX, int n_prefix, int n_prefix_grid, int col_groups, int n_chunks,
    int prefix_tokens, int chunk, int own_x, int own_y)
{
    // a workgroup runs one of the two passes: one LDS area serves either
    constexpr int LP = prefix_block_lds<T, D, BS, SHARED_PREFIX_WAVES>();
    constexpr int LO = decode_mfma_lds<T, D, BS, SHARED_PREFIX_WAVES, true>();
    __shared__ __attribute__((aligned(16))) unsigned char lds[LP > LO ? LP : LO];
    const int b = blockIdx.x;
    if (b < n_prefix_grid) {
        const int lg_id = (b & 7) * (n_prefix_grid >> 3) + (b >> 3);
        if (lg_id < n_prefix)
            prefix_block<T, D, BS, SHARED_PREFIX_WAVES>(PX, lg_id, col_groups, n_chunks, prefix_tokens, chunk,
                                                        (unsigned char PA_LDS *)lds);
        return;
    }
    const int o = b - n_prefix_grid;
    decode_mfma_block<T, D, BS, SHARED_PREFIX_WAVES, true>(P, o % own_x, (o / own_x) % own_y, o / (own_x * own_y),
                                                           (unsigned char PA_LDS *)lds);
}

// GT: q heads per workgroup of the vector own-blocks pass (1 or 2), or 0 for
// the matrix-core own-blocks pass
template <typename T, int D, int BS, int GT>
hipError_t launch_shared_prefix_shape(const DecodeParams &own, const DecodeParams &px, int prefix_tokens, int chunk,
                                      hipStream_t st)
{
    if (chunk <= 0 || chunk % (2 * GQA_TILE) != 0)
        return hipErrorInvalidValue;
    const int rows = GQA_TILE / (px.group / px.group_split);
    const int col_tiles = (px.num_seqs + rows - 1) / rows;
    const int col_groups = (col_tiles + SHARED_PREFIX_WAVES - 1) / SHARED_PREFIX_WAVES;
    const int n_chunks = (prefix_tokens + chunk - 1) / chunk;
    if (n_chunks != px.first_partition || n_chunks != own.first_partition)
        return hipErrorInvalidValue;
    const long long n_prefix = (long long)col_groups * n_chunks * px.num_kv_heads * px.group_split;
    const long long n_prefix_grid = (n_prefix + 7) / 8 * 8;
    const long long own_x = own.max_partitions - own.first_partition;
    const long long own_y = (long long)own.num_kv_heads * own.group_split;
    const long long total = n_prefix_grid + own_x * own_y * own.num_seqs;
    if (own_x <= 0 || total > (1LL << 30))
        return hipErrorInvalidValue;
    if constexpr (GT == 0)
        hipLaunchKernelGGL((shared_prefix_mfma_kernel<T, D, BS>), dim3((unsigned)total),
                           dim3(SHARED_PREFIX_WAVES * 64), 0, st, own, px, (int)n_prefix, (int)n_prefix_grid,
                           col_groups, n_chunks, prefix_tokens, chunk, (int)own_x, (int)own_y);
    else
        hipLaunchKernelGGL((shared_prefix_kernel<T, D, BS, GT>), dim3((unsigned)total),
                           dim3(SHARED_PREFIX_WAVES * 64), 0, st, own, px, (int)n_prefix, (int)n_prefix_grid,
                           col_groups, n_chunks, prefix_tokens, chunk, (int)own_x, (int)own_y);
    return hipGetLastError();
}

template <typename T, int D, int BS>
hipError_t launch_shared_prefix_gt(const DecodeParams &own, const DecodeParams &px, int gt, int prefix_tokens,
                                   int chunk, hipStream_t st)
{
    switch (gt) {
    case 0: return launch_shared_prefix_shape<T, D, BS, 0>(own, px, prefix_tokens, chunk, st);
    case 1: return launch_shared_prefix_shape<T, D, BS, 1>(own, px, prefix_tokens, chunk, st);
    case 2: return launch_shared_prefix_shape<T, D, BS, 2>(own, px, prefix_tokens, chunk, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_shared_prefix_dtype(const DecodeParams &own, const DecodeParams &px, int head_dim, int bs, int gt,
                                      int prefix_tokens, int chunk, hipStream_t st)
{
    switch (head_dim * 64 + bs) {
    case 128 * 64 + 8: return launch_shared_prefix_gt<T, 128, 8>(own, px, gt, prefix_tokens, chunk, st);
    case 128 * 64 + 16: return launch_shared_prefix_gt<T, 128, 16>(own, px, gt, prefix_tokens, chunk, st);
    case 128 * 64 + 32: return launch_shared_prefix_gt<T, 128, 32>(own, px, gt, prefix_tokens, chunk, st);
    case 256 * 64 + 8: return launch_shared_prefix_gt<T, 256, 8>(own, px, gt, prefix_tokens, chunk, st);
    case 256 * 64 + 16: return launch_shared_prefix_gt<T, 256, 16>(own, px, gt, prefix_tokens, chunk, st);
    case 256 * 64 + 32: return launch_shared_prefix_gt<T, 256, 32>(own, px, gt, prefix_tokens, chunk, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
