// pa_internal.h -- launchers shared between the C ABI (pa_api.hip) and the
// kernel translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"

namespace pa {

enum DType { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// Vector-path decode (any q-head group size; `gt` q heads per workgroup) and
// the split-K reduce.  Each returns hipSuccess or the launch error.
hipError_t launch_decode_f32(const DecodeParams &p, int head_dim, int block_size, int gt, hipStream_t st);
hipError_t launch_decode_f16(const DecodeParams &p, int head_dim, int block_size, int gt, hipStream_t st);
hipError_t launch_decode_bf16(const DecodeParams &p, int head_dim, int block_size, int gt, hipStream_t st);
// Grouped-query decode on the matrix cores: f16 / bf16, head_dim 128 or 256,
// at most 16 q heads per workgroup (group / group_split).
hipError_t launch_mfma_f16(const DecodeParams &p, int head_dim, int block_size, hipStream_t st);
hipError_t launch_mfma_bf16(const DecodeParams &p, int head_dim, int block_size, hipStream_t st);
hipError_t launch_reduce(const DecodeParams &p, int dtype, int head_dim, int block_size, hipStream_t st);
// Balanced (stream) schedule.  With occ == nullptr: launch the stream kernel
// for this shape on st.  With occ != nullptr: store the workgroups (one wave
// each) of that kernel that one compute unit holds at once, launch nothing.
hipError_t stream_vec_f32(const DecodeParams *p, int head_dim, int block_size, int gt, hipStream_t st, int *occ);
hipError_t stream_vec_f16(const DecodeParams *p, int head_dim, int block_size, int gt, hipStream_t st, int *occ);
hipError_t stream_vec_bf16(const DecodeParams *p, int head_dim, int block_size, int gt, hipStream_t st, int *occ);
hipError_t stream_mfma_f16(const DecodeParams *p, int head_dim, int block_size, hipStream_t st, int *occ);
hipError_t stream_mfma_bf16(const DecodeParams *p, int head_dim, int block_size, hipStream_t st, int *occ);
// merge the pieces the stream kernel left (one workgroup per unit)
hipError_t launch_stream_reduce(const DecodeParams &p, int dtype, int head_dim, int heads_per_unit, hipStream_t st);
hipError_t launch_append(const AppendParams &p, hipStream_t st);
hipError_t launch_copy_blocks(const CopyParams &p, hipStream_t st);
// multi-token paged attention on the matrix cores (f16 / bf16, head_dim 128 or 256)
hipError_t launch_prefill_f16(const DecodeParams &p, int head_dim, int block_size, int max_query_len, hipStream_t st);
hipError_t launch_prefill_bf16(const DecodeParams &p, int head_dim, int block_size, int max_query_len, hipStream_t st);
// the shared-prefix form of it at head_dim 128: the prefix's keys (p.part_base_blocks blocks of table row 0)
// for the rows of every sequence at once, partials to p.ws_ml / p.ws_acc; then each sequence's own keys,
// merged with those partials
hipError_t launch_prefill_shared_f16(const DecodeParams &p, int block_size, int max_query_len, hipStream_t st);
hipError_t launch_prefill_shared_bf16(const DecodeParams &p, int block_size, int max_query_len, hipStream_t st);
// shared-prefix decode, first pass: the prefix's split-K partitions 0 .. first_partition - 1,
// one per chunk of the prefix; a chunk is a multiple of 32 tokens in [SHARED_PREFIX_CHUNK_MIN,
// SHARED_PREFIX_CHUNK_MAX], chosen per call
constexpr int SHARED_PREFIX_CHUNK_MIN = 128;
constexpr int SHARED_PREFIX_CHUNK_MAX = 512;
constexpr int SHARED_PREFIX_SUFFIX_PARTITION = 512;   // tokens per split-K partition after the prefix
hipError_t launch_prefix_f16(const DecodeParams &p, int head_dim, int block_size, int prefix_tokens, int chunk,
                             hipStream_t st);
hipError_t launch_prefix_bf16(const DecodeParams &p, int head_dim, int block_size, int prefix_tokens, int chunk,
                              hipStream_t st);
// workgroups the prefix pass starts per chunk of the prefix
int prefix_workgroups(int num_seqs, int group, int group_split, int num_kv_heads);
// both passes of a shared-prefix decode in one launch (pa_shared_prefix.h):
// `own` the own-blocks pass's parameters (`gt` q heads per workgroup of the
// vector kernel, 1 or 2, or 0 for the matrix-core kernel), `prefix` the prefix
// pass's; f16 / bf16, head_dim 128 or 256
hipError_t launch_shared_prefix_f16(const DecodeParams &own, const DecodeParams &prefix, int head_dim, int block_size,
                                    int gt, int prefix_tokens, int chunk, hipStream_t st);
hipError_t launch_shared_prefix_bf16(const DecodeParams &own, const DecodeParams &prefix, int head_dim, int block_size,
                                     int gt, int prefix_tokens, int chunk, hipStream_t st);

}  // namespace pa
