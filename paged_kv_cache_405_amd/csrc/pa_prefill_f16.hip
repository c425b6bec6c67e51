// pa_prefill_f16.hip -- multi-token paged attention instances for f16.
#include "pa_internal.h"
#include "pa_prefill.h"

namespace pa {

hipError_t launch_prefill_f16(const DecodeParams &p, int head_dim, int block_size, int max_query_len, hipStream_t st)
{
    return launch_prefill_dtype<f16_t>(p, head_dim, block_size, max_query_len, st);
}

hipError_t launch_prefill_shared_f16(const DecodeParams &p, int block_size, int max_query_len, hipStream_t st)
{
    return launch_prefill_shared_bs<f16_t>(p, block_size, max_query_len, st);
}

hipError_t launch_prefix_f16(const DecodeParams &p, int head_dim, int block_size, int prefix_tokens, int chunk,
                             hipStream_t st)
{
    return launch_prefix_dtype<f16_t>(p, head_dim, block_size, prefix_tokens, chunk, st);
}

int prefix_workgroups(int num_seqs, int group, int group_split, int num_kv_heads)
{
    return prefix_workgroups_per_chunk(num_seqs, group, group_split, num_kv_heads);
}

}  // namespace pa
