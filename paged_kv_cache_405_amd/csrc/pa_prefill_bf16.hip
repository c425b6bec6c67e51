// pa_prefill_bf16.hip -- multi-token paged attention instances for bf16.
#include "pa_internal.h"
#include "pa_prefill.h"

namespace pa {

hipError_t launch_prefill_bf16(const DecodeParams &p, int head_dim, int block_size, int max_query_len, hipStream_t st)
{
    return launch_prefill_dtype<bf16_t>(p, head_dim, block_size, max_query_len, st);
}

hipError_t launch_prefill_shared_bf16(const DecodeParams &p, int block_size, int max_query_len, hipStream_t st)
{
    return launch_prefill_shared_bs<bf16_t>(p, block_size, max_query_len, st);
}

hipError_t launch_prefix_bf16(const DecodeParams &p, int head_dim, int block_size, int prefix_tokens, int chunk,
                              hipStream_t st)
{
    return launch_prefix_dtype<bf16_t>(p, head_dim, block_size, prefix_tokens, chunk, st);
}

}  // namespace pa
