// pa_shared_prefix_bf16.hip -- the combined shared-prefix launch, bf16 instances.
#include "pa_internal.h"
#include "pa_shared_prefix.h"

namespace pa {

hipError_t launch_shared_prefix_bf16(const DecodeParams &own, const DecodeParams &prefix, int head_dim, int block_size,
                                   int gt, int prefix_tokens, int chunk, hipStream_t st)
{
    return launch_shared_prefix_dtype<bf16_t>(own, prefix, head_dim, block_size, gt, prefix_tokens, chunk, st);
}

}  // namespace pa
