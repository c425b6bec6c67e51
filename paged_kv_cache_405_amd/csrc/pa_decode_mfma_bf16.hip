// pa_decode_mfma_bf16.hip -- instantiates the grouped-query (matrix core) decode
// kernels for bf16 storage.
#include "pa_decode_mfma.h"
#include "pa_internal.h"

namespace pa {

hipError_t launch_mfma_bf16(const DecodeParams &p, int head_dim, int block_size, hipStream_t st)
{
    return launch_mfma_dtype<bf16_t>(p, head_dim, block_size, st);
}

hipError_t stream_mfma_bf16(const DecodeParams *p, int head_dim, int block_size, hipStream_t st, int *occ)
{
    return mfma_stream_dtype<bf16_t>(p, head_dim, block_size, st, occ);
}

}  // namespace pa
