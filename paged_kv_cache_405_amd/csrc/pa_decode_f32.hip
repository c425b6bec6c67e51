// pa_decode_f32.hip -- instantiates the vector-path decode kernels for f32
// storage (one translation unit per element type keeps builds parallel).
#include "pa_decode_vec.h"
#include "pa_internal.h"

namespace pa {

hipError_t launch_decode_f32(const DecodeParams &p, int head_dim, int block_size, int gt, hipStream_t st)
{
    return launch_decode_dtype<f32_t>(p, head_dim, block_size, gt, st);
}

hipError_t stream_vec_f32(const DecodeParams *p, int head_dim, int block_size, int gt, hipStream_t st, int *occ)
{
    return vec_stream_dtype<f32_t>(p, head_dim, block_size, gt, st, occ);
}

}  // namespace pa
