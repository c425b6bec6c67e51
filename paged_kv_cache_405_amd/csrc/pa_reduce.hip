// pa_reduce.hip -- instantiates the split-K reduce kernel (one wave per
// (q head, sequence)) for every element type, head_dim and block_size.
#include "pa_decode_vec.h"
#include "pa_stream.h"
#include "pa_internal.h"

namespace pa {

template <typename T, int D>
static hipError_t launch_reduce_d(const DecodeParams &p, int bs, hipStream_t st)
{
    dim3 grid(p.num_q_heads, p.num_seqs);
    switch (bs) {
    case 8: hipLaunchKernelGGL((reduce_kernel<T, D, 8>), grid, dim3(64), 0, st, p); break;
    case 16: hipLaunchKernelGGL((reduce_kernel<T, D, 16>), grid, dim3(64), 0, st, p); break;
    case 32: hipLaunchKernelGGL((reduce_kernel<T, D, 32>), grid, dim3(64), 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_reduce_t(const DecodeParams &p, int head_dim, int bs, hipStream_t st)
{
    switch (head_dim) {
    case 32: return launch_reduce_d<T, 32>(p, bs, st);
    case 64: return launch_reduce_d<T, 64>(p, bs, st);
    case 128: return launch_reduce_d<T, 128>(p, bs, st);
    case 256: return launch_reduce_d<T, 256>(p, bs, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reduce(const DecodeParams &p, int dtype, int head_dim, int block_size, hipStream_t st)
{
    switch (dtype) {
    case DT_F32: return launch_reduce_t<f32_t>(p, head_dim, block_size, st);
    case DT_F16: return launch_reduce_t<f16_t>(p, head_dim, block_size, st);
    case DT_BF16: return launch_reduce_t<bf16_t>(p, head_dim, block_size, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t launch_stream_reduce_t(const DecodeParams &p, int head_dim, int heads_per_unit, hipStream_t st)
{
    if (heads_per_unit < 1 || heads_per_unit > 65535)
        return hipErrorInvalidValue;
    dim3 grid(p.num_seqs, p.num_kv_heads * p.group_split, heads_per_unit);
    switch (head_dim) {
    case 32: hipLaunchKernelGGL((stream_reduce_kernel<T, 32>), grid, dim3(64), 0, st, p, heads_per_unit); break;
    case 64: hipLaunchKernelGGL((stream_reduce_kernel<T, 64>), grid, dim3(64), 0, st, p, heads_per_unit); break;
    case 128: hipLaunchKernelGGL((stream_reduce_kernel<T, 128>), grid, dim3(64), 0, st, p, heads_per_unit); break;
    case 256: hipLaunchKernelGGL((stream_reduce_kernel<T, 256>), grid, dim3(64), 0, st, p, heads_per_unit); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_stream_reduce(const DecodeParams &p, int dtype, int head_dim, int heads_per_unit, hipStream_t st)
{
    switch (dtype) {
    case DT_F32: return launch_stream_reduce_t<f32_t>(p, head_dim, heads_per_unit, st);
    case DT_F16: return launch_stream_reduce_t<f16_t>(p, head_dim, heads_per_unit, st);
    case DT_BF16: return launch_stream_reduce_t<bf16_t>(p, head_dim, heads_per_unit, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
