// pa_blocks.hip -- whole-block copies: copy on write inside a pool pair, and
// swapping between a GPU pool pair and a CPU one.
//
// Method: "vLLM 与 PagedAttention" (inference.mavenzero.com/case-studies/vllm),
// section 二 "PagedAttention 的解法": requests with a common prefix share
// physical blocks and copy one when they diverge (copy on write); section 三
// and "4. vLLM初识" 4.3: a preempted request's KV moves to CPU memory and back.
//
// A block is one contiguous run of block_bytes in both cache layouts, so a
// copy is a plain 16-byte-chunk move.  Grid x walks the pairs, grid y the
// 4 KiB pieces of a block (one 16-byte load and store per thread each), so a
// call with many pairs fills the device; K and V pieces alternate in y.  The
// source is read once: its loads carry the non-temporal hint.  Pool pointers
// may address device memory or device-mapped pinned host memory: the same
// loads and stores reach either.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int COPY_THREADS = 256;
constexpr int COPY_PIECE = COPY_THREADS * 16;   // bytes one workgroup moves per block piece

__global__ __launch_bounds__(COPY_THREADS) void copy_blocks_kernel(const CopyParams C)
{
    const int i = blockIdx.x;
    const int32_t src = C.pairs[2 * i];
    const int32_t dst = C.pairs[2 * i + 1];
    if (src < 0 || src >= C.num_src_blocks || dst < 0 || dst >= C.num_dst_blocks)
        return;
    const int pieces = (int)((C.block_bytes + COPY_PIECE - 1) / COPY_PIECE);
    for (int y = blockIdx.y; y < 2 * pieces; y += gridDim.y) {
        const bool is_v = y >= pieces;
        const int64_t off = (int64_t)(is_v ? y - pieces : y) * COPY_PIECE + threadIdx.x * 16;
        if (off >= C.block_bytes)
            continue;
        const char *s = static_cast<const char *>(is_v ? C.src_v : C.src_k) + (int64_t)src * C.block_bytes + off;
        char *d = static_cast<char *>(is_v ? C.dst_v : C.dst_k) + (int64_t)dst * C.block_bytes + off;
        st16(d, ld16_kv<true>(s));
    }
}

hipError_t launch_copy_blocks(const CopyParams &p, hipStream_t st)
{
    const int pieces = (int)((p.block_bytes + COPY_PIECE - 1) / COPY_PIECE);
    const int gy = 2 * pieces < 64 ? 2 * pieces : 64;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(p.num_pairs, gy), dim3(COPY_THREADS), 0, st, p);
    return hipGetLastError();
}

}  // namespace pa
