// pa_append.hip -- reshape_and_cache: copy each new token's K and V rows into
// its slot of the paged pool, bit for bit.
//
// Method: "vLLM 与 PagedAttention" (inference.mavenzero.com/case-studies/vllm),
// section 二, sub-section "PagedAttention 的解法": a sequence grows into its
// last block and takes a new physical block only when that one is full; the
// caller encodes the destination as slot = physical_block * block_size + offset.
//
// One workgroup per token; each thread moves 16-byte chunks of the token's
// Hkv x head_dim rows for K and for V.  Invalid slots (negative, or past the
// pool) are skipped, so a bad slot can never write outside the pool.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void append_kernel(const AppendParams A)
{
    const int i = blockIdx.x;
    const int64_t slot = A.slots[i];
    if (slot < 0 || slot >= A.num_slots)
        return;
    const int64_t b = slot / A.block_size;
    const int64_t off = slot - b * A.block_size;
    const int per_tensor = A.num_kv_heads * A.chunks_per_head;
    const int64_t row_bytes = (int64_t)A.chunks_per_head * 16;
    for (int c = threadIdx.x; c < 2 * per_tensor; c += blockDim.x) {
        const bool is_v = c >= per_tensor;
        const int cc = is_v ? c - per_tensor : c;
        const int g = cc / A.chunks_per_head;
        const int ch = cc - g * A.chunks_per_head;
        const char *src = static_cast<const char *>(is_v ? A.v : A.k) +
                          ((int64_t)i * A.num_kv_heads + g) * row_bytes + ch * 16;
        char *dst = static_cast<char *>(is_v ? A.v_cache : A.k_cache) +
                    (b * A.block_stride + g * A.head_stride + off * A.token_stride) * A.elem_bytes + ch * 16;
        st16(dst, ld16(src));
    }
}

hipError_t launch_append(const AppendParams &p, hipStream_t st)
{
    const int per_token = 2 * p.num_kv_heads * p.chunks_per_head;
    const int threads = per_token >= 256 ? 256 : ((per_token + 63) / 64) * 64;
    hipLaunchKernelGGL(append_kernel, dim3(p.num_tokens), dim3(threads), 0, st, p);
    return hipGetLastError();
}

}  // namespace pa
