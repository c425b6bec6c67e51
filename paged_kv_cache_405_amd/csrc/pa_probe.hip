// pa_probe.hip -- a streaming-read probe: how fast this GPU reads a large
// buffer from HBM, the bound the decode kernels are measured against.
//
// Decode attention is bound by memory bandwidth ("vLLM 与 PagedAttention"
// (inference.mavenzero.com/case-studies/vllm), section 一: each generated
// token re-reads the whole KV history for little arithmetic).  The
// published HBM peak is not what a read stream reaches; this kernel gives
// the rate the chip does reach with the access pattern that suits it best,
// so that a decode kernel's fraction of the peak can be read next to it.
//
// Every workgroup (256 threads) reads 16-byte words with the non-temporal
// hint, UNROLL loads per thread in flight, and folds them into an XOR that
// one thread stores to sink[workgroup] (so no load is dead).
//   mode 0: workgroup b reads one contiguous chunk, the b-th of `workgroups`
//           equal chunks of the buffer;
//   mode 1: grid stride: iteration i of workgroup b reads the 32 KiB step
//           i * workgroups + b of the buffer;
//   mode 2: the buffer as 4 KiB blocks (a power-of-two count of them) read in
//           a scattered order -- logical block i is physical block
//           (i * 0x9E3779B1) mod count, a bijection -- and each workgroup
//           takes one contiguous 1/workgroups share of the logical blocks:
//           the access pattern of a paged K/V pool (one 4 KiB (block, head)
//           tile at a time, wherever the block manager placed it).
#include "pa_device.h"
#include "pa_probe.h"

namespace pa {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_UNROLL = 8;

__device__ __forceinline__ uint32_t fold(const pa_u32x4 &v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(PROBE_THREADS) void stream_read_kernel(const pa_u32x4 *src, uint64_t n16,
                                                                     int mode, uint32_t *sink)
{
    const uint64_t nwg = gridDim.x;
    const uint64_t b = blockIdx.x;
    const uint64_t t = threadIdx.x;
    constexpr uint64_t STEP = (uint64_t)PROBE_THREADS * PROBE_UNROLL;   // words per workgroup iteration
    uint32_t x = 0;
    if (mode == 0) {
        const uint64_t per = (n16 + nwg - 1) / nwg;
        const uint64_t lo = b * per;
        const uint64_t hi = lo + per < n16 ? lo + per : n16;
        uint64_t i = lo;
        for (; i + STEP <= hi; i += STEP) {
            pa_u32x4 v[PROBE_UNROLL];
#pragma unroll
            for (int u = 0; u < PROBE_UNROLL; ++u)
                v[u] = __builtin_nontemporal_load(src + i + (uint64_t)u * PROBE_THREADS + t);
#pragma unroll
            for (int u = 0; u < PROBE_UNROLL; ++u)
                x ^= fold(v[u]);
        }
        for (uint64_t j = i + t; j < hi; j += PROBE_THREADS)
            x ^= fold(__builtin_nontemporal_load(src + j));
    } else if (mode == 2) {
        constexpr uint64_t BLK = 4096 / 16;                         // words per block: one per thread
        const uint64_t nblk = n16 / BLK;
        const uint64_t per = (nblk + nwg - 1) / nwg;
        const uint64_t lo = b * per;
        const uint64_t hi = lo + per < nblk ? lo + per : nblk;
        uint64_t i = lo;
        for (; i + PROBE_UNROLL <= hi; i += PROBE_UNROLL) {
            pa_u32x4 v[PROBE_UNROLL];
#pragma unroll
            for (int u = 0; u < PROBE_UNROLL; ++u) {
                const uint64_t phys = ((i + u) * 0x9E3779B1ull) & (nblk - 1);
                v[u] = __builtin_nontemporal_load(src + phys * BLK + t);
            }
#pragma unroll
            for (int u = 0; u < PROBE_UNROLL; ++u)
                x ^= fold(v[u]);
        }
        for (; i < hi; ++i)
            x ^= fold(__builtin_nontemporal_load(src + ((i * 0x9E3779B1ull) & (nblk - 1)) * BLK + t));
    } else {
        uint64_t i = b * STEP;
        for (; i + STEP <= n16; i += nwg * STEP) {
            pa_u32x4 v[PROBE_UNROLL];
#pragma unroll
            for (int u = 0; u < PROBE_UNROLL; ++u)
                v[u] = __builtin_nontemporal_load(src + i + (uint64_t)u * PROBE_THREADS + t);
#pragma unroll
            for (int u = 0; u < PROBE_UNROLL; ++u)
                x ^= fold(v[u]);
        }
        // the partial last iteration: the workgroup whose turn it is
        if (i < n16)
            for (uint64_t j = i + t; j < n16; j += PROBE_THREADS)
                x ^= fold(__builtin_nontemporal_load(src + j));
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
        x ^= __shfl_xor(x, off);
    __shared__ uint32_t part[PROBE_THREADS / 64];
    if ((t & 63) == 0)
        part[t >> 6] = x;
    __syncthreads();
    if (t == 0) {
        uint32_t r = 0;
#pragma unroll
        for (int w = 0; w < PROBE_THREADS / 64; ++w)
            r ^= part[w];
        sink[b] = r;
    }
}

}  // namespace pa

extern "C" pa_status pa_probe_stream_read(const void *src, size_t bytes, uint32_t *sink, int workgroups, int mode,
                                          void *stream)
{
    if (!src || !sink || bytes == 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > (1 << 20))
        return PA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
        return PA_ERR_INVALID_ARG;
    if (mode != 0 && mode != 1 && mode != 2)
        return PA_ERR_INVALID_ARG;
    // mode 2: a power-of-two number of 4 KiB blocks
    if (mode == 2 && (bytes % 4096 != 0 || ((bytes / 4096) & (bytes / 4096 - 1)) != 0))
        return PA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(pa::stream_read_kernel, dim3(workgroups), dim3(pa::PROBE_THREADS), 0,
                       static_cast<hipStream_t>(stream), static_cast<const pa::pa_u32x4 *>(src),
                       (uint64_t)(bytes / 16), mode, sink);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
