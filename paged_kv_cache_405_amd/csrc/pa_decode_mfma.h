// pa_decode_mfma.h -- launchers of the grouped-query (matrix core) decode
// path for gfx950: the grid schedule (one workgroup per partition, head group
// and sequence; waves merged through LDS) and the balanced stream schedule,
// both over the per-wave worker of pa_decode_gqa.h.
//
// Method: "vLLM 与 PagedAttention" (inference.mavenzero.com/case-studies/vllm),
// section 二 "注意力计算改造": K/V read block by block, per-block results
// accumulated; partitions of one context are merged the same way.
#pragma once

#include "pa_decode_gqa.h"
#include "pa_device.h"
#include "pa_stream.h"

namespace pa {

// LDS bytes of one grid workgroup of NW waves: the waves' tile slots, later
// their merge area
template <typename T, int D, int BS, int NW, bool STREAM_KV>
constexpr int decode_mfma_lds()
{
    constexpr int MERGE_BYTES = NW * 16 * (D + 2) * 4;
    constexpr int TILES = NW * GqaWorker<T, D, BS, STREAM_KV>::LDS_BYTES;
    return TILES > MERGE_BYTES ? TILES : MERGE_BYTES;
}

// Grid schedule (partition_tokens != 0): one workgroup of NW waves per
// (partition, head group, sequence); the waves take the partition's tiles
// round robin and merge through LDS, reusing the tile slots.  The workgroup
// (partition bx of head group by of grid row bz) as a function of its block
// coordinates, over decode_mfma_lds() bytes of LDS at `lds`: the
// shared-prefix decode runs it inside a launch of its own (pa_shared_prefix.h).
template <typename T, int D, int BS, int NW, bool STREAM_KV>
__device__ __forceinline__ void decode_mfma_block(const DecodeParams &P, int bx, int by, int bz,
                                                  unsigned char PA_LDS *lds)
{
    static_assert(D % 128 == 0, "the grouped-query kernel needs head_dim 128 or 256");
    static_assert(BS % 8 == 0, "block size 8, 16 or 32");
    using W = GqaWorker<T, D, BS, STREAM_KV>;

    const int p = bx + P.first_partition;
    const int hg = by;
    int ctx;
    const int s = seq_of_row(P, bz, BS, ctx);
    const int nblk = (ctx + BS - 1) / BS;
    const int npart = num_partitions(P, nblk);
    if (p >= npart)
        return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    W w;
    w.init_lane(lane);
    w.init_lds(lds + wave * W::LDS_BYTES);
    w.bind(P, s, hg, ctx);
    const int gh = w.gh;
    const int qh0 = w.qh0;

    // tokens [t_lo, t_hi) of this partition, covered by 16-token tiles [k0, k1)
    const int b0 = partition_first_block(P, p);
    const int b1 = min(nblk, b0 + P.partition_blocks);
    w.t_lo = b0 * BS;
    w.t_hi = w.t_vlim = w.t_full = min(b1 * BS, ctx);
    const int k0 = w.t_lo / GQA_TILE;
    const int k1 = (w.t_hi + GQA_TILE - 1) / GQA_TILE;
    w.reset();
    w.run(k0 + wave, k1, NW);

    // every load of every wave (the LDS ones included) has landed before the
    // tile slots become the merge area
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float *sm_m = (float *)lds;   // the tile slots as the merge area (a generic pointer)
    float *sm_l = sm_m + NW * 16;
    float *sm_acc = sm_l + NW * 16;
    w.export_lds(sm_m + wave * 16, sm_l + wave * 16, sm_acc + wave * 16 * D);
    __syncthreads();

    const bool single = npart == 1 && P.first_partition == 0;
    for (int idx = threadIdx.x; idx < gh * D; idx += NW * 64) {
        const int g = idx / D;
        const int d = idx - g * D;
        float M = sm_m[g];
#pragma unroll
        for (int v = 1; v < NW; ++v)
            M = fmaxf(M, sm_m[v * 16 + g]);
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const float c = fast_exp2(sm_m[v * 16 + g] - M);
            L = fmaf(sm_l[v * 16 + g], c, L);
            A = fmaf(sm_acc[(v * 16 + g) * D + d], c, A);
        }
        const int64_t sh = (int64_t)s * P.num_q_heads + qh0 + g;
        if (single) {
            Store<T>::one(P.out, sh * D + d, L > 0.f ? A / L : 0.f);
        } else {
            P.ws_acc[(sh * P.max_partitions + p) * D + d] = A;
            if (d == 0)
                P.ws_ml[sh * P.max_partitions + p] = make_float2(M, L);
        }
    }
}

template <typename T, int D, int BS, int NW, bool STREAM_KV>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(const DecodeParams P)
{
    __shared__ __attribute__((aligned(16))) unsigned char lds[decode_mfma_lds<T, D, BS, NW, STREAM_KV>()];
    decode_mfma_block<T, D, BS, NW, STREAM_KV>(P, blockIdx.x, blockIdx.y, blockIdx.z, (unsigned char PA_LDS *)lds);
}

constexpr int MFMA_WAVES = 4;

template <typename T, int D, int BS>
hipError_t launch_mfma_shape(const DecodeParams &p, hipStream_t st)
{
    dim3 grid(p.max_partitions - p.first_partition, p.num_kv_heads * p.group_split, p.num_seqs);
    if (p.kv_cached)
        hipLaunchKernelGGL((decode_mfma_kernel<T, D, BS, MFMA_WAVES, false>), grid, dim3(MFMA_WAVES * 64), 0, st, p);
    else
        hipLaunchKernelGGL((decode_mfma_kernel<T, D, BS, MFMA_WAVES, true>), grid, dim3(MFMA_WAVES * 64), 0, st, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_mfma_bs(const DecodeParams &p, int bs, hipStream_t st)
{
    switch (bs) {
    case 8: return launch_mfma_shape<T, D, 8>(p, st);
    case 16: return launch_mfma_shape<T, D, 16>(p, st);
    case 32: return launch_mfma_shape<T, D, 32>(p, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_mfma_dtype(const DecodeParams &p, int head_dim, int bs, hipStream_t st)
{
    switch (head_dim) {
    case 128: return launch_mfma_bs<T, 128>(p, bs, st);
    case 256: return launch_mfma_bs<T, 256>(p, bs, st);
    default: return hipErrorInvalidValue;
    }
}

// Balanced schedule: launch (occ == nullptr) or report the workgroups per
// compute unit of the stream kernel for this shape (occ != nullptr).
template <typename T, int D, int BS>
hipError_t mfma_stream_shape(const DecodeParams *p, hipStream_t st, int *occ)
{
    // the two load policies compile to the same registers: the occupancy of one is that of both
    if (occ) {
        *occ = stream_occupancy<GqaWorker<T, D, BS, true>, BS>();
        return hipSuccess;
    }
    return p->kv_cached ? launch_stream<GqaWorker<T, D, BS, false>, BS>(*p, st)
                        : launch_stream<GqaWorker<T, D, BS, true>, BS>(*p, st);
}

template <typename T>
hipError_t mfma_stream_dtype(const DecodeParams *p, int head_dim, int bs, hipStream_t st, int *occ)
{
    switch (head_dim * 64 + bs) {
    case 128 * 64 + 8: return mfma_stream_shape<T, 128, 8>(p, st, occ);
    case 128 * 64 + 16: return mfma_stream_shape<T, 128, 16>(p, st, occ);
    case 128 * 64 + 32: return mfma_stream_shape<T, 128, 32>(p, st, occ);
    case 256 * 64 + 8: return mfma_stream_shape<T, 256, 8>(p, st, occ);
    case 256 * 64 + 16: return mfma_stream_shape<T, 256, 16>(p, st, occ);
    case 256 * 64 + 32: return mfma_stream_shape<T, 256, 32>(p, st, occ);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
