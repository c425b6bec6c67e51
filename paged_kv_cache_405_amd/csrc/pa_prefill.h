// pa_prefill.h -- multi-token paged attention on the matrix cores: several
// query rows per sequence (a prefill chunk, drafted tokens to verify), causal
// over the sequence's paged history.
//
// Method: "vLLM 与 PagedAttention" (inference.mavenzero.com/case-studies/vllm),
// section 二: K/V sit in blocks reached through the sequence's table and are
// read block by block, the per-block results accumulated; section 六
// ("关键的工程优化"): a long prompt's prefill runs in chunks next to decode;
// "指南" ("Speculative Decoding"): the large model checks several drafted
// tokens in one pass.  Query row i of a chunk of n rows over a context of L
// tokens sits at position L - n + i and attends tokens 0 .. L - n + i.
//
// The per-wave worker is the grouped-query decode worker of pa_decode_gqa.h
// with its 16 score columns taken by (query row, q head) pairs -- 16 / gh rows
// of the chunk times the gh q heads of one kv head -- each column with its own
// causal limit.  One workgroup of NW waves per (column tile, head group,
// sequence) takes the key tiles round robin up to the tile's last position
// and merges through LDS, as the grid decode kernel does.
#pragma once

#include "pa_decode_gqa.h"
#include "pa_device.h"

namespace pa {

template <typename T, int D, int BS, int NW, bool STREAM_KV>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(const DecodeParams P)
{
    static_assert(D % 128 == 0, "the matrix-core worker needs head_dim 128 or 256");
    using W = GqaWorker<T, D, BS, STREAM_KV>;
    constexpr int MERGE_BYTES = NW * 16 * (D + 2) * 4;
    constexpr int LDS_TOTAL = NW * W::LDS_BYTES > MERGE_BYTES ? NW * W::LDS_BYTES : MERGE_BYTES;

    const int ct = blockIdx.x;
    const int hg = blockIdx.y;
    const int s = blockIdx.z;
    int ctx = P.ctx[s];
    const int cap = P.max_blocks * BS;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    // this sequence's q rows, kept inside [0, total_q) whatever query_start holds
    const int q_first = P.query_start[s];
    int nq = P.query_start[s + 1] - q_first;
    if (q_first < 0 || q_first >= P.total_q)
        return;
    nq = nq > P.total_q - q_first ? P.total_q - q_first : nq;
    const int gh = P.group / P.group_split;
    const int i0 = ct * (GQA_TILE / gh);
    if (i0 >= nq)
        return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_TOTAL];

    W w;
    w.init_lane(lane);
    w.init_lds((unsigned char PA_LDS *)lds + wave * W::LDS_BYTES);
    w.bind_rows(P, s, hg, ctx, q_first, nq, i0);
    const int k1 = (w.t_last + GQA_TILE - 1) / GQA_TILE;
    w.reset();
    w.run(wave, k1, NW);

    // every load of every wave has landed before the tile slots become the merge area
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float *sm_m = reinterpret_cast<float *>(lds);
    float *sm_l = sm_m + NW * 16;
    float *sm_acc = sm_l + NW * 16;
    w.export_lds(sm_m + wave * 16, sm_l + wave * 16, sm_acc + wave * 16 * D);
    __syncthreads();

    for (int idx = threadIdx.x; idx < w.ncols * D; idx += NW * 64) {
        const int g = idx / D;
        const int d = idx - g * D;
        const int i = i0 + g / gh;
        if (i >= nq)
            continue;
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
        const int64_t row = (int64_t)(q_first + i) * P.num_q_heads + w.qh0 + g % gh;
        Store<T>::one(P.out, row * D + d, L > 0.f ? A / L : 0.f);
    }
}

constexpr int PREFILL_WAVES = 4;

template <typename T, int D, int BS>
hipError_t launch_prefill_shape(const DecodeParams &p, int max_query_len, hipStream_t st)
{
    const int rows = GQA_TILE / (p.group / p.group_split);
    dim3 grid((max_query_len + rows - 1) / rows, p.num_kv_heads * p.group_split, p.num_seqs);
    if (p.kv_cached)
        hipLaunchKernelGGL((prefill_kernel<T, D, BS, PREFILL_WAVES, false>), grid, dim3(PREFILL_WAVES * 64), 0, st, p);
    else
        hipLaunchKernelGGL((prefill_kernel<T, D, BS, PREFILL_WAVES, true>), grid, dim3(PREFILL_WAVES * 64), 0, st, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_prefill_bs(const DecodeParams &p, int bs, int max_query_len, hipStream_t st)
{
    switch (bs) {
    case 8: return launch_prefill_shape<T, D, 8>(p, max_query_len, st);
    case 16: return launch_prefill_shape<T, D, 16>(p, max_query_len, st);
    case 32: return launch_prefill_shape<T, D, 32>(p, max_query_len, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_prefill_dtype(const DecodeParams &p, int head_dim, int bs, int max_query_len, hipStream_t st)
{
    switch (head_dim) {
    case 128: return launch_prefill_bs<T, 128>(p, bs, max_query_len, st);
    case 256: return launch_prefill_bs<T, 256>(p, bs, max_query_len, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
