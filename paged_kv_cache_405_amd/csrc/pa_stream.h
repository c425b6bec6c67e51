// pa_stream.h -- the balanced ("stream") schedule of paged decode attention.
//
// Method: "vLLM 与 PagedAttention" (inference.mavenzero.com/case-studies/vllm),
// section 二 "注意力计算改造": K/V are read block by block and the per-block
// results accumulated.  Accumulating in any grouping gives the same answer
// (online softmax, up to rounding), so the work can be cut wherever the
// hardware wants it cut.  This file cuts it so that every wave of the GPU
// gets the same number of tokens.
//
// The work is a stream of steps (a step is STEP_TOK tokens of one unit; a
// unit is one sequence and the q heads that one worker handles for one kv
// head), ordered head group major, then sequence, then step:
//
//     unit (hg, s) holds n(s) = max(1, ceil(ctx_s / STEP_TOK)) steps,
//     stream position of (hg, s, j) = hg * sum_s n(s) + prefix_s + j.
//
// With T positions and N waves, logical wave w owns [floor(wT/N),
// floor((w+1)T/N)): all waves get the same work to within one step, so none
// finishes late.  A wave walks its range unit by unit.  A unit that lies
// wholly in the range is finished in place (normalised and stored to out); a
// unit cut by a range edge leaves a piece (max, sum, unnormalised output) in
// the workspace, chained to the piece of the next wave, and the reduce kernel
// merges each chain in order -- a fixed order, so results are reproducible.
// A sequence with an empty context still has one (empty) step, so that one
// wave writes its zero rows.
//
// Logical wave ids are assigned XCD-major: dispatch places workgroup b on XCD
// b % 8, and logical wave (b % 8) * N/8 + b / 8 makes each XCD's L2 see one
// contiguous eighth of the stream (head group major), so blocks that several
// sequences share (a common prefix) are fetched once per XCD L2 and then hit.
#pragma once

#include "pa_device.h"

namespace pa {

// wave-wide sum and inclusive prefix sum of a 64-bit value
__device__ __forceinline__ int64_t wave_sum64(int64_t x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
        x += __shfl_xor(x, off);
    return x;
}
__device__ __forceinline__ int64_t wave_incl_scan64(int64_t x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(x, off);
        if (lane >= off)
            x += y;
    }
    return x;
}

// first stream position of logical wave w: floor(w * T / N) without overflow
__device__ __forceinline__ uint64_t range_start(int w, uint64_t T, int N) {
    const uint64_t q = T / (uint64_t)N, r = T % (uint64_t)N;
    return q * (uint64_t)w + (r * (uint64_t)w) / (uint64_t)N;
}

// logical wave whose range holds position c (c < T): the largest w with
// range_start(w) <= c, i.e. floor(((c + 1) N - 1) / T)
__device__ __forceinline__ int wave_of(uint64_t c, uint64_t T, int N) {
    const unsigned __int128 x = (unsigned __int128)(c + 1) * (unsigned)N - 1;
    return (int)(x / T);
}

template <class W, int BS>
__global__ __launch_bounds__(64) void decode_stream_kernel(const DecodeParams P)
{
    constexpr int STEP = W::STEP_TOK;
    const int lane = threadIdx.x;
    const int S = P.num_seqs;
    const int HG = P.num_kv_heads * P.group_split;
    const int N = P.n_waves;
    const int cap = P.max_blocks * BS;
    auto clamp_ctx = [&](int c) { return c < 0 ? 0 : (c > cap ? cap : c); };

    // steps per head group: Tseq = sum over sequences of n(s)
    int64_t tseq = 0;
    for (int b = 0; b < S; b += 64) {
        const int i = b + lane;
        const int64_t n = i < S ? max(1, (clamp_ctx(P.ctx[i]) + STEP - 1) / STEP) : 0;
        tseq += wave_sum64(n);
    }
    const uint64_t T = (uint64_t)tseq * (uint64_t)HG;
    const int bid = blockIdx.x;
    const int w = (bid & 7) * (N >> 3) + (bid >> 3);
    const uint64_t c_lo = range_start(w, T, N);
    const uint64_t c_hi = range_start(w + 1, T, N);
    if (c_lo >= c_hi)
        return;

    // locate c_lo: head group, then the sequence by a prefix scan, then the step
    int hg = (int)(c_lo / (uint64_t)tseq);
    const int64_t r0 = (int64_t)(c_lo - (uint64_t)hg * (uint64_t)tseq);
    int s = 0;
    int64_t base = 0;
    for (int b = 0; b < S; b += 64) {
        const int i = b + lane;
        const int64_t n = i < S ? max(1, (clamp_ctx(P.ctx[i]) + STEP - 1) / STEP) : 0;
        const int64_t incl = wave_incl_scan64(n, lane);
        const int64_t tot = __shfl(incl, 63);
        if (r0 < base + tot) {
            const uint64_t hit = __ballot(i < S && base + incl > r0);
            const int k = __ffsll((unsigned long long)hit) - 1;
            s = b + k;
            base += __shfl(incl - n, k);
            break;
        }
        base += tot;
    }
    int j = (int)(r0 - base);

    W wk;
    wk.init_lane(lane);
    uint64_t pos = c_lo;
    bool first = true;
    for (;;) {
        const int ctx = clamp_ctx(P.ctx[s]);
        const int nreal = (ctx + STEP - 1) / STEP;
        const int nsched = max(1, nreal);
        const uint64_t left = c_hi - pos;
        const int jend = (uint64_t)(nsched - j) <= left ? nsched : j + (int)left;
        wk.bind(P, s, hg, ctx);
        wk.reset();
        wk.run(j, min(jend, nreal), 1);
        const int64_t u = (int64_t)hg * S + s;
        if (j == 0 && jend == nsched) {
            wk.finish_out(P);
            if (lane == 0)
                P.unit_first[u] = -1;
        } else {
            const int piece = 2 * w + (first ? 0 : 1);
            wk.finish_piece(P, piece);
            if (lane == 0) {
                if (j == 0)
                    P.unit_first[u] = piece;
                P.piece_next[piece] = jend == nsched ? -1 : 2 * wave_of(pos + (uint64_t)(jend - j), T, N);
            }
        }
        pos += (uint64_t)(jend - j);
        if (pos >= c_hi)
            break;
        first = false;
        j = 0;
        if (++s == S) {
            s = 0;
            ++hg;
        }
    }
}

// Merge the pieces of every unit the stream kernel cut: one workgroup per
// unit (grid x = sequence, y = head group), threads over (head, dim).
template <typename T, int D>
__global__ __launch_bounds__(128) void stream_reduce_kernel(const DecodeParams P, int heads_per_unit)
{
    const int s = blockIdx.x;
    const int hg = blockIdx.y;
    const int first = P.unit_first[(int64_t)hg * P.num_seqs + s];
    if (first < 0)
        return;
    const int kvh = hg / P.group_split;
    const int qh0 = kvh * P.group + (hg - kvh * P.group_split) * heads_per_unit;
    const int max_pieces = 2 * P.n_waves;
    for (int idx = threadIdx.x; idx < heads_per_unit * D; idx += blockDim.x) {
        const int g = idx / D;
        const int d = idx - g * D;
        float M = NEG_BIG, L = 0.f, A = 0.f;
        int p = first;
        for (int it = 0; p >= 0 && it < max_pieces; ++it) {
            const float2 ml = P.piece_ml[(int64_t)p * heads_per_unit + g];
            const float a = P.piece_acc[((int64_t)p * heads_per_unit + g) * D + d];
            const float mn = fmaxf(M, ml.x);
            const float c0 = fast_exp2(M - mn);
            const float c1 = fast_exp2(ml.x - mn);
            L = L * c0 + ml.y * c1;
            A = A * c0 + a * c1;
            M = mn;
            p = P.piece_next[p];
        }
        Store<T>::one(P.out, ((int64_t)s * P.num_q_heads + qh0 + g) * D + d, L > 0.f ? A / L : 0.f);
    }
}

template <class W, int BS>
hipError_t launch_stream(const DecodeParams &p, hipStream_t st)
{
    hipLaunchKernelGGL((decode_stream_kernel<W, BS>), dim3(p.n_waves), dim3(64), 0, st, p);
    return hipGetLastError();
}

// Workgroups (one wave each) of decode_stream_kernel<W, BS> that one compute
// unit holds at once.
template <class W, int BS>
int stream_occupancy()
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_stream_kernel<W, BS>, 64, 0) != hipSuccess)
        return 0;
    return n;
}

}  // namespace pa
