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

// a value that is the same in every lane, as a scalar (uniform) value
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// wave-wide sum and inclusive prefix sum of a 64-bit value
__device__ __forceinline__ int64_t wave_sum64(int64_t x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
        x += __shfl_xor(x, off);
    return uniform64(x);
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

// first stream position of logical wave w: floor(w * T / N) without
// overflow.  With T < 2^32 and N <= 2^16 (the host keeps N there) every
// division is a 32-bit one: r * w < N^2 <= 2^32.
__device__ __forceinline__ uint64_t range_start(int w, uint64_t T, int N) {
    if (T < (1ull << 32)) {
        const uint32_t t = (uint32_t)T, n = (uint32_t)N, q = t / n, r = t - q * n;
        return (uint64_t)q * (uint32_t)w + (uint64_t)((r * (uint32_t)w) / n);
    }
    const uint64_t q = T / (uint64_t)N, r = T % (uint64_t)N;
    return q * (uint64_t)w + (r * (uint64_t)w) / (uint64_t)N;
}

constexpr int STREAM_WAVES_PER_EU = 1;   // waves per SIMD the register allocation must allow (1 = no limit)

template <class W, int BS>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(STREAM_WAVES_PER_EU)))
void decode_stream_kernel(const DecodeParams P)
{
    constexpr int STEP = W::STEP_TOK;
    const int lane = threadIdx.x;
    const int S = P.num_seqs;
    const int HG = P.num_kv_heads * P.group_split;
    const int N = P.n_waves;
    const int cap = P.max_blocks * BS;
    auto clamp_ctx = [&](int c) { return c < 0 ? 0 : (c > cap ? cap : c); };

    // steps per head group: Tseq = sum over sequences of n(s).  Up to 64
    // sequences (one per lane) the context lengths are read once and kept:
    // the running sum that gives Tseq also locates the wave's first unit
    const bool few = S <= 64;
    int ctx_lane = 0;              // few: lane i holds sequence i's clamped context
    int64_t incl_lane = 0, n_lane = 0;
    int64_t tseq = 0;
    if (few) {
        ctx_lane = lane < S ? clamp_ctx(P.ctx[lane]) : 0;
        n_lane = lane < S ? max(1, (ctx_lane + STEP - 1) / STEP) : 0;
        incl_lane = wave_incl_scan64(n_lane, lane);
        tseq = uniform64(__shfl(incl_lane, 63));
    } else {
        for (int b = 0; b < S; b += 64) {
            const int i = b + lane;
            const int64_t n = i < S ? max(1, (clamp_ctx(P.ctx[i]) + STEP - 1) / STEP) : 0;
            tseq += wave_sum64(n);
        }
    }
    const uint64_t T = (uint64_t)tseq * (uint64_t)HG;
    const int bid = blockIdx.x;
    const int w = (bid & 7) * (N >> 3) + (bid >> 3);   // logical waves XCD-major
    if (bid == 0 && lane == 0)
        P.stream_total[0] = T;
    const uint64_t c_lo = range_start(w, T, N);
    const uint64_t c_hi = range_start(w + 1, T, N);
    if (c_lo >= c_hi)
        return;

    // locate c_lo: the head group, then the sequence by a prefix scan over
    // the units' step counts, then the step
    int hg = c_lo < (1ull << 32) && (uint64_t)tseq < (1ull << 32) ? (int)((uint32_t)c_lo / (uint32_t)tseq)
                                                                  : (int)(c_lo / (uint64_t)tseq);
    const int64_t r0 = (int64_t)(c_lo - (uint64_t)hg * (uint64_t)tseq);
    int s = 0;
    int64_t base = 0;
    if (few) {
        const uint64_t hit = __ballot(lane < S && incl_lane > r0);
        const int k = __ffsll((unsigned long long)hit) - 1;
        s = __builtin_amdgcn_readfirstlane(k);
        base = uniform64(__shfl(incl_lane - n_lane, k));
    }
    for (int b = 0; b < (few ? 0 : S); b += 64) {
        const int i = b + lane;
        const int64_t n = i < S ? max(1, (clamp_ctx(P.ctx[i]) + STEP - 1) / STEP) : 0;
        const int64_t incl = wave_incl_scan64(n, lane);
        const int64_t tot = __shfl(incl, 63);
        if (r0 < base + tot) {
            const uint64_t hit = __ballot(i < S && base + incl > r0);
            const int k = __ffsll((unsigned long long)hit) - 1;
            s = __builtin_amdgcn_readfirstlane(b + k);
            base += uniform64(__shfl(incl - n, k));
            break;
        }
        base += uniform64(tot);
    }
    int j = __builtin_amdgcn_readfirstlane((int)(r0 - base));

    W wk;
    wk.init_lane(lane);
    // at least W::STREAM_LDS_MIN bytes: a worker may size its workgroups so
    // that a compute unit holds only a few of them (one wave per SIMD)
    constexpr int LDS_N = W::LDS_BYTES > W::STREAM_LDS_MIN ? W::LDS_BYTES : W::STREAM_LDS_MIN;
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_N > 0 ? LDS_N : 16];
    wk.init_lds((unsigned char __attribute__((address_space(3))) *)lds);
    uint64_t pos = c_lo;
    bool first = true;
    for (;;) {
        // the cursor is the same in every lane; say so, so that addresses
        // derived from it (table row, tile indices) stay scalar
        s = __builtin_amdgcn_readfirstlane(s);
        hg = __builtin_amdgcn_readfirstlane(hg);
        j = __builtin_amdgcn_readfirstlane(j);
        const int ctx = few ? __builtin_amdgcn_readlane(ctx_lane, s) : clamp_ctx(P.ctx[s]);
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
                if (jend == nsched)
                    P.unit_last[u] = piece;
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

// Merge the pieces of every unit the stream kernel cut: one wave per (unit,
// head of the unit), grid x = sequence, y = head group, z = head.  The piece
// list is known from its two ends, so no load waits on another: lane i loads
// the (max, sum) of piece i and the wave the outputs of the first FEW_PIECES
// pieces (lanes over dims), all at once; then the reference max, the weights
// and the rescaled sums, with further batches of FEW_PIECES outputs as needed
// (past 64 pieces, rounds of 64 weights, the max taken in a pass of its
// own).  Pieces are added in order, so results are
// bit-reproducible.  A unit of a small batch can be cut over many waves (32
// sequences of one kv head over 1024 waves: about 33 pieces each); with one
// load in flight per piece its merge took 32 us, batched it takes a few.
constexpr int FEW_PIECES = 16;   // pieces whose loads the reduce issues in one batch

template <typename T, int D>
__global__ __launch_bounds__(64) void stream_reduce_kernel(const DecodeParams P, int heads_per_unit)
{
    const int s = blockIdx.x;
    const int hg = blockIdx.y;
    const int g = blockIdx.z;
    const int64_t u = (int64_t)hg * P.num_seqs + s;
    const int first = P.unit_first[u];
    if (first < 0)
        return;
    const int w0 = first >> 1;
    const int w1 = P.unit_last[u] >> 1;   // the last piece is 2 w1
    const uint64_t total = P.stream_total[0];
    const int N = P.n_waves;
    const bool every_wave = total >= (uint64_t)N;   // then no range is empty
    auto empty = [&](int w) {
        return !every_wave && w > w0 && range_start(w, total, N) == range_start(w + 1, total, N);
    };
    auto slot = [&](int w) { return (int64_t)(w == w0 ? first : 2 * w) * heads_per_unit + g; };

    const int lane = threadIdx.x;
    constexpr int E = (D + 63) / 64;
    float A[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        A[e] = 0.f;
    const int np = w1 - w0 + 1;

    // the reference max: beyond 64 pieces a pass of its own (one piece per
    // lane, 64 at a time); up to 64 from the weights' own loads below, taken
    // once the first batch of outputs is in flight
    const bool one_round = np <= 64;
    float M = NEG_BIG;
    if (!one_round) {
        for (int w = w0 + lane; w <= w1; w += 64)
            if (!empty(w))
                M = fmaxf(M, P.piece_ml[slot(w)].x);
        M = group_max<64>(M);
    }

    float L = 0.f;
    for (int r0 = 0; r0 < np; r0 += 64) {
        // lane i weighs piece r0 + i (an empty range left no piece: weight 0)
        const int wl = w0 + r0 + lane;
        const bool has = r0 + lane < np && !empty(wl);
        const float2 ml = has ? P.piece_ml[slot(wl)] : make_float2(NEG_BIG, 0.f);
        float c = 0.f;
        const int cnt = min(64, np - r0);
        for (int b0 = 0; b0 < cnt; b0 += FEW_PIECES) {
            // every load of the batch first; a piece past the end or of an
            // empty range is selected out, never multiplied by its weight
            float a[FEW_PIECES][E];
#pragma unroll
            for (int i = 0; i < FEW_PIECES; ++i) {
                const int w = w0 + r0 + b0 + i;
                const bool ok = b0 + i < cnt && !empty(w);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    a[i][e] = ok && lane + 64 * e < D ? P.piece_acc[slot(w) * D + lane + 64 * e] : 0.f;
            }
            if (b0 == 0) {
                if (one_round)
                    M = group_max<64>(ml.x);
                c = has ? fast_exp2(ml.x - M) : 0.f;
                L = fmaf(ml.y, c, L);
            }
#pragma unroll
            for (int i = 0; i < FEW_PIECES; ++i) {
                const int k = min(b0 + i, 63);
                const float ci = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), k));
#pragma unroll
                for (int e = 0; e < E; ++e)
                    A[e] = fmaf(a[i][e], ci, A[e]);   // pieces past the end hold 0
            }
        }
    }
    L = group_sum<64>(L);
    const int kvh = hg / P.group_split;
    const int qh = kvh * P.group + (hg - kvh * P.group_split) * heads_per_unit + g;
    const int64_t o = ((int64_t)s * P.num_q_heads + qh) * D;
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (lane + 64 * e < D)
            Store<T>::one(P.out, o + lane + 64 * e, L > 0.f ? A[e] / L : 0.f);
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
