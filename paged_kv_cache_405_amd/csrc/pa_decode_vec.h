// pa_decode_vec.h -- paged decode attention, vector (VALU) path for gfx950.
//
// Method: "vLLM 与 PagedAttention" (inference.mavenzero.com/case-studies/vllm),
// section 二: the context of a sequence is stored in fixed-size blocks of a
// shared pool that a per-sequence block table maps (sub-section
// "PagedAttention 的解法"); attention reads K/V one block at a time and
// accumulates the per-block results (sub-section "注意力计算改造").  The
// accumulation is done as an online softmax: a running max m, a running sum
// l and an unnormalised output acc, rescaled by exp(m_old - m_new) whenever
// the max grows.  Partitions of one context (split-K) are merged the same way.
//
// Work decomposition (one workgroup per (partition, kv-head group, sequence)):
//   - a wave reads a step -- NLD wave-wide loads of K and of V, a slab of one
//     (block, kv head) tile -- with 16-byte loads: lane -> (token row, 16-byte
//     chunk of head_dim); LPT lanes cover one token's row, so a wave-wide load
//     covers TPL = 64/LPT tokens;
//   - q.k is a per-lane dot over the lane's chunk followed by a DPP sum over
//     the LPT lanes of the row (no LDS);
//   - each token row keeps its own (m, l, acc) over the tokens it sees; the
//     rows are merged with cross-lane shuffles after the block loop, and the
//     waves of the workgroup through LDS;
//   - the waves of a workgroup take the partition's steps round robin, and
//     each wave issues the next step's loads before it computes the current
//     one (register double buffering), so two steps per wave are in flight;
//     no step past the last context token is read.
//   - GT q heads that share one kv head (grouped-query attention) are handled
//     by one workgroup, so each K/V element is read once per GT heads.
//
// Scores are kept in log2 units (scale * log2(e) folded into one factor) so
// that exponentials are single v_exp_f32 instructions.
#pragma once

#include "pa_device.h"
#include "pa_stream.h"

namespace pa {

constexpr int VEC_STAGES = 2;          // steps in the register pipeline of the vector kernel
constexpr int VEC_NLD = 2;             // most wave-wide loads of K (and of V) per step
constexpr int VEC_WAVES_PER_EU = 1;    // occupancy floor handed to the register allocator (1 = none)

// One wave's share of the work on one (sequence, kv head): the online-softmax
// state of GT query heads and the step pipeline that feeds it.  A step is a
// slab of NLD wave-wide loads of K and of V inside one (block, kv head) tile.
// The pipeline is the one of the grouped-query kernel: two register buffers
// alternate, the next step's loads are issued unconditionally before the
// current step's math, and block-table entries are wave-uniform scalar loads
// fetched one step further ahead.
template <typename T, int D, int BS, int GT, bool STREAM_KV>
struct VecWorker {
    using V = Vec<T>;
    static constexpr int VEC = V::N;                 // elements per 16 bytes
    static constexpr int ES = 16 / VEC;              // element bytes
    static constexpr int LPT = D / VEC;              // lanes per token row
    static_assert(LPT >= 1 && LPT <= 64 && (64 % LPT) == 0, "head_dim / dtype combination");
    static constexpr int TPL = 64 / LPT;             // token rows per wave-wide load
    static constexpr int ROWS = TPL < BS ? TPL : BS; // rows that carry tokens
    static constexpr bool ALL_ROWS = TPL <= BS;
    static constexpr int NLD_TILE = BS / ROWS;       // wave-wide loads per (block, kv head) tile
    static constexpr int NLD = NLD_TILE < VEC_NLD ? NLD_TILE : VEC_NLD;   // loads per step (a slab of the tile)
    static constexpr int NSLAB = NLD_TILE / NLD;     // steps per tile
    static constexpr int SLAB_TOK = NLD * ROWS;      // tokens per step

    static constexpr int STEP_TOK = SLAB_TOK;        // tokens per step of the schedule
    static constexpr int STREAM_LDS_MIN = 0;          // the stream kernel's LDS: its own needs only
    static constexpr int LOADS_PER_TILE = 2 * NLD;   // vector-memory operations load() issues
    static constexpr int LDS_BYTES = 0;              // no LDS staging
    __device__ __forceinline__ void init_lds(unsigned char __attribute__((address_space(3))) *) {}

    struct Buf;
    __device__ __forceinline__ void bind_buf(Buf &, int) const {}
    struct Buf {
        uint4 k[NLD];
        uint4 v[NLD];
        bool ok;
    };

    int seq, qh0;             // the unit bound to the worker: a sequence and GT q heads
    int chunk;                // this lane's 16-byte chunk of a row
    const char *kpool;        // K of this kv head (wave-uniform)
    const char *vpool;        // V of this kv head (wave-uniform)
    int lane_off;             // this lane's (row, chunk) byte offset inside a slab
    const int32_t *trow;
    int64_t blk_bytes, ld_bytes;
    int num_blocks;
    int ctx;
    float scale_log2;
    int row;
    bool row_on;
    float qf[GT][VEC];

    float m[GT], l[GT], acc[GT][VEC];   // per token row; rows are merged at the end

    __device__ __forceinline__ void init_lane(int lane) {
        row = lane / LPT;
        chunk = lane % LPT;
        row_on = ALL_ROWS || row < ROWS;
    }

    // attach the worker to head group hg of sequence s (context ctx, already
    // clamped to the table): q of its GT heads, its kv head's pools, the table row
    __device__ __forceinline__ void bind(const DecodeParams &P, int s, int hg, int ctx_) {
        const int kvh = hg / P.group_split;
        seq = s;
        qh0 = kvh * P.group + (hg - kvh * P.group_split) * GT;
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            const int64_t qi = ((int64_t)s * P.num_q_heads + qh0 + g) * D + chunk * VEC;
            V::widen(ld16(static_cast<const char *>(P.q) + qi * ES), qf[g]);
        }
        const int row_c = row_on ? row : 0;
        kpool = static_cast<const char *>(P.k) + (int64_t)kvh * P.head_stride * ES;
        vpool = static_cast<const char *>(P.v) + (int64_t)kvh * P.head_stride * ES;
        lane_off = (int)((int64_t)row_c * P.token_stride * ES) + chunk * 16;
        blk_bytes = P.block_stride * ES;
        ld_bytes = (int64_t)ROWS * P.token_stride * ES;
        trow = P.tables + (int64_t)s * P.max_blocks;
        num_blocks = P.num_blocks;
        ctx = ctx_;
        scale_log2 = P.scale_log2;
    }

    // the unit was finished by this wave: merge the rows, normalise, store
    // out[seq, qh0 + g, :] from the lanes of row 0
    __device__ __forceinline__ void finish_out(const DecodeParams &P) {
        merge_rows();
        if (row != 0)
            return;
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            float v[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                v[e] = l[g] > 0.f ? acc[g][e] / l[g] : 0.f;
            char *o = static_cast<char *>(P.out) + (((int64_t)seq * P.num_q_heads + qh0 + g) * D + chunk * VEC) * ES;
            st16(o, V::narrow(v));
        }
    }

    // part of the unit: store the wave's (max, sum, unnormalised output) as piece `piece`
    __device__ __forceinline__ void finish_piece(const DecodeParams &P, int piece) {
        merge_rows();
        if (row != 0)
            return;
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            float *a = P.piece_acc + ((int64_t)piece * GT + g) * D + chunk * VEC;
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
                st16(a + e, make_uint4(__float_as_uint(acc[g][e]), __float_as_uint(acc[g][e + 1]),
                                       __float_as_uint(acc[g][e + 2]), __float_as_uint(acc[g][e + 3])));
            if (chunk == 0)
                P.piece_ml[(int64_t)piece * GT + g] = make_float2(m[g], l[g]);
        }
    }

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            m[g] = NEG_BIG;
            l[g] = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                acc[g][e] = 0.f;
        }
    }

    // step q of the sequence: block q / NSLAB (a scalar load), slab q % NSLAB
    __device__ __forceinline__ int2 tile_phys(int q) const {
        const int ph = trow[q / NSLAB];
        return make_int2(ph, ph);
    }

    __device__ __forceinline__ void load(int q, int2 pp, Buf &b) const {
        const int ph = pp.x;
        b.ok = (unsigned)ph < (unsigned)num_blocks;
        // slab base (wave-uniform) plus a 32-bit lane offset
        const int64_t boff = (int64_t)(b.ok ? ph : 0) * blk_bytes + (int64_t)(q % NSLAB) * NLD * ld_bytes;
        const char *ks = kpool + boff;
        const char *vs = vpool + boff;
#pragma unroll
        for (int i = 0; i < NLD; ++i)
            b.k[i] = ld16_kv<STREAM_KV>(ks + i * ld_bytes + lane_off);
#pragma unroll
        for (int i = 0; i < NLD; ++i)
            b.v[i] = ld16_kv<STREAM_KV>(vs + i * ld_bytes + lane_off);
    }

    // the loads are the compiler's own: it places the waits
    template <int BEHIND>
    __device__ __forceinline__ void wait(Buf &) const {}

    template <int BEHIND>
    __device__ __forceinline__ void compute(int q, const Buf &b) {
        const int t0 = q * SLAB_TOK;             // first token of the step
        // scores of this step, log2 units
        float sc[GT][NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            float kf[VEC];
            V::widen(b.k[i], kf);
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    d = fmaf(qf[g][e], kf[e], d);
                sc[g][i] = group_sum<LPT>(d) * scale_log2;
            }
        }
        float vf[NLD][VEC];
#pragma unroll
        for (int i = 0; i < NLD; ++i)
            V::widen(b.v[i], vf[i]);

        // tokens past the context, of an unmapped block, or of an idle row:
        // select (never multiply) so that whatever the memory holds is ignored
        const bool full = b.ok && t0 + SLAB_TOK <= ctx && ALL_ROWS;
        if (!full) {
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int t = t0 + i * ROWS + row;
                const bool valid = b.ok && row_on && t < ctx;
                if (!valid) {
#pragma unroll
                    for (int g = 0; g < GT; ++g)
                        sc[g][i] = -INFINITY;
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        vf[i][e] = 0.f;
                }
            }
        }

#pragma unroll
        for (int g = 0; g < GT; ++g) {
            float mx = sc[g][0];
#pragma unroll
            for (int i = 1; i < NLD; ++i)
                mx = fmaxf(mx, sc[g][i]);
            const float mn = fmaxf(m[g], mx);
            const float alpha = fast_exp2(m[g] - mn);
            float pr[NLD];
            float ps = 0.f;
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                pr[i] = fast_exp2(sc[g][i] - mn);
                ps += pr[i];
            }
            l[g] = fmaf(l[g], alpha, ps);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float a = acc[g][e] * alpha;
#pragma unroll
                for (int i = 0; i < NLD; ++i)
                    a = fmaf(pr[i], vf[i][e], a);
                acc[g][e] = a;
            }
            m[g] = mn;
        }
    }

    // steps qbeg, qbeg + stride, ... below qend (wave-uniform)
    __device__ __forceinline__ void run(int qbeg, int qend, int stride) {
        pipeline<VEC_STAGES>(*this, qbeg, qend, stride);
    }

    // merge the token rows of the wave (lanes that differ in the row bits)
    __device__ __forceinline__ void merge_rows() {
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                const float mo = __shfl_xor(m[g], off);
                const float lo = __shfl_xor(l[g], off);
                const float mn = fmaxf(m[g], mo);
                const float a = fast_exp2(m[g] - mn);
                const float c = fast_exp2(mo - mn);
                l[g] = l[g] * a + lo * c;
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    acc[g][e] = acc[g][e] * a + __shfl_xor(acc[g][e], off) * c;
                m[g] = mn;
            }
        }
    }
};

// The grid kernels' workgroup (partition bx of head group by of grid row bz),
// as a function of its block coordinates: the shared-prefix decode runs it
// inside a launch of its own (pa_shared_prefix.h).
template <typename T, int D, int BS, int GT, int NW, bool STREAM_KV>
__device__ __forceinline__ void decode_vec_block(const DecodeParams &P, int bx, int by, int bz)
{
    using W = VecWorker<T, D, BS, GT, STREAM_KV>;
    constexpr int VEC = W::VEC;

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
    w.bind(P, s, hg, ctx);
    w.reset();
    const int row = w.row;
    const int chunk = w.chunk;
    const int qh0 = w.qh0;

    // the partition's steps, taken round robin by the waves; a step past
    // the last context token is not read (the last block may be partly full)
    const int b0 = partition_first_block(P, p);
    const int b1 = min(nblk, b0 + P.partition_blocks);
    const int q_end = (min(ctx, b1 * BS) + W::SLAB_TOK - 1) / W::SLAB_TOK;
    w.run(b0 * W::NSLAB + wave, q_end, NW);
    w.merge_rows();

    const bool single = npart == 1 && P.first_partition == 0;
    auto emit = [&](int g, int d, float M, float L, float A) {
        const int qh = qh0 + g;
        const int64_t sh = (int64_t)s * P.num_q_heads + qh;
        if (single) {
            Store<T>::one(P.out, sh * D + d, L > 0.f ? A / L : 0.f);
        } else {
            P.ws_acc[(sh * P.max_partitions + p) * D + d] = A;
            if (d == 0)
                P.ws_ml[sh * P.max_partitions + p] = make_float2(M, L);
        }
    };

    if constexpr (NW == 1) {
        if (row == 0) {
#pragma unroll
            for (int g = 0; g < GT; ++g)
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    emit(g, chunk * VEC + e, w.m[g], w.l[g], w.acc[g][e]);
        }
    } else {
        __shared__ float sm_m[NW][GT], sm_l[NW][GT];
        __shared__ float sm_acc[NW][GT][D];
        if (row == 0) {
#pragma unroll
            for (int g = 0; g < GT; ++g)
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    sm_acc[wave][g][chunk * VEC + e] = w.acc[g][e];
        }
        if (lane == 0) {
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                sm_m[wave][g] = w.m[g];
                sm_l[wave][g] = w.l[g];
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < GT * D; idx += NW * 64) {
            const int g = idx / D;
            const int d = idx - g * D;
            float M = sm_m[0][g];
#pragma unroll
            for (int v = 1; v < NW; ++v)
                M = fmaxf(M, sm_m[v][g]);
            float L = 0.f, A = 0.f;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const float c = fast_exp2(sm_m[v][g] - M);
                L = fmaf(sm_l[v][g], c, L);
                A = fmaf(sm_acc[v][g][d], c, A);
            }
            emit(g, d, M, L, A);
        }
    }
}

template <typename T, int D, int BS, int GT, int NW, bool STREAM_KV>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(VEC_WAVES_PER_EU)))
void decode_vec_kernel(const DecodeParams P)
{
    decode_vec_block<T, D, BS, GT, NW, STREAM_KV>(P, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Split-K reduce: one wave per (q head, sequence) merges the partitions'
// (max, sum, unnormalised output) and writes the normalised output.  Every
// (q head, sequence) has max_partitions slots, so the slots of the first
// REDUCE_FEW partitions are loaded at once, beside the context length that
// says how many of them are real: one memory round trip instead of three.
// Slots past the real partitions hold whatever an earlier call left there;
// they are selected out, never multiplied by a zero weight.  Partitions are
// added in order whatever the path, so results are bit-reproducible.
constexpr int REDUCE_FEW = 8;

template <typename T, int D, int BS>
__global__ __launch_bounds__(64) void reduce_kernel(const DecodeParams P)
{
    constexpr int E = (D + 63) / 64;
    const int qh = blockIdx.x;
    const int s = blockIdx.y;
    const int lane = threadIdx.x;
    const int64_t sh = (int64_t)s * P.num_q_heads + qh;
    const float2 *ml = P.ws_ml + sh * P.max_partitions;
    const float *acc = P.ws_acc + sh * P.max_partitions * D;
    const int nfew = min(REDUCE_FEW, P.max_partitions);
    const int nlane = min(64, P.max_partitions);
    const float2 mlv = lane < nlane ? ml[lane] : make_float2(NEG_BIG, 0.f);
    float a[REDUCE_FEW][E];
#pragma unroll
    for (int i = 0; i < REDUCE_FEW; ++i)
#pragma unroll
        for (int e = 0; e < E; ++e)
            a[i][e] = i < nfew && lane + 64 * e < D ? acc[(int64_t)i * D + lane + 64 * e] : 0.f;

    int ctx = P.ctx[s];
    const int cap = P.max_blocks * BS;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int nblk = (ctx + BS - 1) / BS;
    const int npart = num_partitions(P, nblk);
    if (npart <= 1 && P.first_partition == 0)
        return;

    // lane i < 64 holds partition i; partitions past 64 in a loop
    float mx = lane < npart ? mlv.x : NEG_BIG;
    for (int i = lane + 64; i < npart; i += 64)
        mx = fmaxf(mx, ml[i].x);
    const float M = group_max<64>(mx);
    const float c = lane < npart ? fast_exp2(mlv.x - M) : 0.f;
    float L = lane < npart ? mlv.y * c : 0.f;
    for (int i = lane + 64; i < npart; i += 64) {
        const float2 v = ml[i];
        L = fmaf(v.y, fast_exp2(v.x - M), L);
    }
    L = group_sum<64>(L);

    float A[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        A[e] = 0.f;
#pragma unroll
    for (int i = 0; i < REDUCE_FEW; ++i) {
        if (i < npart) {
            const float ci = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), i));
#pragma unroll
            for (int e = 0; e < E; ++e)
                A[e] = fmaf(a[i][e], ci, A[e]);
        }
    }
    for (int i = REDUCE_FEW; i < npart; ++i) {
        const float ci = i < 64 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), i))
                                : fast_exp2(ml[i].x - M);
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (lane + 64 * e < D)
                A[e] = fmaf(acc[(int64_t)i * D + lane + 64 * e], ci, A[e]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (lane + 64 * e < D)
            Store<T>::one(P.out, sh * D + lane + 64 * e, L > 0.f ? A[e] / L : 0.f);
}

// ---------------------------------------------------------------------------
// host-side dispatch over the compile-time shape
// ---------------------------------------------------------------------------
constexpr int DECODE_WAVES = 4;

template <typename T, int D, int BS, int GT>
hipError_t launch_decode_shape(const DecodeParams &p, hipStream_t st)
{
    dim3 grid(p.max_partitions - p.first_partition, p.num_kv_heads * p.group_split, p.num_seqs);
    if (p.kv_cached)
        hipLaunchKernelGGL((decode_vec_kernel<T, D, BS, GT, DECODE_WAVES, false>), grid, dim3(DECODE_WAVES * 64), 0, st, p);
    else
        hipLaunchKernelGGL((decode_vec_kernel<T, D, BS, GT, DECODE_WAVES, true>), grid, dim3(DECODE_WAVES * 64), 0, st, p);
    return hipGetLastError();
}

template <typename T, int D, int BS>
hipError_t launch_decode_gt(const DecodeParams &p, int gt, hipStream_t st)
{
    switch (gt) {
    case 1: return launch_decode_shape<T, D, BS, 1>(p, st);
    case 2: return launch_decode_shape<T, D, BS, 2>(p, st);
    case 4: return launch_decode_shape<T, D, BS, 4>(p, st);
    case 8: return launch_decode_shape<T, D, BS, 8>(p, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int D>
hipError_t launch_decode_bs(const DecodeParams &p, int bs, int gt, hipStream_t st)
{
    switch (bs) {
    case 8: return launch_decode_gt<T, D, 8>(p, gt, st);
    case 16: return launch_decode_gt<T, D, 16>(p, gt, st);
    case 32: return launch_decode_gt<T, D, 32>(p, gt, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_decode_dtype(const DecodeParams &p, int head_dim, int bs, int gt, hipStream_t st)
{
    switch (head_dim) {
    case 32: return launch_decode_bs<T, 32>(p, bs, gt, st);
    case 64: return launch_decode_bs<T, 64>(p, bs, gt, st);
    case 128: return launch_decode_bs<T, 128>(p, bs, gt, st);
    case 256: return launch_decode_bs<T, 256>(p, bs, gt, st);
    default: return hipErrorInvalidValue;
    }
}

// Balanced schedule: launch (occ == nullptr) or report the workgroups per
// compute unit of the stream kernel for this shape (occ != nullptr).
template <typename T, int D, int BS, int GT>
hipError_t vec_stream_shape(const DecodeParams *p, hipStream_t st, int *occ)
{
    // the two load policies compile to the same registers: the occupancy of one is that of both
    if (occ) {
        *occ = stream_occupancy<VecWorker<T, D, BS, GT, true>, BS>();
        return hipSuccess;
    }
    return p->kv_cached ? launch_stream<VecWorker<T, D, BS, GT, false>, BS>(*p, st)
                        : launch_stream<VecWorker<T, D, BS, GT, true>, BS>(*p, st);
}

template <typename T, int D, int BS>
hipError_t vec_stream_gt(const DecodeParams *p, int gt, hipStream_t st, int *occ)
{
    switch (gt) {
    case 1: return vec_stream_shape<T, D, BS, 1>(p, st, occ);
    case 2: return vec_stream_shape<T, D, BS, 2>(p, st, occ);
    case 4: return vec_stream_shape<T, D, BS, 4>(p, st, occ);
    case 8: return vec_stream_shape<T, D, BS, 8>(p, st, occ);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int D>
hipError_t vec_stream_bs(const DecodeParams *p, int bs, int gt, hipStream_t st, int *occ)
{
    switch (bs) {
    case 8: return vec_stream_gt<T, D, 8>(p, gt, st, occ);
    case 16: return vec_stream_gt<T, D, 16>(p, gt, st, occ);
    case 32: return vec_stream_gt<T, D, 32>(p, gt, st, occ);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t vec_stream_dtype(const DecodeParams *p, int head_dim, int bs, int gt, hipStream_t st, int *occ)
{
    switch (head_dim) {
    case 32: return vec_stream_bs<T, 32>(p, bs, gt, st, occ);
    case 64: return vec_stream_bs<T, 64>(p, bs, gt, st, occ);
    case 128: return vec_stream_bs<T, 128>(p, bs, gt, st, occ);
    case 256: return vec_stream_bs<T, 256>(p, bs, gt, st, occ);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
