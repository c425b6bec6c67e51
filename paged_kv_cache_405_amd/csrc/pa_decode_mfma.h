// pa_decode_mfma.h -- paged decode attention for grouped-query heads on the
// CDNA4 matrix cores (gfx950).
//
// Method: "vLLM 与 PagedAttention" (inference.mavenzero.com/case-studies/vllm),
// section 二: a sequence's K/V history sits in fixed-size blocks of a shared
// pool reached through its block table ("PagedAttention 的解法"); attention
// reads K/V block by block and accumulates the per-block results ("注意力计算
// 改造").  The accumulation is an online softmax (running max m, running sum
// l, unnormalised output acc rescaled by exp(m_old - m_new)); partitions of a
// long context are merged the same way by the reduce kernel.
//
// When G query heads share one kv head, the G dot products against a K row
// and the G weighted sums of a V row form a small dense contraction.  One
// wave handles a 16-token tile of one kv head against up to 16 query heads:
//
//   scores  S^T[16 tok x 16 heads] = K[16 tok x D] . Q^T[D x 16 heads]
//           D/32 v_mfma_f32_16x16x32_{bf16,f16}: lane l holds K row (l % 16),
//           dims [32c + 8(l/16), +8) -- one 16-byte load -- as the A operand,
//           and q head (l % 16) over the same dims as the B operand.  The
//           result gives lane l the scores of head (l % 16) for tokens
//           4(l/16) + r, r = 0..3.
//   output  O^T[D x 16 heads] += V^T[D x 4 tok] . P^T[4 tok x 16 heads]
//           v_mfma_f32_16x16x4_f32, fp32 operands: lane l supplies one V
//           element as A[row l%16][k l/16] and one probability as
//           B[k l/16][col l%16].  Step i of the tile takes tokens 4k' + i
//           (k' = 0..3) -- a permutation of the tile's tokens, which a sum over
//           tokens does not see -- so lane l's own score r = i is exactly the
//           B element it must supply, and its V element comes from a 16-byte
//           load of token 4(l/16) + i, dims [8(l%16), +8): four such loads
//           cover the tile in 256-byte runs.  Element e of the load feeds the
//           e-th accumulator, whose rows are dims 8(4(l/16) + r) + e.
//
// Probabilities stay fp32 all the way (no rounding of P to 16 bits), and K
// and q enter the score MFMA exactly as stored, so the products are exact.
// Heads past the group (the tile has 16 columns, G may be smaller) see q = 0
// and are never written.  Tokens outside the context, outside the partition
// or in an unmapped block get score -inf and a V row of zeros (a select, not
// a product, so whatever the memory holds cannot leak in).
#pragma once

#include "pa_device.h"
#include "pa_stream.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T> struct ScoreMfma;
template <> struct ScoreMfma<bf16_t> {
    __device__ __forceinline__ static f32x4_t run(const uint4 &a, const uint4 &b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
};
template <> struct ScoreMfma<f16_t> {
    __device__ __forceinline__ static f32x4_t run(const uint4 &a, const uint4 &b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
};

constexpr int MFMA_TILE = 16;   // tokens per wave step
constexpr int MFMA_MAX_HEADS = 16;

// One wave's share of the work on one (sequence, kv head): the online-softmax
// state of up to 16 query heads, and the tile pipeline that feeds it.
//
// Pipeline.  Two register buffers alternate (ping-pong, no copies): while
// the wave computes tile k from one buffer, the loads of its next tile are in
// flight into the other, so the wait before a tile's math is for that tile's
// loads only (vmcnt of one tile), never for the loads behind it.  Block-table
// entries are wave-uniform and read with scalar loads one tile further ahead;
// scalar loads are counted apart from vector loads, so a table lookup never
// waits behind K/V traffic.
template <typename T, int D, int BS>
struct MfmaWorker {
    static constexpr int ES = 2;
    static constexpr int NC = D / 32;      // score MFMAs per tile (32 dims each)
    static constexpr int NU = D / 128;     // 16-byte V chunks per lane per token row
    using V = Vec<T>;

    struct Buf {
        uint4 k[NC];
        uint4 v[4][NU];
        bool okv;
    };

    static constexpr int STEP_TOK = MFMA_TILE;   // tokens per step of the schedule

    // the unit bound to the worker: a sequence and up to 16 q heads of one kv head
    int seq, qh0, gh;
    // addressing of one (sequence, kv head)
    const char *kbase;        // K of this kv head, plus this lane's dim offset in a K row
    const char *vbase;        // V of this kv head, plus this lane's dim offset in a V row
    const int32_t *trow;      // the sequence's block-table row
    int64_t blk_bytes, tok_bytes;
    int nblk, num_blocks;
    int t_lo, t_hi;           // tokens this worker may use
    float scale_log2;
    int lr, lg;               // lane % 16, lane / 16
    uint4 qb[NC];             // q of head lr (zero past the group): B operand of the scores

    // online softmax state
    f32x4_t acc[NU][8];
    float m;                  // running max of head lr (log2 units), equal in the 4 lane rows
    float lp;                 // running sum over this lane's tokens

    __device__ __forceinline__ void init_lane(int lane) {
        lr = lane & 15;
        lg = lane >> 4;
    }

    // attach the worker to head group hg of sequence s (context ctx, already
    // clamped to the table): q of its heads, its kv head's pools, the table
    // row.  The token window [t_lo, t_hi) is the whole context.
    __device__ __forceinline__ void bind(const DecodeParams &P, int s, int hg, int ctx) {
        const int kvh = hg / P.group_split;
        seq = s;
        gh = P.group / P.group_split;
        qh0 = kvh * P.group + (hg - kvh * P.group_split) * gh;
        const bool on = lr < gh;
        const char *qp = static_cast<const char *>(P.q) +
                         (((int64_t)s * P.num_q_heads + qh0 + (on ? lr : 0)) * D + 8 * lg) * ES;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            qb[c] = ld16(qp + 32 * c * ES);
            if (!on)
                qb[c] = make_uint4(0u, 0u, 0u, 0u);
        }
        blk_bytes = P.block_stride * ES;
        tok_bytes = P.token_stride * ES;
        kbase = static_cast<const char *>(P.k) + (int64_t)kvh * P.head_stride * ES + 8 * lg * ES;
        vbase = static_cast<const char *>(P.v) + (int64_t)kvh * P.head_stride * ES + 8 * lr * ES;
        trow = P.tables + (int64_t)s * P.max_blocks;
        nblk = (ctx + BS - 1) / BS;
        num_blocks = P.num_blocks;
        scale_log2 = P.scale_log2;
        t_lo = 0;
        t_hi = ctx;
    }

    // sum of head lr over all of the wave's tokens (every lane must call it)
    __device__ __forceinline__ float total_l() const {
        const float l = lp + __shfl_xor(lp, 16);
        return l + __shfl_xor(l, 32);
    }

    // the unit was finished by this wave: normalise and store out[seq, qh0 + lr, :]
    __device__ __forceinline__ void finish_out(const DecodeParams &P) const {
        const float l = total_l();
        if (lr >= gh)
            return;
        char *o = static_cast<char *>(P.out) + ((int64_t)seq * P.num_q_heads + qh0 + lr) * D * ES;
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = l > 0.f ? acc[u][e][r] / l : 0.f;
                st16(o + 8 * (4 * lg + r + 16 * u) * ES, V::narrow(v));
            }
    }

    // part of the unit: store the wave's (max, sum, unnormalised output) as piece `piece`
    __device__ __forceinline__ void finish_piece(const DecodeParams &P, int piece) const {
        const float l = total_l();
        if (lr >= gh)
            return;
        float *a = P.piece_acc + ((int64_t)piece * gh + lr) * D;
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float *d = a + 8 * (4 * lg + r + 16 * u);
                st16(d, make_uint4(__float_as_uint(acc[u][0][r]), __float_as_uint(acc[u][1][r]),
                                   __float_as_uint(acc[u][2][r]), __float_as_uint(acc[u][3][r])));
                st16(d + 4, make_uint4(__float_as_uint(acc[u][4][r]), __float_as_uint(acc[u][5][r]),
                                       __float_as_uint(acc[u][6][r]), __float_as_uint(acc[u][7][r])));
            }
        if (lg == 0)
            P.piece_ml[(int64_t)piece * gh + lr] = make_float2(m, l);
    }

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[u][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m = NEG_BIG;
        lp = 0.f;
    }

    // physical blocks of tile kt's rows 0.. and (block size 8) rows 8..:
    // wave-uniform indices, so these are scalar loads
    __device__ __forceinline__ int2 phys(int kt) const {
        const int ja = kt * MFMA_TILE / BS;      // < nblk: a tile starts before t_hi <= ctx
        int2 r;
        r.x = trow[ja];
        r.y = BS < MFMA_TILE ? trow[min(ja + 1, nblk - 1)] : r.x;   // rows past the context are masked
        return r;
    }

    __device__ __forceinline__ void load(int kt, int2 pp, Buf &b) const {
        const int t0 = kt * MFMA_TILE;
        const int pk = (BS < MFMA_TILE && lr >= BS) ? pp.y : pp.x;
        const int pv = (BS < MFMA_TILE && 4 * lg >= BS) ? pp.y : pp.x;
        const bool okk = (unsigned)pk < (unsigned)num_blocks;
        b.okv = (unsigned)pv < (unsigned)num_blocks;
        const char *ka = kbase + (int64_t)(okk ? pk : 0) * blk_bytes + (int64_t)((t0 + lr) % BS) * tok_bytes;
        const char *va = vbase + (int64_t)(b.okv ? pv : 0) * blk_bytes + (int64_t)((t0 + 4 * lg) % BS) * tok_bytes;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            b.k[c] = ld16(ka + 32 * c * ES);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int u = 0; u < NU; ++u)
                b.v[i][u] = ld16(va + i * tok_bytes + 128 * u * ES);
    }

    __device__ __forceinline__ void compute(int kt, const Buf &b) {
        f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c)
            sc = ScoreMfma<T>::run(b.k[c], qb[c], sc);
        const int tv = kt * MFMA_TILE + 4 * lg;
        bool valid[4];
        float sv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tv + r;
            valid[r] = b.okv && t >= t_lo && t < t_hi;
            sv[r] = valid[r] ? sc[r] * scale_log2 : -INFINITY;
        }
        float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m, mx);
        const float alpha = fast_exp2(m - mn);
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            pr[r] = fast_exp2(sv[r] - mn);
        lp = fmaf(lp, alpha, (pr[0] + pr[1]) + (pr[2] + pr[3]));
        m = mn;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[u][e] *= alpha;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                float vf[8];
                V::widen(b.v[i][u], vf);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float a = valid[i] ? vf[e] : 0.f;
                    acc[u][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, pr[i], acc[u][e], 0, 0, 0);
                }
            }
        }
    }

    // tiles kbeg, kbeg + stride, ... below kend (all wave-uniform).  The loop
    // runs over pairs of tiles with a single back edge, and the next tile's
    // loads are issued unconditionally (past the end they reload the last tile
    // and are never used), so the wait before each tile's math is the same on
    // every path: that tile's loads, never the ones issued behind them.
    __device__ __forceinline__ void run(int kbeg, int kend, int stride) {
        if (kbeg >= kend)
            return;
        const int n = (kend - 1 - kbeg) / stride + 1;        // tiles of this wave
        const int klast = kbeg + (n - 1) * stride;
        Buf b0, b1;
        int kt = kbeg;
        load(kt, phys(kt), b0);
        int2 pn = phys(min(kt + stride, klast));
        for (int it = 1; it < n; it += 2) {
            load(min(kt + stride, klast), pn, b1);
            pn = phys(min(kt + 2 * stride, klast));
            __builtin_amdgcn_sched_barrier(0);   // next loads go out before this tile's math
            compute(kt, b0);
            load(min(kt + 2 * stride, klast), pn, b0);
            pn = phys(min(kt + 3 * stride, klast));
            __builtin_amdgcn_sched_barrier(0);
            compute(kt + stride, b1);
            kt += 2 * stride;
        }
        if (n & 1)
            compute(kt, b0);
    }
};

template <typename T, int D, int BS, int NW>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(const DecodeParams P)
{
    static_assert(D % 128 == 0, "the grouped-query kernel needs head_dim 128 or 256");
    static_assert(BS % 8 == 0, "block size 8, 16 or 32");
    using W = MfmaWorker<T, D, BS>;
    constexpr int NU = W::NU;

    const int p = blockIdx.x;
    const int hg = blockIdx.y;
    const int s = blockIdx.z;

    int ctx = P.ctx[s];
    const int cap = P.max_blocks * BS;
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int nblk = (ctx + BS - 1) / BS;
    const int npart = nblk == 0 ? 1 : (nblk + P.partition_blocks - 1) / P.partition_blocks;
    if (p >= npart)
        return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    W w;
    w.init_lane(lane);
    w.bind(P, s, hg, ctx);
    const int gh = w.gh;
    const int qh0 = w.qh0;

    // tokens [t_lo, t_hi) of this partition, covered by 16-token tiles [k0, k1);
    // the waves take the tiles round robin
    const int b0 = p * P.partition_blocks;
    const int b1 = min(nblk, b0 + P.partition_blocks);
    w.t_lo = b0 * BS;
    w.t_hi = min(b1 * BS, ctx);
    const int k0 = w.t_lo / MFMA_TILE;
    const int k1 = (w.t_hi + MFMA_TILE - 1) / MFMA_TILE;
    w.reset();
    w.run(k0 + wave, k1, NW);

    // total of head lr over the wave's tokens
    const int lr = w.lr, lg = w.lg;
    const float l = w.total_l();

    // merge the waves through LDS
    __shared__ float sm_m[NW][MFMA_MAX_HEADS], sm_l[NW][MFMA_MAX_HEADS];
    __shared__ float sm_acc[NW][MFMA_MAX_HEADS][D];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sm_acc[wave][lr][8 * (4 * lg + r + 16 * u) + e] = w.acc[u][e][r];
    if (lg == 0) {
        sm_m[wave][lr] = w.m;
        sm_l[wave][lr] = l;
    }
    __syncthreads();

    const bool single = npart == 1;
    for (int idx = threadIdx.x; idx < gh * D; idx += NW * 64) {
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

constexpr int MFMA_WAVES = 4;

template <typename T, int D, int BS>
hipError_t launch_mfma_shape(const DecodeParams &p, hipStream_t st)
{
    dim3 grid(p.max_partitions, p.num_kv_heads * p.group_split, p.num_seqs);
    hipLaunchKernelGGL((decode_mfma_kernel<T, D, BS, MFMA_WAVES>), grid, dim3(MFMA_WAVES * 64), 0, st, p);
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
    using W = MfmaWorker<T, D, BS>;
    if (occ) {
        *occ = stream_occupancy<W, BS>();
        return hipSuccess;
    }
    return launch_stream<W, BS>(*p, st);
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
