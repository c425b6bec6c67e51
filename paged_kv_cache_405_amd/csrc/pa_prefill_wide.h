// pa_prefill_wide.h -- multi-token paged attention at head_dim 128 on the
// 32x32x16 matrix-core products of gfx950 (v_mfma_f32_32x32x16_{f16,bf16}).
//
// Method: "vLLM 与 PagedAttention" (inference.mavenzero.com/case-studies/vllm),
// section 二: K/V sit in fixed-size blocks reached through the sequence's
// block table and are read block by block, the per-block results merged by an
// online softmax; section 六 ("关键的工程优化"): a long prompt is prefilled in
// chunks.  Query row i of a chunk of n rows over a context of L tokens sits at
// position L - n + i and attends tokens 0 .. L - n + i (causal).
//
// A prefill reads each key for many query rows, so the work is a dense
// product per (sequence, kv head) and wants the widest matrix tiles the
// registers allow.  One wave owns 32 score columns -- 32 / gh query rows
// times the gh q heads of one kv head -- and takes the keys 32 at a time:
//
//   S^T[32 keys x 32 cols] = K . Q^T     one per step, 8 products (d = 128)
//       A operand K from LDS (lane l: key l % 32, dims 16c + 8(l / 32) .. +8),
//       B operand Q held in registers for the whole kernel.  Lane l then holds
//       column l % 32 at keys 8(v / 4) + 4(l / 32) + v % 4 of the tile, v < 16.
//   softmax   per column: the lane and its partner l ^ 32 hold all 32 keys; the
//       reference max changes only when a step's max exceeds it by 2^8, so
//       the accumulators are rarely rescaled.
//   O^T[32 dims x 32 cols] += V^T . P^T  four dim tiles x two 16-key chunks
//       B operand P^T straight from the lane's own probabilities (the eight of
//       chunk c are registers 8c .. +8 of the scores: keys 16c +
//       {4h .. 4h + 3, 8 + 4h .. 8 + 4h + 3} for h = l / 32), A operand V^T
//       read from LDS with two transposed reads (ds_read_b64_tr_b16) whose
//       keys follow that same order.
//
// The four waves of a workgroup (128 columns) share each step's K and V
// tiles, staged in LDS by direct-to-LDS loads (no registers), three steps in
// rotation, so the loads run two steps (64 keys) ahead of the products.  The
// 48 KB of stages and 156 registers a lane let three workgroups -- three
// waves per SIMD -- share a CU, whose other waves hide a wave's load and
// product latencies.  A tile is 32 rows of 256 bytes, written in 1 KiB
// pieces of four rows; inside a piece, 16-byte unit u of row k sits at slot
// 16 (k % 4) + (u ^ s(k)) with s(k) = 4 (k % 4) + (k / 4) % 4.  Each
// 16-lane group of a load then reads one whole 256-byte row (coalesced), the
// K operand reads (16 rows, one unit) and the transposed V reads (4 rows x 4
// units per 32 lanes) fall on distinct LDS banks.
//
// Rows past the context or in a block outside the pool are staged as zeros
// (their loads read a zero buffer), and partial steps (the causal diagonal,
// the context's end, such blocks) mask the scores to -inf: whatever that
// memory holds -- NaN included -- never reaches the accumulators.  f16 rounds P once and the
// running sum adds the rounded values (v_dot2_f32_f16); bf16 keeps P as
// hi + lo in two products.
//
// Shared prefix ("vLLM 与 PagedAttention" section 四, prefix caching: requests
// that reuse a cached prompt point at its blocks).  The same kernel in two
// launches: WIDE_OWN runs each sequence from the last whole step inside the
// shared prefix on and writes each (row, q head)'s (reference max, sum,
// unnormalised output); WIDE_PREFIX then takes the steps below that split
// once, with the rows of every sequence packed as the columns (each capped at
// its own causal limit), merges each column's partial and normalises.  The
// long pass, whose memory is idle under its products, carries the merge's
// loads and the output's stores.  Merging two online-softmax partials is
// exact up to rounding, as for split-K decode.
#pragma once

#include <type_traits>

#include "pa_decode_gqa.h"
#include "pa_device.h"

namespace pa {

typedef float wide_f32x16 __attribute__((ext_vector_type(16)));

template <typename T> struct WideOps;
template <> struct WideOps<f16_t> {
    __device__ __forceinline__ static wide_f32x16 mma(const uint4 &a, const uint4 &b, wide_f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(gqa_f16x8, a),
                                                      __builtin_bit_cast(gqa_f16x8, b), c, 0, 0, 0);
    }
};
template <> struct WideOps<bf16_t> {
    __device__ __forceinline__ static wide_f32x16 mma(const uint4 &a, const uint4 &b, wide_f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(gqa_bf16x8, a),
                                                       __builtin_bit_cast(gqa_bf16x8, b), c, 0, 0, 0);
    }
};

constexpr int WIDE_WAVES = 4;                        // waves per workgroup
constexpr int WIDE_COLS = 32;                        // score columns per wave
constexpr int WIDE_STEP = PREFILL_WIDE_STEP;         // the shared-prefix split's unit (keys)
constexpr int WIDE_SK = 32;                          // keys per step of the kernel
constexpr int WIDE_LDS = 3 * 2 * WIDE_SK * 256;      // LDS of the tile stages: three steps of K and V (48 KB)
constexpr int WIDE_WAVES_PER_EU = 3;                 // three workgroups per CU (registers and LDS allow it)
constexpr float WIDE_RESCALE_LOG2 = 8.f;

// what a launch computes (the shared-prefix form runs WIDE_OWN, then WIDE_PREFIX)
constexpr int WIDE_PLAIN = 0;    // every row over its whole causal history
constexpr int WIDE_PREFIX = 1;   // the shared prefix only, the rows of all sequences as columns, merged with
                                 // the own pass's partials
constexpr int WIDE_OWN = 2;      // each sequence's keys past the prefix: partials out

// the sequence whose rows hold q row r: the largest s < num_seqs with
// query_start[s] <= r (r wave-uniform).  Each round narrows the range with 64
// probes, one per lane (three rounds cover 65535 sequences); entries out of
// order end the search early, never out of range.
__device__ __forceinline__ int wide_seq_of_row(const DecodeParams &P, int r)
{
    const int lane = threadIdx.x & 63;
    int lo = 0, hi = P.num_seqs;
    while (hi - lo > 1) {
        const int step = (hi - lo + 63) / 64;
        const int k = lo + lane * step;
        const uint64_t m = __ballot(k < hi && P.query_start[k] <= r);
        if (m == 0)
            break;
        const int last = 63 - __builtin_clzll(m);
        lo = __builtin_amdgcn_readfirstlane(lo + last * step);
        hi = __builtin_amdgcn_readfirstlane(min(hi, lo + step));
    }
    return lo;
}

__device__ __forceinline__ int wide_wave_min(int x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
        x = min(x, __shfl_xor(x, off));
    return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ int wide_wave_max(int x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
        x = max(x, __shfl_xor(x, off));
    return __builtin_amdgcn_readfirstlane(x);
}

// the source of every direct-load lane whose row lies past the context or in a
// block outside the pool
static __device__ __attribute__((aligned(16))) const uint4 wide_zero = {0u, 0u, 0u, 0u};

// MODE: WIDE_PLAIN, WIDE_PREFIX or WIDE_OWN (above).  The shared prefix holds
// P.part_base_blocks blocks, split at its last whole step: in WIDE_PREFIX the
// keys are the tokens below the split (table row 0) and one virtual sequence
// holds all total_q rows, each column capped at its own sequence's causal
// limit and written only where the own pass computed the row (P.own_rows
// rows of each sequence); in WIDE_OWN each sequence's keys start at the split.
template <typename T, int BS, int MODE>
__global__ __launch_bounds__(WIDE_WAVES * 64) __attribute__((amdgpu_waves_per_eu(WIDE_WAVES_PER_EU))) void prefill_wide_kernel(
    const DecodeParams P, int col_groups, int total_wg)
{
    constexpr int D = 128;
    constexpr int ES = 2;
    constexpr bool HILO = std::is_same<T, bf16_t>::value;
    constexpr int SK = WIDE_SK;                        // keys per step
    static_assert(SK == 32 || SK == 64, "keys per step");
    static_assert(WIDE_LDS % (2 * SK * 256) == 0 && WIDE_LDS / (2 * SK * 256) >= 2 && WIDE_LDS / (2 * SK * 256) <= 4,
                  "two to four stages");
    static_assert(WIDE_STEP % SK == 0, "the shared-prefix split is a step boundary");
    constexpr int TILE = SK * 256;                     // bytes of K (or V) per step at head_dim 128
    constexpr int STAGE = 2 * TILE;                    // K then V
    constexpr int NST = WIDE_LDS / STAGE;              // stages in rotation: loads run NST - 1 steps ahead
    constexpr int KT = SK / 32;                        // 32-key score tiles per step
    constexpr int NCH = SK / 16;                       // 16-key chunks of the weighted sums per step
    constexpr int PPW = SK / 8;                        // 1 KiB pieces each wave loads per step
    constexpr int RPW = SK / 2;                        // rows of K (or V) each wave loads per step
    constexpr int NE = SK / BS;                        // table entries per step
    static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
    __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[NST * STAGE];
    unsigned char PA_LDS *const lds = (unsigned char PA_LDS *)lds_raw;

    // logical workgroups XCD-major (dispatch puts workgroup b on XCD b % 8):
    // the column groups of one (head group, sequence) run together on one XCD
    const int per_xcd = (total_wg + 7) / 8;
    const int lg_id = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (lg_id >= total_wg)
        return;
    const int HG = P.num_kv_heads * P.group_split;
    const int cg = lg_id % col_groups;
    const int hg = (lg_id / col_groups) % HG;
    const int s = lg_id / col_groups / HG;

    const int cap = P.max_blocks * BS;
    // the passes split the keys at the last whole step inside the shared prefix: the prefix pass takes the
    // steps below it, unmasked by the prefix's end, and the own pass starts on a step boundary
    const int prefix_tok = MODE == WIDE_PLAIN ? 0 : wide_prefix_split(P.part_base_blocks, BS);
    // the keys this launch reads end at ctx; its rows are q[q_first .. q_first + nq)
    int ctx, q_first, nq;
    if constexpr (MODE == WIDE_PREFIX) {
        ctx = prefix_tok;
        q_first = 0;
        nq = P.total_q;
    } else {
        ctx = P.ctx[s];
        ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
        q_first = P.query_start[s];
        nq = P.query_start[s + 1] - q_first;
        if (q_first < 0 || q_first >= P.total_q)
            return;
        nq = nq > P.total_q - q_first ? P.total_q - q_first : nq;
    }
    const int gh = P.group / P.group_split;
    const int R = WIDE_COLS / gh;                       // query rows per wave
    const int ncols = R * gh;
    const int i0g = cg * WIDE_WAVES * R;
    if (i0g >= nq)
        return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i0 = i0g + wave * R;
    const bool wave_on = i0 < nq;
    const int j = lane & 31;                            // score column
    const int h = lane >> 5;                            // key half of the column's scores
    const int row = i0 + j / gh;
    const bool on = wave_on && j < ncols && row < nq;
    auto limit = [&](int r) { const int t = ctx - nq + r + 1; return t < 0 ? 0 : (t > ctx ? ctx : t); };
    int t_full, t_hi, wave_end, n_steps;   // every column of the wave sees keys below t_full; this column's keys
                                           // are [0, t_hi); the wave's below wave_end; the workgroup's n_steps steps
    bool own_done = true;                  // WIDE_PREFIX: the own pass wrote this column's partial
    if constexpr (MODE == WIDE_PREFIX) {
        // each column's own sequence caps it: its row's causal limit, within the prefix
        int lim = 0;
        if (wave_on) {
            const int r_last = min(i0 + R, nq) - 1;
            int sj = wide_seq_of_row(P, i0);
            for (int s2 = sj + 1; s2 < P.num_seqs; ++s2) {
                const int b = __builtin_amdgcn_readfirstlane(P.query_start[s2]);
                if (b > r_last)
                    break;
                if (row >= b)
                    sj = s2;
            }
            int c = P.ctx[sj];
            c = c < 0 ? 0 : (c > cap ? cap : c);
            const int qf = P.query_start[sj];
            int n = P.query_start[sj + 1] - qf;
            n = n > P.total_q - qf ? P.total_q - qf : n;
            const int t = c - n + (row - qf) + 1;
            lim = t < 0 ? 0 : (t > c ? c : t);
            // the rows the own pass computed: a sequence whose rows start inside q, the first own_rows of them
            own_done = qf >= 0 && qf < P.total_q && row - qf < n && row - qf < P.own_rows;
        }
        const int mine = on ? (lim < prefix_tok ? lim : prefix_tok) : prefix_tok;
        t_full = wide_wave_min(mine);
        t_hi = on ? mine : t_full;
        wave_end = wave_on ? wide_wave_max(on ? mine : 0) : 0;
        n_steps = (prefix_tok + SK - 1) / SK;
    } else {
        t_full = limit(i0);
        t_hi = on ? limit(row) : t_full;
        wave_end = wave_on ? limit(min(i0 + R, nq) - 1) : 0;
        const int wg_end = limit(min(i0g + WIDE_WAVES * R, nq) - 1);
        n_steps = (wg_end + SK - 1) / SK;
    }
    // WIDE_OWN: the keys below the split are the prefix pass's (the split is a step boundary)
    const int t_lo = MODE == WIDE_OWN ? prefix_tok : 0;
    const int s_first = t_lo / SK;

    const int kvh = hg / P.group_split;
    const int qh0 = kvh * P.group + (hg - kvh * P.group_split) * gh;
    const int64_t blk_bytes = P.block_stride * ES;
    const int64_t tok_bytes = P.token_stride * ES;
    const char *kpool = static_cast<const char *>(P.k) + (int64_t)kvh * P.head_stride * ES;
    const char *vpool = static_cast<const char *>(P.v) + (int64_t)kvh * P.head_stride * ES;
    const int32_t __attribute__((address_space(4))) *trow =
        (const int32_t __attribute__((address_space(4))) *)(P.tables + (int64_t)s * P.max_blocks);
    const int nblk = (ctx + BS - 1) / BS;
    const int num_blocks = P.num_blocks;
    const float sl2 = P.scale_log2;

    // Q^T operand of column j: dims 16c + 8h .. +8 for c < 8.  Every lane
    // loads (an idle column reads the sequence's first row) and the select
    // waits for the loads here: none is still counted as in flight inside
    // the loop, whose own vector-memory waits must cover the tile loads only
    uint4 qb[8];
    {
        const char *qp = static_cast<const char *>(P.q) +
                         (((int64_t)(q_first + (on ? row : 0)) * P.num_q_heads + qh0 + (on ? j % gh : 0)) * D + 8 * h) *
                             ES;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint4 v = ld16(qp + 32 * c);
            qb[c] = on ? v : make_uint4(0u, 0u, 0u, 0u);
        }
    }

    // direct loads: lane p brings row p / 16 of the piece, unit (p % 16) ^ s(row)
    // (rows are a multiple of 256 bytes apart, so piece jj's unit is ld_addr ^ 16 (jj % 4))
    uint32_t ld_addr = (uint32_t)((lane >> 4) * tok_bytes) + (uint32_t)((16 * (lane & 15)) ^ (64 * (lane >> 4)));
    // K operand: key l % 32 of the tile, unit 2c + h
    const int kl = lane & 31;
    // (row offset 1024 (kl / 4) + 256 (kl % 4), unit k_x ^ 2c: byte k_addr ^ 32c of the tile)
    uint32_t k_addr = (1024 * (kl >> 2) + 256 * (kl & 3)) | (16u * (uint32_t)(h ^ (4 * (kl & 3) + ((kl >> 2) & 3))));
    // V operand, transposed reads: source lane (group g, index i) addresses key
    // 16c + 8rho + 4h + i / 4, dims 32dt + 16(g % 2) + 4(i % 4) .. +4
    const int vi = lane & 15;
    const int vgd = (lane >> 4) & 1;
    // (dim tile dt at byte v_addr ^ 64dt of a 16-key chunk, the second read at that ^ 32, 2048 on)
    uint32_t v_addr = (1024 * h + 256 * (vi >> 2) + 16 * ((2 * vgd + ((vi & 3) >> 1)) ^ h) + 8 * (vi & 1)) | (64 * (vi >> 2));

    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    // the table entries of a step (clamped to the sequence's last block; a
    // block past it holds only rows past the context).  Each step's entries
    // are fetched a step before its tile loads are issued, so the scalar
    // loads have a whole step's products to land in.
    auto fetch = [&](int step, int (&ent)[NE]) {
        const int b = step * NE;
        if (b + NE <= nblk) {
#pragma unroll
            for (int e = 0; e < NE; ++e)
                ent[e] = trow[b + e];
        } else {
#pragma unroll
            for (int e = 0; e < NE; ++e)
                ent[e] = trow[min(b + e, nblk - 1)];
        }
    };

    // step `step` into stage `st`: waves 0-1 bring K, 2-3 bring V, PPW 1 KiB
    // pieces each (rows RPW (wave % 2) + 4jj .. +4 of the step).  A row past
    // the context or in a block outside the pool is read from 16 zero bytes
    // instead: its K scores are masked, and its V row, all zero, adds nothing
    // (the products never see what such memory holds)
    auto issue = [&](int step, int st, const int (&ent)[NE]) {
        const int tok = step * SK + RPW * (wave & 1);
        const char *pool = (wave >> 1) ? vpool : kpool;
        const uint32_t dst = lds0 + st * STAGE + (wave >> 1) * TILE + (TILE / 2) * (wave & 1);
        constexpr int PER_BLK = BS / 4 < PPW ? BS / 4 : PPW;   // pieces per block entry
#pragma unroll
        for (int g = 0; g < PPW / PER_BLK; ++g) {
            // the entry of the group's rows in either half (constant indices: the array stays in registers)
            const int lo_e = ent[(4 * PER_BLK * g) / BS], hi_e = ent[(RPW + 4 * PER_BLK * g) / BS];
            const int raw = (wave & 1) ? hi_e : lo_e;
            const int row0 = (RPW * (wave & 1) + 4 * PER_BLK * g) % BS;   // the group's first row in its block
            const bool mapped = (unsigned)raw < (unsigned)num_blocks;
            const char *blk = pool + (uint64_t)(uint32_t)(mapped ? raw : 0) * (uint64_t)blk_bytes +
                              (int64_t)row0 * tok_bytes;
            const int t_e = tok + 4 * PER_BLK * g;             // first row of the group's pieces
            if (mapped && t_e + 4 * PER_BLK <= ctx) {
#pragma unroll
                for (int i = 0; i < PER_BLK; ++i) {
                    const int jj = g * PER_BLK + i;
                    load_lds_sbase<false>(blk + (int64_t)(4 * i) * tok_bytes,
                                          (ld_addr ^ (16u * (jj & 3))), dst + 1024 * jj);
                }
            } else {
#pragma unroll
                for (int i = 0; i < PER_BLK; ++i) {
                    const int jj = g * PER_BLK + i;
                    const bool ok = mapped && t_e + 4 * i + (lane >> 4) < ctx;
                    const char *src = blk + (int64_t)(4 * i) * tok_bytes + (ld_addr ^ (16u * (jj & 3)));
                    load_lds_asm<false>(ok ? src : reinterpret_cast<const char *>(&wide_zero), dst + 1024 * jj);
                }
            }
        }
    };

    wide_f32x16 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc[dt][v] = 0.f;
    float m = NEG_BIG;                                  // reference max of column j (log2 units)
    float lp = 0.f;                                     // this lane's share of the column's sum

    // the products and the softmax of one step
    auto compute = [&](int t0, uint32_t okm, auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        const unsigned char PA_LDS *stg = lds + ST * STAGE;
        // (a negative scale also takes the masked path: the other one takes the
        // max of the raw scores)
        const bool masked = t0 + SK > t_full || t0 + SK > ctx || okm != (1u << NE) - 1u ||
                            !(sl2 >= 0.f) || (MODE == WIDE_OWN && t0 < t_lo);

        // all the K fragments of the step are requested before the first
        // product: the reads' latency is paid once per step, not per product
        gqa_u32x4 kf[KT][8];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int c = 0; c < 8; ++c)
                kf[kt][c] = *reinterpret_cast<const gqa_u32x4 PA_LDS *>(stg + 8192 * kt + (k_addr ^ (32u * c)));
        __builtin_amdgcn_sched_barrier(0);
        wide_f32x16 sc[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                sc[kt][v] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
                sc[kt] = WideOps<T>::mma(make_uint4(kf[kt][c].x, kf[kt][c].y, kf[kt][c].z, kf[kt][c].w), qb[c], sc[kt]);

        // the step's max of column j in log2 units, and the factor that takes
        // a raw score there (masked steps scale and mask first)
        float mx, f;
        if (masked) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int kr = 32 * kt + 8 * (v >> 2);             // first key of the 8-key group
                    const int key = t0 + kr + 4 * h + (v & 3);
                    const bool ok = ((okm >> (kr / BS)) & 1u) && key < t_hi && (MODE != WIDE_OWN || key >= t_lo);
                    sc[kt][v] = ok ? sc[kt][v] * sl2 : -INFINITY;
                }
            mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    mx = fmaxf(mx, sc[kt][v]);
            f = 1.f;
        } else {
            float hi = sc[0][0];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    hi = fmaxf(hi, sc[kt][v]);
            mx = hi * sl2;
            f = sl2;
        }
        {
            const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
        }
        const bool grow = mx > m + WIDE_RESCALE_LOG2;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float mn = grow ? mx : m;
            const float alpha = fast_exp2(m - mn);
            m = mn;
            lp *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[dt][v] *= alpha;
        }

#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int kt = c >> 1, v0 = 8 * (c & 1);
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                p[e] = fast_exp2(__builtin_fmaf(sc[kt][v0 + e], f, -m));
            uint4 phi, plo = make_uint4(0u, 0u, 0u, 0u);
            if constexpr (HILO) {
                phi = make_uint4(GqaOps<T>::pack(p[0], p[1]), GqaOps<T>::pack(p[2], p[3]),
                                 GqaOps<T>::pack(p[4], p[5]), GqaOps<T>::pack(p[6], p[7]));
                float w[8];
                GqaOps<T>::unpack(phi.x, w[0], w[1]);
                GqaOps<T>::unpack(phi.y, w[2], w[3]);
                GqaOps<T>::unpack(phi.z, w[4], w[5]);
                GqaOps<T>::unpack(phi.w, w[6], w[7]);
                plo = make_uint4(GqaOps<T>::pack(p[0] - w[0], p[1] - w[1]), GqaOps<T>::pack(p[2] - w[2], p[3] - w[3]),
                                 GqaOps<T>::pack(p[4] - w[4], p[5] - w[5]), GqaOps<T>::pack(p[6] - w[6], p[7] - w[7]));
                lp += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            } else {
                phi = make_uint4(GqaOps<T>::pack(p[0], p[1]), GqaOps<T>::pack(p[2], p[3]),
                                 GqaOps<T>::pack(p[4], p[5]), GqaOps<T>::pack(p[6], p[7]));
                const half2v one = {(_Float16)1.f, (_Float16)1.f};
                lp = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, phi.x), one, lp, false);
                lp = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, phi.y), one, lp, false);
                lp = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, phi.z), one, lp, false);
                lp = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, phi.w), one, lp, false);
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const unsigned char PA_LDS *vs = stg + TILE + 4096 * c;
                const uint2 r0 = GqaOps<T>::read_tr(vs + (v_addr ^ (64u * dt)));
                const uint2 r1 = GqaOps<T>::read_tr(vs + 2048 + (v_addr ^ (32u + 64u * dt)));
                const uint4 va = make_uint4(r0.x, r0.y, r1.x, r1.y);
                acc[dt] = WideOps<T>::mma(va, phi, acc[dt]);
                if constexpr (HILO)
                    acc[dt] = WideOps<T>::mma(va, plo, acc[dt]);
            }
        }
    };

    // one step out of stage ST (a constant, so that every LDS read takes its
    // stage as an immediate offset: the loop below runs NST steps per turn).
    // The loads run NST - 1 steps ahead: step t's tiles go to stage
    // (t - s_first) % NST.  ent_n holds the table entries of the step the
    // next issue loads; o0 .. o2 the in-pool blocks (bit e: keys e BS .. +BS)
    // of this step and the next ones already issued.  The next entries are
    // fetched after the products, so that their scalar loads stay in flight
    // across the barrier (which waits for vector loads only: every LDS read
    // of the stage the next loads fill has been consumed by then)
    int ent_n[NE] = {};
    uint32_t o0 = 0u, o1 = 0u, o2 = 0u;
    auto okm_of = [&](const int (&ent)[NE]) {
        uint32_t o = 0u;
#pragma unroll
        for (int e = 0; e < NE; ++e)
            o |= ((unsigned)ent[e] < (unsigned)num_blocks ? 1u : 0u) << e;
        return o;
    };
    auto run_step = [&](int step, auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        // this wave's loads of the step have landed (those of the later steps
        // already issued may still be in flight: loads complete in the order
        // they were issued, PPW per step); at the barrier every wave's have,
        // and every wave is done with the stage the next loads fill
        const int later = min(NST - 2, n_steps - 1 - step);
        if (later <= 0)
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        else if (later == 1)
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(PPW) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * PPW) : "memory");
        // one register per address family: the per-piece and per-fragment
        // addresses are recomputed (one xor each) rather than kept live
        asm volatile("" : "+v"(k_addr), "+v"(v_addr), "+v"(ld_addr));
        if (step + NST - 1 < n_steps)
            issue(step + NST - 1, (ST + NST - 1) % NST, ent_n);
        const uint32_t okm = o0;
        const uint32_t on = okm_of(ent_n);
        if constexpr (NST == 2) {
            o0 = on;
        } else if constexpr (NST == 3) {
            o0 = o1;
            o1 = on;
        } else {
            o0 = o1;
            o1 = o2;
            o2 = on;
        }
        const int t0 = step * SK;
        if (t0 < wave_end)
            compute(t0, okm, st_c);
        if (step + NST < n_steps)
            fetch(step + NST, ent_n);
    };

    if (n_steps > s_first) {
#pragma unroll
        for (int i = 0; i < NST - 1; ++i) {
            if (s_first + i < n_steps) {
                int e0[NE];
                fetch(s_first + i, e0);
                issue(s_first + i, i, e0);
                const uint32_t o = okm_of(e0);
                if (i == 0)
                    o0 = o;
                else if (i == 1)
                    o1 = o;
                else
                    o2 = o;
            }
        }
        if (s_first + NST - 1 < n_steps)
            fetch(s_first + NST - 1, ent_n);
    }
    for (int step = s_first; step < n_steps; step += NST) {
        run_step(step, std::integral_constant<int, 0>());
        if (step + 1 < n_steps)
            run_step(step + 1, std::integral_constant<int, 1>());
        if constexpr (NST > 2) {
            if (step + 2 < n_steps)
                run_step(step + 2, std::integral_constant<int, 2 % NST>());
        }
        if constexpr (NST > 3) {
            if (step + 3 < n_steps)
                run_step(step + 3, std::integral_constant<int, 3 % NST>());
        }
    }

    // every load into LDS has landed before the workgroup ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!wave_on)
        return;
    {
        const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(lp), __float_as_uint(lp), false, false);
        lp = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    }
    if (!on)
        return;
    const int64_t col = (int64_t)(q_first + row) * P.num_q_heads + qh0 + j % gh;   // (q row, q head)
    if constexpr (MODE == WIDE_OWN) {
        // the column's partial past the split: (reference max, sum, unnormalised output)
        float *ap = P.ws_acc + col * D + 4 * h;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<float4 *>(ap + 32 * dt + 8 * g) =
                    make_float4(acc[dt][4 * g], acc[dt][4 * g + 1], acc[dt][4 * g + 2], acc[dt][4 * g + 3]);
        if (h == 0)
            P.ws_ml[col] = make_float2(m, lp);
        return;
    }
    if constexpr (MODE == WIDE_PREFIX) {
        // merge the own pass's partial of the column (a row it did not compute stays as it is)
        if (!own_done)
            return;
        const float2 mlp = P.ws_ml[col];
        const float *ap = P.ws_acc + col * D + 4 * h;
        float4 pa[4][4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                pa[dt][g] = *reinterpret_cast<const float4 *>(ap + 32 * dt + 8 * g);
        const float mm = fmaxf(m, mlp.x);
        const float a = fast_exp2(m - mm), b = fast_exp2(mlp.x - mm);
        lp = lp * a + mlp.y * b;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                acc[dt][4 * g] = acc[dt][4 * g] * a + pa[dt][g].x * b;
                acc[dt][4 * g + 1] = acc[dt][4 * g + 1] * a + pa[dt][g].y * b;
                acc[dt][4 * g + 2] = acc[dt][4 * g + 2] * a + pa[dt][g].z * b;
                acc[dt][4 * g + 3] = acc[dt][4 * g + 3] * a + pa[dt][g].w * b;
            }
    }
    const float inv = lp > 0.f ? 1.f / lp : 0.f;
    char *op = static_cast<char *>(P.out) +
               (col * D + 4 * h) * ES;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                o[r] = acc[dt][4 * g + r] * inv;
            uint2 w;
            if constexpr (HILO) {
                w.x = (uint32_t)f32_to_bf16_bits(o[0]) | ((uint32_t)f32_to_bf16_bits(o[1]) << 16);
                w.y = (uint32_t)f32_to_bf16_bits(o[2]) | ((uint32_t)f32_to_bf16_bits(o[3]) << 16);
            } else {
                w.x = (uint32_t)f32_to_f16_bits(o[0]) | ((uint32_t)f32_to_f16_bits(o[1]) << 16);
                w.y = (uint32_t)f32_to_f16_bits(o[2]) | ((uint32_t)f32_to_f16_bits(o[3]) << 16);
            }
            *reinterpret_cast<uint2 *>(op + (32 * dt + 8 * g) * ES) = w;
        }
}

// WIDE_PREFIX: one virtual sequence of p.total_q rows (max_query_len unused)
template <typename T, int BS, int MODE = WIDE_PLAIN>
hipError_t launch_prefill_wide(const DecodeParams &p, int max_query_len, hipStream_t st)
{
    const int rows = WIDE_COLS / (p.group / p.group_split);
    const int per_wg = WIDE_WAVES * rows;
    const int n_rows = MODE == WIDE_PREFIX ? p.total_q : max_query_len;
    const int col_groups = (n_rows + per_wg - 1) / per_wg;
    const long long total =
        (long long)col_groups * p.num_kv_heads * p.group_split * (MODE == WIDE_PREFIX ? 1 : p.num_seqs);
    if (total > (1LL << 30))
        return hipErrorInvalidValue;
    if (total == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((total + 7) / 8 * 8));
    hipLaunchKernelGGL((prefill_wide_kernel<T, BS, MODE>), grid, dim3(WIDE_WAVES * 64), 0, st, p, col_groups,
                       (int)total);
    return hipGetLastError();
}

// the shared-prefix form: each sequence's own keys, then the prefix pass over all rows (which merges)
template <typename T, int BS>
hipError_t launch_prefill_shared_wide(const DecodeParams &p, int max_query_len, hipStream_t st)
{
    const int per_wg = WIDE_WAVES * (WIDE_COLS / (p.group / p.group_split));
    DecodeParams q = p;
    q.own_rows = (max_query_len + per_wg - 1) / per_wg * per_wg;   // the rows the own pass's grid covers
    const hipError_t e = launch_prefill_wide<T, BS, WIDE_OWN>(q, max_query_len, st);
    if (e != hipSuccess)
        return e;
    return launch_prefill_wide<T, BS, WIDE_PREFIX>(q, max_query_len, st);
}

}  // namespace pa
