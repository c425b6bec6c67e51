// pa_device.h -- device helpers shared by the gfx950 kernels of the library:
// storage types, 16-byte vector moves, wave64 reductions, the launch
// parameter blocks.  Written for CDNA4 (wave64, DPP within 16-lane rows).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// ---------------------------------------------------------------------------
// storage types: fp32, fp16 and bf16 (bf16 handled as raw 16-bit patterns)
// ---------------------------------------------------------------------------
struct f32_t { using storage = float; };
struct f16_t { using storage = uint16_t; };
struct bf16_t { using storage = uint16_t; };

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Widen the 16 bytes of one uint4 into VEC fp32 values (VEC = 16 / sizeof).
template <typename T> struct Vec;

template <> struct Vec<f32_t> {
    static constexpr int N = 4;
    __device__ __forceinline__ static void widen(const uint4 &u, float *f) {
        f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
    }
    __device__ __forceinline__ static uint4 narrow(const float *f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
};

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x);
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x);

template <> struct Vec<f16_t> {
    static constexpr int N = 8;
    // 8 fp32 values -> 8 f16 (nearest even) in 16 bytes
    __device__ __forceinline__ static uint4 narrow(const float *f) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)f32_to_f16_bits(f[2 * i]) | ((uint32_t)f32_to_f16_bits(f[2 * i + 1]) << 16);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
    __device__ __forceinline__ static void widen2(uint32_t w, float &a, float &b) {
        half2v h = __builtin_bit_cast(half2v, w);
        a = (float)h.x; b = (float)h.y;
    }
    __device__ __forceinline__ static void widen(const uint4 &u, float *f) {
        widen2(u.x, f[0], f[1]); widen2(u.y, f[2], f[3]);
        widen2(u.z, f[4], f[5]); widen2(u.w, f[6], f[7]);
    }
};

template <> struct Vec<bf16_t> {
    static constexpr int N = 8;
    // 8 fp32 values -> 8 bf16 (nearest even) in 16 bytes
    __device__ __forceinline__ static uint4 narrow(const float *f) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)f32_to_bf16_bits(f[2 * i]) | ((uint32_t)f32_to_bf16_bits(f[2 * i + 1]) << 16);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
    __device__ __forceinline__ static void widen2(uint32_t w, float &a, float &b) {
        a = __uint_as_float(w << 16);
        b = __uint_as_float(w & 0xffff0000u);
    }
    __device__ __forceinline__ static void widen(const uint4 &u, float *f) {
        widen2(u.x, f[0], f[1]); widen2(u.y, f[2], f[3]);
        widen2(u.z, f[4], f[5]); widen2(u.w, f[6], f[7]);
    }
};

// fp32 -> storage, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    _Float16 h = (_Float16)x;                 // v_cvt_f16_f32, RNE
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u)      // NaN: keep it a (quiet) NaN
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename T> struct Store;
template <> struct Store<f32_t> {
    __device__ __forceinline__ static void one(void *base, int64_t i, float x) {
        reinterpret_cast<float *>(base)[i] = x;
    }
};
template <> struct Store<f16_t> {
    __device__ __forceinline__ static void one(void *base, int64_t i, float x) {
        reinterpret_cast<uint16_t *>(base)[i] = f32_to_f16_bits(x);
    }
};
template <> struct Store<bf16_t> {
    __device__ __forceinline__ static void one(void *base, int64_t i, float x) {
        reinterpret_cast<uint16_t *>(base)[i] = f32_to_bf16_bits(x);
    }
};

// ---------------------------------------------------------------------------
// 16-byte global moves
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 ld16(const void *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

// A K or V row load.  NT: with the non-temporal hint, for rows that this call
// reads once (private blocks): measured on gfx950, it streams 8 % faster than
// a plain load, and it makes the caches drop the line first, so it is wrong
// for blocks that several sequences read (a shared prefix), which then come
// from HBM again instead of from L2.
typedef unsigned int pa_u32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 ld16_kv(const void *p) {
    if constexpr (NT) {
        const pa_u32x4 v = __builtin_nontemporal_load(static_cast<const pa_u32x4 *>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return ld16(p);
    }
}
__device__ __forceinline__ void st16(void *p, const uint4 &v) {
    *reinterpret_cast<uint4 *>(p) = v;
}

// ---------------------------------------------------------------------------
// wave64 reductions.  Within a 16-lane row: DPP (quad_perm xor 1 and xor 2,
// then half-row and row mirrors, which pair lanes whose partial results are
// already equal within their quad / half row).  Across rows: ds_bpermute.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// keys per step of the head_dim-128 prefill kernel, and the keys its
// shared-prefix form reads once for every row: the whole steps inside a
// prefix of `blocks` blocks of `bs` tokens (host and device)
constexpr int PREFILL_WIDE_STEP = 64;
__host__ __device__ constexpr int wide_prefix_split(int blocks, int bs)
{
    return blocks * bs / PREFILL_WIDE_STEP * PREFILL_WIDE_STEP;
}

constexpr int DPP_XOR1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_HMIRROR = 0x141; // row_half_mirror
constexpr int DPP_MIRROR = 0x140;  // row_mirror

// Sum over aligned groups of W lanes (W = 1, 2, 4, 8, 16, 32, 64); every
// lane of a group receives the group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (W >= 2) x += dpp<DPP_XOR1>(x);
    if constexpr (W >= 4) x += dpp<DPP_XOR2>(x);
    if constexpr (W >= 8) x += dpp<DPP_HMIRROR>(x);
    if constexpr (W >= 16) x += dpp<DPP_MIRROR>(x);
    if constexpr (W >= 32) x += __shfl_xor(x, 16);
    if constexpr (W >= 64) x += __shfl_xor(x, 32);
    return x;
}

template <int W>
__device__ __forceinline__ float group_max(float x) {
    if constexpr (W >= 2) x = fmaxf(x, dpp<DPP_XOR1>(x));
    if constexpr (W >= 4) x = fmaxf(x, dpp<DPP_XOR2>(x));
    if constexpr (W >= 8) x = fmaxf(x, dpp<DPP_HMIRROR>(x));
    if constexpr (W >= 16) x = fmaxf(x, dpp<DPP_MIRROR>(x));
    if constexpr (W >= 32) x = fmaxf(x, __shfl_xor(x, 16));
    if constexpr (W >= 64) x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Finite stand-in for -infinity as the running max: exp2(m_old - m_new)
// stays well defined (1 when both are the stand-in, 0 against a real score).
constexpr float NEG_BIG = -1.0e30f;

// ---------------------------------------------------------------------------
// The tile pipeline shared by the decode workers.  A worker W provides
//   W::Buf                          registers of one tile's K and V loads
//   int2 W::tile_phys(int k)        physical block(s) of tile k (scalar loads)
//   void W::load(int k, int2, Buf&) issue tile k's loads
//   void W::wait<B>(Buf&)           wait until the tile's register loads have
//                                   landed, B = tiles issued after it
//   void W::compute<B>(int k, Buf&) the tile's math
//   W::LOADS_PER_TILE               vector-memory operations load() issues
// and pipeline<STAGES>() runs tiles kbeg, kbeg + stride, ... below kend (all
// wave-uniform) with STAGES buffers in rotation: while tile k is computed,
// the loads of the next STAGES-1 tiles are in flight.  The loop runs over
// groups of STAGES tiles with one back edge and issues every load
// unconditionally (past the end it reloads the last tile, never used), so
// the wait before a tile's math is the same on every path and step: that
// tile's loads, never those issued behind it.  The last n % STAGES tiles
// follow in straight-line code that issues no loads, so there the count of
// loads behind a tile falls by one tile per step.  Every buffer that was
// loaded is waited for exactly once, on every path, whether its tile is
// computed or not: a load whose result the compiler thought unused would
// leave its registers free for other values while the load is still in
// flight.  Table entries are fetched one load ahead, as scalar loads,
// counted apart from the vector loads.
// ---------------------------------------------------------------------------
// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding and leaves the other counters alone (gfx9 encoding:
// vmcnt[3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
__host__ __device__ constexpr int vmcnt_imm(int n) {
    return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8);
}

// tail step I of pipeline(): buffer I has the loads of the STAGES - 2 - I
// buffers after it behind it
template <int STAGES, int I, class W, class B>
__device__ __forceinline__ void pipeline_tail(W &w, B (&b)[STAGES], int kt, int stride, int left)
{
    if constexpr (I < STAGES - 1) {
        w.template wait<STAGES - 2 - I>(b[I]);
        if (I < left)
            w.template compute<STAGES - 2 - I>(kt + I * stride, b[I]);
        pipeline_tail<STAGES, I + 1>(w, b, kt, stride, left);
    }
}

template <int STAGES, class W>
__device__ __forceinline__ void pipeline(W &w, int kbeg, int kend, int stride)
{
    static_assert(STAGES >= 2 && STAGES <= 4, "two to four stages");
    kbeg = __builtin_amdgcn_readfirstlane(kbeg);
    kend = __builtin_amdgcn_readfirstlane(kend);
    stride = __builtin_amdgcn_readfirstlane(stride);
    if (kbeg >= kend)
        return;
    const int n = (kend - 1 - kbeg) / stride + 1;   // tiles of this wave
    const int klast = kbeg + (n - 1) * stride;
    typename W::Buf b[STAGES];
#pragma unroll
    for (int i = 0; i < STAGES; ++i)
        w.bind_buf(b[i], i);
    int2 pn = w.tile_phys(kbeg);
#pragma unroll
    for (int i = 0; i < STAGES - 1; ++i) {
        w.load(min(kbeg + i * stride, klast), pn, b[i]);
        pn = w.tile_phys(min(kbeg + (i + 1) * stride, klast));
    }
    int kt = kbeg;
    int it = 0;
    for (; it + STAGES <= n; it += STAGES) {
#pragma unroll
        for (int i = 0; i < STAGES; ++i) {
            w.load(min(kt + (i + STAGES - 1) * stride, klast), pn, b[(i + STAGES - 1) % STAGES]);
            pn = w.tile_phys(min(kt + (i + STAGES) * stride, klast));
            __builtin_amdgcn_sched_barrier(0);   // the loads go out before this tile's math
            w.template wait<STAGES - 1>(b[i]);
            w.template compute<STAGES - 1>(kt + i * stride, b[i]);
        }
        kt += STAGES * stride;
    }
    pipeline_tail<STAGES, 0>(w, b, kt, stride, n - it);
    // retire every load still in flight (direct-to-LDS loads of unused
    // reloads included) before any LDS slot is reused
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// launch parameters
// ---------------------------------------------------------------------------
struct DecodeParams {
    void *out;
    const void *q;
    const void *k;
    const void *v;
    const int32_t *tables;
    const int32_t *ctx;
    float *ws_acc;            // [S, Hq, P, D] unnormalised partial outputs
    float2 *ws_ml;            // [S, Hq, P] (running max in log2 units, sum)
    int64_t block_stride;     // elements between physical blocks
    int64_t head_stride;      // elements between kv heads inside a block
    int64_t token_stride;     // elements between tokens inside a block
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int max_blocks;           // table row length
    int num_blocks;           // pool size (entries outside [0, num_blocks) contribute nothing)
    int partition_blocks;     // blocks per split-K partition
    int max_partitions;       // P (grid x extent)
    // shared-prefix decode: partitions [0, first_partition) hold the prefix
    // (written by the prefix pass); partition p >= first_partition covers the
    // blocks from part_base_blocks + (p - first_partition) * partition_blocks
    int first_partition;
    int part_base_blocks;
    int group;                // q heads per kv head
    int group_split;          // workgroups sharing one kv head (each takes group/group_split q heads)
    float scale_log2;         // scale * log2(e)
    // balanced (stream) schedule: waves take equal shares of the step stream of
    // all (head group, sequence) units; a unit cut between waves leaves pieces
    int n_waves;              // logical waves of the stream kernel (a multiple of 8)
    int kv_cached;            // 1: blocks may be shared across sequences -- plain (cached) K/V loads
    int order_rows;           // grid kernels: 1 = take sequences longest first (seq_of_row), 0 = in order
    const int32_t *query_start;   // multi-token calls: [num_seqs + 1] first q row of each sequence
    int total_q;                  // multi-token calls: rows of q and out
    int own_rows;                 // shared-prefix prefill: the rows of each sequence its own pass computes
    uint64_t *stream_total;   // [1] steps of the whole stream (T), written by the stream kernel
    int32_t *unit_first;      // [HG * S] first piece of each unit, -1 when one wave finished it
    int32_t *unit_last;       // [HG * S] last piece of each cut unit
    float2 *piece_ml;         // [2 * n_waves][heads per unit] (max in log2 units, sum)
    float *piece_acc;         // [2 * n_waves][heads per unit][D] unnormalised partial outputs
};

// The sequence that grid row z works on, and its context length (clamped to
// the table).  Rows take the sequences of each window of 64 consecutive
// sequences in order of decreasing context length (ties by index).  The
// hardware starts workgroups roughly in grid order, as earlier ones finish;
// with the long units of a window started first, the ones that start last
// are short, and the call does not end on a few long units running alone
// (measured on MI355X, 64 sequences of U[1, 2048] tokens at 7B heads: 181.6
// against 191.4 us in drawn order).  Every wave ranks the window itself from
// one context length per lane, so the result needs no workspace and no
// extra launch; it is wave-uniform.  The ranking delays the start of every
// workgroup a little, which costs more than it saves when no unit can be
// long: the host turns it off then (order_rows = 0).
__device__ __forceinline__ int seq_of_row(const DecodeParams &P, int z, int bs, int &ctx_out) {
    const int cap = P.max_blocks * bs;
    if (!P.order_rows) {
        const int v = P.ctx[z];
        ctx_out = v < 0 ? 0 : (v > cap ? cap : v);
        return z;
    }
    const int base = z & ~63;
    const int n = __builtin_amdgcn_readfirstlane(min(64, P.num_seqs - base));
    const int lane = (int)(threadIdx.x & 63);
    int c = -1;
    if (lane < n) {
        const int v = P.ctx[base + lane];
        c = v < 0 ? 0 : (v > cap ? cap : v);
    }
    int rank = 0;
    for (int j = 0; j < n; ++j) {
        const int cj = __builtin_amdgcn_readlane(c, j);
        rank += (cj > c || (cj == c && j < lane)) ? 1 : 0;
    }
    const uint64_t hit = __ballot(lane < n && rank == z - base);
    const int i = (int)__builtin_ctzll(hit);
    ctx_out = __builtin_amdgcn_readlane(c, i);
    return base + i;
}

// split-K partitions of a sequence of nblk blocks, and the first block of
// partition p (shared-prefix decode: the prefix partitions come first and
// hold no blocks of the sequence's own; a sequence with nothing past the
// prefix has only those)
__device__ __forceinline__ int num_partitions(const DecodeParams &P, int nblk) {
    if (P.first_partition == 0)
        return nblk == 0 ? 1 : (nblk + P.partition_blocks - 1) / P.partition_blocks;
    const int rest = nblk - P.part_base_blocks;
    return P.first_partition + (rest > 0 ? (rest + P.partition_blocks - 1) / P.partition_blocks : 0);
}
__device__ __forceinline__ int partition_first_block(const DecodeParams &P, int p) {
    return P.part_base_blocks + (p - P.first_partition) * P.partition_blocks;
}

struct AppendParams {
    const void *k;
    const void *v;
    void *k_cache;
    void *v_cache;
    const int64_t *slots;
    int64_t block_stride, head_stride, token_stride;   // elements
    int num_tokens;
    int num_kv_heads;
    int block_size;
    int64_t num_slots;        // num_blocks * block_size
    int chunks_per_head;      // head_dim * elem_bytes / 16
    int elem_bytes;
};

// whole-block copies (pa_copy_blocks, pa_swap_blocks)
struct CopyParams {
    void *dst_k;
    void *dst_v;
    const void *src_k;
    const void *src_v;
    const int32_t *pairs;     // [num_pairs][2] (source block, destination block)
    int num_pairs;
    int num_src_blocks, num_dst_blocks;
    int64_t block_bytes;      // a multiple of 16
};

}  // namespace pa
