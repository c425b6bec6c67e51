// pa_decode_gqa.h -- paged decode attention for grouped-query heads on the
// CDNA4 matrix cores, with V staged through LDS (gfx950).
//
// Method: "vLLM 与 PagedAttention" (inference.mavenzero.com/case-studies/vllm),
// section 二: the K/V history of a sequence sits in fixed-size blocks of a
// shared pool reached through its block table ("PagedAttention 的解法"), and
// attention reads K/V block by block and accumulates the per-block results
// ("注意力计算改造"), here as an online softmax (a reference max per head, a
// running sum, an unnormalised output).
//
// One wave handles 16-token tiles of one kv head against the G <= 16 query
// heads that share it.  Per tile:
//
//   K   four 16-byte loads per lane into registers: lane l holds K row l % 16,
//       dims [32c + 8(l/16), +8) -- the A operand of
//   S^T[16 tok x 16 cols] = K . Q^T    (D/32 x v_mfma_f32_16x16x32_{bf16,f16})
//       Lane l gets the scores of column l % 16 for tokens 4(l/16) + r.  With
//       G <= 8 the eight q heads are entered twice (columns h and h + 8 carry
//       head h), so both halves of the tile compute the same probabilities.
//   V   direct 16-byte loads from global memory into LDS (no registers): load
//       i, lane l moves token 4i + l % 4, 16-byte chunk l / 4, so LDS holds
//       [token group][chunk][token][16 bytes], with 128 bytes of padding
//       after each load's kilobyte.
//   PV  O[16 rows x 16 dims] += P[16 rows x 16 tok] . V[16 tok x 16 dims]
//       (v_mfma_f32_16x16x16_{bf16,f16}, D/16 of them per tile).  The A
//       operand needs, in lane l, row l % 16 at tokens 4(l/16) + kk -- exactly
//       the lane's own four probabilities.  The B operand needs four
//       consecutive tokens of one dim per lane, which is a transposed read of
//       the row-major V tile: ds_read_b64_tr_b16 gives output lane i of each
//       16-lane group element i % 4 of the 8 bytes addressed by source lane
//       4r + i / 4, so source lane s of group g addresses dims
//       [16t + 4(s % 4), +4) of token 4g + s / 4.  The padding makes the 16
//       lanes of a group read 128 distinct bytes: no bank conflicts.
//   P   stays fp32 up to the products: p = hi + lo with hi = round16(p) and
//       lo = round16(p - hi), so P carries 16 (bf16) or 22 (f16) significant
//       bits.  With G <= 8, rows 0-7 of the A operand hold hi parts and rows
//       8-15 the lo parts of the same heads (the columns were duplicated for
//       that), and O[h] = row h + row h + 8: one MFMA per 16 dims.  With
//       8 < G <= 16 the hi and lo parts go through two MFMAs.
//
// The softmax keeps a reference max per head and rescales the accumulators
// only when a tile's max exceeds it by more than 2^8 (log2 units), so the
// probabilities stay below 256 and a rescale is rare after the first tile.
//
// Tokens outside the worker's window or in an unmapped block get score -inf
// (a select); their V values are zeroed in the B operand (a mask on the
// 16-bit lanes, partial tiles only), so whatever the memory holds -- NaN
// included -- cannot reach the accumulators.
#pragma once

#include "pa_device.h"

namespace pa {

typedef __bf16 gqa_bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 gqa_f16x4 __attribute__((ext_vector_type(4)));
typedef short gqa_s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 gqa_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 gqa_f16x8 __attribute__((ext_vector_type(8)));
typedef float gqa_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int gqa_u32x2 __attribute__((ext_vector_type(2)));
typedef __fp16 gqa_fp16x4_tr __attribute__((__vector_size__(4 * sizeof(__fp16))));   // transposed-read result

#define PA_LDS __attribute__((address_space(3)))

template <typename T> struct GqaOps;
template <> struct GqaOps<bf16_t> {
    __device__ __forceinline__ static gqa_f32x4 score(const uint4 &a, const uint4 &b, gqa_f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gqa_bf16x8, a),
                                                       __builtin_bit_cast(gqa_bf16x8, b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static uint2 read_tr(const unsigned char PA_LDS *p) {
        return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((gqa_bf16x4 PA_LDS *)p));
    }
    __device__ __forceinline__ static gqa_f32x4 pv(uint2 a, gqa_u32x2 b, gqa_f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(gqa_s16x4, a),
                                                         __builtin_bit_cast(gqa_s16x4, b), c, 0, 0, 0);
    }
    // two fp32 values rounded to the storage type (nearest even), packed, and back
    __device__ __forceinline__ static uint32_t pack(float a, float b) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 v = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
    __device__ __forceinline__ static void unpack(uint32_t w, float &a, float &b) {
        a = __uint_as_float(w << 16);
        b = __uint_as_float(w & 0xffff0000u);
    }
};
template <> struct GqaOps<f16_t> {
    __device__ __forceinline__ static gqa_f32x4 score(const uint4 &a, const uint4 &b, gqa_f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(gqa_f16x8, a),
                                                      __builtin_bit_cast(gqa_f16x8, b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static uint2 read_tr(const unsigned char PA_LDS *p) {
        return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((gqa_fp16x4_tr PA_LDS *)p));
    }
    __device__ __forceinline__ static gqa_f32x4 pv(uint2 a, gqa_u32x2 b, gqa_f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(gqa_f16x4, a),
                                                     __builtin_bit_cast(gqa_f16x4, b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static uint32_t pack(float a, float b) {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        const f16x2 v = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
    __device__ __forceinline__ static void unpack(uint32_t w, float &a, float &b) {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        const f16x2 v = __builtin_bit_cast(f16x2, w);
        a = (float)v.x;
        b = (float)v.y;
    }
};

constexpr int GQA_STAGES = 3;          // tiles in flight per wave (registers for K, LDS for V)
constexpr int GQA_TILE = 16;    // tokens per tile
constexpr float GQA_RESCALE_LOG2 = 8.f;   // rescale when a head's max grows by more than 2^8

typedef unsigned int gqa_u32x4 __attribute__((ext_vector_type(4)));

// The tile loads are issued by hand: the compiler classes direct-to-LDS
// loads apart from register loads and, with both in flight, could only wait
// for all of them.  Vector-memory loads return in issue order, so the waits
// below count exactly: a tile's K is in registers once at most `n` loads
// issued after it are still in flight, and likewise its V in LDS.
template <bool NT>
__device__ __forceinline__ gqa_u32x4 load_k_asm(const char *p, int off_bytes) {
    gqa_u32x4 r;
    if constexpr (NT)
        asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(r) : "v"(p + off_bytes) : "memory");
    else
        asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p + off_bytes) : "memory");
    return r;
}
// M0 carries the LDS destination of a direct load; the clobber tells the
// compiler it changed (it warns that M0 is reserved, which is the point)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT>
__device__ __forceinline__ void load_lds_asm(const char *src, uint32_t lds_addr) {
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
                     :: "v"(src), "s"(lds_addr) : "m0", "memory");
    else
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                     :: "v"(src), "s"(lds_addr) : "m0", "memory");
}
#pragma clang diagnostic pop
// wait for the K loads of one tile: the registers are operands of the
// wait itself, so that from the load to here the compiler keeps them for
// the load (it cannot see that the load writes them late) and nothing that
// reads them can move above the wait
template <int N>
__device__ __forceinline__ void vm_wait_tied(gqa_u32x4 (&k)[4]) {
    asm volatile("s_waitcnt vmcnt(%4)" : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]) : "i"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void vm_wait_tied(gqa_u32x4 (&k)[8]) {
    asm volatile("s_waitcnt vmcnt(%8)"
                 : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]), "+v"(k[4]), "+v"(k[5]), "+v"(k[6]), "+v"(k[7])
                 : "i"(N) : "memory");
}
// The same two loads with the address split into a wave-uniform 64-bit base
// (scalar registers) and a 32-bit per-lane offset: no vector arithmetic per
// load.  Usable when a tile's 16 rows lie in one block.
template <int OFF, bool NT>
__device__ __forceinline__ gqa_u32x4 load_k_sbase(const char *base, uint32_t voff) {
    gqa_u32x4 r;
    if constexpr (NT)
        asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3 nt" : "=v"(r) : "v"(voff), "s"(base), "i"(OFF) : "memory");
    else
        asm volatile("global_load_dwordx4 %0, %1, %2 offset:%3" : "=v"(r) : "v"(voff), "s"(base), "i"(OFF) : "memory");
    return r;
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// no instruction offset here: on a load into LDS it moves the LDS
// destination as well as the source, so the whole offset goes into the base
template <bool NT>
__device__ __forceinline__ void load_lds_sbase(const char *base, uint32_t voff, uint32_t lds_addr) {
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                     :: "v"(voff), "s"(base), "s"(lds_addr) : "m0", "memory");
    else
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(voff), "s"(base), "s"(lds_addr) : "m0", "memory");
}
#pragma clang diagnostic pop

// max over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four token groups
// of one score column): gfx950's lane swaps exchange the upper 32 lanes of
// one register with the lower 32 of another, and odd 16-lane rows with even
// ones, so swapping a value with itself pairs lane l with l ^ 32 (then l ^ 16)
__device__ __forceinline__ float max_token_groups(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "i"(N) : "memory");
}

// ds_read_b64_tr_b16 issued by hand (see the wait in compute()); the
// offset is an immediate
template <int OFF>
__device__ __forceinline__ gqa_u32x2 read_tr_at(const unsigned char PA_LDS *p) {
    gqa_u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(p), "i"(OFF) : "memory");
    return r;
}
__device__ __forceinline__ gqa_u32x2 read_tr_asm(const unsigned char PA_LDS *p, int off) {
    switch (off) {
    case 0: return read_tr_at<0>(p);
    case 128: return read_tr_at<128>(p);
    case 256: return read_tr_at<256>(p);
    case 384: return read_tr_at<384>(p);
    case 512: return read_tr_at<512>(p);
    case 640: return read_tr_at<640>(p);
    case 768: return read_tr_at<768>(p);
    default: return read_tr_at<896>(p);
    }
}
// wait for every LDS read; as with the K loads, the results are operands of
// the wait
__device__ __forceinline__ void lgkm_wait_tied(gqa_u32x2 (&v)[8]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
                 :: "memory");
}
__device__ __forceinline__ void lgkm_wait_tied(gqa_u32x2 (&v)[16]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
                   "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]),
                   "+v"(v[15])
                 :: "memory");
}
// two sets of reads, each held by a wait of its own (the first retires all)
template <int N>
__device__ __forceinline__ void lgkm_wait_tied(gqa_u32x2 (&a)[N], gqa_u32x2 (&b)[N]) {
    lgkm_wait_tied(a);
    lgkm_wait_tied(b);
}

template <typename T, int D, int BS, bool STREAM_KV>
struct GqaWorker {
    static constexpr int ES = 2;
    static constexpr int NC = D / 32;           // score MFMAs per tile
    static constexpr int NT = D / 16;           // PV MFMAs (16-dim column tiles) per tile
    static constexpr int NL = D / 32;           // direct LDS loads per tile (1 KiB each)
    static constexpr int LOAD_LDS = 1024 + 128; // bytes of LDS per direct load (with padding)
    static constexpr int TILE_LDS = NL * LOAD_LDS;
    // head_dim 256 holds twice the K registers per tile: two tiles in rotation
    static constexpr int STAGES = D <= 128 ? GQA_STAGES : 2;
    static constexpr int LDS_BYTES = STAGES * TILE_LDS;
    static constexpr int STEP_TOK = GQA_TILE;   // tokens per step of the schedule
    static constexpr int LOADS_PER_TILE = NC + NL;   // vector-memory operations load() issues
    // In the balanced schedule, one wave per SIMD: the stream kernel's
    // one-wave workgroups take a quarter of the compute unit's 160 KiB of LDS
    // each, so four fit.  Two waves on one SIMD do not share it evenly (the
    // older wave issues first and ends its share far earlier), and the
    // kernel ended ragged; one wave per SIMD, holding the same tiles in
    // flight, also halves the waves, the cut units and their pieces.
    static constexpr int STREAM_LDS_MIN = 160 * 1024 / 4;
    using Ops = GqaOps<T>;

    struct Buf {
        gqa_u32x4 k[NC];
        unsigned char PA_LDS *v;   // this buffer's LDS slot
        bool oka, okb;             // blocks of rows 0.. and (block size 8) rows 8.. mapped
    };

    // the unit bound to the worker: a sequence and gh <= 16 q heads of one kv head
    int seq, qh0, gh;
    bool dup;                 // gh <= 8: heads entered twice, hi and lo parts in one MFMA
    bool lo_lane;             // dup and this lane's A-operand row is a lo row (8 .. 15)
    const char *kpool, *vpool;
    const int32_t __attribute__((address_space(4))) *trow;   // constant space: read-only during the kernel, always scalar loads
    int64_t blk_bytes, tok_bytes;
    int nblk, num_blocks;
    // token limits of the unit: a token t enters the scores of this lane's
    // column when t_lo <= t < t_hi (t_hi differs per column when columns are
    // query rows at different positions); its V rows are read only when
    // t < t_vlim (the tokens inside the context); tiles below t_full are
    // valid for every column (the unmasked path)
    int t_lo, t_hi, t_vlim, t_full;
    int ncols;                // score columns that carry an output row
    float scale_log2;
    int lr, lg;
    int k_lane;               // byte offset of this lane's K row / dims inside a tile
    int v_src;                // byte offset of this lane's direct-load source inside 4 token rows
    int tr_off;               // byte offset of this lane's transposed read inside a tile slot
    unsigned char PA_LDS *lds;
    uint4 qb[NC];

    gqa_f32x4 acc[NT];        // rows 4 lg + r of each 16-dim column tile
    float m;                  // reference max of column lr's head (log2 units)
    float lp;                 // this lane's running sum over its tokens

    __device__ __forceinline__ void init_lane(int lane) {
        lr = lane & 15;
        lg = lane >> 4;
    }
    __device__ __forceinline__ void init_lds(unsigned char PA_LDS *base) { lds = base; }
    __device__ __forceinline__ void bind_buf(Buf &b, int slot) const { b.v = lds + slot * TILE_LDS; }

    // the parts of a unit that do not depend on what the columns are
    __device__ __forceinline__ void bind_kv(const DecodeParams &P, int s, int hg, int ctx) {
        const int kvh = hg / P.group_split;
        seq = s;
        gh = P.group / P.group_split;
        qh0 = kvh * P.group + (hg - kvh * P.group_split) * gh;
        blk_bytes = P.block_stride * ES;
        tok_bytes = P.token_stride * ES;
        kpool = static_cast<const char *>(P.k) + (int64_t)kvh * P.head_stride * ES;
        vpool = static_cast<const char *>(P.v) + (int64_t)kvh * P.head_stride * ES;
        trow = (const int32_t __attribute__((address_space(4))) *)(P.tables + (int64_t)s * P.max_blocks);
        nblk = (ctx + BS - 1) / BS;
        num_blocks = P.num_blocks;
        scale_log2 = P.scale_log2;
        constexpr int RW = BS < GQA_TILE ? BS : GQA_TILE;
        k_lane = (int)((lr % RW) * tok_bytes) + 8 * lg * ES;
        // direct load i, lane l: token 4i + l % 4 (of the tile), 16-byte chunk l / 4 (plus 16 per
        // extra 128 dims at head_dim 256)
        const int lane = 16 * lg + lr;
        v_src = (int)((lane % 4) * tok_bytes) + 16 * (lane / 4);
        // transposed read, column tile 0: token group lg, token lr / 4, dims 4(lr % 4) .. +3,
        // which sit in 16-byte chunk (lr % 4) / 2 at byte 8 (lr % 2)
        tr_off = lg * (D / 128) * LOAD_LDS + (lr / 4) * 16 + ((lr % 4) / 2) * 64 + (lr % 2) * 8;
    }

    __device__ __forceinline__ void load_q(const char *qp, bool on) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            qb[c] = ld16(qp + 32 * c * ES);
            if (!on)
                qb[c] = make_uint4(0u, 0u, 0u, 0u);
        }
    }

    // decode: the columns are the unit's gh q heads (entered twice when gh <= 8)
    __device__ __forceinline__ void bind(const DecodeParams &P, int s, int hg, int ctx) {
        bind_kv(P, s, hg, ctx);
        dup = gh <= 8;
        lo_lane = dup && lr >= 8;
        ncols = gh;
        const int hq = dup ? (lr & 7) : lr;          // head of this lane's column
        const bool on = hq < gh;
        load_q(static_cast<const char *>(P.q) + (((int64_t)s * P.num_q_heads + qh0 + (on ? hq : 0)) * D + 8 * lg) * ES,
               on);
        t_lo = 0;
        t_hi = t_vlim = t_full = ctx;
    }

    // several query rows: column c is query row i0 + c / gh (at position
    // ctx - nq + that row), head c % gh, for the 16 / gh rows of the tile;
    // row q_first of q is query row 0 of the sequence.  Columns past the
    // tile's rows read nothing and write nothing; they follow the first row's
    // limit so that they never force the masked path.
    __device__ __forceinline__ void bind_rows(const DecodeParams &P, int s, int hg, int ctx, int q_first, int nq,
                                              int i0) {
        bind_kv(P, s, hg, ctx);
        dup = false;
        lo_lane = false;
        const int rows = GQA_TILE / gh;
        ncols = rows * gh;
        const int i = i0 + lr / gh;
        const bool on = lr < ncols && i < nq;
        load_q(static_cast<const char *>(P.q) +
                   (((int64_t)(q_first + (on ? i : i0))) * P.num_q_heads + qh0 + (on ? lr % gh : 0)) * D * ES +
                   8 * lg * ES,
               on);
        auto limit = [&](int row) { const int t = ctx - nq + row + 1; return t < 0 ? 0 : (t > ctx ? ctx : t); };
        t_lo = 0;
        t_vlim = ctx;
        t_full = limit(i0);
        t_hi = on ? limit(i) : t_full;
        t_last = limit(min(i0 + rows, nq) - 1);
    }
    int t_last;               // bind_rows: one past the last token any column attends

    // shared-prefix pass of decode: column c is sequence i0 + c / gh (its
    // query row of q [num_seqs, Hq, D]), head c % gh, and sees the tokens
    // [c0, c1) of the prefix that every table starts with (sequence 0's table
    // is read), below its own context.  Columns past the batch read nothing
    // and write nothing.
    __device__ __forceinline__ void bind_prefix(const DecodeParams &P, int hg, int i0, int c0, int c1) {
        bind_kv(P, 0, hg, c1);
        dup = false;
        lo_lane = false;
        const int rows = GQA_TILE / gh;
        ncols = rows * gh;
        const int i = i0 + lr / gh;
        const bool on = lr < ncols && i < P.num_seqs;
        load_q(static_cast<const char *>(P.q) +
                   (((int64_t)(on ? i : i0)) * P.num_q_heads + qh0 + (on ? lr % gh : 0)) * D * ES + 8 * lg * ES,
               on);
        const int cap = P.max_blocks * BS;
        int c = on ? P.ctx[i] : c1;
        c = c < 0 ? 0 : (c > cap ? cap : c);
        t_lo = c0;
        t_vlim = c1;
        t_hi = c < c1 ? c : c1;
        int tf = t_hi;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
            tf = min(tf, __shfl_xor(tf, off));
        t_full = __builtin_amdgcn_readfirstlane(tf);
        t_last = c1;
    }

    // bind_prefix columns: each (sequence, q head) leaves its (max, sum,
    // unnormalised output) as split-K partition `part` of the workspace
    __device__ __forceinline__ void finish_partials(const DecodeParams &P, int i0, int part) {
        finalize();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = row_head(r);
            const int i = i0 + c / gh;
            if (!owns(r) || i >= P.num_seqs)
                continue;
            const int64_t sh = (int64_t)i * P.num_q_heads + qh0 + c % gh;
            float *a = P.ws_acc + (sh * P.max_partitions + part) * D + lr;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                a[16 * t] = acc[t][r];
            if (lr == 0)
                P.ws_ml[sh * P.max_partitions + part] = make_float2(mrow[r], lrow[r]);
        }
    }
    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = gqa_f32x4{0.f, 0.f, 0.f, 0.f};
        m = NEG_BIG;
        lp = 0.f;
    }

    // physical blocks of tile kt's rows 0.. and (block size 8) rows 8..
    __device__ __forceinline__ int2 tile_phys(int kt) const {
        const int ja = kt * GQA_TILE / BS;
        int2 r;
        r.x = trow[ja];
        r.y = BS < GQA_TILE ? trow[min(ja + 1, nblk - 1)] : r.x;
        return r;
    }

    // K rows into registers, V rows into the buffer's LDS slot (scalar base)
    template <int C = 0>
    __device__ __forceinline__ void load_k_rows(const char *base, Buf &b) const {
        if constexpr (C < NC) {
            b.k[C] = load_k_sbase<32 * C * ES, STREAM_KV>(base, (uint32_t)k_lane);
            load_k_rows<C + 1>(base, b);
        }
    }
    template <int I = 0>
    __device__ __forceinline__ void load_v_rows(const char *base, uint32_t slot) const {
        if constexpr (I < NL) {
            constexpr int grp = I / (D / 128);        // token group: tokens 4 grp .. 4 grp + 3
            constexpr int half = I % (D / 128);       // which 128 dims
            load_lds_sbase<STREAM_KV>(base + (int64_t)(4 * grp) * tok_bytes + 256 * half, (uint32_t)v_src, slot + I * LOAD_LDS);
            load_v_rows<I + 1>(base, slot);
        }
    }

    __device__ __forceinline__ void load(int kt, int2 pp, Buf &b) const {
        const int t0 = kt * GQA_TILE;
        b.oka = (unsigned)pp.x < (unsigned)num_blocks;
        b.okb = (unsigned)pp.y < (unsigned)num_blocks;
        const int64_t row0 = (int64_t)(t0 % BS) * tok_bytes;
        const uint32_t slot = (uint32_t)(uintptr_t)b.v;
        if constexpr (BS >= GQA_TILE) {
            // the tile is 16 rows of one block: every address is that block's
            // base plus a per-lane offset
            const int64_t blk = b.oka ? (int64_t)pp.x * blk_bytes : 0;
            load_k_rows(kpool + blk + row0, b);
            load_v_rows(vpool + blk + row0, slot);
        } else {
            // rows 0 .. BS-1 of the tile in block pp.x, the rest in block pp.y
            const char *ba = (b.oka ? kpool + (int64_t)pp.x * blk_bytes : kpool) + row0;
            const char *bb = (b.okb ? kpool + (int64_t)pp.y * blk_bytes : kpool) + row0;
            const char *ka = lr >= BS ? bb : ba;
#pragma unroll
            for (int c = 0; c < NC; ++c)
                b.k[c] = load_k_asm<STREAM_KV>(ka, k_lane + 32 * c * ES);
            const char *va = (b.oka ? vpool + (int64_t)pp.x * blk_bytes : vpool) + row0;
            const char *vb = (b.okb ? vpool + (int64_t)pp.y * blk_bytes : vpool) + row0;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int grp = i / (D / 128);
                const int half = i % (D / 128);
                const char *src = 4 * grp >= BS ? vb - (int64_t)BS * tok_bytes : va;
                load_lds_asm<STREAM_KV>(src + (int64_t)(4 * grp) * tok_bytes + (v_src + 256 * half), slot + i * LOAD_LDS);
            }
        }
    }

    // this tile's K: the loads behind it are its own V (NL) and those of
    // the BEHIND tiles issued after it
    template <int BEHIND>
    __device__ __forceinline__ void wait(Buf &b) const {
        vm_wait_tied<NL + LOADS_PER_TILE * BEHIND>(b.k);
    }

    // V_READY: the tile's V is known to be in LDS already (a workgroup that
    // stages tiles for all its waves has waited and met at a barrier)
    template <int BEHIND, bool V_READY = false>
    __device__ __forceinline__ void compute(int kt, const Buf &b) {
        gqa_f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c)
            sc = Ops::score(make_uint4(b.k[c].x, b.k[c].y, b.k[c].z, b.k[c].w), qb[c], sc);
        const int t0 = kt * GQA_TILE;
        const int tv = t0 + 4 * lg;                   // this lane's four tokens tv + r
        const bool full = b.oka && b.okb && t0 >= t_lo && t0 + GQA_TILE <= t_full;
        const bool okv = (BS < GQA_TILE && 4 * lg >= BS) ? b.okb : b.oka;
        float sv[4];
        uint32_t keep[2] = {0xffffffffu, 0xffffffffu};   // 16-bit lanes of the V fragment to keep
#pragma unroll
        for (int r = 0; r < 4; ++r)
            sv[r] = sc[r] * scale_log2;
        if (!full) {
            bool valid[4], readable[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                readable[r] = okv && tv + r >= t_lo && tv + r < t_vlim;   // its V rows may be used
                valid[r] = readable[r] && tv + r < t_hi;                 // it enters this column's scores
                sv[r] = valid[r] ? sv[r] : -INFINITY;
            }
            keep[0] = (readable[0] ? 0x0000ffffu : 0u) | (readable[1] ? 0xffff0000u : 0u);
            keep[1] = (readable[2] ? 0x0000ffffu : 0u) | (readable[3] ? 0xffff0000u : 0u);
        }
        const float mx = max_token_groups(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
        // lazy rescale: move the reference max only when this tile's max exceeds it by 2^8
        const bool grow = mx > m + GQA_RESCALE_LOG2;
        if (__any(grow)) {
            const float mn = grow ? mx : m;
            const float alpha = fast_exp2(m - mn);
            lp *= alpha;
            m = mn;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * lg + r;
                const float ar = __shfl(alpha, dup ? (row & 7) : row);
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[t][r] *= ar;
            }
        }
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            pr[r] = fast_exp2(sv[r] - m);
        lp += (pr[0] + pr[1]) + (pr[2] + pr[3]);

        // P = hi + lo in the storage type; A operand: row lr, tokens tv .. tv + 3
        const uint2 phi = make_uint2(Ops::pack(pr[0], pr[1]), Ops::pack(pr[2], pr[3]));
        float w[4];
        Ops::unpack(phi.x, w[0], w[1]);
        Ops::unpack(phi.y, w[2], w[3]);
        const uint2 plo = make_uint2(Ops::pack(pr[0] - w[0], pr[1] - w[1]), Ops::pack(pr[2] - w[2], pr[3] - w[3]));
        const uint2 pa = lo_lane ? plo : phi;

        // V of this tile is in LDS once the loads issued after it (those of
        // the BEHIND tiles behind) are the only ones left in flight: the
        // compiler cannot see which direct load an LDS read depends on, so
        // the reads are issued by hand after that exact wait.
        if constexpr (!V_READY)
            vm_wait<LOADS_PER_TILE * BEHIND>();
        gqa_u32x2 vb[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
            vb[t] = read_tr_asm(b.v + tr_off + ((16 * t) / 128) * LOAD_LDS, (t % 8) * 128);
        lgkm_wait_tied(vb);
        if (!full) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                vb[t].x &= keep[0];
                vb[t].y &= keep[1];
            }
        }
        if (dup) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = Ops::pv(pa, vb[t], acc[t]);
        } else {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                acc[t] = Ops::pv(phi, vb[t], acc[t]);
                acc[t] = Ops::pv(plo, vb[t], acc[t]);
            }
        }
    }

    // Two consecutive key tiles (kt, kt + 1) whose K fragments and V are in
    // LDS (a workgroup that stages tiles for its waves), with the weighted
    // sums done by 16x16x32 products: the A operand of one product takes the
    // lane's four probabilities of each tile (k slots 8g + r and 8g + 4 + r
    // for tokens 4g + r of the first and of the second tile, g = lane / 16),
    // and the B operand the two transposed reads of those tokens' V rows, in
    // the same order -- one product where the single-tile path makes two.
    // HILO: P as hi + lo (two products); otherwise P is rounded once to the
    // storage type and the running sum adds the rounded values, so that the
    // weights the products use are exactly the ones normalised by.
    template <bool HILO>
    __device__ __forceinline__ void compute_pair(int kt, const Buf &b0, const Buf &b1) {
        gqa_f32x4 sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            sc0 = Ops::score(make_uint4(b0.k[c].x, b0.k[c].y, b0.k[c].z, b0.k[c].w), qb[c], sc0);
            sc1 = Ops::score(make_uint4(b1.k[c].x, b1.k[c].y, b1.k[c].z, b1.k[c].w), qb[c], sc1);
        }
        float sv[8];
        uint32_t keep[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
        bool any_masked = false;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const Buf &b = h ? b1 : b0;
            const gqa_f32x4 &sc = h ? sc1 : sc0;
            const int t0 = (kt + h) * GQA_TILE;
            const int tv = t0 + 4 * lg;
            const bool full = b.oka && b.okb && t0 >= t_lo && t0 + GQA_TILE <= t_full;
            const bool okv = (BS < GQA_TILE && 4 * lg >= BS) ? b.okb : b.oka;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sv[4 * h + r] = sc[r] * scale_log2;
            if (!full) {
                any_masked = true;
                bool readable[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    readable[r] = okv && tv + r >= t_lo && tv + r < t_vlim;
                    sv[4 * h + r] = readable[r] && tv + r < t_hi ? sv[4 * h + r] : -INFINITY;
                }
                keep[2 * h] = (readable[0] ? 0x0000ffffu : 0u) | (readable[1] ? 0xffff0000u : 0u);
                keep[2 * h + 1] = (readable[2] ? 0x0000ffffu : 0u) | (readable[3] ? 0xffff0000u : 0u);
            }
        }
        float mx = sv[0];
#pragma unroll
        for (int r = 1; r < 8; ++r)
            mx = fmaxf(mx, sv[r]);
        mx = max_token_groups(mx);
        const bool grow = mx > m + GQA_RESCALE_LOG2;
        if (__any(grow)) {
            const float mn = grow ? mx : m;
            const float alpha = fast_exp2(m - mn);
            lp *= alpha;
            m = mn;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * lg + r);
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[t][r] *= ar;
            }
        }
        float pr[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
            pr[r] = fast_exp2(sv[r] - m);
        const uint4 phi = make_uint4(Ops::pack(pr[0], pr[1]), Ops::pack(pr[2], pr[3]), Ops::pack(pr[4], pr[5]),
                                     Ops::pack(pr[6], pr[7]));
        float w[8];
        Ops::unpack(phi.x, w[0], w[1]);
        Ops::unpack(phi.y, w[2], w[3]);
        Ops::unpack(phi.z, w[4], w[5]);
        Ops::unpack(phi.w, w[6], w[7]);
        uint4 plo = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (HILO) {
            lp += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
            plo = make_uint4(Ops::pack(pr[0] - w[0], pr[1] - w[1]), Ops::pack(pr[2] - w[2], pr[3] - w[3]),
                             Ops::pack(pr[4] - w[4], pr[5] - w[5]), Ops::pack(pr[6] - w[6], pr[7] - w[7]));
        } else {
            lp += ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
        }
        gqa_u32x2 va[NT], vb[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            va[t] = read_tr_asm(b0.v + tr_off + ((16 * t) / 128) * LOAD_LDS, (t % 8) * 128);
            vb[t] = read_tr_asm(b1.v + tr_off + ((16 * t) / 128) * LOAD_LDS, (t % 8) * 128);
        }
        lgkm_wait_tied(va, vb);
        if (any_masked) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                va[t].x &= keep[0];
                va[t].y &= keep[1];
                vb[t].x &= keep[2];
                vb[t].y &= keep[3];
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint4 vop = make_uint4(va[t].x, va[t].y, vb[t].x, vb[t].y);
            acc[t] = Ops::score(phi, vop, acc[t]);
            if constexpr (HILO)
                acc[t] = Ops::score(plo, vop, acc[t]);
        }
    }

    __device__ __forceinline__ void run(int kbeg, int kend, int stride) {
        pipeline<STAGES>(*this, kbeg, kend, stride);
    }

    // ---- results ---------------------------------------------------------
    // After finalize(): lanes with owns() hold the unnormalised output of head
    // row_head(r) at dims 16 t + lr in acc[t][r], and mrow[r] / lrow[r] its
    // reference max and total sum.  Every lane must call finalize().
    float mrow[4], lrow[4];

    __device__ __forceinline__ void finalize() {
        float l = lp + __shfl_xor(lp, 16);
        l += __shfl_xor(l, 32);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * lg + r;
            const int src = dup ? (row & 7) : row;
            mrow[r] = __shfl(m, src);
            lrow[r] = __shfl(l, src);
        }
        if (dup) {   // O[h] = hi row h + lo row h + 8 (lanes 32.. hold rows 8..15)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[t][r] += __shfl_xor(acc[t][r], 32);
        }
    }
    __device__ __forceinline__ bool owns(int r) const {
        return (!dup || lg < 2) && 4 * lg + r < ncols;
    }
    __device__ __forceinline__ int row_head(int r) const { return 4 * lg + r; }

    __device__ __forceinline__ void finish_out(const DecodeParams &P) {
        finalize();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (!owns(r))
                continue;
            const float L = lrow[r];
            const int64_t base = ((int64_t)seq * P.num_q_heads + qh0 + row_head(r)) * D + lr;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                Store<T>::one(P.out, base + 16 * t, L > 0.f ? acc[t][r] / L : 0.f);
        }
    }

    __device__ __forceinline__ void finish_piece(const DecodeParams &P, int piece) {
        finalize();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (!owns(r))
                continue;
            const int h = row_head(r);
            float *a = P.piece_acc + ((int64_t)piece * gh + h) * D + lr;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                a[16 * t] = acc[t][r];
            if (lr == 0)
                P.piece_ml[(int64_t)piece * gh + h] = make_float2(mrow[r], lrow[r]);
        }
    }

    // bind_rows columns, every key of theirs seen: normalised rows of out
    // (row q_first + i0 + c / gh, head qh0 + c % gh for column c)
    __device__ __forceinline__ void finish_rows(const DecodeParams &P, int q_first, int i0, int nq) {
        finalize();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = row_head(r);
            const int i = i0 + c / gh;
            if (!owns(r) || i >= nq)
                continue;
            const float L = lrow[r];
            const int64_t base = ((int64_t)(q_first + i) * P.num_q_heads + qh0 + c % gh) * D + lr;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                Store<T>::one(P.out, base + 16 * t, L > 0.f ? acc[t][r] / L : 0.f);
        }
    }

    // the wave's partial result into LDS arrays [16] and [16][D] (grid kernel merge)
    __device__ __forceinline__ void export_lds(float *sm, float *sl, float *sacc) {
        finalize();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (!owns(r))
                continue;
            const int h = row_head(r);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                sacc[h * D + 16 * t + lr] = acc[t][r];
            if (lr == 0) {
                sm[h] = mrow[r];
                sl[h] = lrow[r];
            }
        }
    }
};

}  // namespace pa
