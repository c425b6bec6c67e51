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
// The per-wave math is the grouped-query decode worker of pa_decode_gqa.h
// with its 16 score columns taken by (query row, q head) pairs -- 16 / gh rows
// of the chunk times the gh q heads of one kv head -- each column with its own
// causal limit.  What differs from decode is where K and V come from: a
// prefill reads every key tile for many columns, so a workgroup brings each
// tile into LDS once and all its waves take it from there.
#pragma once

#include <type_traits>

#include "pa_decode_gqa.h"
#include "pa_device.h"
#include "pa_prefill_wide.h"

namespace pa {

// One workgroup of NW waves per (group of NW column tiles, head group,
// sequence): wave i owns column tile NW * g + i and sees every
// key tile its columns attend.  A key tile goes from memory into LDS once for
// the whole workgroup -- its K and V moved by direct-to-LDS loads that the
// waves share out -- and every wave reads it there:
//
//   K  chunk c (32 dims) of the 16 rows is one 1 KiB load: lane i brings row
//      i / 4, piece p = (i % 4) ^ ((row / 2) % 4) (16 bytes, 8 dims), so that
//      LDS slot 4 row + (p ^ ((row / 2) % 4)) holds piece p.  The worker's A
//      operand (lane l: row l % 16, piece l / 16) then reads 16 bytes per lane
//      with every 8 lanes on 8 different 16-byte bank groups: no conflicts.
//   V  the worker's own layout (its transposed reads, unchanged).
//
// A slot holds a pair of tiles, which the worker takes in one step
// (compute_pair: 16x16x32 products for the weighted sums as well as for the
// scores).  Per step: each wave waits for its own loads of the slot, the
// waves meet at a barrier (the slot is complete in LDS, and every wave is done
// with the slot before, which the next loads then fill), the loads STAGES - 1
// slots ahead go out, and the wave's 16 columns take the pair (K fragments
// from LDS).  Past the last pair the loads repeat the last one into the free
// slot, so the wait count is the same on every step; a tile past the last is
// read as unmapped, so it contributes nothing.
//
// Logical workgroups are XCD-major (dispatch puts workgroup b on XCD b % 8):
// the column groups of one (head group, sequence) are consecutive and run
// together on one XCD, whose L2 then serves their re-reads of the same K/V.
//
// pa_prefill takes this kernel at head_dim 256 (head_dim 128 has the 32x32x16
// kernel of pa_prefill_wide.h), with 8 waves per workgroup: the worker needs
// more registers than four waves per SIMD leave.  The shared-prefix pass
// below runs 8-wave workgroups at both head dims (its 128 sequences fill 8
// column tiles; 16 waves measured 64.7 against 64.2 us per call).
constexpr int PREFILL_WAVES = 8;
constexpr int PREFIX_WAVES = 8;
constexpr int PF_STAGES = 2;    // slots (tile pairs) in rotation

template <typename T, int D, int BS, bool STREAM_KV, int NW>
struct PrefillTiles {
    using W = GqaWorker<T, D, BS, STREAM_KV>;
    static constexpr int NC = W::NC;                    // K chunks (and loads) per tile
    static constexpr int NL = W::NL;                    // V loads per tile
    static constexpr int K_BYTES = NC * 1024;
    static constexpr int TILE_BYTES = K_BYTES + W::TILE_LDS;   // one tile: K, then V
    static constexpr int BYTES = 2 * TILE_BYTES;        // one slot: a pair of tiles
    static constexpr int TILE_LOADS = NC + NL;
    static constexpr int LOADS = 2 * TILE_LOADS;
    static constexpr int PER_WAVE = LOADS / NW;
    static constexpr int STAGES = PF_STAGES;
    static_assert(LOADS % NW == 0, "the loads of a slot share out evenly");
    // bf16 keeps P as hi + lo (8 significant bits would not meet the accuracy bound); f16 rounds it once
    static constexpr bool HILO = std::is_same<T, bf16_t>::value;
};

// Key tiles t_begin .. t_end - 1 of the worker's kv head, staged in pairs
// through LDS for all the waves of the workgroup (every wave calls this with
// the same range); the wave computes the pairs that start below my_end.
template <typename T, int D, int BS, bool STREAM_KV, int NW>
__device__ __forceinline__ void staged_tiles(GqaWorker<T, D, BS, STREAM_KV> &w, unsigned char PA_LDS *base, int wave,
                                             int lane, int t_begin, int t_end, int my_end)
{
    using PT = PrefillTiles<T, D, BS, STREAM_KV, NW>;
    using W = typename PT::W;
    constexpr int STAGES = PT::STAGES;
    // K source rows of this lane (K loads: row i / 4, swizzled piece)
    const int k_row = lane >> 2;
    const int k_piece = (lane & 3) ^ ((k_row >> 1) & 3);
    // K slot of this lane's A operand (row lane % 16, piece lane / 16)
    const int a_row = lane & 15, a_piece = lane >> 4;
    const int a_off = 16 * (4 * a_row + (a_piece ^ ((a_row >> 1) & 3)));

    // slot st <- tiles 2 step and 2 step + 1 (a tile past the last repeats the last: same bytes, never used)
    auto issue = [&](int step, int st) {
        const uint32_t slot = (uint32_t)(uintptr_t)(base + st * PT::BYTES);
#pragma unroll
        for (int p = 0; p < PT::PER_WAVE; ++p) {
            const int j = wave * PT::PER_WAVE + p;          // wave-uniform
            const int h = j / PT::TILE_LOADS, jj = j % PT::TILE_LOADS;
            const int kt = min(t_begin + 2 * step + h, t_end - 1);
            const int2 pp = w.tile_phys(kt);
            const bool oka = (unsigned)pp.x < (unsigned)w.num_blocks;
            const bool okb = (unsigned)pp.y < (unsigned)w.num_blocks;
            const int t0 = kt * GQA_TILE;
            const uint32_t tslot = slot + h * PT::TILE_BYTES;
            if (jj < PT::NC) {
                // K chunk jj: this lane's row and piece
                const bool second = BS < GQA_TILE && k_row >= BS;
                const int64_t blk = second ? (okb ? pp.y : 0) : (oka ? pp.x : 0);
                const int in_row = BS < GQA_TILE ? (k_row & (BS - 1)) : (t0 % BS) + k_row;
                const char *src = w.kpool + blk * w.blk_bytes + (int64_t)in_row * w.tok_bytes + 64 * jj + 16 * k_piece;
                load_lds_asm<STREAM_KV>(src, tslot + jj * 1024);
            } else {
                // V load i, as the worker lays V out: token 4 grp + lane % 4, chunk lane / 4
                const int i = jj - PT::NC;
                const int grp = i / (D / 128), half = i % (D / 128);
                const bool second = BS < GQA_TILE && 4 * grp >= BS;
                const int64_t blk = second ? (okb ? pp.y : 0) : (oka ? pp.x : 0);
                const int in_row = BS < GQA_TILE ? (4 * grp) & (BS - 1) : (t0 % BS) + 4 * grp;
                const char *src = w.vpool + blk * w.blk_bytes + (int64_t)in_row * w.tok_bytes + 256 * half + w.v_src;
                load_lds_asm<STREAM_KV>(src, tslot + PT::K_BYTES + i * W::LOAD_LDS);
            }
        }
    };
    // the wave's view of tile kt in slot st: K fragments from LDS, V in place; a
    // tile past the last is unmapped (masked out)
    auto view = [&](int kt, const unsigned char PA_LDS *ts, typename W::Buf &b) {
#pragma unroll
        for (int c = 0; c < PT::NC; ++c)
            b.k[c] = *reinterpret_cast<const gqa_u32x4 PA_LDS *>(ts + c * 1024 + a_off);
        b.v = const_cast<unsigned char PA_LDS *>(ts + PT::K_BYTES);
        const int2 pp = kt < t_end ? w.tile_phys(kt) : make_int2(-1, -1);
        b.oka = (unsigned)pp.x < (unsigned)w.num_blocks;
        b.okb = (unsigned)pp.y < (unsigned)w.num_blocks;
    };

    const int n_steps = (t_end - t_begin + 1) / 2;
    if (n_steps > 0) {
#pragma unroll
        for (int i = 0; i < STAGES - 1; ++i)
            issue(min(i, n_steps - 1), i);
        for (int step = 0; step < n_steps; ++step) {
            vm_wait<PT::PER_WAVE * (STAGES - 2)>();        // this wave's loads of this step's slot
            asm volatile("s_barrier" ::: "memory");       // the slot complete; the one before done by all
            issue(min(step + STAGES - 1, n_steps - 1), (step + STAGES - 1) % STAGES);
            const int kt = t_begin + 2 * step;
            if (kt < my_end) {
                const unsigned char PA_LDS *ss = base + (step % STAGES) * PT::BYTES;
                typename W::Buf b0, b1;
                view(kt, ss, b0);
                view(kt + 1, ss + PT::TILE_BYTES, b1);
                w.template compute_pair<PT::HILO>(kt, b0, b1);
            }
        }
        // every load into LDS has landed before the workgroup ends
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
}

template <typename T, int D, int BS, bool STREAM_KV>
__global__ __launch_bounds__(PREFILL_WAVES * 64) void prefill_kernel(const DecodeParams P, int col_groups,
                                                                             int total_wg)
{
    static_assert(D % 128 == 0, "the matrix-core worker needs head_dim 128 or 256");
    constexpr int NW = PREFILL_WAVES;
    using PT = PrefillTiles<T, D, BS, STREAM_KV, NW>;
    using W = typename PT::W;
    constexpr int STAGES = PT::STAGES;
    __shared__ __attribute__((aligned(16))) unsigned char lds[STAGES * PT::BYTES];

    const int per_xcd = (total_wg + 7) / 8;
    const int lg_id = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (lg_id >= total_wg)
        return;
    const int HG = P.num_kv_heads * P.group_split;
    const int cg = lg_id % col_groups;
    const int hg = (lg_id / col_groups) % HG;
    const int s = lg_id / col_groups / HG;

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
    const int rows = GQA_TILE / gh;                       // query rows per column tile
    const int i0g = cg * NW * rows;
    if (i0g >= nq)
        return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i0 = i0g + wave * rows;
    const bool active = i0 < nq;
    W w;
    w.init_lane(lane);
    w.bind_rows(P, s, hg, ctx, q_first, nq, active ? i0 : i0g);
    // key tiles of the group: up to the last position any of its rows attends
    const int last_row = min(i0g + NW * rows, nq) - 1;
    const int t_end = min(ctx, max(0, ctx - nq + last_row + 1));
    const int n_tiles = (t_end + GQA_TILE - 1) / GQA_TILE;
    const int my_tiles = active ? (w.t_last + GQA_TILE - 1) / GQA_TILE : 0;

    w.reset();
    staged_tiles<T, D, BS, STREAM_KV, NW>(w, (unsigned char PA_LDS *)lds, wave, lane, 0, n_tiles, my_tiles);
    if (active)
        w.finish_rows(P, q_first, i0, nq);
}

template <typename T, int D, int BS>
hipError_t launch_prefill_shape(const DecodeParams &p, int max_query_len, hipStream_t st)
{
    const int rows = GQA_TILE / (p.group / p.group_split);
    constexpr int NW = PREFILL_WAVES;
    const int col_tiles = (max_query_len + rows - 1) / rows;
    const int col_groups = (col_tiles + NW - 1) / NW;
    const long long total = (long long)col_groups * p.num_kv_heads * p.group_split * p.num_seqs;
    if (total > (1LL << 30))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)((total + 7) / 8 * 8));
    // every column group of a (head group, sequence) reads the same key tiles:
    // K and V are loaded with the caches' normal policy, whatever the flags say
    hipLaunchKernelGGL((prefill_kernel<T, D, BS, false>), grid, dim3(NW * 64), 0, st, p, col_groups, (int)total);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Shared-prefix decode, first pass.  When every table of a decode batch
// starts with the same blocks (a common system prompt, copy-on-write sharing:
// "vLLM 与 PagedAttention" section 二, "指南" "Copy-on-Write：Prefix Caching
// 的基础"), those blocks' K/V need to be read once, not once per sequence:
// the batch's query rows are the columns of one pass over them, like a
// prefill's rows but with no causal order -- each sequence sees the prefix
// tokens below its own context.  The prefix is cut into chunks of `chunk`
// tokens (a multiple of two tiles, chosen per call by the host), one
// workgroup per (group of PREFIX_WAVES column tiles, chunk, head group); each
// (sequence, q head) leaves the chunk's (max, sum, unnormalised output) as
// split-K partition `chunk`.  The decode kernels then take the sequences' own
// blocks as the partitions after these, and the split-K reduce merges them
// all.

// workgroups the prefix pass starts per chunk: column groups x head groups
inline int prefix_workgroups_per_chunk(int num_seqs, int group, int group_split, int num_kv_heads)
{
    const int rows = GQA_TILE / (group / group_split);
    const int col_tiles = (num_seqs + rows - 1) / rows;
    const int col_groups = (col_tiles + PREFIX_WAVES - 1) / PREFIX_WAVES;
    return col_groups * num_kv_heads * group_split;
}

// LDS bytes of one prefix-pass workgroup of NW waves
template <typename T, int D, int BS, int NW>
constexpr int prefix_block_lds()
{
    using PT = PrefillTiles<T, D, BS, false, NW>;
    return PT::STAGES * PT::BYTES;
}

// One workgroup of the prefix pass (NW waves; logical workgroup lg_id of
// total_wg), over prefix_block_lds() bytes of LDS at `lds`: also run inside
// the shared-prefix decode's combined launch (pa_shared_prefix.h), next to
// the workgroups of the own-blocks pass, sharing their LDS.
template <typename T, int D, int BS, int NW>
__device__ __forceinline__ void prefix_block(const DecodeParams &P, int lg_id, int col_groups, int n_chunks,
                                             int prefix_tokens, int chunk, unsigned char PA_LDS *lds)
{
    static_assert(D % 128 == 0, "the matrix-core worker needs head_dim 128 or 256");
    using PT = PrefillTiles<T, D, BS, false, NW>;
    using W = typename PT::W;

    const int cg = lg_id % col_groups;
    const int c = (lg_id / col_groups) % n_chunks;
    const int hg = lg_id / col_groups / n_chunks;
    const int gh = P.group / P.group_split;
    const int rows = GQA_TILE / gh;
    const int i0g = cg * NW * rows;                      // first sequence of the group (inside the batch)
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i0 = i0g + wave * rows;
    const bool active = i0 < P.num_seqs;
    const int c0 = c * chunk;
    const int c1 = min(prefix_tokens, c0 + chunk);
    W w;
    w.init_lane(lane);
    w.bind_prefix(P, hg, active ? i0 : i0g, c0, c1);
    w.reset();
    const int t_end = (c1 + GQA_TILE - 1) / GQA_TILE;
    staged_tiles<T, D, BS, false, NW>(w, lds, wave, lane, c0 / GQA_TILE, t_end,
                                      active ? t_end : 0);
    if (active)
        w.finish_partials(P, i0, c);
}

template <typename T, int D, int BS>
__global__ __launch_bounds__(PREFIX_WAVES * 64) void prefix_kernel(const DecodeParams P, int col_groups, int n_chunks,
                                                               int prefix_tokens, int chunk, int total_wg)
{
    // XCD-major, column groups fastest: the groups reading one chunk of one kv head share an L2
    const int per_xcd = (total_wg + 7) / 8;
    const int lg_id = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (lg_id >= total_wg)
        return;
    __shared__ __attribute__((aligned(16))) unsigned char lds[prefix_block_lds<T, D, BS, PREFIX_WAVES>()];
    prefix_block<T, D, BS, PREFIX_WAVES>(P, lg_id, col_groups, n_chunks, prefix_tokens, chunk,
                                         (unsigned char PA_LDS *)lds);
}

template <typename T, int D, int BS>
hipError_t launch_prefix_shape(const DecodeParams &p, int prefix_tokens, int chunk, hipStream_t st)
{
    if (chunk <= 0 || chunk % (2 * GQA_TILE) != 0)
        return hipErrorInvalidValue;
    const int rows = GQA_TILE / (p.group / p.group_split);
    const int col_tiles = (p.num_seqs + rows - 1) / rows;
    const int col_groups = (col_tiles + PREFIX_WAVES - 1) / PREFIX_WAVES;
    const int n_chunks = (prefix_tokens + chunk - 1) / chunk;
    if (n_chunks != p.first_partition)
        return hipErrorInvalidValue;
    const long long total = (long long)col_groups * n_chunks * p.num_kv_heads * p.group_split;
    if (total > (1LL << 30))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)((total + 7) / 8 * 8));
    hipLaunchKernelGGL((prefix_kernel<T, D, BS>), grid, dim3(PREFIX_WAVES * 64), 0, st, p, col_groups, n_chunks,
                       prefix_tokens, chunk, (int)total);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_prefix_dtype(const DecodeParams &p, int head_dim, int bs, int prefix_tokens, int chunk,
                               hipStream_t st)
{
    switch (head_dim * 64 + bs) {
    case 128 * 64 + 8: return launch_prefix_shape<T, 128, 8>(p, prefix_tokens, chunk, st);
    case 128 * 64 + 16: return launch_prefix_shape<T, 128, 16>(p, prefix_tokens, chunk, st);
    case 128 * 64 + 32: return launch_prefix_shape<T, 128, 32>(p, prefix_tokens, chunk, st);
    case 256 * 64 + 8: return launch_prefix_shape<T, 256, 8>(p, prefix_tokens, chunk, st);
    case 256 * 64 + 16: return launch_prefix_shape<T, 256, 16>(p, prefix_tokens, chunk, st);
    case 256 * 64 + 32: return launch_prefix_shape<T, 256, 32>(p, prefix_tokens, chunk, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int D>
hipError_t launch_prefill_bs(const DecodeParams &p, int bs, int max_query_len, hipStream_t st)
{
    if constexpr (D == 128) {
        switch (bs) {
        case 8: return launch_prefill_wide<T, 8>(p, max_query_len, st);
        case 16: return launch_prefill_wide<T, 16>(p, max_query_len, st);
        case 32: return launch_prefill_wide<T, 32>(p, max_query_len, st);
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (bs) {
        case 8: return launch_prefill_shape<T, D, 8>(p, max_query_len, st);
        case 16: return launch_prefill_shape<T, D, 16>(p, max_query_len, st);
        case 32: return launch_prefill_shape<T, D, 32>(p, max_query_len, st);
        default: return hipErrorInvalidValue;
        }
    }
}

template <typename T>
hipError_t launch_prefill_shared_bs(const DecodeParams &p, int bs, int max_query_len, hipStream_t st)
{
    switch (bs) {
    case 8: return launch_prefill_shared_wide<T, 8>(p, max_query_len, st);
    case 16: return launch_prefill_shared_wide<T, 16>(p, max_query_len, st);
    case 32: return launch_prefill_shared_wide<T, 32>(p, max_query_len, st);
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
