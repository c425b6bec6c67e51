// pa_api.hip -- the C ABI declared in include/pa.h: host-side argument
// checks, the launch plan (split-K partition, q-head grouping, workspace
// carving) and the kernel launches on the caller's stream.
//
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and touches no device state.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "pa.h"
#include "pa_blocks.h"
#include "pa_internal.h"

namespace {

constexpr size_t WS_ALIGN = 256;
// split-K partition after a shared prefix, in tokens: a multiple of the block size
#define PA_SUFFIX_TOKENS(bs) (pa::SHARED_PREFIX_SUFFIX_PARTITION / (bs) * (bs))

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool supported_head_dim(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }
bool supported_block_size(int b) { return b == 8 || b == 16 || b == 32; }
bool supported_dtype(pa_dtype t) { return t == PA_F32 || t == PA_F16 || t == PA_BF16; }
bool supported_layout(pa_layout l) { return l == PA_LAYOUT_BHTD || l == PA_LAYOUT_BTHD; }
bool supported_kernel(pa_kernel k) { return k == PA_KERNEL_AUTO || k == PA_KERNEL_VECTOR || k == PA_KERNEL_MFMA; }

// The matrix-core kernel needs 16-bit elements, head_dim a multiple of 128
// and q-head groups that fill at most 16 columns per workgroup.
bool mfma_shape(pa_dtype dtype, int head_dim, int group)
{
    return dtype != PA_F32 && (head_dim == 128 || head_dim == 256) && (group <= 16 || group % 16 == 0);
}

// Smallest q-head group the library sends to the matrix cores on its own:
// below it the per-token vector work is small enough for the VALU.
constexpr int MFMA_MIN_GROUP = 4;
constexpr long long AUTO_UNITS_PER_CU = 4;   // single pass at or above this many units per compute unit
// grid kernels take sequences longest first (seq_of_row) when a unit can
// hold more than this many tokens; below it the ranking costs more than the
// tail it saves (measured on MI355X: the shared-prefix call, whose suffix
// pass has units of at most 208 tokens, 73.2 us with the ranking against
// 69.2 us without)
constexpr long long ORDER_ROWS_MIN_TOKENS = 512;

// Tokens per step of the vector worker (its schedule unit): one or two
// wave-wide loads of 64 / (head_dim * elem_bytes / 16) token rows each, as
// many as a block holds.  Mirrors VecWorker's STEP_TOK.
long long vec_step_tokens(pa_dtype dtype, int head_dim, int block_size)
{
    const int vec = dtype == PA_F32 ? 4 : 8;           // elements per 16 bytes
    const int rows_per_load = 64 / (head_dim / vec);
    const int rows = rows_per_load < block_size ? rows_per_load : block_size;
    const int loads_per_block = block_size / rows;
    return (long long)(loads_per_block < 2 ? loads_per_block : 2) * rows;
}

struct Plan {
    bool mfma = false;          // grouped-query matrix-core kernel
    bool stream = false;        // balanced schedule (partition_tokens == 0)
    int n_waves = 0;            // stream: logical waves (one workgroup each)
    size_t off_first = 0, off_last = 0, off_ml = 0, off_acc = 0;   // stream: workspace sections
    int partition_blocks = 0;   // blocks per partition
    int max_partitions = 1;     // grid x extent
    int gt = 1;                 // q heads per workgroup
    int group_split = 1;        // workgroups per kv head
    size_t ml_bytes = 0;        // (max, sum) pairs, first in the workspace
    size_t ws_bytes = 0;        // total workspace (0 = single pass)
};

pa_status check_sizes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int max_blocks_per_seq, pa_dtype dtype, int partition_tokens)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0)
        return PA_ERR_INVALID_ARG;
    if (num_q_heads % num_kv_heads != 0)
        return PA_ERR_INVALID_ARG;
    if (!supported_dtype(dtype) || !supported_head_dim(head_dim) || !supported_block_size(block_size))
        return PA_ERR_UNSUPPORTED;
    if (partition_tokens < PA_PARTITION_BALANCED || (partition_tokens > 0 && partition_tokens % block_size != 0))
        return PA_ERR_INVALID_ARG;
    if ((long long)max_blocks_per_seq * block_size > (1LL << 30))
        return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

// Workgroups of the stream kernel for this shape that one compute unit of the
// current device holds at once, cached per (device, kernel shape).  Returns 0
// when there is no device or the query fails.
int stream_occupancy(pa_dtype dtype, bool mfma, int head_dim, int block_size, int gt, int *cus)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || *cus <= 0)
        return 0;
    static std::mutex mu;
    static std::map<std::tuple<int, int, int, int, int, int>, int> cache;
    const auto key = std::make_tuple(dev, (int)dtype, (int)mfma, head_dim, block_size, gt);
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find(key);
        if (it != cache.end())
            return it->second;
    }
    int occ = 0;
    hipError_t e;
    if (mfma)
        e = dtype == PA_F16 ? pa::stream_mfma_f16(nullptr, head_dim, block_size, nullptr, &occ)
                            : pa::stream_mfma_bf16(nullptr, head_dim, block_size, nullptr, &occ);
    else if (dtype == PA_F32)
        e = pa::stream_vec_f32(nullptr, head_dim, block_size, gt, nullptr, &occ);
    else if (dtype == PA_F16)
        e = pa::stream_vec_f16(nullptr, head_dim, block_size, gt, nullptr, &occ);
    else
        e = pa::stream_vec_bf16(nullptr, head_dim, block_size, gt, nullptr, &occ);
    if (e != hipSuccess || occ <= 0)
        return 0;
    std::lock_guard<std::mutex> lock(mu);
    cache[key] = occ;
    return occ;
}

pa_status make_plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                    int max_blocks_per_seq, pa_dtype dtype, int partition_tokens, pa_kernel kernel, Plan *pl)
{
    pa_status st = check_sizes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                               max_blocks_per_seq, dtype, partition_tokens);
    if (st != PA_OK)
        return st;
    if (!supported_kernel(kernel))
        return PA_ERR_UNSUPPORTED;
    const int group = num_q_heads / num_kv_heads;
    const bool mfma_ok = mfma_shape(dtype, head_dim, group);
    if (kernel == PA_KERNEL_MFMA && !mfma_ok)
        return PA_ERR_UNSUPPORTED;
    pl->mfma = kernel == PA_KERNEL_MFMA || (kernel == PA_KERNEL_AUTO && mfma_ok && group >= MFMA_MIN_GROUP);
    if (pl->mfma)
        pl->gt = group <= 16 ? group : 16;
    else
        pl->gt = group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
    pl->group_split = group / pl->gt;
    int pt = partition_tokens;
    if (pt == PA_PARTITION_AUTO) {
        // enough (sequence, head group) units that whole units, handed out by
        // the hardware as workgroups finish, keep every compute unit busy:
        // one pass, no reduce; else cut contexts into equal shares
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return PA_ERR_HIP;
        const long long units = (long long)num_seqs * num_kv_heads * pl->group_split;
        pt = units >= AUTO_UNITS_PER_CU * (long long)cus ? PA_PARTITION_SINGLE : PA_PARTITION_BALANCED;
    }
    const long long max_tokens = (long long)block_size * max_blocks_per_seq;
    if (pt <= 0 || pt >= max_tokens) {      // balanced schedule or single pass
        pl->partition_blocks = max_blocks_per_seq;
        pl->max_partitions = 1;
    } else {
        pl->partition_blocks = pt / block_size;
        pl->max_partitions = (max_blocks_per_seq + pl->partition_blocks - 1) / pl->partition_blocks;
    }
    if ((long long)num_kv_heads * pl->group_split > 65535 || num_seqs > 65535)
        return PA_ERR_UNSUPPORTED;
    if (pt == PA_PARTITION_BALANCED) {
        // balanced schedule: as many one-wave workgroups as the device holds at
        // once (a multiple of 8, one share per XCD), pieces for cut units
        int cus = 0;
        const int occ = stream_occupancy(dtype, pl->mfma, head_dim, block_size, pl->gt, &cus);
        if (occ <= 0)
            return PA_ERR_HIP;
        long long waves = (long long)cus * occ / 8 * 8;
        // never more waves than the stream can hold steps: a small batch
        // would otherwise start thousands of workgroups that find their
        // range empty (the tiny workload: 18 steps at most, 8192 waves)
        const long long step_tok = pl->mfma ? 16 : vec_step_tokens(dtype, head_dim, block_size);
        const long long max_steps = (long long)num_seqs * num_kv_heads * pl->group_split *
                                    (((long long)max_blocks_per_seq * block_size + step_tok - 1) / step_tok);
        waves = std::min(waves, (max_steps + 7) / 8 * 8);
        waves = waves < 8 ? 8 : (waves > (1 << 16) ? (1 << 16) : waves);   // N <= 2^16: 32-bit range arithmetic
        pl->stream = true;
        pl->n_waves = (int)waves;
        pl->partition_blocks = max_blocks_per_seq;
        pl->max_partitions = 1;
        const size_t units = (size_t)num_seqs * num_kv_heads * pl->group_split;
        const size_t pieces = 2 * (size_t)pl->n_waves;
        // [total steps T][unit_first][unit_last][piece max, sum][piece outputs]
        pl->off_first = WS_ALIGN;
        pl->off_last = pl->off_first + round_up(units * sizeof(int32_t), WS_ALIGN);
        pl->off_ml = pl->off_last + round_up(units * sizeof(int32_t), WS_ALIGN);
        pl->off_acc = pl->off_ml + round_up(pieces * pl->gt * sizeof(float2), WS_ALIGN);
        pl->ws_bytes = pl->off_acc + pieces * pl->gt * (size_t)head_dim * sizeof(float);
        pl->ml_bytes = 0;
        return PA_OK;
    }
    if (pl->max_partitions > 1) {
        const size_t units = (size_t)num_seqs * num_q_heads * pl->max_partitions;
        pl->ml_bytes = round_up(units * sizeof(float2), WS_ALIGN);
        pl->ws_bytes = pl->ml_bytes + units * (size_t)head_dim * sizeof(float);
    } else {
        pl->ml_bytes = 0;
        pl->ws_bytes = 0;
    }
    return PA_OK;
}

void layout_strides(pa_layout layout, int num_kv_heads, int block_size, int head_dim,
                    int64_t *block_stride, int64_t *head_stride, int64_t *token_stride)
{
    *block_stride = (int64_t)num_kv_heads * block_size * head_dim;
    if (layout == PA_LAYOUT_BHTD) {
        *head_stride = (int64_t)block_size * head_dim;
        *token_stride = head_dim;
    } else {
        *head_stride = head_dim;
        *token_stride = (int64_t)num_kv_heads * head_dim;
    }
}

int elem_bytes(pa_dtype t) { return t == PA_F32 ? 4 : 2; }

}  // namespace

// Device memory of pa_decode_noalloc: the split-K / balanced-schedule
// workspace of a decode call, owned by the library instead of the caller.
// Each GPU the library runs on holds its own copy until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host it names
// a stand-in, not device memory): it passes the address hipGetSymbolAddress
// gives for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_ptr[SCRATCH_MAX_DEVICES] = {};

// the address of `scratch` on the current device (looked up on the first
// call on that device, with the device current); null on failure
void *scratch_address()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES)
        return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        scratch_ptr[dev] = ptr;
    }
    return scratch_ptr[dev];
}

}  // namespace

namespace {

// The new K/V rows of a decode step: one token per sequence, sequence s's
// rows k_new/v_new[s] going to slot slots[s] (pa_decode_append).
struct AppendRows {
    const void *k_new;
    const void *v_new;
    const int64_t *slots;
};

pa_status launch_append_rows(const void *k, const void *v, void *k_cache, void *v_cache, const int64_t *slots,
                             int num_tokens, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             pa_dtype dtype, pa_layout layout, hipStream_t stream);

// pa_decode_ex, and pa_decode_append when app is given: every argument is
// checked before anything is enqueued, then the append kernel goes ahead of
// the decode
pa_status decode_call(void *out, const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens,
                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                      pa_dtype dtype, pa_layout layout, int partition_tokens, pa_kernel kernel,
                      unsigned flags, void *workspace, size_t workspace_bytes, void *stream, const AppendRows *app,
                      bool use_scratch = false)
{
    if (flags & ~(unsigned)PA_DECODE_SHARED_BLOCKS)
        return PA_ERR_INVALID_ARG;
    // argument checks (no HIP call), then the launch plan (which may query the
    // device for the balanced schedule), then the workspace
    pa_status st = check_sizes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                               dtype, partition_tokens);
    if (st != PA_OK)
        return st;
    if (!supported_kernel(kernel) || (kernel == PA_KERNEL_MFMA &&
                                      !mfma_shape(dtype, head_dim, num_q_heads / num_kv_heads)))
        return PA_ERR_UNSUPPORTED;
    if (!supported_layout(layout))
        return PA_ERR_UNSUPPORTED;
    if (num_blocks <= 0 || !std::isfinite(scale))
        return PA_ERR_INVALID_ARG;
    if (num_seqs == 0)
        return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
        return PA_ERR_INVALID_ARG;
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4))
        return PA_ERR_INVALID_ARG;
    Plan pl;
    st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, dtype,
                   partition_tokens, kernel, &pl);
    if (st != PA_OK)
        return st;
    if (use_scratch && pl.ws_bytes > 0) {
        // the library's own scratch, once every argument has been checked
        if (pl.ws_bytes > PA_NOALLOC_SCRATCH_BYTES)
            return PA_ERR_WORKSPACE;
        workspace = scratch_address();
        if (!workspace)
            return PA_ERR_HIP;
        workspace_bytes = PA_NOALLOC_SCRATCH_BYTES;
    }
    if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes || !aligned(workspace, 16)))
        return PA_ERR_WORKSPACE;

    pa::DecodeParams p;
    std::memset(&p, 0, sizeof(p));
    p.out = out;
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.tables = block_tables;
    p.ctx = context_lens;
    p.kv_cached = (flags & PA_DECODE_SHARED_BLOCKS) ? 1 : 0;
    p.order_rows = (int64_t)max_blocks_per_seq * block_size > ORDER_ROWS_MIN_TOKENS ? 1 : 0;
    if (pl.stream) {
        char *ws = static_cast<char *>(workspace);
        p.n_waves = pl.n_waves;
        p.stream_total = reinterpret_cast<uint64_t *>(ws);
        p.unit_first = reinterpret_cast<int32_t *>(ws + pl.off_first);
        p.unit_last = reinterpret_cast<int32_t *>(ws + pl.off_last);
        p.piece_ml = reinterpret_cast<float2 *>(ws + pl.off_ml);
        p.piece_acc = reinterpret_cast<float *>(ws + pl.off_acc);
    } else if (pl.ws_bytes > 0) {
        p.ws_ml = reinterpret_cast<float2 *>(workspace);
        p.ws_acc = reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.ml_bytes);
    }
    layout_strides(layout, num_kv_heads, block_size, head_dim, &p.block_stride, &p.head_stride, &p.token_stride);
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    p.partition_blocks = pl.partition_blocks;
    p.max_partitions = pl.max_partitions;
    p.group = num_q_heads / num_kv_heads;
    p.group_split = pl.group_split;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (app && launch_append_rows(app->k_new, app->v_new, const_cast<void *>(k_cache), const_cast<void *>(v_cache),
                                  app->slots, num_seqs, num_kv_heads, head_dim, block_size, num_blocks, dtype,
                                  layout, s) != PA_OK)
        return PA_ERR_HIP;
    if (pl.stream) {
        if (pl.mfma)
            e = dtype == PA_F16 ? pa::stream_mfma_f16(&p, head_dim, block_size, s, nullptr)
                                : pa::stream_mfma_bf16(&p, head_dim, block_size, s, nullptr);
        else if (dtype == PA_F32)
            e = pa::stream_vec_f32(&p, head_dim, block_size, pl.gt, s, nullptr);
        else if (dtype == PA_F16)
            e = pa::stream_vec_f16(&p, head_dim, block_size, pl.gt, s, nullptr);
        else
            e = pa::stream_vec_bf16(&p, head_dim, block_size, pl.gt, s, nullptr);
        if (e != hipSuccess)
            return PA_ERR_HIP;
        return pa::launch_stream_reduce(p, (int)dtype, head_dim, pl.gt, s) == hipSuccess ? PA_OK : PA_ERR_HIP;
    }
    if (pl.mfma) {
        e = dtype == PA_F16 ? pa::launch_mfma_f16(p, head_dim, block_size, s)
                            : pa::launch_mfma_bf16(p, head_dim, block_size, s);
    } else {
        switch (dtype) {
        case PA_F32: e = pa::launch_decode_f32(p, head_dim, block_size, pl.gt, s); break;
        case PA_F16: e = pa::launch_decode_f16(p, head_dim, block_size, pl.gt, s); break;
        default: e = pa::launch_decode_bf16(p, head_dim, block_size, pl.gt, s); break;
        }
    }
    if (e != hipSuccess)
        return PA_ERR_HIP;
    if (pl.max_partitions > 1) {
        e = pa::launch_reduce(p, (int)dtype, head_dim, block_size, s);
        if (e != hipSuccess)
            return PA_ERR_HIP;
    }
    return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_path(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                         int max_blocks_per_seq, pa_dtype dtype, int partition_tokens, pa_kernel kernel,
                         int *partition_out, pa_kernel *kernel_out)
{
    if (!partition_out || !kernel_out)
        return PA_ERR_INVALID_ARG;
    Plan pl;
    const pa_status st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                   max_blocks_per_seq, dtype, partition_tokens, kernel, &pl);
    if (st != PA_OK)
        return st;
    *partition_out = pl.stream ? PA_PARTITION_BALANCED
                   : pl.max_partitions > 1 ? pl.partition_blocks * block_size : PA_PARTITION_SINGLE;
    *kernel_out = pl.mfma ? PA_KERNEL_MFMA : PA_KERNEL_VECTOR;
    return PA_OK;
}

pa_status pa_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, int max_blocks_per_seq, pa_dtype dtype,
                                    int partition_tokens, size_t *bytes_out)
{
    if (!bytes_out)
        return PA_ERR_INVALID_ARG;
    // enough for whichever kernel the call picks
    *bytes_out = 0;
    Plan pl;
    pa_status st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             max_blocks_per_seq, dtype, partition_tokens, PA_KERNEL_VECTOR, &pl);
    if (st != PA_OK)
        return st;
    size_t bytes = pl.ws_bytes;
    if (mfma_shape(dtype, head_dim, num_q_heads / num_kv_heads)) {
        Plan pm;
        st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, dtype,
                       partition_tokens, PA_KERNEL_MFMA, &pm);
        if (st != PA_OK)
            return st;
        bytes = pm.ws_bytes > bytes ? pm.ws_bytes : bytes;
    }
    *bytes_out = bytes;
    return PA_OK;
}

pa_status pa_decode_ex(void *out, const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, const int32_t *context_lens,
                       int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                       int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                       pa_dtype dtype, pa_layout layout, int partition_tokens, pa_kernel kernel,
                       unsigned flags, void *workspace, size_t workspace_bytes, void *stream)
{
    return decode_call(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, max_blocks_per_seq, num_blocks, scale, dtype, layout, partition_tokens,
                       kernel, flags, workspace, workspace_bytes, stream, nullptr);
}

pa_status pa_decode_append(void *out, const void *q, const void *k_new, const void *v_new, void *k_cache,
                           void *v_cache, const int64_t *slot_mapping, const int32_t *block_tables,
                           const int32_t *context_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                           int head_dim, int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                           pa_dtype dtype, pa_layout layout, int partition_tokens, pa_kernel kernel,
                           unsigned flags, void *workspace, size_t workspace_bytes, void *stream)
{
    if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping))
        return PA_ERR_INVALID_ARG;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slot_mapping, 8))
        return PA_ERR_INVALID_ARG;
    const AppendRows app{k_new, v_new, slot_mapping};
    return decode_call(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, max_blocks_per_seq, num_blocks, scale, dtype, layout, partition_tokens,
                       kernel, flags, workspace, workspace_bytes, stream, &app);
}

pa_status pa_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, const int32_t *context_lens,
                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                    int block_size, int max_blocks_per_seq, float scale, pa_dtype dtype,
                    void *workspace, size_t workspace_bytes, void *stream)
{
    return pa_decode_ex(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                        num_kv_heads, head_dim, block_size, max_blocks_per_seq, INT32_MAX, scale, dtype,
                        PA_LAYOUT_BHTD, PA_PARTITION_AUTO, PA_KERNEL_AUTO, 0u, workspace, workspace_bytes, stream);
}

pa_status pa_decode_noalloc(void *out, const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, const int32_t *context_lens,
                            int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                            int block_size, int max_blocks_per_seq, float scale, pa_dtype dtype, void *stream)
{
    return decode_call(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, max_blocks_per_seq, INT32_MAX, scale, dtype, PA_LAYOUT_BHTD,
                       PA_PARTITION_AUTO, PA_KERNEL_AUTO, 0u, nullptr, 0, stream, nullptr, true);
}

}  // extern "C"

namespace {

// the launch plan of a shared-prefix decode (host only; checks included)
struct PrefixPlan {
    Plan suffix;                  // the split-K decode over the blocks after the prefix
    int chunk = 0, n_chunks = 0, max_partitions = 0, prefix_group_split = 1;
    size_t ml_bytes = 0, ws_bytes = 0;
};

// The prefix chunk of a call: the smallest multiple of 32 tokens that keeps
// the prefix pass to about one workgroup per compute unit, within
// [SHARED_PREFIX_CHUNK_MIN, SHARED_PREFIX_CHUNK_MAX].  Smaller chunks start
// more workgroups but leave more partials to write and merge; the pass does
// best when its workgroups just cover the compute units (measured on MI355X,
// 128 sequences over a 1504-token prefix at 32 kv heads: 192-token chunks,
// 8 x 32 = 256 workgroups, 63.4 us per call against 65.0 at 256 tokens and
// 67.5 at 128).
int prefix_chunk(int prefix_tokens, int workgroups_per_chunk, int cus)
{
    const int chunks = std::max(1, cus / std::max(1, workgroups_per_chunk));
    int c = (prefix_tokens + chunks - 1) / chunks;
    c = (c + 31) / 32 * 32;
    return std::min(std::max(c, pa::SHARED_PREFIX_CHUNK_MIN), pa::SHARED_PREFIX_CHUNK_MAX);
}

// chunk: the prefix chunk of the call; the workspace query plans with the
// smallest chunk, whose partition count bounds every call's
pa_status make_prefix_plan(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                           int max_blocks_per_seq, pa_dtype dtype, int prefix_blocks, int chunk, PrefixPlan *pp)
{
    pa_status st = check_sizes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, dtype,
                               PA_PARTITION_SINGLE);
    if (st != PA_OK)
        return st;
    if (prefix_blocks < 0 || prefix_blocks > max_blocks_per_seq)
        return PA_ERR_INVALID_ARG;
    const int group = num_q_heads / num_kv_heads;
    if (!mfma_shape(dtype, head_dim, group))
        return PA_ERR_UNSUPPORTED;
    const int pt = PA_SUFFIX_TOKENS(block_size);
    st = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, dtype, pt,
                   PA_KERNEL_AUTO, &pp->suffix);
    if (st != PA_OK)
        return st;
    pp->chunk = chunk;
    pp->n_chunks = (prefix_blocks * block_size + chunk - 1) / chunk;
    const int rest = max_blocks_per_seq - prefix_blocks;
    const int pb = pt / block_size;
    pp->max_partitions = pp->n_chunks + (rest + pb - 1) / pb;
    pp->prefix_group_split = group <= 16 ? 1 : group / 16;
    if ((long long)num_kv_heads * pp->prefix_group_split > 65535 || pp->max_partitions > 65535)
        return PA_ERR_UNSUPPORTED;
    const size_t units = (size_t)num_seqs * num_q_heads * pp->max_partitions;
    pp->ml_bytes = round_up(units * sizeof(float2), WS_ALIGN);
    pp->ws_bytes = pp->ml_bytes + units * (size_t)head_dim * sizeof(float);
    return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_shared_prefix_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                                  int block_size, int max_blocks_per_seq, pa_dtype dtype,
                                                  int prefix_blocks, size_t *bytes_out)
{
    if (!bytes_out)
        return PA_ERR_INVALID_ARG;
    PrefixPlan pp;
    const pa_status st = make_prefix_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                          max_blocks_per_seq, dtype, prefix_blocks, pa::SHARED_PREFIX_CHUNK_MIN, &pp);
    if (st != PA_OK)
        return st;
    *bytes_out = pp.ws_bytes;
    return PA_OK;
}

pa_status pa_decode_shared_prefix(void *out, const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                                  int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                  int max_blocks_per_seq, int num_blocks, int prefix_blocks, float scale,
                                  pa_dtype dtype, pa_layout layout, void *workspace, size_t workspace_bytes,
                                  void *stream)
{
    if (!supported_layout(layout))
        return PA_ERR_UNSUPPORTED;
    if (num_blocks <= 0 || !std::isfinite(scale))
        return PA_ERR_INVALID_ARG;
    PrefixPlan pp;
    pa_status st = make_prefix_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                    dtype, prefix_blocks, pa::SHARED_PREFIX_CHUNK_MIN, &pp);
    if (st != PA_OK)
        return st;
    if (num_seqs == 0)
        return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
        return PA_ERR_INVALID_ARG;
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4))
        return PA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < pp.ws_bytes || !aligned(workspace, 16))
        return PA_ERR_WORKSPACE;
    // Both passes go in one launch (pa_shared_prefix.h) when the own blocks
    // take the matrix-core kernel or the vector one with 1 or 2 q heads per
    // workgroup: the prefix pass's workgroups then run beside the own-blocks
    // pass instead of before it.
    const bool combined = prefix_blocks > 0 && pp.max_partitions > pp.n_chunks &&
                          (pp.suffix.mfma || pp.suffix.gt == 1 || pp.suffix.gt == 2);
    // every argument checked (the workspace against the smallest chunk's plan,
    // as the query states it): the chunk of the call.  Beside the own-blocks
    // pass, few long chunks: fewer prefix workgroups taking room from it and
    // fewer partials for the reduce (measured on the shared-prefix workload:
    // 64.2 us per call as two launches, 62.8 / 61.1 / 57.9 / 54.7 / 54.5 /
    // 59.9 / 69.3 us combined with chunks of 192 / 256 / 384 / 512 / 768 /
    // 1024 / 1504 tokens).  Alone, about one workgroup per compute unit.
    if (prefix_blocks > 0) {
        const int prefix_tokens = prefix_blocks * block_size;
        int chunk;
        if (combined) {
            chunk = std::min(pa::SHARED_PREFIX_CHUNK_MAX,
                             std::max(pa::SHARED_PREFIX_CHUNK_MIN, (prefix_tokens + 31) / 32 * 32));
        } else {
            int dev = 0, cus = 0;
            if (hipGetDevice(&dev) != hipSuccess ||
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
                return PA_ERR_HIP;
            const int group = num_q_heads / num_kv_heads;
            chunk = prefix_chunk(prefix_tokens,
                                 pa::prefix_workgroups(num_seqs, group, pp.prefix_group_split, num_kv_heads), cus);
        }
        st = make_prefix_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, dtype,
                              prefix_blocks, chunk, &pp);
        if (st != PA_OK)
            return st;
    }

    pa::DecodeParams p;
    std::memset(&p, 0, sizeof(p));
    p.out = out;
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.tables = block_tables;
    p.ctx = context_lens;
    p.ws_ml = reinterpret_cast<float2 *>(workspace);
    p.ws_acc = reinterpret_cast<float *>(static_cast<char *>(workspace) + pp.ml_bytes);
    layout_strides(layout, num_kv_heads, block_size, head_dim, &p.block_stride, &p.head_stride, &p.token_stride);
    p.num_seqs = num_seqs;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    p.group = num_q_heads / num_kv_heads;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);
    p.max_partitions = pp.max_partitions;
    p.first_partition = pp.n_chunks;
    p.part_base_blocks = prefix_blocks;
    p.order_rows = (int64_t)(max_blocks_per_seq - prefix_blocks) * block_size > ORDER_ROWS_MIN_TOKENS ? 1 : 0;
    p.partition_blocks = PA_SUFFIX_TOKENS(block_size) / block_size;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    // both passes in one launch (their data is disjoint; the reduce follows both)
    if (combined) {
        pa::DecodeParams px = p, sx = p;
        px.group_split = pp.prefix_group_split;
        sx.group_split = pp.suffix.group_split;
        const int gt = pp.suffix.mfma ? 0 : pp.suffix.gt;
        e = dtype == PA_F16 ? pa::launch_shared_prefix_f16(sx, px, head_dim, block_size, gt,
                                                          prefix_blocks * block_size, pp.chunk, s)
                            : pa::launch_shared_prefix_bf16(sx, px, head_dim, block_size, gt,
                                                           prefix_blocks * block_size, pp.chunk, s);
        if (e != hipSuccess)
            return PA_ERR_HIP;
        return pa::launch_reduce(p, (int)dtype, head_dim, block_size, s) == hipSuccess ? PA_OK : PA_ERR_HIP;
    }
    // the prefix, once for the whole batch
    if (pp.n_chunks > 0) {
        pa::DecodeParams px = p;
        px.group_split = pp.prefix_group_split;
        e = dtype == PA_F16 ? pa::launch_prefix_f16(px, head_dim, block_size, prefix_blocks * block_size, pp.chunk, s)
                            : pa::launch_prefix_bf16(px, head_dim, block_size, prefix_blocks * block_size, pp.chunk, s);
        if (e != hipSuccess)
            return PA_ERR_HIP;
    }
    // each sequence's own blocks
    if (pp.max_partitions > pp.n_chunks) {
        pa::DecodeParams sx = p;
        sx.group_split = pp.suffix.group_split;
        if (pp.suffix.mfma) {
            e = dtype == PA_F16 ? pa::launch_mfma_f16(sx, head_dim, block_size, s)
                                : pa::launch_mfma_bf16(sx, head_dim, block_size, s);
        } else {
            e = dtype == PA_F16 ? pa::launch_decode_f16(sx, head_dim, block_size, pp.suffix.gt, s)
                                : pa::launch_decode_bf16(sx, head_dim, block_size, pp.suffix.gt, s);
        }
        if (e != hipSuccess)
            return PA_ERR_HIP;
    }
    return pa::launch_reduce(p, (int)dtype, head_dim, block_size, s) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_reshape_and_cache(const void *k, const void *v, void *k_cache, void *v_cache,
                               const int64_t *slot_mapping, int num_tokens, int num_kv_heads,
                               int head_dim, int block_size, int num_blocks, pa_dtype dtype,
                               pa_layout layout, void *stream)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0)
        return PA_ERR_INVALID_ARG;
    if (!supported_dtype(dtype) || !supported_head_dim(head_dim) || !supported_block_size(block_size) ||
        !supported_layout(layout))
        return PA_ERR_UNSUPPORTED;
    if (num_tokens == 0)
        return PA_OK;
    if (!k || !v || !k_cache || !v_cache || !slot_mapping)
        return PA_ERR_INVALID_ARG;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(slot_mapping, 8))
        return PA_ERR_INVALID_ARG;

    return launch_append_rows(k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
                              block_size, num_blocks, dtype, layout, static_cast<hipStream_t>(stream));
}

namespace {

// the checks and launch parameters of the prefill entry points; *done: nothing to compute
pa_status prefill_setup(void *out, const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *block_tables, const int32_t *context_lens, const int32_t *query_start,
                        int num_seqs, int total_q, int max_query_len, int num_q_heads, int num_kv_heads,
                        int head_dim, int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                        pa_dtype dtype, pa_layout layout, unsigned flags, pa::DecodeParams *p, bool *done)
{
    *done = false;
    if (flags & ~(unsigned)PA_DECODE_SHARED_BLOCKS)
        return PA_ERR_INVALID_ARG;
    pa_status st = check_sizes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                               dtype, PA_PARTITION_SINGLE);
    if (st != PA_OK)
        return st;
    const int group = num_q_heads / num_kv_heads;
    if (!mfma_shape(dtype, head_dim, group) || !supported_layout(layout))
        return PA_ERR_UNSUPPORTED;
    if (total_q < 0 || max_query_len < 0 || num_blocks <= 0 || !std::isfinite(scale))
        return PA_ERR_INVALID_ARG;
    if (num_seqs > 65535 || (long long)num_kv_heads * (group <= 16 ? 1 : group / 16) > 65535)
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0 || total_q == 0 || max_query_len == 0) {
        *done = true;
        return PA_OK;
    }
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
        return PA_ERR_INVALID_ARG;
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4))
        return PA_ERR_INVALID_ARG;

    std::memset(p, 0, sizeof(*p));
    p->out = out;
    p->q = q;
    p->k = k_cache;
    p->v = v_cache;
    p->tables = block_tables;
    p->ctx = context_lens;
    p->query_start = query_start;
    p->total_q = total_q;
    p->kv_cached = (flags & PA_DECODE_SHARED_BLOCKS) ? 1 : 0;
    layout_strides(layout, num_kv_heads, block_size, head_dim, &p->block_stride, &p->head_stride, &p->token_stride);
    p->num_seqs = num_seqs;
    p->num_q_heads = num_q_heads;
    p->num_kv_heads = num_kv_heads;
    p->max_blocks = max_blocks_per_seq;
    p->num_blocks = num_blocks;
    p->partition_blocks = max_blocks_per_seq;
    p->max_partitions = 1;
    p->group = group;
    p->group_split = group <= 16 ? 1 : group / 16;
    p->scale_log2 = (float)((double)scale * 1.4426950408889634);
    return PA_OK;
}

// the prefix partials of the shared-prefix prefill: (max, sum) then the
// unnormalised output of every (q row, q head)
size_t prefill_partial_ml_bytes(int total_q, int num_q_heads)
{
    return round_up((size_t)total_q * num_q_heads * sizeof(float2), WS_ALIGN);
}

}  // namespace

pa_status pa_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_tables, const int32_t *context_lens, const int32_t *query_start,
                     int num_seqs, int total_q, int max_query_len, int num_q_heads, int num_kv_heads, int head_dim,
                     int block_size, int max_blocks_per_seq, int num_blocks, float scale, pa_dtype dtype,
                     pa_layout layout, unsigned flags, void *stream)
{
    pa::DecodeParams p;
    bool done = false;
    const pa_status st = prefill_setup(out, q, k_cache, v_cache, block_tables, context_lens, query_start, num_seqs,
                                       total_q, max_query_len, num_q_heads, num_kv_heads, head_dim, block_size,
                                       max_blocks_per_seq, num_blocks, scale, dtype, layout, flags, &p, &done);
    if (st != PA_OK || done)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = dtype == PA_F16 ? pa::launch_prefill_f16(p, head_dim, block_size, max_query_len, s)
                                         : pa::launch_prefill_bf16(p, head_dim, block_size, max_query_len, s);
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_prefill_shared_prefix_workspace_bytes(int total_q, int num_q_heads, int head_dim, int block_size,
                                                   int prefix_blocks, size_t *bytes_out)
{
    if (!bytes_out)
        return PA_ERR_INVALID_ARG;
    *bytes_out = 0;
    if (total_q < 0 || num_q_heads <= 0 || prefix_blocks < 0)
        return PA_ERR_INVALID_ARG;
    if (!supported_head_dim(head_dim) || !supported_block_size(block_size))
        return PA_ERR_UNSUPPORTED;
    if (head_dim != 128 || pa::wide_prefix_split(prefix_blocks, block_size) == 0 || total_q == 0)
        return PA_OK;   // computed as pa_prefill: no workspace
    *bytes_out = prefill_partial_ml_bytes(total_q, num_q_heads) +
                 (size_t)total_q * num_q_heads * head_dim * sizeof(float);
    return PA_OK;
}

pa_status pa_prefill_shared_prefix(void *out, const void *q, const void *k_cache, const void *v_cache,
                                   const int32_t *block_tables, const int32_t *context_lens,
                                   const int32_t *query_start, int num_seqs, int total_q, int max_query_len,
                                   int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                   int max_blocks_per_seq, int num_blocks, int prefix_blocks, float scale,
                                   pa_dtype dtype, pa_layout layout, void *workspace, size_t workspace_bytes,
                                   void *stream)
{
    pa::DecodeParams p;
    bool done = false;
    pa_status st = prefill_setup(out, q, k_cache, v_cache, block_tables, context_lens, query_start, num_seqs,
                                 total_q, max_query_len, num_q_heads, num_kv_heads, head_dim, block_size,
                                 max_blocks_per_seq, num_blocks, scale, dtype, layout, 0u, &p, &done);
    if (st != PA_OK)
        return st;
    if (prefix_blocks < 0 || prefix_blocks > max_blocks_per_seq)
        return PA_ERR_INVALID_ARG;
    if (done)
        return PA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (head_dim != 128 || pa::wide_prefix_split(prefix_blocks, block_size) == 0) {
        // less than one whole step to share, or the head_dim-256 kernel (no shared-prefix form): every row
        // over its whole history
        e = dtype == PA_F16 ? pa::launch_prefill_f16(p, head_dim, block_size, max_query_len, s)
                            : pa::launch_prefill_bf16(p, head_dim, block_size, max_query_len, s);
        return e == hipSuccess ? PA_OK : PA_ERR_HIP;
    }
    size_t need = 0;
    st = pa_prefill_shared_prefix_workspace_bytes(total_q, num_q_heads, head_dim, block_size, prefix_blocks, &need);
    if (st != PA_OK)
        return st;
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16))
        return PA_ERR_WORKSPACE;
    p.part_base_blocks = prefix_blocks;
    p.ws_ml = reinterpret_cast<float2 *>(workspace);
    p.ws_acc = reinterpret_cast<float *>(static_cast<char *>(workspace) + prefill_partial_ml_bytes(total_q, num_q_heads));
    e = dtype == PA_F16 ? pa::launch_prefill_shared_f16(p, block_size, max_query_len, s)
                        : pa::launch_prefill_shared_bf16(p, block_size, max_query_len, s);
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

static pa_status copy_blocks_common(void *dst_k, void *dst_v, const void *src_k, const void *src_v,
                                    const int32_t *pairs, int num_pairs, int num_dst_blocks, int num_src_blocks,
                                    int block_size, int num_kv_heads, int head_dim, pa_dtype dtype, void *stream)
{
    if (num_pairs < 0 || num_dst_blocks <= 0 || num_src_blocks <= 0 || num_kv_heads <= 0)
        return PA_ERR_INVALID_ARG;
    if (!supported_dtype(dtype) || !supported_head_dim(head_dim) || !supported_block_size(block_size))
        return PA_ERR_UNSUPPORTED;
    if (num_pairs == 0)
        return PA_OK;
    if (!dst_k || !dst_v || !src_k || !src_v || !pairs)
        return PA_ERR_INVALID_ARG;
    if (!aligned(dst_k, 16) || !aligned(dst_v, 16) || !aligned(src_k, 16) || !aligned(src_v, 16) ||
        !aligned(pairs, 4))
        return PA_ERR_INVALID_ARG;
    pa::CopyParams c;
    c.dst_k = dst_k;
    c.dst_v = dst_v;
    c.src_k = src_k;
    c.src_v = src_v;
    c.pairs = pairs;
    c.num_pairs = num_pairs;
    c.num_src_blocks = num_src_blocks;
    c.num_dst_blocks = num_dst_blocks;
    c.block_bytes = (int64_t)block_size * num_kv_heads * head_dim * elem_bytes(dtype);
    return pa::launch_copy_blocks(c, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs, int num_pairs, int num_blocks,
                         int block_size, int num_kv_heads, int head_dim, pa_dtype dtype, void *stream)
{
    return copy_blocks_common(k_cache, v_cache, k_cache, v_cache, pairs, num_pairs, num_blocks, num_blocks,
                              block_size, num_kv_heads, head_dim, dtype, stream);
}

// The address a kernel uses for p: p itself for device (or managed) memory,
// the device mapping of pinned host memory.  False for memory the device
// cannot reach (pageable host memory), which must never get to a kernel.
static bool device_address(const void *p, const void **out)
{
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) {
        *out = p;
        return true;
    }
    if (a.type == hipMemoryTypeHost && a.devicePointer) {
        const ptrdiff_t off = a.hostPointer ? static_cast<const char *>(p) - static_cast<const char *>(a.hostPointer) : 0;
        *out = static_cast<const char *>(a.devicePointer) + off;
        return true;
    }
    return false;
}

pa_status pa_swap_blocks(void *dst_k, void *dst_v, const void *src_k, const void *src_v, const int32_t *pairs,
                         int num_pairs, int num_dst_blocks, int num_src_blocks, int block_size, int num_kv_heads,
                         int head_dim, pa_dtype dtype, void *stream)
{
    if (num_pairs > 0 && dst_k && dst_v && src_k && src_v && pairs) {
        const void *dk, *dv, *sk, *sv, *pp;
        if (!device_address(dst_k, &dk) || !device_address(dst_v, &dv) || !device_address(src_k, &sk) ||
            !device_address(src_v, &sv) || !device_address(pairs, &pp))
            return PA_ERR_INVALID_ARG;
        return copy_blocks_common(const_cast<void *>(dk), const_cast<void *>(dv), sk, sv,
                                  static_cast<const int32_t *>(pp), num_pairs, num_dst_blocks, num_src_blocks,
                                  block_size, num_kv_heads, head_dim, dtype, stream);
    }
    return copy_blocks_common(dst_k, dst_v, src_k, src_v, pairs, num_pairs, num_dst_blocks, num_src_blocks,
                              block_size, num_kv_heads, head_dim, dtype, stream);
}

const char *pa_status_string(pa_status status)
{
    switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape, element type or layout";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch failed";
    case PA_ERR_NO_BLOCKS: return "not enough free blocks";
    default: return "unknown status";
    }
}

int pa_abi_version(void) { return 203; }

}  // extern "C"

namespace {

// the append kernel over num_tokens new rows (arguments already checked)
pa_status launch_append_rows(const void *k, const void *v, void *k_cache, void *v_cache, const int64_t *slots,
                             int num_tokens, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             pa_dtype dtype, pa_layout layout, hipStream_t stream)
{
    pa::AppendParams a;
    std::memset(&a, 0, sizeof(a));
    a.k = k;
    a.v = v;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.slots = slots;
    layout_strides(layout, num_kv_heads, block_size, head_dim, &a.block_stride, &a.head_stride, &a.token_stride);
    a.num_tokens = num_tokens;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.num_slots = (int64_t)num_blocks * block_size;
    a.elem_bytes = elem_bytes(dtype);
    a.chunks_per_head = head_dim * a.elem_bytes / 16;
    return pa::launch_append(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

