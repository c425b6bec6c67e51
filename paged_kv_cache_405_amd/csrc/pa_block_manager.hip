// pa_block_manager.hip -- the host block manager of pa_blocks.h (host code
// only: it launches nothing).
//
// Method: "vLLM 与 PagedAttention" (inference.mavenzero.com/case-studies/vllm),
// section 二 "PagedAttention 的解法": one table per request maps its logical
// blocks to physical blocks of a shared pool; a block is taken only when the
// request's last block is full; requests with a common prefix share blocks
// and copy one on write.  "指南", "Copy-on-Write：Prefix Caching 的基础":
// shared blocks are read-only until a request diverges.  Section 三 of the
// first page and "4. vLLM初识" 4.3: preempted requests move to CPU memory.
//
// Free blocks are ordered sets, so the lowest-numbered one is taken first and
// every run is reproducible.  Every operation checks all its preconditions --
// ids, pools, output sizes, free blocks -- before it changes anything, so a
// failed call leaves the manager as it was.
#include <climits>
#include <cstdint>
#include <mutex>
#include <set>
#include <unordered_map>
#include <vector>

#include "pa_blocks.h"

namespace {

enum Pool { GPU = 0, CPU = 1 };

struct Request {
    std::vector<int32_t> table;   // physical blocks, logical order
    int64_t len = 0;              // tokens
    Pool pool = GPU;
};

}  // namespace

struct pa_block_manager {
    int bs = 0;
    std::vector<int> ref[2];
    std::set<int32_t> free_blocks[2];
    std::unordered_map<int64_t, Request> reqs;
    std::mutex mu;

    int32_t take(Pool p) {
        const int32_t b = *free_blocks[p].begin();
        free_blocks[p].erase(free_blocks[p].begin());
        ref[p][b] = 1;
        return b;
    }
    void drop(Pool p, int32_t b) {
        if (--ref[p][b] == 0)
            free_blocks[p].insert(b);
    }
    Request *find(int64_t seq) {
        auto it = reqs.find(seq);
        return it == reqs.end() ? nullptr : &it->second;
    }
    // free GPU blocks an append of n tokens takes: the new blocks, plus a copy
    // when the last block is shared and only partly filled
    int64_t needed(const Request &r, int n) const {
        const int64_t blocks_after = (r.len + n + bs - 1) / bs;
        const int64_t fresh = blocks_after - (int64_t)r.table.size();
        const bool cow = n > 0 && r.len % bs != 0 && ref[GPU][r.table[r.len / bs]] > 1;
        return fresh + (cow ? 1 : 0);
    }
};

extern "C" {

pa_status pa_bm_create(int num_gpu_blocks, int num_cpu_blocks, int block_size, pa_block_manager **out)
{
    if (!out || num_gpu_blocks < 0 || num_cpu_blocks < 0 || block_size <= 0)
        return PA_ERR_INVALID_ARG;
    auto *bm = new pa_block_manager;
    bm->bs = block_size;
    bm->ref[GPU].assign(num_gpu_blocks, 0);
    bm->ref[CPU].assign(num_cpu_blocks, 0);
    for (int i = 0; i < num_gpu_blocks; ++i)
        bm->free_blocks[GPU].insert(bm->free_blocks[GPU].end(), i);
    for (int i = 0; i < num_cpu_blocks; ++i)
        bm->free_blocks[CPU].insert(bm->free_blocks[CPU].end(), i);
    *out = bm;
    return PA_OK;
}

void pa_bm_destroy(pa_block_manager *bm) { delete bm; }

pa_status pa_bm_add(pa_block_manager *bm, int64_t seq)
{
    if (!bm)
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    if (bm->find(seq))
        return PA_ERR_INVALID_ARG;
    bm->reqs.emplace(seq, Request{});
    return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager *bm, int64_t parent, int64_t child)
{
    if (!bm)
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    Request *p = bm->find(parent);
    if (!p || p->pool != GPU || bm->find(child))
        return PA_ERR_INVALID_ARG;
    Request c = *p;
    for (int32_t b : c.table)
        ++bm->ref[GPU][b];
    bm->reqs.emplace(child, std::move(c));
    return PA_OK;
}

pa_status pa_bm_blocks_needed(pa_block_manager *bm, int64_t seq, int n, int *out)
{
    if (!bm || !out || n < 0)
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    const Request *r = bm->find(seq);
    if (!r || r->pool != GPU)
        return PA_ERR_INVALID_ARG;
    const int64_t need = bm->needed(*r, n);
    if (need > INT_MAX)
        return PA_ERR_INVALID_ARG;
    *out = (int)need;
    return PA_OK;
}

pa_status pa_bm_append(pa_block_manager *bm, int64_t seq, int n, int64_t *slots, int32_t *copies, int max_copies,
                       int *num_copies)
{
    if (!bm || !num_copies || n < 0 || max_copies < 0 || (n > 0 && !slots))
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    Request *r = bm->find(seq);
    if (!r || r->pool != GPU)
        return PA_ERR_INVALID_ARG;
    const int bs = bm->bs;
    const bool cow = n > 0 && r->len % bs != 0 && bm->ref[GPU][r->table[r->len / bs]] > 1;
    if (cow && (max_copies < 1 || !copies))
        return PA_ERR_INVALID_ARG;
    if (bm->needed(*r, n) > (int64_t)bm->free_blocks[GPU].size())
        return PA_ERR_NO_BLOCKS;
    int nc = 0;
    for (int64_t t = r->len; t < r->len + n; ++t) {
        const int64_t j = t / bs;
        if (j == (int64_t)r->table.size()) {
            r->table.push_back(bm->take(GPU));                 // the last block is full: take one
        } else if (bm->ref[GPU][r->table[j]] > 1) {            // writing into a shared block: copy it first
            const int32_t fresh = bm->take(GPU);
            copies[2 * nc] = r->table[j];
            copies[2 * nc + 1] = fresh;
            ++nc;
            bm->drop(GPU, r->table[j]);
            r->table[j] = fresh;
        }
        slots[t - r->len] = (int64_t)r->table[j] * bs + t % bs;
    }
    r->len += n;
    *num_copies = nc;
    return PA_OK;
}

pa_status pa_bm_free(pa_block_manager *bm, int64_t seq)
{
    if (!bm)
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    Request *r = bm->find(seq);
    if (!r)
        return PA_ERR_INVALID_ARG;
    for (int32_t b : r->table)
        bm->drop(r->pool, b);
    bm->reqs.erase(seq);
    return PA_OK;
}

// move a request's blocks from pool `from` to fresh blocks of the other pool
static pa_status move_request(pa_block_manager *bm, int64_t seq, Pool from, int32_t *pairs, int max_pairs,
                              int *num_pairs)
{
    if (!bm || !num_pairs || max_pairs < 0)
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    Request *r = bm->find(seq);
    if (!r || r->pool != from)
        return PA_ERR_INVALID_ARG;
    const Pool to = from == GPU ? CPU : GPU;
    const int64_t nb = (int64_t)r->table.size();
    if (nb > max_pairs || (nb > 0 && !pairs))
        return PA_ERR_INVALID_ARG;
    if (nb > (int64_t)bm->free_blocks[to].size())
        return PA_ERR_NO_BLOCKS;
    for (int64_t j = 0; j < nb; ++j) {
        const int32_t dst = bm->take(to);
        pairs[2 * j] = r->table[j];
        pairs[2 * j + 1] = dst;
        bm->drop(from, r->table[j]);
        r->table[j] = dst;
    }
    r->pool = to;
    *num_pairs = (int)nb;
    return PA_OK;
}

pa_status pa_bm_swap_out(pa_block_manager *bm, int64_t seq, int32_t *pairs, int max_pairs, int *num_pairs)
{
    return move_request(bm, seq, GPU, pairs, max_pairs, num_pairs);
}

pa_status pa_bm_swap_in(pa_block_manager *bm, int64_t seq, int32_t *pairs, int max_pairs, int *num_pairs)
{
    return move_request(bm, seq, CPU, pairs, max_pairs, num_pairs);
}

pa_status pa_bm_block_tables(pa_block_manager *bm, const int64_t *seqs, int n, int max_blocks, int32_t *tables,
                             int32_t *context_lens)
{
    if (!bm || n < 0 || max_blocks <= 0 || (n > 0 && (!seqs || !tables || !context_lens)))
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    for (int i = 0; i < n; ++i) {
        const Request *r = bm->find(seqs[i]);
        if (!r || r->pool != GPU || (int64_t)r->table.size() > max_blocks || r->len > INT32_MAX)
            return PA_ERR_INVALID_ARG;
    }
    for (int i = 0; i < n; ++i) {
        const Request &r = *bm->find(seqs[i]);
        int32_t *row = tables + (int64_t)i * max_blocks;
        for (int j = 0; j < max_blocks; ++j)
            row[j] = j < (int)r.table.size() ? r.table[j] : -1;
        context_lens[i] = (int32_t)r.len;
    }
    return PA_OK;
}

pa_status pa_bm_num_free(pa_block_manager *bm, int pool, int *out)
{
    if (!bm || !out || (pool != GPU && pool != CPU))
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    *out = (int)bm->free_blocks[pool].size();
    return PA_OK;
}

pa_status pa_bm_ref_count(pa_block_manager *bm, int pool, int block, int *out)
{
    if (!bm || !out || (pool != GPU && pool != CPU))
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    if (block < 0 || block >= (int)bm->ref[pool].size())
        return PA_ERR_INVALID_ARG;
    *out = bm->ref[pool][block];
    return PA_OK;
}

pa_status pa_bm_info(pa_block_manager *bm, int64_t seq, int64_t *num_tokens, int *num_blocks, int *on_gpu)
{
    if (!bm || !num_tokens || !num_blocks || !on_gpu)
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    const Request *r = bm->find(seq);
    if (!r)
        return PA_ERR_INVALID_ARG;
    *num_tokens = r->len;
    *num_blocks = (int)r->table.size();
    *on_gpu = r->pool == GPU ? 1 : 0;
    return PA_OK;
}

}  // extern "C"
