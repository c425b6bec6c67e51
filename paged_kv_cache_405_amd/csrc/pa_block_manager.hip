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
// Section 四 "Prefix Caching": the KV of a prompt's prefix stays in a
// least-recently-used cache, and a later request with the same prefix reuses
// it and computes only the rest.
//
// Free blocks are ordered sets, so the lowest-numbered one is taken first and
// every run is reproducible.  Every operation checks all its preconditions --
// ids, pools, output sizes, free blocks -- before it changes anything, so a
// failed call leaves the manager as it was.
//
// Prefix cache: a full GPU block of a request whose every token is known is
// entered under a 64-bit chain hash of its whole token prefix (the hash of the
// block before it and the block's own tokens, mixed with the SplitMix64
// finaliser); a lookup accepts an entry only if its tokens and its parent's
// hash match as well.  A cached block that no request holds stays cached but
// can be taken: an allocation takes a free block first, else the cached block
// released longest ago (ties: lowest index), which then leaves the cache.
// A request's blocks are released last block first, so the head of a prefix
// outlives its tail.
#include <climits>
#include <cstdint>
#include <mutex>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pa_blocks.h"

namespace {

enum Pool { GPU = 0, CPU = 1 };

struct Request {
    std::vector<int32_t> table;   // physical blocks, logical order
    int64_t len = 0;              // tokens
    Pool pool = GPU;
    // prefix cache bookkeeping
    bool known = true;                 // every token given (add_cached / append_tokens)
    std::vector<int32_t> tokens;       // those tokens, while known
    std::vector<uint64_t> chain;       // chain hash of each full block's prefix
    size_t registered = 0;             // full blocks already offered to the cache
};

struct CacheEntry {
    uint64_t hash = 0, parent = 0;     // chain hash of the prefix through this block, and of the one before
    std::vector<int32_t> toks;         // the block's own tokens
    uint64_t released = 0;             // clock when its last holder let go
};

constexpr uint64_t CHAIN_SEED = 0x243F6A8885A308D3ull;   // the hash "before" a request's first block

uint64_t mix64(uint64_t x)
{
    x ^= x >> 30;
    x *= 0xBF58476D1CE4E5B9ull;
    x ^= x >> 27;
    x *= 0x94D049BB133111EBull;
    x ^= x >> 31;
    return x;
}

uint64_t block_hash(uint64_t parent, const int32_t *t, int bs)
{
    uint64_t h = mix64(parent ^ 0x9E3779B97F4A7C15ull);
    for (int i = 0; i < bs; ++i)
        h = mix64(h + (uint64_t)(uint32_t)t[i] + 0x9E3779B97F4A7C15ull);
    return h;
}

}  // namespace

struct pa_block_manager {
    int bs = 0;
    std::vector<int> ref[2];
    std::set<int32_t> free_blocks[2];
    std::unordered_map<int64_t, Request> reqs;
    std::unordered_map<uint64_t, int32_t> by_hash;       // prefix cache: chain hash -> block
    std::unordered_map<int32_t, CacheEntry> entries;     // cached block -> entry
    std::set<std::pair<uint64_t, int32_t>> evictable;    // (released, block) of cached blocks nobody holds
    uint64_t clock = 0;
    std::mutex mu;

    // blocks an allocation from pool p can take
    size_t available(Pool p) const { return free_blocks[p].size() + (p == GPU ? evictable.size() : 0); }

    int32_t take(Pool p) {
        int32_t b;
        if (!free_blocks[p].empty()) {
            b = *free_blocks[p].begin();
            free_blocks[p].erase(free_blocks[p].begin());
        } else {
            // the cached block released longest ago leaves the cache
            b = evictable.begin()->second;
            evictable.erase(evictable.begin());
            by_hash.erase(entries[b].hash);
            entries.erase(b);
        }
        ref[p][b] = 1;
        return b;
    }
    void drop(Pool p, int32_t b) {
        if (--ref[p][b] != 0)
            return;
        auto it = p == GPU ? entries.find(b) : entries.end();
        if (it != entries.end()) {
            it->second.released = ++clock;
            evictable.insert({it->second.released, b});
        } else {
            free_blocks[p].insert(b);
        }
    }
    // a cache hit: the block is held again
    void hold(int32_t b) {
        if (ref[GPU][b] == 0)
            evictable.erase({entries[b].released, b});
        ++ref[GPU][b];
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
    // offer the request's newly full blocks to the cache
    void register_blocks(Request &r) {
        if (!r.known)
            return;
        const size_t full = r.tokens.size() / (size_t)bs;
        for (size_t j = r.chain.size(); j < full; ++j)
            r.chain.push_back(block_hash(j == 0 ? CHAIN_SEED : r.chain[j - 1], r.tokens.data() + j * bs, bs));
        for (size_t j = r.registered; j < full; ++j) {
            const uint64_t parent = j == 0 ? CHAIN_SEED : r.chain[j - 1];
            const uint64_t h = r.chain[j];
            const int32_t b = r.table[j];
            if (by_hash.count(h) || entries.count(b))
                continue;
            CacheEntry e;
            e.hash = h;
            e.parent = parent;
            e.toks.assign(r.tokens.begin() + j * bs, r.tokens.begin() + (j + 1) * bs);
            entries.emplace(b, std::move(e));
            by_hash.emplace(h, b);
        }
        if (full > r.registered)
            r.registered = full;
    }
};

namespace {

// grow r by n tokens (checks done by the caller, lock held)
void grow(pa_block_manager *bm, Request *r, int n, int64_t *slots, int32_t *copies, int *num_copies)
{
    const int bs = bm->bs;
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
}

// the checks an append of n tokens to seq needs; on success *out is the request
pa_status check_append(pa_block_manager *bm, int64_t seq, int n, int64_t *slots, int32_t *copies, int max_copies,
                       int *num_copies, Request **out)
{
    if (!num_copies || n < 0 || max_copies < 0 || (n > 0 && !slots))
        return PA_ERR_INVALID_ARG;
    Request *r = bm->find(seq);
    if (!r || r->pool != GPU)
        return PA_ERR_INVALID_ARG;
    const bool cow = n > 0 && r->len % bm->bs != 0 && bm->ref[GPU][r->table[r->len / bm->bs]] > 1;
    if (cow && (max_copies < 1 || !copies))
        return PA_ERR_INVALID_ARG;
    if (bm->needed(*r, n) > (int64_t)bm->available(GPU))
        return PA_ERR_NO_BLOCKS;
    *out = r;
    return PA_OK;
}

}  // namespace

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
    if (!bm)
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    Request *r = nullptr;
    const pa_status st = check_append(bm, seq, n, slots, copies, max_copies, num_copies, &r);
    if (st != PA_OK)
        return st;
    grow(bm, r, n, slots, copies, num_copies);
    if (n > 0) {   // tokens not given: the request's blocks stay out of the prefix cache
        r->known = false;
        r->tokens.clear();
    }
    return PA_OK;
}

pa_status pa_bm_append_tokens(pa_block_manager *bm, int64_t seq, const int32_t *tokens, int n, int64_t *slots,
                              int32_t *copies, int max_copies, int *num_copies)
{
    if (!bm || (n > 0 && !tokens))
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    Request *r = nullptr;
    const pa_status st = check_append(bm, seq, n, slots, copies, max_copies, num_copies, &r);
    if (st != PA_OK)
        return st;
    grow(bm, r, n, slots, copies, num_copies);
    if (r->known) {
        r->tokens.insert(r->tokens.end(), tokens, tokens + n);
        bm->register_blocks(*r);
    }
    return PA_OK;
}

pa_status pa_bm_add_cached(pa_block_manager *bm, int64_t seq, const int32_t *prompt, int n, int *cached_tokens)
{
    if (!bm || !cached_tokens || n < 0 || (n > 0 && !prompt))
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    if (bm->find(seq))
        return PA_ERR_INVALID_ARG;
    Request r;
    const int bs = bm->bs;
    const int max_blocks = n > 0 ? (n - 1) / bs : 0;     // leave at least one prompt token to compute
    uint64_t prev = CHAIN_SEED;
    for (int i = 0; i < max_blocks; ++i) {
        const int32_t *t = prompt + (int64_t)i * bs;
        const uint64_t h = block_hash(prev, t, bs);
        auto it = bm->by_hash.find(h);
        if (it == bm->by_hash.end())
            break;
        const CacheEntry &e = bm->entries[it->second];
        bool same = e.parent == prev;
        for (int k = 0; same && k < bs; ++k)
            same = e.toks[k] == t[k];
        if (!same)
            break;
        bm->hold(it->second);
        r.table.push_back(it->second);
        r.chain.push_back(h);
        prev = h;
    }
    r.len = (int64_t)r.table.size() * bs;
    r.tokens.assign(prompt, prompt + r.len);
    r.registered = r.table.size();
    *cached_tokens = (int)r.len;
    bm->reqs.emplace(seq, std::move(r));
    return PA_OK;
}

pa_status pa_bm_cache_stats(pa_block_manager *bm, int *cached_blocks, int *evictable_blocks)
{
    if (!bm || !cached_blocks || !evictable_blocks)
        return PA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(bm->mu);
    *cached_blocks = (int)bm->entries.size();
    *evictable_blocks = (int)bm->evictable.size();
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
    for (auto it = r->table.rbegin(); it != r->table.rend(); ++it)   // last block first
        bm->drop(r->pool, *it);
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
    if (nb > (int64_t)bm->available(to))
        return PA_ERR_NO_BLOCKS;
    for (int64_t j = 0; j < nb; ++j) {
        pairs[2 * j] = r->table[j];
        pairs[2 * j + 1] = bm->take(to);
    }
    for (int64_t j = nb - 1; j >= 0; --j)            // the old blocks released last block first
        bm->drop(from, r->table[j]);
    for (int64_t j = 0; j < nb; ++j)
        r->table[j] = pairs[2 * j + 1];
    r->pool = to;
    if (to == GPU)   // fresh copies: their full blocks are not offered to the cache
        r->registered = r->known ? r->tokens.size() / (size_t)bm->bs : r->table.size();
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
    *out = (int)bm->available((Pool)pool);
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
