// Random operation sequences through the host block manager of pa_blocks.h,
// built with AddressSanitizer and UndefinedBehaviorSanitizer on the host (no
// GPU involved: the manager is host code).  Besides the sanitizers' own
// checks, every step checks the manager's bookkeeping against what the
// driver can see from outside: each live request reads back, through its
// table, exactly the token ids written at the slots it was given (copies
// and swaps applied to a shadow pool), reference counts equal the number of
// live tables holding each block, and the free count equals the unheld
// blocks.  Exit status 0 = clean.
//
//   bm_driver <seed> <steps>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "pa_blocks.h"

namespace {

constexpr int BS = 4, NG = 48, NC = 32;

[[noreturn]] void fail(const char *what, long a = 0, long b = 0)
{
    std::fprintf(stderr, "bm_driver: %s (%ld, %ld)\n", what, a, b);
    std::exit(1);
}

struct Req {
    std::vector<int32_t> tokens;   // every token id the request holds, in order
};

struct Shadow {
    std::vector<int32_t> gpu = std::vector<int32_t>(NG * BS, -1);   // token id per slot
    std::vector<int32_t> cpu = std::vector<int32_t>(NC * BS, -1);
};

}  // namespace

int main(int argc, char **argv)
{
    const unsigned seed = argc > 1 ? (unsigned)std::atoi(argv[1]) : 1u;
    const int steps = argc > 2 ? std::atoi(argv[2]) : 2000;
    std::mt19937 rng(seed);
    pa_block_manager *bm = nullptr;
    if (pa_bm_create(NG, NC, BS, &bm) != PA_OK || !bm)
        fail("create");
    std::map<int64_t, Req> live;          // requests on the GPU or the CPU
    std::map<int64_t, bool> on_gpu;
    Shadow sh;
    int64_t next_id = 1;
    int32_t next_tok = 1000;
    // a few prompts that share prefixes, for the prefix cache
    const std::vector<int32_t> system = {7, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16};

    auto apply_copies = [&](const int32_t *cp, int n) {
        for (int i = 0; i < n; ++i)
            for (int o = 0; o < BS; ++o)
                sh.gpu[cp[2 * i + 1] * BS + o] = sh.gpu[cp[2 * i] * BS + o];
    };
    auto write_slots = [&](const int64_t *slots, const int32_t *toks, int n) {
        for (int i = 0; i < n; ++i) {
            if (slots[i] < 0 || slots[i] >= (int64_t)NG * BS)
                fail("slot out of the pool", (long)slots[i]);
            sh.gpu[slots[i]] = toks[i];
        }
    };
    auto check = [&]() {
        std::vector<int> refs(NG, 0);
        for (auto &kv : live) {
            int64_t ntok = 0;
            int nblk = 0, g = 0;
            if (pa_bm_info(bm, kv.first, &ntok, &nblk, &g) != PA_OK)
                fail("info", (long)kv.first);
            if (ntok != (int64_t)kv.second.tokens.size() || nblk != (int)((ntok + BS - 1) / BS) ||
                (g != 0) != on_gpu[kv.first])
                fail("info mismatch", (long)kv.first, (long)ntok);
            if (!g)
                continue;
            std::vector<int32_t> table(NG + 1, -2);
            int32_t len = -1;
            if (pa_bm_block_tables(bm, &kv.first, 1, NG + 1, table.data(), &len) != PA_OK)
                fail("tables", (long)kv.first);
            if (len != ntok)
                fail("table length", (long)len, (long)ntok);
            for (int j = 0; j <= NG; ++j) {
                if (j < nblk) {
                    if (table[j] < 0 || table[j] >= NG)
                        fail("table entry", (long)j, (long)table[j]);
                    ++refs[table[j]];
                } else if (table[j] != -1) {
                    fail("table past the end", (long)j, (long)table[j]);
                }
            }
            for (int64_t t = 0; t < ntok; ++t)
                if (sh.gpu[table[t / BS] * BS + t % BS] != kv.second.tokens[t])
                    fail("read-back", (long)kv.first, (long)t);
        }
        int unheld = 0;
        for (int b = 0; b < NG; ++b) {
            int rc = -1;
            if (pa_bm_ref_count(bm, 0, b, &rc) != PA_OK || rc != refs[b])
                fail("ref count", (long)b, (long)rc);
            unheld += refs[b] == 0;
        }
        int nf = -1;
        if (pa_bm_num_free(bm, 0, &nf) != PA_OK || nf != unheld)
            fail("free count", (long)nf, (long)unheld);
        int cached = -1, evictable = -1;
        if (pa_bm_cache_stats(bm, &cached, &evictable) != PA_OK || evictable > cached || cached > NG)
            fail("cache stats", (long)cached, (long)evictable);
    };

    for (int step = 0; step < steps; ++step) {
        const int op = (int)(rng() % 8);
        std::vector<int64_t> gpu_ids, cpu_ids;
        for (auto &kv : on_gpu)
            (kv.second ? gpu_ids : cpu_ids).push_back(kv.first);
        auto pick = [&](std::vector<int64_t> &v) { return v[rng() % v.size()]; };
        int64_t slots[64];
        int32_t copies[8], pairs[2 * (NG + NC)];
        int ncp = 0, np = 0;
        if (op == 0 || live.empty()) {                        // a new request
            const int64_t id = next_id++;
            if (pa_bm_add(bm, id) != PA_OK)
                fail("add");
            live[id] = Req();
            on_gpu[id] = true;
        } else if (op == 1 && !gpu_ids.empty()) {             // append n tokens (ids given: cacheable)
            const int64_t id = pick(gpu_ids);
            const int n = 1 + (int)(rng() % 9);
            std::vector<int32_t> toks(n);
            for (auto &t : toks)
                t = next_tok++;
            const pa_status st = pa_bm_append_tokens(bm, id, toks.data(), n, slots, copies, 4, &ncp);
            if (st == PA_OK) {
                apply_copies(copies, ncp);
                write_slots(slots, toks.data(), n);
                live[id].tokens.insert(live[id].tokens.end(), toks.begin(), toks.end());
            } else if (st != PA_ERR_NO_BLOCKS) {
                fail("append_tokens", (long)st);
            }
        } else if (op == 2 && !gpu_ids.empty()) {             // append without ids
            const int64_t id = pick(gpu_ids);
            const int n = 1 + (int)(rng() % 6);
            const pa_status st = pa_bm_append(bm, id, n, slots, copies, 4, &ncp);
            if (st == PA_OK) {
                std::vector<int32_t> toks(n);
                for (auto &t : toks)
                    t = next_tok++;
                apply_copies(copies, ncp);
                write_slots(slots, toks.data(), n);
                live[id].tokens.insert(live[id].tokens.end(), toks.begin(), toks.end());
            } else if (st != PA_ERR_NO_BLOCKS) {
                fail("append", (long)st);
            }
        } else if (op == 3 && !gpu_ids.empty()) {             // fork
            const int64_t parent = pick(gpu_ids), child = next_id++;
            if (pa_bm_fork(bm, parent, child) != PA_OK)
                fail("fork");
            live[child] = live[parent];
            on_gpu[child] = true;
        } else if (op == 4) {                                 // free any request
            std::vector<int64_t> all(gpu_ids);
            all.insert(all.end(), cpu_ids.begin(), cpu_ids.end());
            if (!all.empty()) {
                const int64_t id = pick(all);
                if (pa_bm_free(bm, id) != PA_OK)
                    fail("free");
                live.erase(id);
                on_gpu.erase(id);
            }
        } else if (op == 5 && !gpu_ids.empty()) {             // swap out
            const int64_t id = pick(gpu_ids);
            const pa_status st = pa_bm_swap_out(bm, id, pairs, NG + NC, &np);
            if (st == PA_OK) {
                for (int i = 0; i < np; ++i)
                    for (int o = 0; o < BS; ++o)
                        sh.cpu[pairs[2 * i + 1] * BS + o] = sh.gpu[pairs[2 * i] * BS + o];
                on_gpu[id] = false;
            } else if (st != PA_ERR_NO_BLOCKS) {
                fail("swap_out", (long)st);
            }
        } else if (op == 6 && !cpu_ids.empty()) {             // swap in
            const int64_t id = pick(cpu_ids);
            const pa_status st = pa_bm_swap_in(bm, id, pairs, NG + NC, &np);
            if (st == PA_OK) {
                for (int i = 0; i < np; ++i)
                    for (int o = 0; o < BS; ++o)
                        sh.gpu[pairs[2 * i + 1] * BS + o] = sh.cpu[pairs[2 * i] * BS + o];
                on_gpu[id] = true;
            } else if (st != PA_ERR_NO_BLOCKS) {
                fail("swap_in", (long)st);
            }
        } else if (op == 7) {                                 // a prompt that may hit the prefix cache
            const int64_t id = next_id++;
            std::vector<int32_t> prompt(system.begin(), system.begin() + 1 + (int)(rng() % system.size()));
            const int extra = (int)(rng() % 5);
            for (int i = 0; i < extra; ++i)
                prompt.push_back(2000 + (int32_t)(rng() % 3));
            int hit = -1;
            if (pa_bm_add_cached(bm, id, prompt.data(), (int)prompt.size(), &hit) != PA_OK)
                fail("add_cached");
            if (hit < 0 || hit % BS != 0 || hit >= (int)prompt.size())
                fail("cached tokens", (long)hit, (long)prompt.size());
            live[id].tokens.assign(prompt.begin(), prompt.begin() + hit);
            on_gpu[id] = true;
            const int rest = (int)prompt.size() - hit;
            const pa_status st = pa_bm_append_tokens(bm, id, prompt.data() + hit, rest, slots, copies, 4, &ncp);
            if (st == PA_OK) {
                apply_copies(copies, ncp);
                write_slots(slots, prompt.data() + hit, rest);
                live[id].tokens.insert(live[id].tokens.end(), prompt.begin() + hit, prompt.end());
            } else if (st != PA_ERR_NO_BLOCKS) {
                fail("prompt append", (long)st);
            }
        }
        check();
    }
    // argument errors change nothing
    int out = 0;
    if (pa_bm_add(nullptr, 1) != PA_ERR_INVALID_ARG || pa_bm_num_free(bm, 2, &out) != PA_ERR_INVALID_ARG ||
        pa_bm_append(bm, -12345, 1, nullptr, nullptr, 0, nullptr) != PA_ERR_INVALID_ARG)
        fail("argument errors");
    check();
    pa_bm_destroy(bm);
    std::printf("bm_driver: %d steps clean (seed %u)\n", steps, seed);
    return 0;
}
