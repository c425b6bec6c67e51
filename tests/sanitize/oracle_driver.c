/*
 * The CPU oracle (oracle/pa_oracle.c) built with AddressSanitizer and
 * UndefinedBehaviorSanitizer: random shapes in every storage type, empty and
 * one-token contexts, tables padded with -1 past their used length, pools
 * whose unused slots hold NaN bit patterns, appends with skipped slots, and
 * the argument errors the oracle reports instead of reading out of bounds.
 * Besides the sanitizers' checks: a one-token context gives V[0] exactly and
 * every output is finite.  Exit status 0 = clean.
 *
 *   oracle_driver <seed> <cases>
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_paged_decode(double *out, const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_tables, const int32_t *context_lens, int num_seqs, int num_q_heads,
                     int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                     double scale, int dtype);
int orc_reshape_and_cache(const void *k, const void *v, void *k_cache, void *v_cache, const int64_t *slot_mapping,
                          int num_tokens, int num_kv_heads, int head_dim, int block_size, int num_blocks, int dtype);
void orc_decode_array(double *dst, const void *src, int64_t n, int dtype);

static uint64_t state;
static uint32_t next_u32(void)
{
    /* xorshift64*: the driver's own draws (no arithmetic of the oracle's) */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (uint32_t)((state * 0x2545F4914F6CDD1DULL) >> 32);
}
static int rnd(int n) { return (int)(next_u32() % (uint32_t)n); }

static void fail(const char *what, int a)
{
    fprintf(stderr, "oracle_driver: %s (%d)\n", what, a);
    exit(1);
}

/* finite elements with 2^-7 <= |x| < 4 (or zero) in the storage type, as
 * raw bit patterns: sign, an exponent field in range, a random fraction */
static void fill(void *p, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t sign = next_u32() & 1u, zero = rnd(16) == 0;
        if (dtype == 0) {
            const uint32_t bits = zero ? 0u : (sign << 31) | ((uint32_t)(120 + rnd(9)) << 23) | (next_u32() & 0x7fffffu);
            memcpy((float *)p + i, &bits, 4);
        } else if (dtype == 1) {
            ((uint16_t *)p)[i] = zero ? 0 : (uint16_t)((sign << 15) | ((uint32_t)(8 + rnd(9)) << 10) | (next_u32() & 0x3ffu));
        } else {
            ((uint16_t *)p)[i] = zero ? 0 : (uint16_t)((sign << 15) | ((uint32_t)(120 + rnd(9)) << 7) | (next_u32() & 0x7fu));
        }
    }
}

int main(int argc, char **argv)
{
    state = 0x9E3779B97F4A7C15ULL ^ (uint64_t)(argc > 1 ? atoi(argv[1]) : 1);
    const int cases = argc > 2 ? atoi(argv[2]) : 200;
    const int dims[] = {32, 64, 128}, bss[] = {8, 16, 32}, eb[] = {4, 2, 2};
    for (int c = 0; c < cases; ++c) {
        const int dtype = rnd(3), D = dims[rnd(3)], bs = bss[rnd(3)];
        const int Hkv = 1 + rnd(3), G = 1 + rnd(4), Hq = Hkv * G, S = 1 + rnd(5);
        int ctx[8], MB = 1, need = 0;
        for (int s = 0; s < S; ++s) {
            ctx[s] = rnd(4) == 0 ? rnd(2) : rnd(3 * bs + 1);     /* empty and one-token contexts often */
            const int nb = (ctx[s] + bs - 1) / bs;
            MB = nb + 1 > MB ? nb + 1 : MB;
            need += nb;
        }
        const int NB = need + 2;
        const int64_t pool = (int64_t)NB * bs * Hkv * D;
        void *k = malloc((size_t)pool * eb[dtype]), *v = malloc((size_t)pool * eb[dtype]);
        void *q = malloc((size_t)S * Hq * D * eb[dtype]);
        int32_t *tables = malloc(sizeof(int32_t) * (size_t)S * MB);
        double *out = malloc(sizeof(double) * (size_t)S * Hq * D);
        if (!k || !v || !q || !tables || !out)
            fail("malloc", c);
        fill(k, pool, dtype);
        fill(v, pool, dtype);
        fill(q, (int64_t)S * Hq * D, dtype);
        /* blocks 0 .. need-1 handed out in a scrambled order; the last two stay free */
        int perm[64];
        for (int i = 0; i < need; ++i)
            perm[i] = i;
        for (int i = need - 1; i > 0; --i) {
            const int j = rnd(i + 1), t = perm[i];
            perm[i] = perm[j];
            perm[j] = t;
        }
        int used = 0;
        for (int s = 0; s < S; ++s) {
            const int nb = (ctx[s] + bs - 1) / bs;
            for (int j = 0; j < MB; ++j)
                tables[s * MB + j] = j < nb ? perm[used + j] : -1;
            used += nb;
        }
        const double scale = 1.0 / sqrt((double)D);
        if (orc_paged_decode(out, q, k, v, tables, ctx, S, Hq, Hkv, D, bs, MB, NB, scale, dtype) != 0)
            fail("decode", c);
        for (int64_t i = 0; i < (int64_t)S * Hq * D; ++i)
            if (!isfinite(out[i]))
                fail("non-finite output", c);
        for (int s = 0; s < S; ++s) {
            if (ctx[s] != 1)
                continue;
            /* one token: the output is its V row, exactly */
            double vrow[128];
            for (int h = 0; h < Hq; ++h) {
                const int64_t base = (((int64_t)tables[s * MB] * bs) * Hkv + h / G) * D;
                orc_decode_array(vrow, (const char *)v + base * eb[dtype], D, dtype);
                for (int d = 0; d < D; ++d)
                    if (out[((int64_t)s * Hq + h) * D + d] != vrow[d])
                        fail("one-token context is not V[0]", c);
            }
        }
        /* append: one row per sequence, some skipped, into the free blocks */
        int64_t slots[8];
        for (int s = 0; s < S; ++s)
            slots[s] = rnd(3) == 0 ? -1 : (int64_t)(NB - 1 - rnd(2)) * bs + rnd(bs);
        void *nk = malloc((size_t)S * Hkv * D * eb[dtype]), *nv = malloc((size_t)S * Hkv * D * eb[dtype]);
        fill(nk, (int64_t)S * Hkv * D, dtype);
        fill(nv, (int64_t)S * Hkv * D, dtype);
        if (orc_reshape_and_cache(nk, nv, k, v, slots, S, Hkv, D, bs, NB, dtype) != 0)
            fail("append", c);
        /* argument errors: reported, nothing read out of bounds */
        tables[0] = NB;
        if (ctx[0] > 0 && orc_paged_decode(out, q, k, v, tables, ctx, S, Hq, Hkv, D, bs, MB, NB, scale, dtype) != -1)
            fail("bad table entry accepted", c);
        slots[0] = (int64_t)NB * bs;
        if (orc_reshape_and_cache(nk, nv, k, v, slots, S, Hkv, D, bs, NB, dtype) != -1)
            fail("slot past the pool accepted", c);
        free(nk);
        free(nv);
        free(k);
        free(v);
        free(q);
        free(tables);
        free(out);
    }
    printf("oracle_driver: %d cases clean\n", cases);
    return 0;
}
