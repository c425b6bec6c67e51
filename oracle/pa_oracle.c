/*
 * pa_oracle.c -- plain, slow CPU reference for paged decode attention and for
 * the KV append ("reshape_and_cache").  TEST INFRASTRUCTURE ONLY: it is used by
 * the tests, by the smoke check and by the CPU-baseline leg of the benchmark.
 * The GPU library never links, loads or calls it, and it shares no code,
 * header or table with the GPU library.
 *
 * Sources (web pages on vLLM / PagedAttention):
 *   [VP]  "vLLM 与 PagedAttention" (inference.mavenzero.com/case-studies/vllm),
 *         section 二 "PagedAttention": sub-section "PagedAttention 的解法"
 *         (KV cache cut into blocks of usually 16 tokens; a per-request block
 *         table maps logical block i to a physical block in one shared pool;
 *         worked table [1,3,7,9]) and sub-section "注意力计算改造" (K/V are read
 *         block by block; kernel sketch whose argument list fixes the cache
 *         layout [num_blocks, block_size, num_heads, d_head], a per-request
 *         block table and a context length).
 *   [VG]  "指南" (illegalscreed.cn .../vllm/guide-line), section "为什么 vLLM 快：
 *         PagedAttention": KV cache holds each layer's and head's K and V for
 *         all earlier tokens; blocks are allocated on demand anywhere in a
 *         shared pool.
 *   [VB]  "vLLM让大模型推理快10倍？..." (298.name/post/186.html), section
 *         "PagedAttention怎么解决？": a request of n tokens needs ceil(n/16) pages.
 *
 * What is computed.  Paging changes where K and V live, not the attention
 * result.  For each sequence s and query head h the oracle gathers the K/V
 * rows of tokens 0..ctx_s-1 through the block table (token t lives in physical
 * block table[s][t / block_size] at offset t % block_size) and evaluates the
 * textbook definition softmax(scale * q K^T) V in double precision, in two
 * plain passes (max, then exponentials and sums).  No blocking, no online
 * rescaling, no split: those belong to the GPU path, not to the definition.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *   - batching: block_tables is [num_seqs, max_blocks_per_seq] int32 row-major,
 *     context_lens is [num_seqs] int32; q and out are [num_seqs, num_q_heads,
 *     head_dim] (the sketch's output shape is garbled; out takes q's shape);
 *   - context_lens counts every cached token, the one appended this step
 *     included; ctx = 0 gives an all-zero output row;
 *   - grouped-query heads: q head h reads kv head h / (num_q_heads/num_kv_heads);
 *   - slot of the append: slot = physical_block * block_size + offset, int64,
 *     negative slots are skipped;
 *   - element types f32 / f16 / bf16 are decoded exactly to double by the
 *     decoders below, written from the IEEE 754 binary16 definition and from
 *     bfloat16's definition as the upper half of a binary32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* ---- element decoders (exact) -------------------------------------------- */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* subnormal: m * 2^-14 / 2^10 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);   /* (1 + m/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double orc_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int m = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);              /* m * 2^-126 / 2^7 */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134);   /* (1 + m/2^7) * 2^(e-127) */
    return sign ? -v : v;
}

static double orc_load(const void *base, int64_t idx, int dtype)
{
    if (dtype == ORC_F32) {
        float f;
        memcpy(&f, (const char *)base + idx * 4, 4);
        return (double)f;                         /* exact widening */
    }
    uint16_t u;
    memcpy(&u, (const char *)base + idx * 2, 2);
    return dtype == ORC_F16 ? orc_f16_to_f64(u) : orc_bf16_to_f64(u);
}

int orc_elem_bytes(int dtype)
{
    return dtype == ORC_F32 ? 4 : (dtype == ORC_F16 || dtype == ORC_BF16) ? 2 : 0;
}

/* ---- rounding of a double to a storage format (round to nearest even) ---- */

/* Format with p significand bits (implicit bit included), smallest normal
 * exponent emin and largest exponent emax.  Below 2^emin the quantum stays
 * 2^(emin-p+1) (gradual underflow).  x / quantum is exact (power-of-two
 * scaling), nearbyint rounds half to even in the default rounding mode. */
static double orc_round_format(double x, int p, int emin, int emax)
{
    if (x == 0.0 || isnan(x) || isinf(x))
        return x;
    int e2;
    frexp(x, &e2);                  /* x = f * 2^e2, 0.5 <= |f| < 1 */
    int lead = e2 - 1;              /* exponent of the leading bit */
    if (lead < emin)
        lead = emin;
    double quantum = ldexp(1.0, lead - (p - 1));
    double r = nearbyint(x / quantum) * quantum;
    double max_finite = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (fabs(r) > max_finite)
        return x > 0 ? INFINITY : -INFINITY;
    return r;
}

double orc_round_to_dtype(double x, int dtype)
{
    switch (dtype) {
    case ORC_F32:  return orc_round_format(x, 24, -126, 127);
    case ORC_F16:  return orc_round_format(x, 11, -14, 15);
    case ORC_BF16: return orc_round_format(x, 8, -126, 127);
    default:       return NAN;
    }
}

void orc_round_array(double *x, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i)
        x[i] = orc_round_to_dtype(x[i], dtype);
}

/* Decode n stored elements to double (used by tests to read GPU output). */
void orc_decode_array(double *dst, const void *src, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = orc_load(src, i, dtype);
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- paged decode attention (fp64) --------------------------------------- */

/*
 * Layout of k_cache and v_cache: [num_blocks, block_size, num_kv_heads,
 * head_dim], the layout of the kernel sketch in [VP] "注意力计算改造".
 * Returns 0, or -1 for arguments that make the definition meaningless
 * (the caller's bug, reported instead of read out of bounds).
 */
int orc_paged_decode(double *out, const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_tables, const int32_t *context_lens,
                     int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                     int block_size, int max_blocks_per_seq, int num_blocks,
                     double scale, int dtype)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
        num_q_heads % num_kv_heads != 0 || orc_elem_bytes(dtype) == 0)
        return -1;
    for (int s = 0; s < num_seqs; ++s) {
        int L = context_lens[s];
        if (L < 0 || L > max_blocks_per_seq * block_size)
            return -1;
        int used = (L + block_size - 1) / block_size;      /* [VB]: ceil(n / 16) */
        for (int j = 0; j < used; ++j) {
            int b = block_tables[(int64_t)s * max_blocks_per_seq + j];
            if (b < 0 || b >= num_blocks)
                return -1;
        }
    }

    const int G = num_q_heads / num_kv_heads;
    const int D = head_dim;
    int bad = 0;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int s = 0; s < num_seqs; ++s) {
        for (int h = 0; h < num_q_heads; ++h) {
            const int L = context_lens[s];
            double *o = out + ((int64_t)s * num_q_heads + h) * D;
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            if (L == 0)
                continue;
            const int g = h / G;
            const int64_t qbase = ((int64_t)s * num_q_heads + h) * D;
            double *score = (double *)malloc(sizeof(double) * (size_t)L);
            if (!score) {
#pragma omp atomic write
                bad = 1;
                continue;
            }

            /* pass 1: scores through the block table */
            for (int t = 0; t < L; ++t) {
                int64_t b = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
                int off = t % block_size;
                int64_t kbase = ((b * block_size + off) * num_kv_heads + g) * D;
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += orc_load(q, qbase + d, dtype) * orc_load(k_cache, kbase + d, dtype);
                score[t] = scale * dot;
            }

            /* pass 2: softmax weights and the weighted sum of V rows */
            double m = score[0];
            for (int t = 1; t < L; ++t)
                if (score[t] > m)
                    m = score[t];
            double Z = 0.0;
            for (int t = 0; t < L; ++t) {
                double w = exp(score[t] - m);
                Z += w;
                int64_t b = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
                int off = t % block_size;
                int64_t vbase = ((b * block_size + off) * num_kv_heads + g) * D;
                for (int d = 0; d < D; ++d)
                    o[d] += w * orc_load(v_cache, vbase + d, dtype);
            }
            for (int d = 0; d < D; ++d)
                o[d] /= Z;
            free(score);
        }
    }
    return bad ? -1 : 0;
}

/* ---- append of new K/V rows into their slots ------------------------------ */

/*
 * k, v: [num_tokens, num_kv_heads, head_dim] in the storage type.  Token i goes
 * to physical block slot / block_size at offset slot % block_size of the same
 * [num_blocks, block_size, num_kv_heads, head_dim] caches; bytes are copied
 * unchanged.  A negative slot skips the token; a slot past the pool is an
 * error (nothing is written for any token then).
 */
int orc_reshape_and_cache(const void *k, const void *v, void *k_cache, void *v_cache,
                          const int64_t *slot_mapping, int num_tokens, int num_kv_heads,
                          int head_dim, int block_size, int num_blocks, int dtype)
{
    const int eb = orc_elem_bytes(dtype);
    if (eb == 0 || num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || num_blocks <= 0)
        return -1;
    for (int i = 0; i < num_tokens; ++i)
        if (slot_mapping[i] >= (int64_t)num_blocks * block_size)
            return -1;
    const size_t row = (size_t)head_dim * eb;
    for (int i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        int64_t b = slot / block_size;
        int64_t off = slot % block_size;
        for (int g = 0; g < num_kv_heads; ++g) {
            int64_t dst = ((b * block_size + off) * num_kv_heads + g) * (int64_t)row;
            int64_t src = ((int64_t)i * num_kv_heads + g) * (int64_t)row;
            memcpy((char *)k_cache + dst, (const char *)k + src, row);
            memcpy((char *)v_cache + dst, (const char *)v + src, row);
        }
    }
    return 0;
}
