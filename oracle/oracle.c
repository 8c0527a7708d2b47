/*
 * CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg may load
 * this library. The GPU library never links, includes or calls it, and it
 * includes no header of the GPU library.
 *
 * Everything here is the plain definition, written out:
 *   - key/value cache writes are byte copies of a token's rows into the slot
 *     the block table gives it ("vLLM and PagedAttention" slides, slide 11:
 *     a new token lands in the next free slot of its sequence's last block);
 *   - block copies are whole-block memcpy (slide 13 of the same deck, on
 *     sampling several outputs from one prompt: copy-on-write duplicates a
 *     shared last block only);
 *   - attention is single-query scaled dot-product attention over the keys
 *     and values gathered through the block table ("PagedAttention: attention
 *     block by block", slide 9: where the bytes come from changes, not what is
 *     computed), evaluated in double precision.
 *
 * Cache layout read here: [num_blocks][num_kv_heads][block_size][head_dim],
 * row-major, head_dim innermost; slot = physical_block * block_size + offset
 * (the block table of the "Week 22 Day 2" lesson note, section 2, maps logical
 * block j, tokens j*B .. j*B+B-1, to one physical block).
 *
 * Element codes: 0 = fp32, 1 = fp16 (IEEE binary16), 2 = bf16 (upper half of
 * an IEEE binary32).  All loops are sequential per (sequence, head); OpenMP
 * only spreads independent (sequence, head) pairs over threads, so results do
 * not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };
enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ENOMEM = -2 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double f16_to_f64(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);            /* subnormal: m * 2^(1-15-10) */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bf16 is the upper 16 bits of a binary32 value. */
static double bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double elem(const void *base, int64_t i, int dtype)
{
    switch (dtype) {
    case ORC_F32: return (double)((const float *)base)[i];
    case ORC_F16: return f16_to_f64(((const uint16_t *)base)[i]);
    default:      return bf16_to_f64(((const uint16_t *)base)[i]);
    }
}

static int elt_size(int dtype)
{
    return dtype == ORC_F32 ? 4 : 2;
}

int oracle_decode_element(double *out, const void *src, int64_t n, int dtype)
{
    if (dtype < 0 || dtype > 2) return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i) out[i] = elem(src, i, dtype);
    return ORC_OK;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Write token i's key and value rows (num_kv_heads x head_dim elements, rows
 * token_stride elements apart in key/value) into slot slot_mapping[i].
 * A negative slot is padding and is skipped.  A slot beyond the pool is an
 * error and nothing is written.
 */
int oracle_reshape_and_cache(const void *key, const void *value, int64_t key_stride,
                             int64_t value_stride, void *k_cache, void *v_cache,
                             int64_t num_blocks, const int64_t *slot_mapping,
                             int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t elt_bytes)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || elt_bytes <= 0)
        return ORC_EINVAL;
    for (int32_t i = 0; i < num_tokens; ++i)
        if (slot_mapping[i] >= num_blocks * (int64_t)block_size) return ORC_EINVAL;
    const size_t row = (size_t)head_dim * elt_bytes;
    for (int32_t i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0) continue;
        int64_t blk = slot / block_size, off = slot % block_size;
        for (int32_t h = 0; h < num_kv_heads; ++h) {
            int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * (int64_t)row;
            memcpy((char *)k_cache + dst,
                   (const char *)key + (i * key_stride + (int64_t)h * head_dim) * elt_bytes, row);
            memcpy((char *)v_cache + dst,
                   (const char *)value + (i * value_stride + (int64_t)h * head_dim) * elt_bytes, row);
        }
    }
    return ORC_OK;
}

/* For each (src, dst) pair in order: the whole of block dst becomes a copy of block src, in K and V. */
int oracle_copy_blocks(void *k_cache, void *v_cache, int64_t num_blocks, int64_t block_bytes,
                       const int32_t *pairs, int32_t num_pairs)
{
    for (int32_t p = 0; p < num_pairs; ++p) {
        int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return ORC_EINVAL;
    }
    for (int32_t p = 0; p < num_pairs; ++p) {
        int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
        memmove((char *)k_cache + dst * block_bytes, (const char *)k_cache + src * block_bytes,
                (size_t)block_bytes);
        memmove((char *)v_cache + dst * block_bytes, (const char *)v_cache + src * block_bytes,
                (size_t)block_bytes);
    }
    return ORC_OK;
}

/*
 * Attention of one query row over n gathered key/value rows.
 * key_row(t) / val_row(t) give the element offset of token t's row.
 *   x_t = scale * sum_d q[d] k_t[d];  m = max_t x_t;  p_t = exp(x_t - m);
 *   l = sum_t p_t;  out[d] = (sum_t p_t v_t[d]) / l
 * n == 0 gives zeros.
 */
typedef int64_t (*row_fn)(const void *ctx, int64_t t);

static void attend_one(double *out, const void *q, int64_t q_off, const void *k, const void *v,
                       row_fn row, const void *rctx, int64_t t_begin, int64_t t_end, int32_t head_dim,
                       double scale, int dtype, double *x, double *m_out, double *l_out)
{
    int64_t n = t_end - t_begin;
    for (int32_t d = 0; d < head_dim; ++d) out[d] = 0.0;
    if (n <= 0) {
        if (m_out) *m_out = -INFINITY;
        if (l_out) *l_out = 0.0;
        return;
    }
    double m = -INFINITY;
    for (int64_t t = t_begin; t < t_end; ++t) {
        int64_t r = row(rctx, t);
        double dot = 0.0;
        for (int32_t d = 0; d < head_dim; ++d)
            dot += elem(q, q_off + d, dtype) * elem(k, r + d, dtype);
        x[t - t_begin] = scale * dot;
        if (x[t - t_begin] > m) m = x[t - t_begin];
    }
    double l = 0.0;
    for (int64_t t = t_begin; t < t_end; ++t) {
        double p = exp(x[t - t_begin] - m);
        int64_t r = row(rctx, t);
        l += p;
        for (int32_t d = 0; d < head_dim; ++d) out[d] += p * elem(v, r + d, dtype);
    }
    for (int32_t d = 0; d < head_dim; ++d) out[d] /= l;
    if (m_out) *m_out = m;
    if (l_out) *l_out = l;
}

struct paged_rows {
    const int32_t *table; /* this sequence's row of the block table */
    int64_t kvh, hkv, bs, d;
};

static int64_t paged_row(const void *c, int64_t t)
{
    const struct paged_rows *p = (const struct paged_rows *)c;
    int64_t pb = p->table[t / p->bs];
    return ((pb * p->hkv + p->kvh) * p->bs + t % p->bs) * p->d;
}

struct contig_rows {
    int64_t base, d; /* element offset of row 0 of (sequence, kv head) */
};

static int64_t contig_row(const void *c, int64_t t)
{
    const struct contig_rows *p = (const struct contig_rows *)c;
    return p->base + t * p->d;
}

static int check_tables(const int32_t *tables, int32_t max_blocks, const int32_t *ctx, int32_t S,
                        int32_t bs, int64_t num_blocks)
{
    for (int32_t s = 0; s < S; ++s) {
        if (ctx[s] < 0 || (int64_t)ctx[s] > (int64_t)max_blocks * bs) return ORC_EINVAL;
        int32_t nb = (ctx[s] + bs - 1) / bs;
        for (int32_t j = 0; j < nb; ++j) {
            int32_t b = tables[(int64_t)s * max_blocks + j];
            if (b < 0 || b >= num_blocks) return ORC_EINVAL;
        }
    }
    return ORC_OK;
}

/*
 * out[s][h][:] for every sequence s and query head h, in double precision.
 * Query head h reads key/value head h / (num_q_heads / num_kv_heads).
 * partition_size == 0: one softmax over the whole context.
 * partition_size  > 0: the context is cut into [p*P, min((p+1)*P, ctx)); each
 *   part gets its own m_p, l_p and normalised output o_p; the parts are merged
 *   with M = max_p m_p, w_p = l_p exp(m_p - M), out = sum_p w_p o_p / sum_p w_p.
 *   In exact arithmetic both give the same result.
 */
int oracle_paged_attention(double *out, const void *q, const void *k_cache, const void *v_cache,
                           int64_t num_blocks, const int32_t *block_tables, int32_t max_blocks,
                           const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, double scale,
                           int32_t partition_size, int32_t dtype)
{
    if (num_seqs < 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || head_dim <= 0 ||
        block_size <= 0 || partition_size < 0 || dtype < 0 || dtype > 2)
        return ORC_EINVAL;
    if (check_tables(block_tables, max_blocks, context_lens, num_seqs, block_size, num_blocks))
        return ORC_EINVAL;
    int32_t max_ctx = 0;
    for (int32_t s = 0; s < num_seqs; ++s)
        if (context_lens[s] > max_ctx) max_ctx = context_lens[s];
    const int32_t G = num_q_heads / num_kv_heads;
    int err = ORC_OK;
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * ((size_t)max_ctx + 1));
        if (!x) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for collapse(2) schedule(dynamic, 1)
        for (int32_t s = 0; s < num_seqs; ++s) {
            for (int32_t h = 0; h < num_q_heads; ++h) {
                if (!x) continue;
                struct paged_rows rc = {block_tables + (int64_t)s * max_blocks, h / G, num_kv_heads,
                                        block_size, head_dim};
                double *o = out + ((int64_t)s * num_q_heads + h) * head_dim;
                int64_t q_off = ((int64_t)s * num_q_heads + h) * head_dim;
                int64_t ctx = context_lens[s];
                if (partition_size == 0 || ctx == 0) {
                    attend_one(o, q, q_off, k_cache, v_cache, paged_row, &rc, 0, ctx, head_dim, scale,
                               dtype, x, NULL, NULL);
                    continue;
                }
                int64_t nparts = (ctx + partition_size - 1) / partition_size;
                double M = -INFINITY;
                double *ms = (double *)malloc(sizeof(double) * 2 * nparts);
                double *os = (double *)malloc(sizeof(double) * nparts * head_dim);
                if (!ms || !os) {
                    free(ms);
                    free(os);
#pragma omp atomic write
                    err = ORC_ENOMEM;
                    continue;
                }
                for (int64_t p = 0; p < nparts; ++p) {
                    int64_t t0 = p * partition_size, t1 = t0 + partition_size < ctx ? t0 + partition_size : ctx;
                    attend_one(os + p * head_dim, q, q_off, k_cache, v_cache, paged_row, &rc, t0, t1,
                               head_dim, scale, dtype, x, &ms[2 * p], &ms[2 * p + 1]);
                    if (ms[2 * p] > M) M = ms[2 * p];
                }
                double W = 0.0;
                for (int32_t d = 0; d < head_dim; ++d) o[d] = 0.0;
                for (int64_t p = 0; p < nparts; ++p) {
                    double w = ms[2 * p + 1] * exp(ms[2 * p] - M);
                    W += w;
                    for (int32_t d = 0; d < head_dim; ++d) o[d] += w * os[p * head_dim + d];
                }
                for (int32_t d = 0; d < head_dim; ++d) o[d] /= W;
                free(ms);
                free(os);
            }
        }
        free(x);
    }
    return err;
}

/*
 * Prefill (chunked) attention over the paged cache, in double precision: sequence s holds
 * context_lens[s] tokens, of which the last n_s = query_start[s+1] - query_start[s] are
 * queries (rows query_start[s] .. query_start[s+1]-1 of q and out, [T][num_q_heads][head_dim]).
 * Query i of s sits at position p = context_lens[s] - n_s + i and attends, causally, to the
 * keys at positions 0 .. p ("vLLM and PagedAttention" slide 3: the prompt is processed in
 * parallel; the cache holds every earlier token, shared prefix blocks included).
 */
int oracle_paged_prefill(double *out, const void *q, const void *k_cache, const void *v_cache, int64_t num_blocks,
                         const int32_t *block_tables, int32_t max_blocks, const int32_t *context_lens,
                         const int32_t *query_start, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, double scale, int32_t dtype)
{
    if (num_seqs < 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || head_dim <= 0 || block_size <= 0 ||
        dtype < 0 || dtype > 2)
        return ORC_EINVAL;
    if (check_tables(block_tables, max_blocks, context_lens, num_seqs, block_size, num_blocks))
        return ORC_EINVAL;
    int32_t max_ctx = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t n = query_start[s + 1] - query_start[s];
        if (n < 0 || n > context_lens[s]) return ORC_EINVAL;
        if (context_lens[s] > max_ctx) max_ctx = context_lens[s];
    }
    const int32_t G = num_q_heads / num_kv_heads;
    const int64_t T = query_start[num_seqs];
    int err = ORC_OK;
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * ((size_t)max_ctx + 1));
        if (!x) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for collapse(2) schedule(dynamic, 4)
        for (int64_t r = 0; r < T; ++r) {
            for (int32_t h = 0; h < num_q_heads; ++h) {
                if (!x) continue;
                int32_t s = 0;
                while (query_start[s + 1] <= r) ++s;
                const int64_t pos = (int64_t)context_lens[s] - (query_start[s + 1] - query_start[s]) + (r - query_start[s]);
                struct paged_rows rc = {block_tables + (int64_t)s * max_blocks, h / G, num_kv_heads, block_size,
                                        head_dim};
                const int64_t off = (r * num_q_heads + h) * head_dim;
                attend_one(out + off, q, off, k_cache, v_cache, paged_row, &rc, 0, pos + 1, head_dim, scale, dtype, x,
                           NULL, NULL);
            }
        }
        free(x);
    }
    return err;
}

/*
 * The same attention over a contiguous cache k, v: [num_seqs][num_kv_heads][lmax][head_dim];
 * token t of (s, kv head) is row t of that slab.
 */
int oracle_contiguous_attention(double *out, const void *q, const void *k, const void *v, int32_t lmax,
                                const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, double scale, int32_t dtype)
{
    if (num_seqs < 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || head_dim <= 0 || lmax < 0 ||
        dtype < 0 || dtype > 2)
        return ORC_EINVAL;
    for (int32_t s = 0; s < num_seqs; ++s)
        if (context_lens[s] < 0 || context_lens[s] > lmax) return ORC_EINVAL;
    const int32_t G = num_q_heads / num_kv_heads;
    int err = ORC_OK;
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * ((size_t)lmax + 1));
        if (!x) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for collapse(2) schedule(dynamic, 1)
        for (int32_t s = 0; s < num_seqs; ++s) {
            for (int32_t h = 0; h < num_q_heads; ++h) {
                if (!x) continue;
                struct contig_rows rc = {(((int64_t)s * num_kv_heads + h / G) * lmax) * head_dim, head_dim};
                attend_one(out + ((int64_t)s * num_q_heads + h) * head_dim, q,
                           ((int64_t)s * num_q_heads + h) * head_dim, k, v, contig_row, &rc, 0,
                           context_lens[s], head_dim, scale, dtype, x, NULL, NULL);
            }
        }
        free(x);
    }
    return err;
}

int oracle_elt_size(int dtype)
{
    return elt_size(dtype);
}
