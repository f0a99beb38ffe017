/*
 * pkv_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU reference for paged KV-cache decode
 * attention, written in C with every arithmetic step in double precision.
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load it. It shares no code, header or table with the GPU
 * library: it has its own dtype codes, its own element decoders and its own
 * reading of the cache layout.
 *
 * Sources (the three web pages on paged KV caches):
 *  - "Basics of LLM Inference and vLLM Internals" (ttlab), section 2 "KV Cache
 *    and Sizing Formulas": bytes per token = 2 * L * H_kv * d * b; MQA/GQA
 *    share one K/V head between a group of query heads; an fp8 KV cache has
 *    b = 1.
 *  - same page, section 4 "PagedAttention and Block Management": KV is cut
 *    into fixed 16-token blocks; a per-request block table maps logical block
 *    i to a physical block anywhere in the pool; only the last block is
 *    partly filled; requests with a common prefix may share physical blocks.
 *  - "The Memory Trick Behind Fast LLM Serving" (tarundecipher), sections
 *    "PagedAttention changes the shape of the problem" and "Batching does not
 *    merge the conversations": a flattened batch whose metadata keeps every
 *    sequence's context private.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - query head h uses KV head h / G, G = H_q / H_kv (contiguous groups);
 *  - a slot is phys_block * 16 + (position % 16);
 *  - context_lens[s] counts every token the query attends to, itself included;
 *  - context_lens[s] <= 0 gives an all-zero output row;
 *  - a negative slot in an append is skipped;
 *  - softmax uses the natural exponential of scale * (q . k), max-subtracted;
 *  - fp8 is OCP E4M3FN (bias 7, no infinities, 0x7F/0xFF are NaN, max 448)
 *    with one float scale per tensor: the stored value is code * scale.
 *
 * Layout of one cache tensor (K or V): [num_blocks][H_kv][16][d], so element
 * (blk, g, off, j) sits at ((blk * H_kv + g) * 16 + off) * d + j.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define OR_F32 0
#define OR_F16 1
#define OR_BF16 2
#define OR_FP8 3
#define OR_BLOCK 16

#define OR_OK 0
#define OR_BAD -1

static int elem_size(int dt)
{
    switch (dt) {
    case OR_F32: return 4;
    case OR_F16: return 2;
    case OR_BF16: return 2;
    case OR_FP8: return 1;
    default: return 0;
    }
}

/* Threads the OpenMP loops below will use. */
int oracle_num_threads(void)
{
    return omp_get_max_threads();
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits. */
double oracle_f16_to_double(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = (m == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (m * 2^-9); there is no infinity and only the
 * pattern S.1111.111 is NaN. */
double oracle_fp8_e4m3_to_double(uint8_t c)
{
    int s = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Quantise x with per-tensor scale c to E4M3FN: RNE(clamp(x / c, -448, 448)).
 * Written as a search over the 127 non-negative finite codes so that it
 * depends on nothing but the decoder above: the nearest code wins and an exact
 * tie goes to the code with an even mantissa. NaN maps to 0x7F. */
uint8_t oracle_fp8_e4m3_encode(double x, double c)
{
    double y = x / c;
    if (isnan(y))
        return 0x7F;
    int neg = signbit(y) ? 1 : 0;
    double a = fabs(y);
    if (a > 448.0)
        a = 448.0;
    int best = 0;
    double best_err = INFINITY;
    for (int code = 0; code < 0x7F; ++code) {
        double err = fabs(oracle_fp8_e4m3_to_double((uint8_t)code) - a);
        if (err < best_err || (err == best_err && (code & 1) == 0 && (best & 1) == 1)) {
            best = code;
            best_err = err;
        }
    }
    return (uint8_t)(best | (neg << 7));
}

/* The same rounding applied to a quotient taken in float32: y = x / c as one
 * IEEE single-precision division (round to nearest even), then the nearest
 * code of y as above. The pages give fp8 storage with a per-tensor scale
 * but no precision for the division; a code is an integer decided by
 * floating point, so both the checked side and this one must take it in one
 * stated precision, and float32 is the narrowest IEEE type that holds every
 * incoming element (16-bit or float32 rows) and the scale exactly. Only a
 * quotient within rounding of a midpoint between two codes can differ from
 * the exact one; with c a power of two the quotient is exact and this
 * equals oracle_fp8_e4m3_encode(x, c). */
uint8_t oracle_fp8_e4m3_encode_f32(float x, float c)
{
    volatile float y = x / c;
    return oracle_fp8_e4m3_encode((double)y, 1.0);
}

/* Element idx of an array of dtype dt, converted exactly to double. */
static double load_elem(const void *base, size_t idx, int dt)
{
    switch (dt) {
    case OR_F32: {
        float f;
        memcpy(&f, (const char *)base + 4 * idx, 4);
        return (double)f;
    }
    case OR_F16: {
        uint16_t h;
        memcpy(&h, (const char *)base + 2 * idx, 2);
        return oracle_f16_to_double(h);
    }
    case OR_BF16: {
        uint16_t b;
        memcpy(&b, (const char *)base + 2 * idx, 2);
        return oracle_bf16_to_double(b);
    }
    case OR_FP8:
        return oracle_fp8_e4m3_to_double(((const uint8_t *)base)[idx]);
    default:
        return NAN;
    }
}

/* Sizing (ttlab page, section 2): 2 (K and V) * L * H_kv * d * b bytes. */
uint64_t oracle_kv_bytes_per_token(int64_t num_layers, int64_t num_kv_heads, int64_t head_dim,
                                   int64_t elem_bytes)
{
    return (uint64_t)(2 * num_layers * num_kv_heads * head_dim * elem_bytes);
}

/* Index of element (blk, g, off, j) in one cache tensor. */
static size_t cache_index(int64_t blk, int64_t g, int64_t off, int64_t j, int64_t num_kv_heads,
                          int64_t head_dim)
{
    return (size_t)(((blk * num_kv_heads + g) * OR_BLOCK + off) * head_dim + j);
}

/* Append: for every new token i whose slot is non-negative, copy its K and V
 * rows (one per KV head) byte for byte into row slot % 16 of physical block
 * slot / 16. k and v are [T][H_kv][d] in the cache dtype. */
int oracle_kv_append(const void *k, const void *v, int dtype, const int64_t *slot_mapping,
                     int64_t num_tokens, void *k_cache, void *v_cache, int64_t num_blocks,
                     int64_t num_kv_heads, int64_t head_dim)
{
    int b = elem_size(dtype);
    if (b == 0)
        return OR_BAD;
    for (int64_t i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        if (slot >= num_blocks * OR_BLOCK)
            return OR_BAD;
        int64_t blk = slot / OR_BLOCK;
        int64_t off = slot % OR_BLOCK;
        for (int64_t g = 0; g < num_kv_heads; ++g) {
            size_t dst = cache_index(blk, g, off, 0, num_kv_heads, head_dim) * b;
            size_t src = (size_t)((i * num_kv_heads + g) * head_dim) * b;
            memcpy((char *)k_cache + dst, (const char *)k + src, (size_t)(head_dim * b));
            memcpy((char *)v_cache + dst, (const char *)v + src, (size_t)(head_dim * b));
        }
    }
    return OR_OK;
}

/* Gather: the logical K/V rows of every sequence, in token order, as raw
 * bytes: k_out and v_out are [S][H_kv][max_ctx][d]. Position t of sequence s
 * lives in physical block block_tables[s][t / 16], row t % 16. Rows at or past
 * the sequence's context length are left untouched. */
/* Quantising append into an fp8 cache (ttlab page, section 2: fp8 halves the
 * bytes per element; section 4: rows are written slot by slot). Each new
 * token's rows, in float32, float16 or bfloat16 (src_dtype), go to block
 * slot / 16, row slot % 16 like oracle_kv_append, every element x becoming
 * oracle_fp8_e4m3_encode_f32(x, k_scale) in K and (x, v_scale) in V. A negative
 * slot skips the token. Returns OR_BAD for a slot past the pool. */
int oracle_kv_append_fp8(const void *k, const void *v, int src_dtype,
                         const int64_t *slot_mapping, int64_t num_tokens, uint8_t *k_cache,
                         uint8_t *v_cache, int64_t num_blocks, int64_t num_kv_heads,
                         int64_t head_dim, float k_scale, float v_scale)
{
    if (src_dtype != OR_F32 && src_dtype != OR_F16 && src_dtype != OR_BF16)
        return OR_BAD;
    for (int64_t i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        if (slot >= num_blocks * OR_BLOCK)
            return OR_BAD;
        int64_t blk = slot / OR_BLOCK;
        int64_t off = slot % OR_BLOCK;
        for (int64_t g = 0; g < num_kv_heads; ++g) {
            size_t dst = cache_index(blk, g, off, 0, num_kv_heads, head_dim);
            size_t src = (size_t)((i * num_kv_heads + g) * head_dim);
            for (int64_t j = 0; j < head_dim; ++j) {
                /* every float16 / bfloat16 value is exactly a float32 value */
                float kx = (float)load_elem(k, src + j, src_dtype);
                float vx = (float)load_elem(v, src + j, src_dtype);
                k_cache[dst + j] = oracle_fp8_e4m3_encode_f32(kx, k_scale);
                v_cache[dst + j] = oracle_fp8_e4m3_encode_f32(vx, v_scale);
            }
        }
    }
    return OR_OK;
}

int oracle_gather(const void *k_cache, const void *v_cache, int dtype, int64_t num_blocks,
                  int64_t num_kv_heads, int64_t head_dim, const int32_t *block_tables,
                  int64_t max_blocks_per_seq, const int32_t *context_lens, int64_t num_seqs,
                  int64_t max_ctx, void *k_out, void *v_out)
{
    int b = elem_size(dtype);
    if (b == 0)
        return OR_BAD;
    for (int64_t s = 0; s < num_seqs; ++s) {
        int64_t n = context_lens[s];
        if (n > max_ctx)
            n = max_ctx;
        for (int64_t t = 0; t < n; ++t) {
            int64_t phys = block_tables[s * max_blocks_per_seq + t / OR_BLOCK];
            if (phys < 0 || phys >= num_blocks)
                return OR_BAD;
            for (int64_t g = 0; g < num_kv_heads; ++g) {
                size_t src = cache_index(phys, g, t % OR_BLOCK, 0, num_kv_heads, head_dim) * b;
                size_t dst = (size_t)(((s * num_kv_heads + g) * max_ctx + t) * head_dim) * b;
                memcpy((char *)k_out + dst, (const char *)k_cache + src, (size_t)(head_dim * b));
                memcpy((char *)v_out + dst, (const char *)v_cache + src, (size_t)(head_dim * b));
            }
        }
    }
    return OR_OK;
}

/* Attention of one query head over the token range [t0, t1) of sequence s:
 * returns the max score m, the sum of exp(score - m) in *l, and the
 * unnormalised weighted sum of V rows in acc[0..d). Scores are
 * scale * sum_j q[j] * K[t][j]; fp8 elements are code * tensor scale. */
static void attend_range(const void *q, int q_dtype, int64_t q_row, const void *k_cache,
                         const void *v_cache, int kv_dtype, double k_scale, double v_scale,
                         int64_t num_kv_heads, int64_t head_dim, int64_t g,
                         const int32_t *bt_row, int64_t t0, int64_t t1, double scale,
                         double *m_out, double *l_out, double *acc)
{
    double m = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) {
        int64_t phys = bt_row[t / OR_BLOCK];
        double dot = 0.0;
        for (int64_t j = 0; j < head_dim; ++j) {
            double qj = load_elem(q, (size_t)(q_row * head_dim + j), q_dtype);
            double kj = load_elem(k_cache, cache_index(phys, g, t % OR_BLOCK, j, num_kv_heads,
                                                       head_dim), kv_dtype) * k_scale;
            dot += qj * kj;
        }
        double x = scale * dot;
        if (x > m)
            m = x;
    }
    double l = 0.0;
    for (int64_t j = 0; j < head_dim; ++j)
        acc[j] = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
        int64_t phys = bt_row[t / OR_BLOCK];
        double dot = 0.0;
        for (int64_t j = 0; j < head_dim; ++j) {
            double qj = load_elem(q, (size_t)(q_row * head_dim + j), q_dtype);
            double kj = load_elem(k_cache, cache_index(phys, g, t % OR_BLOCK, j, num_kv_heads,
                                                       head_dim), kv_dtype) * k_scale;
            dot += qj * kj;
        }
        double w = exp(scale * dot - m);
        l += w;
        for (int64_t j = 0; j < head_dim; ++j) {
            double vj = load_elem(v_cache, cache_index(phys, g, t % OR_BLOCK, j, num_kv_heads,
                                                       head_dim), kv_dtype) * v_scale;
            acc[j] += w * vj;
        }
    }
    *m_out = m;
    *l_out = l;
}

static int check_decode_args(int64_t num_seqs, int64_t num_q_heads, int64_t num_kv_heads,
                             int64_t head_dim, int64_t num_blocks, const int32_t *block_tables,
                             int64_t max_blocks_per_seq, const int32_t *context_lens)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || head_dim > 1024)
        return OR_BAD;
    if (num_q_heads % num_kv_heads != 0)
        return OR_BAD;
    for (int64_t s = 0; s < num_seqs; ++s) {
        int64_t n = context_lens[s];
        if (n > max_blocks_per_seq * OR_BLOCK)
            return OR_BAD;
        for (int64_t i = 0; i * OR_BLOCK < n; ++i) {
            int32_t phys = block_tables[s * max_blocks_per_seq + i];
            if (phys < 0 || phys >= num_blocks)
                return OR_BAD;
        }
    }
    return OR_OK;
}

/* Paged decode attention, the plain definition: for each sequence s with
 * n = context_lens[s] > 0 and each query head h (KV head g = h / G),
 *   x_t = scale * q[s][h] . K_t   for t < n, K_t read through the block table,
 *   out[s][h] = sum_t exp(x_t - max x) V_t / sum_t exp(x_t - max x).
 * A sequence with n <= 0 gets a zero row. q is [S][H_q][d] in q_dtype and out
 * is [S][H_q][d] in double. Threads split the (s, h) pairs; each pair is one
 * independent sequential loop. */
int oracle_paged_decode(const void *q, int q_dtype, int64_t num_seqs, int64_t num_q_heads,
                        const void *k_cache, const void *v_cache, int kv_dtype, double k_scale,
                        double v_scale, int64_t num_blocks, int64_t num_kv_heads,
                        int64_t head_dim, const int32_t *block_tables, int64_t max_blocks_per_seq,
                        const int32_t *context_lens, double scale, double *out)
{
    if (elem_size(q_dtype) == 0 || elem_size(kv_dtype) == 0)
        return OR_BAD;
    if (check_decode_args(num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_tables,
                          max_blocks_per_seq, context_lens) != OR_OK)
        return OR_BAD;
    int64_t group = num_q_heads / num_kv_heads;
    int64_t pairs = num_seqs * num_q_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
        int64_t s = p / num_q_heads;
        int64_t h = p % num_q_heads;
        int64_t g = h / group;
        int64_t n = context_lens[s];
        double *o = out + p * head_dim;
        if (n <= 0) {
            for (int64_t j = 0; j < head_dim; ++j)
                o[j] = 0.0;
            continue;
        }
        double m, l;
        attend_range(q, q_dtype, p, k_cache, v_cache, kv_dtype, k_scale, v_scale, num_kv_heads,
                     head_dim, g, block_tables + s * max_blocks_per_seq, 0, n, scale, &m, &l, o);
        for (int64_t j = 0; j < head_dim; ++j)
            o[j] /= l;
    }
    return OR_OK;
}

/* Paged chunked-prefill attention, the plain definition. A prompt is fed in
 * chunks within a per-step token budget (ttlab section 6, chunked prefill);
 * the tokens of a chunk attend causally to every earlier token of their
 * sequence and to each other, all read from the paged cache. Sequence s has
 * q_len = query_start[s + 1] - query_start[s] query tokens, the last q_len of
 * its n = context_lens[s] tokens (their K/V already appended). Query token i
 * of s sits at position p = n - q_len + i; for query head h (KV head
 * g = h / G):
 *   out[query_start[s] + i][h] = softmax over t in [0, p] of scale * q . K_t,
 *                                applied to V_t.
 * q and out are [query_start[S]][H_q][d] (out in double). Invalid
 * arguments (q_len < 0 or > n, query_start[0] != 0, out-of-range block ids)
 * return OR_BAD. Threads split the (query row, head) pairs. */
int oracle_paged_prefill(const void *q, int q_dtype, int64_t num_seqs, int64_t num_q_heads,
                         const int32_t *query_start, const void *k_cache, const void *v_cache,
                         int kv_dtype, double k_scale, double v_scale, int64_t num_blocks,
                         int64_t num_kv_heads, int64_t head_dim, const int32_t *block_tables,
                         int64_t max_blocks_per_seq, const int32_t *context_lens, double scale,
                         double *out)
{
    if (elem_size(q_dtype) == 0 || elem_size(kv_dtype) == 0)
        return OR_BAD;
    if (check_decode_args(num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_tables,
                          max_blocks_per_seq, context_lens) != OR_OK)
        return OR_BAD;
    if (num_seqs > 0 && query_start[0] != 0)
        return OR_BAD;
    for (int64_t s = 0; s < num_seqs; ++s) {
        int64_t q_len = (int64_t)query_start[s + 1] - query_start[s];
        if (q_len < 0 || q_len > context_lens[s])
            return OR_BAD;
    }
    int64_t group = num_q_heads / num_kv_heads;
    int64_t total = num_seqs > 0 ? query_start[num_seqs] : 0;
    int64_t pairs = total * num_q_heads;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t pr = 0; pr < pairs; ++pr) {
        int64_t row = pr / num_q_heads; /* query token row of q */
        int64_t h = pr % num_q_heads;
        int64_t s = 0;
        while (query_start[s + 1] <= row)
            ++s;
        int64_t q_len = (int64_t)query_start[s + 1] - query_start[s];
        int64_t pos = context_lens[s] - q_len + (row - query_start[s]);
        double *o = out + pr * head_dim;
        double m, l;
        attend_range(q, q_dtype, pr, k_cache, v_cache, kv_dtype, k_scale, v_scale, num_kv_heads,
                     head_dim, h / group, block_tables + s * max_blocks_per_seq, 0, pos + 1,
                     scale, &m, &l, o);
        for (int64_t j = 0; j < head_dim; ++j)
            o[j] /= l;
    }
    return OR_OK;
}

/* Split-KV form of the same result, used to check the cross-partition
 * log-sum-exp algebra. Partition j covers positions [j*P, min((j+1)*P, n)).
 * For every non-empty partition it records m_j (max score), l_j (sum of
 * exp(x - m_j)) and o_j (the partition's own normalised output) into
 * part_m/part_l [S][H_q][Pn] and part_o [S][H_q][Pn][d]; empty partitions get
 * m = -inf, l = 0, o = 0. It then merges them:
 *   M = max_j m_j, w_j = l_j * exp(m_j - M), out = sum_j w_j o_j / sum_j w_j.
 * Pn = ceil(max_blocks_per_seq * 16 / P). */
int oracle_paged_decode_split(const void *q, int q_dtype, int64_t num_seqs, int64_t num_q_heads,
                              const void *k_cache, const void *v_cache, int kv_dtype,
                              double k_scale, double v_scale, int64_t num_blocks,
                              int64_t num_kv_heads, int64_t head_dim, const int32_t *block_tables,
                              int64_t max_blocks_per_seq, const int32_t *context_lens,
                              double scale, int64_t partition_size, double *part_m,
                              double *part_l, double *part_o, double *out)
{
    if (elem_size(q_dtype) == 0 || elem_size(kv_dtype) == 0)
        return OR_BAD;
    if (partition_size <= 0 || partition_size % OR_BLOCK != 0)
        return OR_BAD;
    if (check_decode_args(num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_tables,
                          max_blocks_per_seq, context_lens) != OR_OK)
        return OR_BAD;
    int64_t group = num_q_heads / num_kv_heads;
    int64_t pn = (max_blocks_per_seq * OR_BLOCK + partition_size - 1) / partition_size;
    int64_t pairs = num_seqs * num_q_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
        int64_t s = p / num_q_heads;
        int64_t h = p % num_q_heads;
        int64_t g = h / group;
        int64_t n = context_lens[s];
        const int32_t *bt_row = block_tables + s * max_blocks_per_seq;
        for (int64_t j = 0; j < pn; ++j) {
            int64_t t0 = j * partition_size;
            int64_t t1 = t0 + partition_size < n ? t0 + partition_size : n;
            double *oj = part_o + (p * pn + j) * head_dim;
            if (t0 >= t1) {
                part_m[p * pn + j] = -INFINITY;
                part_l[p * pn + j] = 0.0;
                for (int64_t e = 0; e < head_dim; ++e)
                    oj[e] = 0.0;
                continue;
            }
            double m, l;
            attend_range(q, q_dtype, p, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                         num_kv_heads, head_dim, g, bt_row, t0, t1, scale, &m, &l, oj);
            for (int64_t e = 0; e < head_dim; ++e)
                oj[e] /= l;
            part_m[p * pn + j] = m;
            part_l[p * pn + j] = l;
        }
        double *o = out + p * head_dim;
        for (int64_t e = 0; e < head_dim; ++e)
            o[e] = 0.0;
        if (n <= 0)
            continue;
        double big_m = -INFINITY;
        for (int64_t j = 0; j < pn; ++j)
            if (part_l[p * pn + j] > 0.0 && part_m[p * pn + j] > big_m)
                big_m = part_m[p * pn + j];
        double wsum = 0.0;
        for (int64_t j = 0; j < pn; ++j) {
            if (!(part_l[p * pn + j] > 0.0))
                continue;
            double w = part_l[p * pn + j] * exp(part_m[p * pn + j] - big_m);
            wsum += w;
            for (int64_t e = 0; e < head_dim; ++e)
                o[e] += w * part_o[(p * pn + j) * head_dim + e];
        }
        for (int64_t e = 0; e < head_dim; ++e)
            o[e] /= wsum;
    }
    return OR_OK;
}
