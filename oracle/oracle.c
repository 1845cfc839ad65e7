/*
 * CPU oracle for the ordered fp32 scatter-reduce.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load this file.  The product library never links or calls
 * it, and the two share no code, headers, tables or constants.
 *
 * What it computes is the defined result of a deterministic, batch-invariant
 * reduction of many contributions into shared destinations.  The sources are:
 *   - a stable order of contributions per destination: sort by
 *     (destination, source id), as in the MoE backward of the DeepSeek-V4 book
 *     (ch. 9, section 3.2: sort tokens by (expert_id, original_token_id), then
 *     merge in sorted order without atomicAdd);
 *   - per-split private buffers reduced in split-id order (same chapter,
 *     section 3.3, mHC backward);
 *   - one fp32 reduction tree, whatever the partitioning (bitwise-determinism
 *     interview note, "why pay the overhead": every EP size goes through the
 *     same fp32 reduction tree);
 *   - the fixed tree's shape: chunks of 8 contributions summed left to right,
 *     chunk sums combined by a balanced pairwise tree, no fused multiply-add.
 *
 * Readings where the pages leave a step open:
 *   - "balanced pairwise tree" over C chunk sums: split at the largest power
 *     of two strictly below C, left part first.
 *   - a left-to-right chunk sum starts from its first element (no +0.0 seed,
 *     which would turn a lone -0.0 into +0.0).
 *   - index_add: the destination's old value is added once, last, as the
 *     left operand: out = old + T(contributions).  Rows with no contribution
 *     are never written.
 *   - combine: a token's contributions are ordered by the row index of the
 *     expert output they come from (ties by slot); each contribution is
 *     fl32(gate * row), rounded before it is added.
 *   - split reduce: the same tree over the split ids 0..S-1.
 *   - sparse-attention key gradient: contribution q * topk + j is
 *     fl32(dS[q][j] * Q[q]), rounded before it is added (like the gate
 *     product), and the source id is q * topk + j; any softmax scale is
 *     folded into dS by the caller.
 *
 * Arithmetic: IEEE-754 binary32, round to nearest even, no contraction
 * (build with -ffp-contract=off), no excess precision (FLT_EVAL_METHOD 0,
 * SSE), subnormals kept (no flush-to-zero).  The split-K reference is fp64.
 *
 * Everything here is plain loops; speed is not a goal.
 */
#include <float.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs float arithmetic evaluated in float"
#endif

#define ORC_OK 0
#define ORC_BAD_ARG 1
#define ORC_INDEX_OUT_OF_RANGE 4
#define ORC_NO_MEMORY 6

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* ------------------------------------------------------------------ */
/* bfloat16 helpers                                                    */
/* ------------------------------------------------------------------ */
static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* float -> bfloat16, round to nearest even; NaN stays NaN (quietened). */
static uint16_t float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static float load_elem(const void* base, int dtype, int64_t idx)
{
    if (dtype == ORC_BF16)
        return bf16_to_float(((const uint16_t*)base)[idx]);
    return ((const float*)base)[idx];
}

/* ------------------------------------------------------------------ */
/* The fixed tree T(v_0 .. v_{L-1}), L >= 1                            */
/* ------------------------------------------------------------------ */

/* Sum of m >= 1 values, left to right, starting from the first. */
static float chunk_sum(const float* v, int64_t m)
{
    float s = v[0];
    for (int64_t i = 1; i < m; ++i)
        s = s + v[i];
    return s;
}

/* Balanced pairwise tree over c >= 1 chunk sums. */
static float pair_tree(const float* s, int64_t c)
{
    if (c == 1)
        return s[0];
    int64_t p = 1;
    while (p * 2 < c)
        p *= 2; /* largest power of two strictly less than c */
    float left = pair_tree(s, p);
    float right = pair_tree(s + p, c - p);
    return left + right;
}

/* T over L >= 1 values.  Returns 0 on success. */
static int tree_sum(const float* v, int64_t L, float* result)
{
    int64_t c = (L + 7) / 8;
    float* sums = (float*)malloc((size_t)c * sizeof(float));
    if (!sums)
        return ORC_NO_MEMORY;
    for (int64_t j = 0; j < c; ++j) {
        int64_t m = L - 8 * j < 8 ? L - 8 * j : 8;
        sums[j] = chunk_sum(v + 8 * j, m);
    }
    *result = pair_tree(sums, c);
    free(sums);
    return ORC_OK;
}

int oracle_tree_sum_f32(const float* v, int64_t L, float* result)
{
    if (!v || !result || L < 1)
        return ORC_BAD_ARG;
    return tree_sum(v, L, result);
}

/* The same tree in a bfloat16 accumulator: every partial sum is rounded to
 * bfloat16.  Test-only: it reproduces worked examples stated in bf16.  A bf16
 * sum is formed as bf16(fl32(a + b)); for the sum of two bf16 values the double
 * rounding is innocuous since 24 >= 2*8 + 2. */
static uint16_t bf16_add(uint16_t a, uint16_t b)
{
    return float_to_bf16(bf16_to_float(a) + bf16_to_float(b));
}

static uint16_t pair_tree_bf16(const uint16_t* s, int64_t c)
{
    if (c == 1)
        return s[0];
    int64_t p = 1;
    while (p * 2 < c)
        p *= 2;
    uint16_t left = pair_tree_bf16(s, p);
    uint16_t right = pair_tree_bf16(s + p, c - p);
    return bf16_add(left, right);
}

int oracle_tree_sum_bf16(const uint16_t* v, int64_t L, uint16_t* result)
{
    if (!v || !result || L < 1)
        return ORC_BAD_ARG;
    int64_t c = (L + 7) / 8;
    uint16_t* sums = (uint16_t*)malloc((size_t)c * sizeof(uint16_t));
    if (!sums)
        return ORC_NO_MEMORY;
    for (int64_t j = 0; j < c; ++j) {
        int64_t m = L - 8 * j < 8 ? L - 8 * j : 8;
        uint16_t s = v[8 * j];
        for (int64_t i = 1; i < m; ++i)
            s = bf16_add(s, v[8 * j + i]);
        sums[j] = s;
    }
    *result = pair_tree_bf16(sums, c);
    free(sums);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Stable order of contributions: sort by (dest, src_id, position)     */
/* ------------------------------------------------------------------ */
typedef struct {
    int32_t dest;
    int32_t src;
    int64_t pos;
} contrib_key;

static int cmp_contrib(const void* a, const void* b)
{
    const contrib_key* x = (const contrib_key*)a;
    const contrib_key* y = (const contrib_key*)b;
    if (x->dest != y->dest)
        return x->dest < y->dest ? -1 : 1;
    if (x->src != y->src)
        return x->src < y->src ? -1 : 1;
    if (x->pos != y->pos)
        return x->pos < y->pos ? -1 : 1;
    return 0;
}

/* perm[r] = input position of the r-th contribution in (dest, src_id) order,
 * ties by input position; seg_offsets[d] = first r with dest d (length D+1);
 * inv_perm (optional) is the inverse: inv_perm[perm[r]] = r.
 * src_id == NULL means src_id[i] = i. */
int oracle_sort_by_dest(const int32_t* dest, const int32_t* src_id, int64_t n, int32_t num_dests,
                        int32_t* perm, int32_t* seg_offsets, int32_t* inv_perm)
{
    if (n < 0 || num_dests < 1 || (n > 0 && (!dest || !perm)) || !seg_offsets)
        return ORC_BAD_ARG;
    for (int64_t i = 0; i < n; ++i)
        if (dest[i] < 0 || dest[i] >= num_dests)
            return ORC_INDEX_OUT_OF_RANGE;
    contrib_key* keys = (contrib_key*)malloc((size_t)(n > 0 ? n : 1) * sizeof(contrib_key));
    if (!keys)
        return ORC_NO_MEMORY;
    for (int64_t i = 0; i < n; ++i) {
        keys[i].dest = dest[i];
        keys[i].src = src_id ? src_id[i] : (int32_t)i;
        keys[i].pos = i;
    }
    qsort(keys, (size_t)n, sizeof(contrib_key), cmp_contrib);
    for (int64_t r = 0; r < n; ++r) {
        perm[r] = (int32_t)keys[r].pos;
        if (inv_perm)
            inv_perm[keys[r].pos] = (int32_t)r;
    }
    /* seg_offsets: exclusive prefix sum of the per-destination counts */
    for (int32_t d = 0; d <= num_dests; ++d)
        seg_offsets[d] = 0;
    for (int64_t i = 0; i < n; ++i)
        seg_offsets[dest[i] + 1] += 1;
    for (int32_t d = 0; d < num_dests; ++d)
        seg_offsets[d + 1] += seg_offsets[d];
    free(keys);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Running independent output rows on several host threads             */
/* ------------------------------------------------------------------ */

/* Every output row (a destination, a key, a token) is computed from its own
 * inputs only, so rows can be handed to threads in contiguous ranges without
 * changing a bit: the threads only divide the row loop.  threads <= 1 runs
 * the loop on the calling thread. */
typedef struct row_job {
    int (*fn)(const struct row_job* job, int64_t r0, int64_t r1);
    const void* ctx;
    int64_t r0, r1;
    int rc;
} row_job;

static void* row_job_main(void* arg)
{
    row_job* j = (row_job*)arg;
    j->rc = j->fn(j, j->r0, j->r1);
    return NULL;
}

static int run_rows(int (*fn)(const row_job*, int64_t, int64_t), const void* ctx, int64_t rows, int32_t threads)
{
    if (threads > 256)
        threads = 256;
    if (threads <= 1 || rows < 2) {
        row_job one = {fn, ctx, 0, rows, ORC_OK};
        return fn(&one, 0, rows);
    }
    row_job jobs[256];
    pthread_t tid[256];
    int started[256];
    int64_t per = (rows + threads - 1) / threads;
    for (int32_t t = 0; t < threads; ++t) {
        int64_t lo = (int64_t)t * per < rows ? (int64_t)t * per : rows;
        int64_t hi = lo + per < rows ? lo + per : rows;
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].r0 = lo;
        jobs[t].r1 = hi;
        jobs[t].rc = ORC_OK;
        started[t] = pthread_create(&tid[t], NULL, row_job_main, &jobs[t]) == 0;
        if (!started[t])
            row_job_main(&jobs[t]); /* no thread: run the range here */
    }
    int rc = ORC_OK;
    for (int32_t t = 0; t < threads; ++t) {
        if (started[t])
            pthread_join(tid[t], NULL);
        if (rc == ORC_OK && jobs[t].rc != ORC_OK)
            rc = jobs[t].rc;
    }
    return rc;
}

/* Longest segment of a CSR offset array (the size of a per-thread buffer). */
static int64_t max_segment(const int32_t* seg, int32_t num_dests)
{
    int64_t m = 1;
    for (int32_t d = 0; d < num_dests; ++d)
        if (seg[d + 1] - seg[d] > m)
            m = seg[d + 1] - seg[d];
    return m;
}

/* ------------------------------------------------------------------ */
/* Scatter-reduce / index_add                                          */
/* ------------------------------------------------------------------ */

/* One reduction problem after the sort: destination d's contributions are
 * perm[seg[d]] .. perm[seg[d+1]-1], in that order.  A contribution i is
 * src row i (scale == NULL), or fl32(scale[i] * src row i / rows_per_src). */
typedef struct {
    float* out;
    int32_t num_dests;
    int64_t H;
    const void* src;
    int src_dtype;
    const float* scale;
    int32_t rows_per_src;
    const int32_t* perm;
    const int32_t* seg;
    const int32_t* dests;
    int64_t max_len;
} reduce_ctx;

static int reduce_rows(const row_job* job, int64_t r0, int64_t r1)
{
    const reduce_ctx* c = (const reduce_ctx*)job->ctx;
    float* vals = (float*)malloc((size_t)c->max_len * sizeof(float));
    if (!vals)
        return ORC_NO_MEMORY;
    int rc = ORC_OK;
    for (int64_t q = r0; q < r1 && rc == ORC_OK; ++q) {
        int32_t d = c->dests ? c->dests[q] : (int32_t)q;
        if (d < 0 || d >= c->num_dests) {
            rc = ORC_INDEX_OUT_OF_RANGE;
            break;
        }
        int64_t lo = c->seg[d], L = c->seg[d + 1] - c->seg[d];
        if (L == 0)
            continue; /* untouched row */
        float* row = c->out + q * c->H;
        for (int64_t h = 0; h < c->H && rc == ORC_OK; ++h) {
            for (int64_t j = 0; j < L; ++j) {
                int64_t i = c->perm[lo + j];
                if (c->scale) {
                    float product = c->scale[i] * load_elem(c->src, c->src_dtype, (i / c->rows_per_src) * c->H + h);
                    vals[j] = product; /* rounded to float before any add */
                } else {
                    vals[j] = load_elem(c->src, c->src_dtype, i * c->H + h);
                }
            }
            float t;
            rc = tree_sum(vals, L, &t);
            if (rc == ORC_OK)
                row[h] = row[h] + t;
        }
    }
    free(vals);
    return rc;
}

/* Sorts the contributions by (index, src_id), then reduces every requested row. */
static int sort_and_reduce(reduce_ctx* c, int64_t n, const int32_t* index, const int32_t* src_id, int64_t rows,
                           int32_t threads)
{
    int32_t* perm = (int32_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
    int32_t* seg = (int32_t*)malloc((size_t)(c->num_dests + 1) * sizeof(int32_t));
    if (!perm || !seg) {
        free(perm); free(seg);
        return ORC_NO_MEMORY;
    }
    int rc = oracle_sort_by_dest(index, src_id, n, c->num_dests, perm, seg, NULL);
    if (rc == ORC_OK) {
        c->perm = perm;
        c->seg = seg;
        c->max_len = max_segment(seg, c->num_dests);
        rc = run_rows(reduce_rows, c, rows, threads);
    }
    free(perm); free(seg);
    return rc;
}

/* For every destination d (or the listed ones), with its contributions taken in
 * (src_id, position) order:  out[d][h] = out[d][h] + T(src[i_0][h], ...).
 *
 * dests == NULL: out is [num_dests][H], updated in place.
 * dests != NULL: out is [ndest][H] and holds the listed destinations' rows
 * (initial contents in, result out); other destinations are not computed.
 * threads: host threads that share the rows (the bits do not depend on it). */
int oracle_scatter_reduce(float* out, int32_t num_dests, int64_t H, const void* src, int src_dtype,
                          int64_t n, const int32_t* index, const int32_t* src_id,
                          const int32_t* dests, int64_t ndest, int32_t threads)
{
    if (!out || H < 1 || num_dests < 1 || n < 0 || (n > 0 && (!src || !index)))
        return ORC_BAD_ARG;
    if (src_dtype != ORC_F32 && src_dtype != ORC_BF16)
        return ORC_BAD_ARG;
    reduce_ctx c = {out, num_dests, H, src, src_dtype, NULL, 1, NULL, NULL, dests, 1};
    return sort_and_reduce(&c, n, index, src_id, dests ? ndest : num_dests, threads);
}

/* ------------------------------------------------------------------ */
/* Sparse-attention key gradient                                       */
/* ------------------------------------------------------------------ */

/* The backward of DeepSeek-V4's sparse attention (ch. 9, section 3.1): every
 * query q selected topk keys, and the gradient of a selected key accumulates,
 * over the queries that selected it, the query's row scaled by that query's
 * score gradient.  Contribution i = q * topk + j is
 *     c_i[h] = fl32(dS[i] * Q[q][h])      (one rounding, never fused)
 * and dK[key][h] = dK[key][h] + T(c_i[h] over i with key_idx[i] == key, in
 * order of i), the index_add order with the contribution formed on the fly.
 * Q is [nq][H] fp32 or bf16, dS and key_idx are [nq][topk].
 * keys == NULL: dK is [num_keys][H], updated in place.
 * keys != NULL: dK is [nkeys][H] holding the listed keys' rows. */
int oracle_sparse_attn_dk(float* dK, int32_t num_keys, int64_t H, const void* Q, int q_dtype, const float* dS,
                          const int32_t* key_idx, int64_t nq, int32_t topk, const int32_t* keys, int64_t nkeys,
                          int32_t threads)
{
    if (!dK || H < 1 || num_keys < 1 || nq < 0 || topk < 1)
        return ORC_BAD_ARG;
    if (q_dtype != ORC_F32 && q_dtype != ORC_BF16)
        return ORC_BAD_ARG;
    const int64_t n = nq * (int64_t)topk;
    if (n > 0 && (!Q || !dS || !key_idx))
        return ORC_BAD_ARG;
    reduce_ctx c = {dK, num_keys, H, Q, q_dtype, dS, topk, NULL, NULL, keys, 1};
    return sort_and_reduce(&c, n, key_idx, NULL, keys ? nkeys : num_keys, threads);
}

/* ------------------------------------------------------------------ */
/* MoE combine                                                         */
/* ------------------------------------------------------------------ */

/* out[t][h] = T over the token's k contributions fl32(gate[t][j] * rows[row_of[t][j]][h]),
 * ordered by row index (ties by slot j).  Written, not accumulated.
 * tokens == NULL: all T tokens, out is [T][H]; else out is [ntok][H].
 * threads: host threads that share the tokens (the bits do not depend on it). */
typedef struct {
    const void* rows;
    int rows_dtype;
    int64_t num_rows, H;
    const int32_t* row_of;
    const float* gates;
    int64_t T;
    int32_t k;
    const int64_t* tokens;
    float* out;
} combine_ctx;

static int combine_rows(const row_job* job, int64_t q0, int64_t q1)
{
    const combine_ctx* c = (const combine_ctx*)job->ctx;
    const int32_t k = c->k;
    int32_t* order = (int32_t*)malloc((size_t)k * sizeof(int32_t));
    float* vals = (float*)malloc((size_t)k * sizeof(float));
    if (!order || !vals) {
        free(order); free(vals);
        return ORC_NO_MEMORY;
    }
    int rc = ORC_OK;
    for (int64_t q = q0; q < q1 && rc == ORC_OK; ++q) {
        int64_t t = c->tokens ? c->tokens[q] : q;
        if (t < 0 || t >= c->T) {
            rc = ORC_INDEX_OUT_OF_RANGE;
            break;
        }
        const int32_t* r = c->row_of + t * k;
        const float* g = c->gates + t * k;
        for (int32_t j = 0; j < k; ++j) {
            if (r[j] < 0 || r[j] >= c->num_rows)
                rc = ORC_INDEX_OUT_OF_RANGE;
        }
        if (rc != ORC_OK)
            break;
        /* insertion sort of the slots by (row, slot): stable */
        for (int32_t j = 0; j < k; ++j)
            order[j] = j;
        for (int32_t a = 1; a < k; ++a) {
            int32_t cur = order[a];
            int32_t b = a - 1;
            while (b >= 0 && r[order[b]] > r[cur]) {
                order[b + 1] = order[b];
                --b;
            }
            order[b + 1] = cur;
        }
        for (int64_t h = 0; h < c->H; ++h) {
            for (int32_t j = 0; j < k; ++j) {
                int32_t slot = order[j];
                float y = load_elem(c->rows, c->rows_dtype, (int64_t)r[slot] * c->H + h);
                float p = g[slot] * y; /* rounded to float before any add */
                vals[j] = p;
            }
            float s;
            rc = tree_sum(vals, k, &s);
            if (rc != ORC_OK)
                break;
            c->out[q * c->H + h] = s;
        }
    }
    free(order); free(vals);
    return rc;
}

int oracle_combine(const void* rows, int rows_dtype, int64_t num_rows, int64_t H,
                   const int32_t* row_of, const float* gates, int64_t T, int32_t k,
                   const int64_t* tokens, int64_t ntok, float* out, int32_t threads)
{
    if (!rows || !row_of || !gates || !out || H < 1 || k < 1 || T < 0 || num_rows < 0)
        return ORC_BAD_ARG;
    if (rows_dtype != ORC_F32 && rows_dtype != ORC_BF16)
        return ORC_BAD_ARG;
    combine_ctx c = {rows, rows_dtype, num_rows, H, row_of, gates, T, k, tokens, out};
    return run_rows(combine_rows, &c, tokens ? ntok : T, threads);
}

/* ------------------------------------------------------------------ */
/* Split-K                                                             */
/* ------------------------------------------------------------------ */

/* out[e] = T(partials[0][e], partials[1][e], ..., partials[S-1][e]) in split-id order. */
int oracle_splitk_reduce(const float* partials, int32_t S, int64_t count, float* out)
{
    if (!partials || !out || S < 1 || count < 0)
        return ORC_BAD_ARG;
    float* vals = (float*)malloc((size_t)S * sizeof(float));
    if (!vals)
        return ORC_NO_MEMORY;
    int rc = ORC_OK;
    for (int64_t e = 0; e < count && rc == ORC_OK; ++e) {
        for (int32_t s = 0; s < S; ++s)
            vals[s] = partials[(int64_t)s * count + e];
        rc = tree_sum(vals, S, &out[e]);
    }
    free(vals);
    return rc;
}

/* Exact reference of dW = X^T dY for bf16 X [K][M], dY [K][N]:
 * exact[m][n] = sum_t x[t][m]*dy[t][n] and absum[m][n] = sum_t |x[t][m]*dy[t][n]|,
 * both in fp64 (each bf16 x bf16 product is exact in fp64). */
int oracle_splitk_reference(const uint16_t* X, const uint16_t* dY, int64_t K, int64_t M, int64_t N,
                            double* exact, double* absum)
{
    if (!X || !dY || !exact || !absum || K < 0 || M < 1 || N < 1)
        return ORC_BAD_ARG;
    double* dy = (double*)malloc((size_t)N * sizeof(double));
    if (!dy)
        return ORC_NO_MEMORY;
    for (int64_t i = 0; i < M * N; ++i) {
        exact[i] = 0.0;
        absum[i] = 0.0;
    }
    for (int64_t t = 0; t < K; ++t) {
        for (int64_t c = 0; c < N; ++c)
            dy[c] = (double)bf16_to_float(dY[t * N + c]);
        for (int64_t m = 0; m < M; ++m) {
            double x = (double)bf16_to_float(X[t * M + m]);
            double* e = exact + m * N;
            double* a = absum + m * N;
            for (int64_t c = 0; c < N; ++c) {
                double p = x * dy[c];
                e[c] += p;
                a[c] += p < 0 ? -p : p;
            }
        }
    }
    free(dy);
    return ORC_OK;
}

/* fp64 per-split sums: P[s][m][n] = sum over tokens t of split s of x[t][m]*dy[t][n].
 * Split s covers tokens [s*c, min(K, (s+1)*c)) with c = ceil(K / S). */
int oracle_splitk_partials(const uint16_t* X, const uint16_t* dY, int64_t K, int64_t M, int64_t N,
                           int32_t S, double* P)
{
    if (!X || !dY || !P || K < 1 || M < 1 || N < 1 || S < 1)
        return ORC_BAD_ARG;
    double* scratch = (double*)malloc((size_t)(M * N) * sizeof(double));
    if (!scratch)
        return ORC_NO_MEMORY;
    int64_t c = (K + S - 1) / S;
    int rc = ORC_OK;
    for (int32_t s = 0; s < S && rc == ORC_OK; ++s) {
        int64_t lo = (int64_t)s * c < K ? (int64_t)s * c : K;
        int64_t hi = lo + c < K ? lo + c : K;
        rc = oracle_splitk_reference(X + lo * M, dY + lo * N, hi - lo, M, N, P + (int64_t)s * M * N, scratch);
    }
    free(scratch);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Fingerprint                                                         */
/* ------------------------------------------------------------------ */

/* SplitMix64's output finaliser (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014). */
uint64_t oracle_splitmix64_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* h = mix(nbytes) + sum_i mix(w_i XOR s_i)  (mod 2^64), where w_i is the i-th
 * little-endian 64-bit word of the bytes in logical order (the last word
 * zero-padded) and s_i = (i + 1) * 0x9e3779b97f4a7c15 is the (i+1)-th state of
 * a SplitMix64 generator started at 0.  For all-zero bytes each term is that
 * generator's published output.  Wrapping addition makes the value
 * independent of the order in which the terms are added.
 * The composition is this library's convention (the pages name a tensor hash
 * without defining one).  It is pinned by the published SplitMix64 outputs:
 * words chosen as s_i XOR s_j turn term i into output j, which fixes the XOR,
 * the word index, the byte order and the zero padding. */
uint64_t oracle_fingerprint(const void* data, int64_t nbytes)
{
    const unsigned char* p = (const unsigned char*)data;
    const uint64_t gamma = 0x9e3779b97f4a7c15ULL;
    uint64_t h = oracle_splitmix64_mix((uint64_t)nbytes);
    int64_t words = (nbytes + 7) / 8;
    for (int64_t i = 0; i < words; ++i) {
        uint64_t w = 0;
        for (int b = 0; b < 8; ++b) {
            int64_t at = i * 8 + b;
            if (at < nbytes)
                w |= (uint64_t)p[at] << (8 * b);
        }
        uint64_t state = (uint64_t)(i + 1) * gamma;
        h += oracle_splitmix64_mix(w ^ state);
    }
    return h;
}
