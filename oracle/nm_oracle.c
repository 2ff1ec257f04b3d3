/*
 * nm_oracle.c -- plain, slow CPU oracle for the N:M bitmask decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or constant with the HIP library.
 *
 * Arithmetic is IEEE fp64 in source order; build with -ffp-contract=off.  Every
 * function validates its inputs and returns a status (0 = ok).
 *
 * Pages this follows (cited by title and section):
 *   [SD-en]    "SparseDecoding: Decoding-Aware Pruning for Accurate and Efficient LLM
 *              Inference" (ai.info AI summary), sections "Main Findings" and
 *              "Methodology in Plain English" (Steps 2 and 3).
 *   [SD-cn]    "SparseDecoding:解码感知的准确高效大模型剪枝框架" (paper.rainbus.top
 *              summary), sections 前置知识 (N:M 半结构化稀疏), 核心方法 (核心创新二),
 *              方法步骤详情 (第三步, 第四步).
 *   [SD-repro] "SparseDecoding：只用解码激活校准的稀疏推理" (daiwk.github.io reproduction
 *              notes), sections 核心公式 and 背景与主要改动.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { NMO_OK = 0, NMO_EARG = 1, NMO_ENONFINITE = 2, NMO_EMASK = 3, NMO_ENOMEM = 4 };

/* bfloat16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_val(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int bf16_finite(uint16_t b) { return (b & 0x7F80u) != 0x7F80u; }

/* ------------------------------------------------------------------ column norms
 * Wanda's per-input-channel activation norm [SD-repro, 核心公式]: for input column j,
 * n_j = sqrt(sum over calibration tokens t of X[t][j]^2).  Reading taken: the sum runs
 * in fp64 in token order, the square root is the IEEE fp64 one, and the result is
 * rounded once to fp32 (the precision the pack step consumes). */
int nmo_col_norm(const uint16_t *X, int64_t T, int64_t K, int64_t ldx, float *n)
{
    if (!X || !n || T < 1 || K < 1 || ldx < K) return NMO_EARG;
    for (int64_t j = 0; j < K; ++j) {
        double s = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            uint16_t b = X[t * ldx + j];
            if (!bf16_finite(b)) return NMO_ENONFINITE;
            double v = bf16_val(b);
            s = s + v * v;
        }
        n[j] = (float)sqrt(s);
    }
    return NMO_OK;
}

/* ------------------------------------------------------------------ select + pack */
typedef struct {
    double score;
    int col;
} scored_t;

/* (score descending, column ascending): a strict total order inside a group. */
static int before(const scored_t *a, const scored_t *b)
{
    if (a->score != b->score) return a->score > b->score;
    return a->col < b->col;
}

/*
 * Wanda N:M selection and bitmask packing.
 *
 * Score [SD-repro, 核心公式]: s_ij = |W_ij| * n_j.  Both factors have short
 * significands (8 and 24 bits), so the fp64 product is exact and comparisons between
 * scores are exact.
 * Selection [SD-cn, 前置知识 N:M; SD-repro, 核心公式]: in every group of M consecutive
 * input columns of a row keep the N highest scores.  Equal scores: the lower column
 * wins (the pages leave ties open; this is the reading taken).
 * Encoding [SD-en, Methodology Step 2; SD-cn, 方法步骤详情 第三步]: one bit per input
 * column, 32 consecutive columns per 32-bit word, bit b of word w <-> column 32w+b;
 * a set bit marks a kept weight (a kept weight that happens to be 0 still sets its
 * bit, which keeps exactly N per group).  Kept values are stored per row in
 * increasing column order, so the t-th set bit of word w (lowest first) owns
 * values[16w + t] at 50% sparsity.
 *
 * Only N = M/2 with M in {4, 8, 16, 32} is accepted: then every aligned word holds
 * exactly 16 kept columns [SD-en, Methodology Step 3].
 */
int nmo_prune_pack(const uint16_t *W, int64_t ldw, int64_t R, int64_t K, const float *n, int N,
                   int M, uint32_t *masks, uint16_t *values)
{
    if (!W || !n || !masks || !values) return NMO_EARG;
    if (R < 1 || K < 32 || K % 32 != 0 || ldw < K) return NMO_EARG;
    if (!(M == 4 || M == 8 || M == 16 || M == 32) || 2 * N != M) return NMO_EARG;
    for (int64_t j = 0; j < K; ++j)
        if (!isfinite(n[j]) || n[j] < 0.0f) return NMO_ENONFINITE;

    scored_t grp[32];
    for (int64_t i = 0; i < R; ++i) {
        const uint16_t *row = W + i * ldw;
        for (int64_t j = 0; j < K; ++j)
            if (!bf16_finite(row[j])) return NMO_ENONFINITE;

        /* 1. select: clear the row's mask words, then set the kept bits group by group */
        for (int64_t w = 0; w < K / 32; ++w) masks[i * (K / 32) + w] = 0u;
        for (int64_t g0 = 0; g0 < K; g0 += M) {
            /* stable insertion sort of the group under (score desc, column asc) */
            for (int k = 0; k < M; ++k) {
                scored_t e;
                e.col = (int)(g0 + k);
                e.score = fabs(bf16_val(row[g0 + k])) * (double)n[g0 + k];
                int p = k;
                while (p > 0 && before(&e, &grp[p - 1])) {
                    grp[p] = grp[p - 1];
                    --p;
                }
                grp[p] = e;
            }
            /* 2. mask emit: the first N of the order are kept */
            for (int k = 0; k < N; ++k) {
                int64_t c = grp[k].col;
                masks[i * (K / 32) + c / 32] |= 1u << (c % 32);
            }
        }
        /* 3. value pack: scan each word from its lowest bit up */
        for (int64_t w = 0; w < K / 32; ++w) {
            uint32_t m = masks[i * (K / 32) + w];
            int t = 0;
            for (int b = 0; b < 32; ++b) {
                if (m & (1u << b)) {
                    if (t >= 16) return NMO_EMASK;
                    values[i * (K / 2) + 16 * w + t] = row[32 * w + b];
                    ++t;
                }
            }
            if (t != 16) return NMO_EMASK;
        }
    }
    return NMO_OK;
}

/* qsort order for a whole row: (score descending, column ascending). */
static int cmp_scored(const void *a, const void *b)
{
    const scored_t *x = (const scored_t *)a, *y = (const scored_t *)b;
    if (before(x, y)) return -1;
    if (before(y, x)) return 1;
    return 0;
}

/*
 * 50% unstructured selection [SD-en, Methodology Step 4: "50% unstructured sparsity",
 * retaining 50% of weights; SD-en, Step 3 on rows of a general sparse matrix].
 * Reading taken: the comparison group is the whole output row (as in Wanda's
 * unstructured setting), each row keeps exactly K/2 weights -- the first K/2 of the
 * row under (score descending, column ascending), score s_ij = |W_ij| * n_j as above.
 * Encoding is unchanged: one bit per column, kept values in increasing column order,
 * now with a varying number of set bits per word (the t-th kept value of the row is
 * values[t]).
 */
int nmo_prune_pack_unstructured(const uint16_t *W, int64_t ldw, int64_t R, int64_t K, const float *n,
                                uint32_t *masks, uint16_t *values)
{
    if (!W || !n || !masks || !values) return NMO_EARG;
    if (R < 1 || K < 32 || K % 32 != 0 || ldw < K) return NMO_EARG;
    for (int64_t j = 0; j < K; ++j)
        if (!isfinite(n[j]) || n[j] < 0.0f) return NMO_ENONFINITE;
    scored_t *order = (scored_t *)malloc((size_t)K * sizeof(scored_t));
    if (!order) return NMO_ENOMEM;
    for (int64_t i = 0; i < R; ++i) {
        const uint16_t *row = W + i * ldw;
        for (int64_t j = 0; j < K; ++j) {
            if (!bf16_finite(row[j])) {
                free(order);
                return NMO_ENONFINITE;
            }
            order[j].col = (int)j;
            order[j].score = fabs(bf16_val(row[j])) * (double)n[j];
        }
        qsort(order, (size_t)K, sizeof(scored_t), cmp_scored);
        for (int64_t w = 0; w < K / 32; ++w) masks[i * (K / 32) + w] = 0u;
        for (int64_t k = 0; k < K / 2; ++k) {
            int64_t c = order[k].col;
            masks[i * (K / 32) + c / 32] |= 1u << (c % 32);
        }
        int64_t t = 0;
        for (int64_t j = 0; j < K; ++j)
            if (masks[i * (K / 32) + j / 32] & (1u << (j % 32))) values[i * (K / 2) + t++] = row[j];
    }
    free(order);
    return NMO_OK;
}

/* Expand one packed row back to a dense row of bf16 patterns (zeros elsewhere). */
static int unpack_row(const uint32_t *mrow, const uint16_t *vrow, int64_t K, uint16_t *out)
{
    for (int64_t w = 0; w < K / 32; ++w) {
        uint32_t m = mrow[w];
        int t = 0;
        for (int b = 0; b < 32; ++b) {
            if (m & (1u << b)) {
                if (t >= 16) return NMO_EMASK;
                out[32 * w + b] = vrow[16 * w + t];
                ++t;
            } else {
                out[32 * w + b] = 0;
            }
        }
        if (t != 16) return NMO_EMASK;
    }
    return NMO_OK;
}

/* Unstructured rows: the t-th set bit of the row (words in order, lowest bit first) owns
 * values[t]; a row must hold exactly K/2 set bits. */
static int unpack_row_rowwise(const uint32_t *mrow, const uint16_t *vrow, int64_t K, uint16_t *out)
{
    int64_t t = 0;
    for (int64_t j = 0; j < K; ++j) {
        if (mrow[j / 32] & (1u << (j % 32))) {
            if (t >= K / 2) return NMO_EMASK;
            out[j] = vrow[t++];
        } else {
            out[j] = 0;
        }
    }
    return t == K / 2 ? NMO_OK : NMO_EMASK;
}

int nmo_unpack_unstructured(const uint32_t *masks, const uint16_t *values, int64_t R, int64_t K, uint16_t *Wout)
{
    if (!masks || !values || !Wout || R < 1 || K < 32 || K % 32 != 0) return NMO_EARG;
    for (int64_t i = 0; i < R; ++i) {
        int rc = unpack_row_rowwise(masks + i * (K / 32), values + i * (K / 2), K, Wout + i * K);
        if (rc) return rc;
    }
    return NMO_OK;
}

int nmo_unpack(const uint32_t *masks, const uint16_t *values, int64_t R, int64_t K, uint16_t *Wout)
{
    if (!masks || !values || !Wout || R < 1 || K < 32 || K % 32 != 0) return NMO_EARG;
    for (int64_t i = 0; i < R; ++i) {
        int rc = unpack_row(masks + i * (K / 32), values + i * (K / 2), K, Wout + i * K);
        if (rc) return rc;
    }
    return NMO_OK;
}

/* ------------------------------------------------------------------ index metadata
 * The formats the bitmask is priced against [SD-en, Main Findings (metadata
 * reduction); SD-cn, 核心方法 (核心创新二)]: 8 bits (a uint8 offset) or 32 bits (an
 * int32 column index) per kept weight instead of 2.  The pages do not spell the
 * layouts out; the readings taken: one entry per kept weight, in the order of the
 * packed values; the uint8 entry of the t-th kept weight of word w is its column
 * minus 32w (0..31), the int32 entry is its column within the row.
 */
#define NMO_META_U8 1
#define NMO_META_I32 2

/* Column of kept weight t (0 <= t < K/2) of row i. */
static int64_t meta_column(const void *meta, int fmt, int64_t i, int64_t t, int64_t K)
{
    const int64_t nnz = K / 2;
    if (fmt == NMO_META_U8) return 32 * (t / 16) + ((const uint8_t *)meta)[i * nnz + t];
    return ((const int32_t *)meta)[i * nnz + t];
}

/* Metadata of canonical masks: the set bits of each word, lowest first. */
int nmo_meta_from_mask(const uint32_t *masks, int64_t R, int64_t K, int fmt, void *meta)
{
    if (!masks || !meta || R < 1 || K < 32 || K % 32 != 0) return NMO_EARG;
    if (fmt != NMO_META_U8 && fmt != NMO_META_I32) return NMO_EARG;
    for (int64_t i = 0; i < R; ++i) {
        for (int64_t w = 0; w < K / 32; ++w) {
            uint32_t m = masks[i * (K / 32) + w];
            int64_t t = 16 * w;
            for (int b = 0; b < 32; ++b) {
                if (!(m & (1u << b))) continue;
                if (t >= 16 * w + 16) return NMO_EMASK;
                if (fmt == NMO_META_U8)
                    ((uint8_t *)meta)[i * (K / 2) + t] = (uint8_t)b;
                else
                    ((int32_t *)meta)[i * (K / 2) + t] = (int32_t)(32 * w + b);
                ++t;
            }
            if (t != 16 * w + 16) return NMO_EMASK;
        }
    }
    return NMO_OK;
}

/* Index metadata is well formed when the columns of each word's 16 kept weights lie in
 * that word and strictly increase (the values are stored in column order). */
static int check_meta(const void *meta, int fmt, int64_t R, int64_t K)
{
    for (int64_t i = 0; i < R; ++i) {
        for (int64_t w = 0; w < K / 32; ++w) {
            int64_t prev = -1;
            for (int64_t t = 16 * w; t < 16 * w + 16; ++t) {
                int64_t c = meta_column(meta, fmt, i, t, K);
                if (c < 32 * w || c >= 32 * w + 32 || c <= prev) return NMO_EMASK;
                prev = c;
            }
        }
    }
    return NMO_OK;
}

/* ------------------------------------------------------------------ matvec references
 * y[b][i] = sum_j Wp[i][j] * x[b][j] with Wp the unpacked pruned matrix (dense
 * reference) or W itself; every product of two bf16 values is exact in fp64 and the
 * sum runs in ascending j.  absum[b][i] = sum_j |Wp[i][j] * x[b][j]| feeds the
 * tolerance.  Rows are split statically over nthreads POSIX threads; each output
 * element is still one sequential fp64 sum, so the thread count never changes a bit.
 */
typedef struct {
    const void *meta;        /* index metadata (nmo_spmv_index), else NULL */
    int fmt;                 /* NMO_META_U8 or NMO_META_I32 when meta is set */
    const uint32_t *masks;   /* NULL for the dense reference */
    int rowwise;             /* masks with a varying count per word (unstructured rows) */
    const uint16_t *values;  /* packed values, or the dense W */
    int64_t ldw;             /* dense only */
    int64_t R, K, ldx;
    const uint16_t *x;
    int B;
    double *y, *absum;
    int64_t r0, r1;
    int rc;
} mv_job;

static void *mv_worker(void *arg)
{
    mv_job *jb = (mv_job *)arg;
    uint16_t *row = NULL;
    if (jb->masks) {
        row = (uint16_t *)malloc((size_t)jb->K * sizeof(uint16_t));
        if (!row) {
            jb->rc = NMO_ENOMEM;
            return NULL;
        }
    }
    jb->rc = NMO_OK;
    if (jb->meta) {
        /* direct definition over the kept weights of each row, in storage order */
        const int64_t nnz = jb->K / 2;
        for (int64_t i = jb->r0; i < jb->r1; ++i) {
            for (int b = 0; b < jb->B; ++b) {
                const uint16_t *xb = jb->x + (int64_t)b * jb->ldx;
                double s = 0.0, a = 0.0;
                for (int64_t t = 0; t < nnz; ++t) {
                    int64_t col = meta_column(jb->meta, jb->fmt, i, t, jb->K);
                    double p = bf16_val(jb->values[i * nnz + t]) * bf16_val(xb[col]);
                    s = s + p;
                    a = a + fabs(p);
                }
                jb->y[(int64_t)b * jb->R + i] = s;
                jb->absum[(int64_t)b * jb->R + i] = a;
            }
        }
        return NULL;
    }
    for (int64_t i = jb->r0; i < jb->r1; ++i) {
        const uint16_t *w;
        if (jb->masks) {
            int rc = jb->rowwise
                         ? unpack_row_rowwise(jb->masks + i * (jb->K / 32), jb->values + i * (jb->K / 2), jb->K, row)
                         : unpack_row(jb->masks + i * (jb->K / 32), jb->values + i * (jb->K / 2), jb->K, row);
            if (rc) {
                jb->rc = rc;
                break;
            }
            w = row;
        } else {
            w = jb->values + i * jb->ldw;
        }
        for (int b = 0; b < jb->B; ++b) {
            const uint16_t *xb = jb->x + (int64_t)b * jb->ldx;
            double s = 0.0, a = 0.0;
            for (int64_t j = 0; j < jb->K; ++j) {
                double p = bf16_val(w[j]) * bf16_val(xb[j]);
                s = s + p;
                a = a + fabs(p);
            }
            jb->y[(int64_t)b * jb->R + i] = s;
            jb->absum[(int64_t)b * jb->R + i] = a;
        }
    }
    free(row);
    return NULL;
}

static int run_mv(mv_job proto, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 1024) nthreads = 1024;
    if ((int64_t)nthreads > proto.R) nthreads = (int)proto.R;
    mv_job *jobs = (mv_job *)calloc((size_t)nthreads, sizeof(mv_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return NMO_ENOMEM;
    }
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].r0 = proto.R * t / nthreads;
        jobs[t].r1 = proto.R * (t + 1) / nthreads;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, mv_worker, &jobs[t]) != 0) break;
        started = t;
    }
    mv_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    for (int t = started + 1; t < nthreads; ++t) mv_worker(&jobs[t]); /* threads that failed to start */
    int rc = NMO_OK;
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].rc) rc = jobs[t].rc;
    free(jobs);
    free(th);
    return rc;
}

static int check_x(const uint16_t *x, int64_t K, int64_t ldx, int B)
{
    for (int b = 0; b < B; ++b)
        for (int64_t j = 0; j < K; ++j)
            if (!bf16_finite(x[(int64_t)b * ldx + j])) return NMO_ENONFINITE;
    return NMO_OK;
}

/* Sparse reference [SD-en, Methodology Step 3]: the matvec of the unpacked pruned
 * matrix, i.e. one product per kept weight per token. */
int nmo_spmv(const uint32_t *masks, const uint16_t *values, int64_t R, int64_t K, const uint16_t *x,
             int64_t ldx, int B, double *y, double *absum, int nthreads)
{
    if (!masks || !values || !x || !y || !absum) return NMO_EARG;
    if (R < 1 || K < 32 || K % 32 != 0 || B < 1 || ldx < K) return NMO_EARG;
    int rc = check_x(x, K, ldx, B);
    if (rc) return rc;
    for (int64_t i = 0; i < R * (K / 2); ++i)
        if (!bf16_finite(values[i])) return NMO_ENONFINITE;
    mv_job p;
    memset(&p, 0, sizeof p);
    p.masks = masks;
    p.values = values;
    p.R = R;
    p.K = K;
    p.ldx = ldx;
    p.x = x;
    p.B = B;
    p.y = y;
    p.absum = absum;
    return run_mv(p, nthreads);
}

/* Dense reference: the same sum over the unpruned bf16 matrix. */
int nmo_dense(const uint16_t *W, int64_t ldw, int64_t R, int64_t K, const uint16_t *x, int64_t ldx, int B,
              double *y, double *absum, int nthreads)
{
    if (!W || !x || !y || !absum) return NMO_EARG;
    if (R < 1 || K < 1 || B < 1 || ldw < K || ldx < K) return NMO_EARG;
    int rc = check_x(x, K, ldx, B);
    if (rc) return rc;
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < K; ++j)
            if (!bf16_finite(W[i * ldw + j])) return NMO_ENONFINITE;
    mv_job p;
    memset(&p, 0, sizeof p);
    p.values = W;
    p.ldw = ldw;
    p.R = R;
    p.K = K;
    p.ldx = ldx;
    p.x = x;
    p.B = B;
    p.y = y;
    p.absum = absum;
    return run_mv(p, nthreads);
}

/* Sparse reference over index metadata: y[b][i] = sum_t values[i][t] * x[b][col(i, t)],
 * summed in storage order (which is ascending column order, so on metadata built from
 * masks the result equals nmo_spmv's bit for bit). */
int nmo_spmv_index(const void *meta, int fmt, const uint16_t *values, int64_t R, int64_t K, const uint16_t *x,
                   int64_t ldx, int B, double *y, double *absum, int nthreads)
{
    if (!meta || !values || !x || !y || !absum) return NMO_EARG;
    if (fmt != NMO_META_U8 && fmt != NMO_META_I32) return NMO_EARG;
    if (R < 1 || K < 32 || K % 32 != 0 || B < 1 || ldx < K) return NMO_EARG;
    int rc = check_x(x, K, ldx, B);
    if (rc) return rc;
    rc = check_meta(meta, fmt, R, K);
    if (rc) return rc;
    for (int64_t i = 0; i < R * (K / 2); ++i)
        if (!bf16_finite(values[i])) return NMO_ENONFINITE;
    mv_job p;
    memset(&p, 0, sizeof p);
    p.meta = meta;
    p.fmt = fmt;
    p.values = values;
    p.R = R;
    p.K = K;
    p.ldx = ldx;
    p.x = x;
    p.B = B;
    p.y = y;
    p.absum = absum;
    return run_mv(p, nthreads);
}

/* Sparse reference for unstructured rows: the matvec of the unpacked pruned matrix. */
int nmo_spmv_unstructured(const uint32_t *masks, const uint16_t *values, int64_t R, int64_t K, const uint16_t *x,
                          int64_t ldx, int B, double *y, double *absum, int nthreads)
{
    if (!masks || !values || !x || !y || !absum) return NMO_EARG;
    if (R < 1 || K < 32 || K % 32 != 0 || B < 1 || ldx < K) return NMO_EARG;
    int rc = check_x(x, K, ldx, B);
    if (rc) return rc;
    for (int64_t i = 0; i < R * (K / 2); ++i)
        if (!bf16_finite(values[i])) return NMO_ENONFINITE;
    mv_job p;
    memset(&p, 0, sizeof p);
    p.masks = masks;
    p.rowwise = 1;
    p.values = values;
    p.R = R;
    p.K = K;
    p.ldx = ldx;
    p.x = x;
    p.B = B;
    p.y = y;
    p.absum = absum;
    return run_mv(p, nthreads);
}
