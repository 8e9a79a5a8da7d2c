/*
 * snack_oracle.c -- plain, slow, obviously-correct fp64 reference of the SNACK
 * truly-sparse linear layer.  TEST INFRASTRUCTURE ONLY: only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load this library.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Source: "Beyond Masked Sparsity: SNACK Enables Truly Sparse Neural Networks
 * on GPU" (Badour, van Keulen, Mocanu, arXiv:2610.04093).
 *
 * Notation: W is out x in (O x I) and holds nnz stored entries as a COO triple
 * (rows[k], cols[k], vals[k]); X is B x I (batch-major), Y = X W^T + b is B x O,
 * dY is B x O, dX = dY W is B x I, dW[k] = sum_b dY[b,rows[k]] X[b,cols[k]].
 * All floating-point work is fp64.  Loops over the batch run in parallel with
 * OpenMP when nthreads > 1; every output is still summed in ascending k (or
 * ascending b), so the result does not depend on the thread count.
 *
 * Every function returns 0 on success or a positive error code:
 *   1 null pointer, 2 bad shape, 3 index out of range, 4 duplicate (row,col),
 *   5 allocation failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_NULL 1
#define OR_SHAPE 2
#define OR_INDEX 3
#define OR_DUP 4
#define OR_NOMEM 5

static void set_threads(int nthreads) {
#ifdef _OPENMP
    omp_set_num_threads(nthreads > 0 ? nthreads : 1);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_num_procs();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* COO construction.  Appendix B (Table 7) defines the COO triple, the CSR    */
/* index pointer (row offsets) and the CSC view; Section 3.1 states that CSR  */
/* and COO are interchangeable.  The oracle sorts with a comparison sort on   */
/* the key row*I + col (and col*O + row for the column view).                 */
/* ------------------------------------------------------------------------ */

typedef struct { int64_t key; int64_t idx; } keyed_t;

static int cmp_keyed(const void *a, const void *b) {
    const keyed_t *x = (const keyed_t *)a, *y = (const keyed_t *)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

/* Sort the triple by (row, col); reject out-of-range indices and repeated
 * pairs.  perm_out[k] = input position of sorted entry k.  row_offsets[r] is
 * the number of entries whose row is < r (r = 0..O).  The column view lists
 * sorted positions in (col, row) order: col_perm[j] is a position in the
 * sorted triple, col_rows/col_cols its row and column, col_offsets[c] the
 * number of entries whose column is < c.  Any output may be NULL. */
int oracle_build(int64_t O, int64_t I, int64_t nnz,
                 const int32_t *rows, const int32_t *cols, const float *vals,
                 int32_t *rows_out, int32_t *cols_out, float *vals_out,
                 int32_t *perm_out, int32_t *row_offsets_out,
                 int32_t *col_perm_out, int32_t *col_rows_out, int32_t *col_cols_out,
                 int32_t *col_offsets_out)
{
    if (O < 0 || I < 0 || nnz < 0) return OR_SHAPE;
    if (O > 2147483647LL || I > 2147483647LL || nnz > 2147483647LL) return OR_SHAPE;
    if (nnz > O * I) return OR_SHAPE;
    if (nnz > 0 && (!rows || !cols)) return OR_NULL;
    for (int64_t k = 0; k < nnz; ++k) {
        if (rows[k] < 0 || rows[k] >= O || cols[k] < 0 || cols[k] >= I) return OR_INDEX;
    }
    keyed_t *e = (keyed_t *)malloc(sizeof(keyed_t) * (size_t)(nnz > 0 ? nnz : 1));
    if (!e) return OR_NOMEM;
    for (int64_t k = 0; k < nnz; ++k) {
        e[k].key = (int64_t)rows[k] * I + cols[k];
        e[k].idx = k;
    }
    qsort(e, (size_t)nnz, sizeof(keyed_t), cmp_keyed);
    for (int64_t k = 1; k < nnz; ++k) {
        if (e[k].key == e[k - 1].key) { free(e); return OR_DUP; }
    }
    for (int64_t k = 0; k < nnz; ++k) {
        int64_t src = e[k].idx;
        if (rows_out) rows_out[k] = rows[src];
        if (cols_out) cols_out[k] = cols[src];
        if (vals_out) vals_out[k] = vals ? vals[src] : 0.0f;
        if (perm_out) perm_out[k] = (int32_t)src;
    }
    if (row_offsets_out) {
        /* row_offsets[r] = #{k : row_k < r} */
        for (int64_t r = 0; r <= O; ++r) row_offsets_out[r] = 0;
        for (int64_t k = 0; k < nnz; ++k) row_offsets_out[rows[e[k].idx] + 1] += 1;
        for (int64_t r = 0; r < O; ++r) row_offsets_out[r + 1] += row_offsets_out[r];
    }
    if (col_perm_out || col_rows_out || col_cols_out || col_offsets_out) {
        keyed_t *t = (keyed_t *)malloc(sizeof(keyed_t) * (size_t)(nnz > 0 ? nnz : 1));
        if (!t) { free(e); return OR_NOMEM; }
        for (int64_t k = 0; k < nnz; ++k) {
            int64_t src = e[k].idx;
            t[k].key = (int64_t)cols[src] * O + rows[src];
            t[k].idx = k; /* position in the row-sorted triple */
        }
        qsort(t, (size_t)nnz, sizeof(keyed_t), cmp_keyed);
        for (int64_t j = 0; j < nnz; ++j) {
            int64_t k = t[j].idx;
            if (col_perm_out) col_perm_out[j] = (int32_t)k;
            if (col_rows_out) col_rows_out[j] = rows[e[k].idx];
            if (col_cols_out) col_cols_out[j] = cols[e[k].idx];
        }
        if (col_offsets_out) {
            for (int64_t c = 0; c <= I; ++c) col_offsets_out[c] = 0;
            for (int64_t k = 0; k < nnz; ++k) col_offsets_out[cols[e[k].idx] + 1] += 1;
            for (int64_t c = 0; c < I; ++c) col_offsets_out[c + 1] += col_offsets_out[c];
        }
        free(t);
    }
    free(e);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Forward.  Algorithm 1 (Section 3.1): start from C = 0, then for every      */
/* stored entry (i, j, a) and every batch column l, C[i,l] += a * B[j,l].     */
/* In the layer's batch-major layout C[i,l] is Y[l][i] and B[j,l] is X[l][j]; */
/* the bias of the nn.Linear drop-in (Section 3.5) is added last.  The batch  */
/* loop is outermost so that threads own disjoint rows of Y; each Y[l][i] is  */
/* still the sum over its entries in ascending k.                             */
/* ------------------------------------------------------------------------ */
int oracle_fwd(int64_t O, int64_t I, int64_t nnz,
               const int32_t *rows, const int32_t *cols, const double *vals,
               int64_t B, const double *X, const double *bias, double *Y, int nthreads)
{
    if (O < 0 || I < 0 || nnz < 0 || B < 0) return OR_SHAPE;
    if ((nnz > 0 && (!rows || !cols || !vals)) || (B > 0 && ((I > 0 && !X) || (O > 0 && !Y))))
        return OR_NULL;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t l = 0; l < B; ++l) {
        double *y = Y + l * O;
        const double *x = X + l * I;
        for (int64_t i = 0; i < O; ++i) y[i] = 0.0;
        for (int64_t k = 0; k < nnz; ++k) y[rows[k]] += vals[k] * x[cols[k]];
        if (bias) for (int64_t i = 0; i < O; ++i) y[i] += bias[i];
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Input gradient.  Section 3.4 / Appendix F: dL/dX = W^T (dL/dA); W^T keeps  */
/* W's entries with row and column swapped, so entry (i, j, a) adds a*dA[i,l] */
/* into dX[j,l].  Batch-major: dX[l][j] += a * dY[l][i], ascending k.         */
/* ------------------------------------------------------------------------ */
int oracle_bwd_input(int64_t O, int64_t I, int64_t nnz,
                     const int32_t *rows, const int32_t *cols, const double *vals,
                     int64_t B, const double *dY, double *dX, int nthreads)
{
    if (O < 0 || I < 0 || nnz < 0 || B < 0) return OR_SHAPE;
    if ((nnz > 0 && (!rows || !cols || !vals)) || (B > 0 && ((O > 0 && !dY) || (I > 0 && !dX))))
        return OR_NULL;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t l = 0; l < B; ++l) {
        double *dx = dX + l * I;
        const double *dy = dY + l * O;
        for (int64_t j = 0; j < I; ++j) dx[j] = 0.0;
        for (int64_t k = 0; k < nnz; ++k) dx[cols[k]] += vals[k] * dy[rows[k]];
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Weight gradient on the support.  Section 3.4 / Appendix F: (dL/dW)_{i,j} = */
/* sum over the batch t of dA[i,t] X[j,t], evaluated only for (i,j) in        */
/* supp(W) and written (not accumulated) in the order of the stored triple.   */
/* ------------------------------------------------------------------------ */
int oracle_grad_weight(int64_t O, int64_t I, int64_t nnz,
                       const int32_t *rows, const int32_t *cols,
                       int64_t B, const double *X, const double *dY, double *dW, int nthreads)
{
    if (O < 0 || I < 0 || nnz < 0 || B < 0) return OR_SHAPE;
    if (nnz > 0 && (!rows || !cols || !dW || (B > 0 && (!X || !dY)))) return OR_NULL;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < nnz; ++k) {
        double s = 0.0;
        for (int64_t t = 0; t < B; ++t) s += dY[t * O + rows[k]] * X[t * I + cols[k]];
        dW[k] = s;
    }
    return OR_OK;
}

/* Bias gradient of the nn.Linear drop-in: db[i] = sum_t dY[t][i]. */
int oracle_grad_bias(int64_t O, int64_t B, const double *dY, double *db)
{
    if (O < 0 || B < 0) return OR_SHAPE;
    if (O > 0 && (!db || (B > 0 && !dY))) return OR_NULL;
    for (int64_t i = 0; i < O; ++i) {
        double s = 0.0;
        for (int64_t t = 0; t < B; ++t) s += dY[t * O + i];
        db[i] = s;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Topology update (Appendix G): prune the n_prune stored entries of smallest */
/* magnitude, then regrow as many fresh positions with the uniform            */
/* initializer of Algorithm 2: draw a row index and a column index, reject    */
/* the pair if it is already in the set S of live positions, else add it.     */
/* getrand(n) maps a SplitMix64 output u to floor(u*n / 2^64).  Ties in |w|   */
/* are broken by the position in the sorted triple; regrown values are 0.     */
/* ------------------------------------------------------------------------ */

/* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014): add the golden-ratio increment to the state and
 * return a mixed copy of it. */
static uint64_t splitmix64_next(uint64_t *state) {
    uint64_t z = (*state += 0x9E3779B97F4A7C15ULL);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

void oracle_splitmix64(uint64_t seed, int64_t n, uint64_t *out) {
    uint64_t s = seed;
    for (int64_t i = 0; i < n; ++i) out[i] = splitmix64_next(&s);
}

static int64_t getrand(uint64_t *state, int64_t n) {
    unsigned __int128 p = (unsigned __int128)splitmix64_next(state) * (unsigned __int128)(uint64_t)n;
    return (int64_t)(p >> 64);
}

void oracle_getrand(uint64_t seed, int64_t n, int64_t count, int64_t *out) {
    uint64_t s = seed;
    for (int64_t i = 0; i < count; ++i) out[i] = getrand(&s, n);
}

typedef struct { float mag; int64_t k; } magkey_t;

static int cmp_mag(const void *a, const void *b) {
    const magkey_t *x = (const magkey_t *)a, *y = (const magkey_t *)b;
    if (x->mag != y->mag) return x->mag < y->mag ? -1 : 1;
    return (x->k > y->k) - (x->k < y->k);
}

/* Input: a sorted triple.  Output: the sorted triple after prune-and-regrow,
 * pruned_out[0..n_prune) = the pruned positions of the input in ascending
 * order (optional), trials_out = number of (row, col) draws (optional). */
/* Uniform initializer (SNACK, Algorithm 2; cost analysis in Appendix F): draw
 * nnz distinct positions of the O x I matrix by rejection.  Each trial draws the
 * row with getrand(O) and then the column with getrand(I) from one SplitMix64
 * stream started at `seed`, and keeps the pair unless it was drawn before.  The
 * positions are returned sorted by (row, col) with their row offsets (or NULL)
 * and the number of trials. */
int oracle_init_uniform(int64_t O, int64_t I, int64_t nnz, uint64_t seed,
                        int32_t *rows_out, int32_t *cols_out, int32_t *row_offsets_out, int64_t *trials_out)
{
    if (O <= 0 || I <= 0 || nnz < 0 || nnz > O * I) return OR_SHAPE;
    if (nnz > 0 && (!rows_out || !cols_out)) return OR_NULL;
    unsigned char *seen = (unsigned char *)calloc((size_t)(O * I), 1);
    int32_t *r = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
    int32_t *c = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
    if (!seen || !r || !c) { free(seen); free(r); free(c); return OR_NOMEM; }
    uint64_t state = seed;
    int64_t trials = 0, n = 0;
    while (n < nnz) {
        const int64_t row = getrand(&state, O);   /* row first, then column */
        const int64_t col = getrand(&state, I);
        trials += 1;
        if (seen[row * I + col]) continue;         /* drawn before: reject */
        seen[row * I + col] = 1;
        r[n] = (int32_t)row; c[n] = (int32_t)col; ++n;
    }
    if (trials_out) *trials_out = trials;
    int st = oracle_build(O, I, nnz, r, c, NULL, rows_out, cols_out, NULL,
                          NULL, row_offsets_out, NULL, NULL, NULL, NULL);
    free(seen); free(r); free(c);
    return st;
}

int oracle_topology(int64_t O, int64_t I, int64_t nnz,
                    const int32_t *rows, const int32_t *cols, const float *vals,
                    int64_t n_prune, uint64_t seed,
                    int32_t *rows_out, int32_t *cols_out, float *vals_out,
                    int32_t *row_offsets_out, int32_t *pruned_out, int64_t *trials_out)
{
    if (O <= 0 || I <= 0 || nnz < 0 || n_prune < 0 || n_prune > nnz || nnz > O * I) return OR_SHAPE;
    if (nnz > 0 && (!rows || !cols || !vals || !rows_out || !cols_out || !vals_out)) return OR_NULL;
    for (int64_t k = 0; k < nnz; ++k)
        if (rows[k] < 0 || rows[k] >= O || cols[k] < 0 || cols[k] >= I) return OR_INDEX;

    magkey_t *m = (magkey_t *)malloc(sizeof(magkey_t) * (size_t)(nnz > 0 ? nnz : 1));
    unsigned char *live = (unsigned char *)calloc((size_t)(O * I), 1);
    char *gone = (char *)calloc((size_t)(nnz > 0 ? nnz : 1), 1);
    int32_t *r2 = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
    int32_t *c2 = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
    float *v2 = (float *)malloc(sizeof(float) * (size_t)(nnz > 0 ? nnz : 1));
    if (!m || !live || !gone || !r2 || !c2 || !v2) {
        free(m); free(live); free(gone); free(r2); free(c2); free(v2);
        return OR_NOMEM;
    }
    for (int64_t k = 0; k < nnz; ++k) { m[k].mag = fabsf(vals[k]); m[k].k = k; }
    qsort(m, (size_t)nnz, sizeof(magkey_t), cmp_mag);
    for (int64_t q = 0; q < n_prune; ++q) gone[m[q].k] = 1;
    if (pruned_out) {
        int64_t at = 0;
        for (int64_t k = 0; k < nnz; ++k) if (gone[k]) pruned_out[at++] = (int32_t)k;
    }
    /* S = survivors; collect them first */
    int64_t n2 = 0;
    for (int64_t k = 0; k < nnz; ++k) {
        if (gone[k]) continue;
        live[(int64_t)rows[k] * I + cols[k]] = 1;
        r2[n2] = rows[k]; c2[n2] = cols[k]; v2[n2] = vals[k]; ++n2;
    }
    /* Algorithm 2 over the pruned count */
    uint64_t state = seed;
    int64_t trials = 0;
    while (n2 < nnz) {
        int64_t i = getrand(&state, O);
        int64_t j = getrand(&state, I);
        ++trials;
        if (live[i * I + j]) continue;
        live[i * I + j] = 1;
        r2[n2] = (int32_t)i; c2[n2] = (int32_t)j; v2[n2] = 0.0f; ++n2;
    }
    if (trials_out) *trials_out = trials;
    int st = oracle_build(O, I, nnz, r2, c2, v2, rows_out, cols_out, vals_out,
                          NULL, row_offsets_out, NULL, NULL, NULL, NULL);
    free(m); free(live); free(gone); free(r2); free(c2); free(v2);
    return st;
}
