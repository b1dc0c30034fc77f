/*
 * snack_oracle.c -- plain, slow, fp64 CPU oracle for the truly sparse COO layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header, table or helper with the HIP
 * path.
 *
 * Sources (cited by page title and section):
 *   [SNACK]  "Beyond Masked Sparsity: SNACK Enables Truly Sparse Neural Networks
 *            on GPU" -- abstract and Figure 1 (weight stored as the COO triple of
 *            values, rows, cols over the non-zeros; the layer is a drop-in
 *            nn.Linear; backward is a sparse outer product over supp(W); DST adds
 *            and drops connections in place); Table 7 (COO / CSR / CSC).
 *   [PCSR]   "Padded-CSR: a sparse storage format for dynamic sparse training on
 *            CPU" -- section 3.2 (sorted COO + row pointer), section 4.1 (CSR),
 *            section 4.3 (DST drops a fraction and grows the same number),
 *            section 6.1 (scalar SpMM loop), section 7.1 (the two gradients and
 *            dW at live slots), section 7.2 (transpose with a permutation map).
 *   SplitMix64: Steele, Lea & Flood, "Fast splittable pseudorandom number
 *            generators" (OOPSLA 2014); output function as in Vigna's public
 *            reference splitmix64.c.
 *
 * Conventions: the layer is nn.Linear-shaped.  W is [M, K] (out, in); X is
 * [B, K], Y and dY are [B, M], dX is [B, K], all row-major fp32 on input.  All
 * arithmetic below is in double.  Every function that produces a floating
 * value also produces the matching sum of absolute terms, which the tests use
 * for the per-element tolerance |got - ref| <= 1e-5 * abs_sum + 1e-6.
 *
 * Parity status of each function: all are pinned by tests (worked examples from
 * the pages, dense brute force, adjoint identity, finite differences,
 * enumeration) except the regrow candidate *stream*, whose choice of generator
 * the pages leave open; its generator is pinned to SplitMix64's published
 * outputs and its positions to a chi-square uniformity test.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
    OR_OK = 0,
    OR_INVALID = 1,
    OR_RANGE = 2,
    OR_DUPLICATE = 3,
    OR_NOMEM = 4
};

/* ------------------------------------------------------------------------- */
/* Canonical order.  [PCSR 3.2]: entries sorted by row, then by column; the   */
/* row pointer has nrows+1 entries and row i owns [row_ptr[i], row_ptr[i+1]). */
/* [PCSR 7.2] / [SNACK Table 7]: the transposed (CSC) view lists the same     */
/* entries sorted by column then row; perm[j] is the canonical slot whose     */
/* value sits at transposed slot j.                                          */
/* ------------------------------------------------------------------------- */

typedef struct {
    int64_t key;
    int64_t slot;
} keyed_t;

static int cmp_keyed(const void* a, const void* b)
{
    const keyed_t* x = (const keyed_t*)a;
    const keyed_t* y = (const keyed_t*)b;
    if (x->key < y->key) return -1;
    if (x->key > y->key) return 1;
    if (x->slot < y->slot) return -1;
    if (x->slot > y->slot) return 1;
    return 0;
}

/*
 * Sort an arbitrary-order COO triple into canonical order and build the row
 * pointer and the transposed index.  Positions must be distinct: the support
 * of W is a set.  Returns OR_RANGE for an index outside the matrix and
 * OR_DUPLICATE when two entries name one position (range is checked first).
 * Any output pointer may be NULL if that output is not wanted.
 */
int oracle_canonicalize(int32_t M, int32_t K, int64_t nnz,
                        const int32_t* rows, const int32_t* cols, const float* vals,
                        int32_t* c_rows, int32_t* c_cols, float* c_vals,
                        int32_t* row_ptr, int32_t* perm, int32_t* rows_t,
                        int32_t* col_ptr)
{
    if (M < 0 || K < 0 || nnz < 0) return OR_INVALID;
    if (nnz > 0 && (rows == NULL || cols == NULL)) return OR_INVALID;
    for (int64_t k = 0; k < nnz; ++k) {
        if (rows[k] < 0 || rows[k] >= M || cols[k] < 0 || cols[k] >= K) return OR_RANGE;
    }
    keyed_t* a = (keyed_t*)malloc(sizeof(keyed_t) * (size_t)(nnz > 0 ? nnz : 1));
    if (!a) return OR_NOMEM;
    for (int64_t k = 0; k < nnz; ++k) {
        a[k].key = (int64_t)rows[k] * (int64_t)K + (int64_t)cols[k];
        a[k].slot = k;
    }
    qsort(a, (size_t)nnz, sizeof(keyed_t), cmp_keyed);
    for (int64_t k = 1; k < nnz; ++k) {
        if (a[k].key == a[k - 1].key) {
            free(a);
            return OR_DUPLICATE;
        }
    }
    int32_t* tmp_rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
    int32_t* tmp_cols = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
    if (!tmp_rows || !tmp_cols) {
        free(a); free(tmp_rows); free(tmp_cols);
        return OR_NOMEM;
    }
    for (int64_t k = 0; k < nnz; ++k) {
        int64_t s = a[k].slot;
        tmp_rows[k] = rows[s];
        tmp_cols[k] = cols[s];
        if (c_vals) c_vals[k] = vals ? vals[s] : 0.0f;
    }
    if (c_rows) memcpy(c_rows, tmp_rows, sizeof(int32_t) * (size_t)nnz);
    if (c_cols) memcpy(c_cols, tmp_cols, sizeof(int32_t) * (size_t)nnz);

    /* Row pointer by counting, then a running sum. */
    if (row_ptr) {
        for (int32_t i = 0; i <= M; ++i) row_ptr[i] = 0;
        for (int64_t k = 0; k < nnz; ++k) row_ptr[tmp_rows[k] + 1] += 1;
        for (int32_t i = 0; i < M; ++i) row_ptr[i + 1] += row_ptr[i];
    }

    /* Transposed view: canonical slots re-sorted by (col, row). */
    for (int64_t k = 0; k < nnz; ++k) {
        a[k].key = (int64_t)tmp_cols[k] * (int64_t)M + (int64_t)tmp_rows[k];
        a[k].slot = k;
    }
    qsort(a, (size_t)nnz, sizeof(keyed_t), cmp_keyed);
    for (int64_t j = 0; j < nnz; ++j) {
        if (perm) perm[j] = (int32_t)a[j].slot;
        if (rows_t) rows_t[j] = tmp_rows[a[j].slot];
    }
    if (col_ptr) {
        for (int32_t c = 0; c <= K; ++c) col_ptr[c] = 0;
        for (int64_t k = 0; k < nnz; ++k) col_ptr[tmp_cols[k] + 1] += 1;
        for (int32_t c = 0; c < K; ++c) col_ptr[c + 1] += col_ptr[c];
    }
    free(a); free(tmp_rows); free(tmp_cols);
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* Forward.  [SNACK Fig. 1]: the block replaces nn.Linear, so Y = X W^T.      */
/* [PCSR 6.1]: for each live entry (row i, col c, value v) the output row    */
/* gains v times the matching input entry -- here written over slots k and   */
/* batch rows b:  Y[b, r_k] += v_k * X[b, c_k].  Rows with no entry stay 0.  */
/* ------------------------------------------------------------------------- */
void oracle_forward(int32_t M, int32_t K, int64_t nnz,
                    const int32_t* rows, const int32_t* cols, const float* vals,
                    int32_t B, const float* X, double* Y, double* Yabs)
{
    for (int64_t e = 0; e < (int64_t)B * M; ++e) {
        Y[e] = 0.0;
        if (Yabs) Yabs[e] = 0.0;
    }
    for (int64_t k = 0; k < nnz; ++k) {
        const int64_t r = rows[k], c = cols[k];
        const double v = (double)vals[k];
        for (int64_t b = 0; b < B; ++b) {
            const double x = (double)X[b * K + c];
            Y[b * M + r] += v * x;
            if (Yabs) Yabs[b * M + r] += fabs(v * x);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Input gradient.  [PCSR 7.1]: dL/dX = W^T dL/dY, an SpMM with the          */
/* transpose; in the nn.Linear layout  dX[b, c_k] += v_k * dY[b, r_k].       */
/* Columns with no entry get 0.                                              */
/* ------------------------------------------------------------------------- */
void oracle_backward_dx(int32_t M, int32_t K, int64_t nnz,
                        const int32_t* rows, const int32_t* cols, const float* vals,
                        int32_t B, const float* dY, double* dX, double* dXabs)
{
    for (int64_t e = 0; e < (int64_t)B * K; ++e) {
        dX[e] = 0.0;
        if (dXabs) dXabs[e] = 0.0;
    }
    for (int64_t k = 0; k < nnz; ++k) {
        const int64_t r = rows[k], c = cols[k];
        const double v = (double)vals[k];
        for (int64_t b = 0; b < B; ++b) {
            const double g = (double)dY[b * M + r];
            dX[b * K + c] += v * g;
            if (dXabs) dXabs[b * K + c] += fabs(v * g);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Weight gradient on the support only.  [PCSR 7.1]: for a live slot at      */
/* (i, c) the gradient is the dot product of the output-gradient row i with  */
/* the input row c over the batch; [SNACK Fig. 1] calls this the sparse      */
/* outer product over supp(W).  Stored zeros still get a gradient.           */
/* ------------------------------------------------------------------------- */
void oracle_backward_dw(int32_t M, int32_t K, int64_t nnz,
                        const int32_t* rows, const int32_t* cols,
                        int32_t B, const float* X, const float* dY,
                        double* dW, double* dWabs)
{
    for (int64_t k = 0; k < nnz; ++k) {
        const int64_t r = rows[k], c = cols[k];
        double s = 0.0, a = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            const double t = (double)dY[b * M + r] * (double)X[b * K + c];
            s += t;
            a += fabs(t);
        }
        dW[k] = s;
        if (dWabs) dWabs[k] = a;
    }
}

/* ------------------------------------------------------------------------- */
/* Training-loop glue (not part of the sparse method itself).               */
/* MSE with mean reduction over n elements: dL/dY = 2 (Y - T) / n.           */
/* Exact GELU: 0.5 x (1 + erf(x / sqrt 2)); derivative Phi(x) + x phi(x).    */
/* SGD: v <- v - lr * g.                                                      */
/* ------------------------------------------------------------------------- */
void oracle_mse_grad(int64_t n, const float* Y, const float* T, double* dY)
{
    for (int64_t e = 0; e < n; ++e) dY[e] = 2.0 * ((double)Y[e] - (double)T[e]) / (double)n;
}

void oracle_gelu_fwd(int64_t n, const float* X, double* Y)
{
    for (int64_t e = 0; e < n; ++e) {
        const double x = (double)X[e];
        Y[e] = 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
    }
}

void oracle_gelu_bwd(int64_t n, const float* X, const float* dY, double* dX)
{
    const double inv_sqrt2pi = 1.0 / sqrt(2.0 * 3.14159265358979323846);
    for (int64_t e = 0; e < n; ++e) {
        const double x = (double)X[e];
        const double cdf = 0.5 * (1.0 + erf(x / sqrt(2.0)));
        const double pdf = inv_sqrt2pi * exp(-0.5 * x * x);
        dX[e] = (double)dY[e] * (cdf + x * pdf);
    }
}

void oracle_sgd(int64_t n, const float* v, const float* g, double lr, double* out)
{
    for (int64_t e = 0; e < n; ++e) out[e] = (double)v[e] - lr * (double)g[e];
}

/* ------------------------------------------------------------------------- */
/* SplitMix64 (Steele, Lea & Flood 2014): the state advances by the golden   */
/* gamma 0x9E3779B97F4A7C15 and each state is passed through the published   */
/* output mix (xor-shift 30, multiply, xor-shift 27, multiply, xor-shift 31).*/
/* ------------------------------------------------------------------------- */
uint64_t oracle_splitmix64_mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Candidate t of the regrow stream of epoch e: the SplitMix64 output number */
/* (e * 2^40 + t) of the generator seeded with `seed`, mapped onto [0, N)    */
/* by the high word of the 64x64-bit product (Lemire's multiply-shift).      */
uint64_t oracle_regrow_candidate(uint64_t seed, uint64_t epoch, uint64_t t, uint64_t N)
{
    const uint64_t gamma = 0x9E3779B97F4A7C15ULL;
    const uint64_t x = seed + ((epoch << 40) + t + 1ULL) * gamma;
    const uint64_t u = oracle_splitmix64_mix(x);
    return (uint64_t)(((unsigned __int128)u * (unsigned __int128)N) >> 64);
}

/* ------------------------------------------------------------------------- */
/* Drop / regrow with nnz fixed.  [PCSR 4.3]: a DST update drops some live   */
/* entries and grows the same number elsewhere; [SNACK Fig. 1]: in place on  */
/* the triple.  SET-style rule: drop the n_drop entries of smallest |v|      */
/* (ties broken by canonical slot; the order key is the IEEE bit pattern of  */
/* |v|, so -0 ties +0 and NaN sorts after +inf), then grow n_drop positions  */
/* drawn uniformly at random among the positions that are empty after the   */
/* drop: walk the candidate stream t = 0, 1, 2, ... and accept a candidate   */
/* when its position is neither kept nor already accepted.  Grown entries    */
/* hold +0.0.  Input: canonical triple; output: the new canonical triple.    */
/* ------------------------------------------------------------------------- */
typedef struct {
    uint32_t mag;
    int64_t slot;
} dropkey_t;

static int cmp_dropkey(const void* a, const void* b)
{
    const dropkey_t* x = (const dropkey_t*)a;
    const dropkey_t* y = (const dropkey_t*)b;
    if (x->mag < y->mag) return -1;
    if (x->mag > y->mag) return 1;
    if (x->slot < y->slot) return -1;
    if (x->slot > y->slot) return 1;
    return 0;
}

static int cmp_i64(const void* a, const void* b)
{
    const int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

int oracle_prune_regrow(int32_t M, int32_t K, int64_t nnz,
                        const int32_t* rows, const int32_t* cols, const float* vals,
                        int64_t n_drop, uint64_t seed, uint64_t epoch,
                        int32_t* o_rows, int32_t* o_cols, float* o_vals,
                        uint64_t* candidates_used)
{
    if (n_drop < 0 || n_drop > nnz) return OR_INVALID;
    const uint64_t N = (uint64_t)M * (uint64_t)K;
    const size_t n1 = (size_t)(nnz > 0 ? nnz : 1);
    dropkey_t* d = (dropkey_t*)malloc(sizeof(dropkey_t) * n1);
    unsigned char* dropped = (unsigned char*)calloc(n1, 1);
    /* one bit per matrix position: set when the position is occupied */
    unsigned char* occ = (unsigned char*)calloc((size_t)(N / 8 + 1), 1);
    int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * n1);
    float* pv = (float*)malloc(sizeof(float) * n1);
    if (!d || !dropped || !occ || !pos || !pv) {
        free(d); free(dropped); free(occ); free(pos); free(pv);
        return OR_NOMEM;
    }
    for (int64_t k = 0; k < nnz; ++k) {
        float a = fabsf(vals[k]);
        uint32_t bits;
        memcpy(&bits, &a, sizeof bits);
        d[k].mag = bits;
        d[k].slot = k;
    }
    qsort(d, (size_t)nnz, sizeof(dropkey_t), cmp_dropkey);
    for (int64_t i = 0; i < n_drop; ++i) dropped[d[i].slot] = 1;

    /* kept entries, in their canonical order */
    int64_t m = 0;
    for (int64_t k = 0; k < nnz; ++k) {
        if (dropped[k]) continue;
        const int64_t p = (int64_t)rows[k] * K + cols[k];
        occ[p >> 3] |= (unsigned char)(1u << (p & 7));
        pos[m] = p;
        pv[m] = vals[k];
        ++m;
    }
    /* grow */
    int64_t* grown = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_drop > 0 ? n_drop : 1));
    if (!grown) {
        free(d); free(dropped); free(occ); free(pos); free(pv);
        return OR_NOMEM;
    }
    int64_t g = 0;
    uint64_t t = 0;
    while (g < n_drop) {
        const uint64_t p = oracle_regrow_candidate(seed, epoch, t, N);
        ++t;
        if (occ[p >> 3] & (1u << (p & 7))) continue;
        occ[p >> 3] |= (unsigned char)(1u << (p & 7));
        grown[g++] = (int64_t)p;
    }
    if (candidates_used) *candidates_used = t;
    qsort(grown, (size_t)n_drop, sizeof(int64_t), cmp_i64);

    /* merge the two position-sorted lists */
    int64_t i = 0, j = 0, o = 0;
    while (i < m || j < n_drop) {
        int take_kept;
        if (i >= m) take_kept = 0;
        else if (j >= n_drop) take_kept = 1;
        else take_kept = pos[i] < grown[j];
        const int64_t p = take_kept ? pos[i] : grown[j];
        o_rows[o] = (int32_t)(p / K);
        o_cols[o] = (int32_t)(p % K);
        o_vals[o] = take_kept ? pv[i] : 0.0f;
        if (take_kept) ++i; else ++j;
        ++o;
    }
    free(d); free(dropped); free(occ); free(pos); free(pv); free(grown);
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* Drop / regrow with the regrow at high-gradient cells (RigL-style).        */
/* [PCSR 4.3]: a RigL update drops a fraction of the live entries and grows   */
/* the same number "at high-gradient locations"; [SNACK Tables 8-9] run RigL  */
/* on the truly sparse layer.  Drop: exactly as oracle_prune_regrow (the      */
/* n_drop smallest |v|, ties by slot).  Grow: among the cells empty after the */
/* drop, the n_drop cells with the largest |dL/dW[r, c]|, where dL/dW[r, c] = */
/* sum over b of dY[b, r] X[b, c] is the dense weight gradient of the layer   */
/* at that cell for the batch (X, dY) ([PCSR 7.1]: the gradient of W is       */
/* dY^T X; on the support it is the sampled product).  The decision is taken */
/* on the fp32 value of that sum accumulated in batch order with a fused      */
/* multiply-add per term (the precision the layer computes in), so both sides */
/* rank the same numbers; the order key is the IEEE bits of |g| (a NaN counts */
/* as 0), larger first, ties by smaller linear position r*K + c.  Grown       */
/* entries hold +0.0.                                                         */
/* ------------------------------------------------------------------------- */
typedef struct {
    uint32_t key;
    int64_t pos;
} growkey_t;

static int cmp_growkey(const void* a, const void* b)
{
    const growkey_t* x = (const growkey_t*)a;
    const growkey_t* y = (const growkey_t*)b;
    if (x->key > y->key) return -1;   /* larger score first */
    if (x->key < y->key) return 1;
    if (x->pos < y->pos) return -1;   /* then smaller position */
    if (x->pos > y->pos) return 1;
    return 0;
}

/* the grow score key of cell (r, c): IEEE bits of |sum_b dY[b, r] X[b, c]| */
uint32_t oracle_grow_key(int32_t M, int32_t K, int32_t B, const float* X, const float* dY, int32_t r, int32_t c)
{
    float g = 0.0f;
    for (int32_t b = 0; b < B; ++b) g = fmaf(dY[(int64_t)b * M + r], X[(int64_t)b * K + c], g);
    if (isnan(g)) return 0u;
    const float a = fabsf(g);
    uint32_t bits;
    memcpy(&bits, &a, sizeof bits);
    return bits;
}

int oracle_prune_regrow_grad(int32_t M, int32_t K, int64_t nnz,
                             const int32_t* rows, const int32_t* cols, const float* vals,
                             int64_t n_drop, int32_t B, const float* X, const float* dY,
                             int32_t* o_rows, int32_t* o_cols, float* o_vals)
{
    if (n_drop < 0 || n_drop > nnz || B < 1) return OR_INVALID;
    const uint64_t N = (uint64_t)M * (uint64_t)K;
    const size_t n1 = (size_t)(nnz > 0 ? nnz : 1);
    dropkey_t* d = (dropkey_t*)malloc(sizeof(dropkey_t) * n1);
    unsigned char* dropped = (unsigned char*)calloc(n1, 1);
    unsigned char* occ = (unsigned char*)calloc((size_t)(N / 8 + 1), 1);
    int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * n1);
    float* pv = (float*)malloc(sizeof(float) * n1);
    const uint64_t nempty = N - (uint64_t)(nnz - n_drop);
    growkey_t* cand = (growkey_t*)malloc(sizeof(growkey_t) * (size_t)(nempty > 0 ? nempty : 1));
    if (!d || !dropped || !occ || !pos || !pv || !cand) {
        free(d); free(dropped); free(occ); free(pos); free(pv); free(cand);
        return OR_NOMEM;
    }
    /* drop: the same total order as the SET-style update */
    for (int64_t k = 0; k < nnz; ++k) {
        float a = fabsf(vals[k]);
        uint32_t bits;
        memcpy(&bits, &a, sizeof bits);
        d[k].mag = bits;
        d[k].slot = k;
    }
    qsort(d, (size_t)nnz, sizeof(dropkey_t), cmp_dropkey);
    for (int64_t i = 0; i < n_drop; ++i) dropped[d[i].slot] = 1;
    int64_t m = 0;
    for (int64_t k = 0; k < nnz; ++k) {
        if (dropped[k]) continue;
        const int64_t p = (int64_t)rows[k] * K + cols[k];
        occ[p >> 3] |= (unsigned char)(1u << (p & 7));
        pos[m] = p;
        pv[m] = vals[k];
        ++m;
    }
    /* grow: every empty cell with its score, best n_drop first */
    uint64_t e = 0;
    for (uint64_t p = 0; p < N; ++p) {
        if (occ[p >> 3] & (1u << (p & 7))) continue;
        cand[e].key = oracle_grow_key(M, K, B, X, dY, (int32_t)(p / (uint64_t)K), (int32_t)(p % (uint64_t)K));
        cand[e].pos = (int64_t)p;
        ++e;
    }
    qsort(cand, (size_t)e, sizeof(growkey_t), cmp_growkey);
    int64_t* grown = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_drop > 0 ? n_drop : 1));
    if (!grown) {
        free(d); free(dropped); free(occ); free(pos); free(pv); free(cand);
        return OR_NOMEM;
    }
    for (int64_t g = 0; g < n_drop; ++g) grown[g] = cand[g].pos;
    qsort(grown, (size_t)n_drop, sizeof(int64_t), cmp_i64);
    /* merge the two position-sorted lists */
    int64_t i = 0, j = 0, o = 0;
    while (i < m || j < n_drop) {
        int take_kept;
        if (i >= m) take_kept = 0;
        else if (j >= n_drop) take_kept = 1;
        else take_kept = pos[i] < grown[j];
        const int64_t p = take_kept ? pos[i] : grown[j];
        o_rows[o] = (int32_t)(p / K);
        o_cols[o] = (int32_t)(p % K);
        o_vals[o] = take_kept ? pv[i] : 0.0f;
        if (take_kept) ++i; else ++j;
        ++o;
    }
    free(d); free(dropped); free(occ); free(pos); free(pv); free(cand); free(grown);
    return OR_OK;
}

/* ------------------------------------------------------------------------- */
/* bf16 rounding of a value for the inference forward with narrower value    */
/* streams ([PCSR 9.3]: narrower index and value encodings).  bf16 keeps 8   */
/* significant bits and fp32's exponent range: a finite x is rounded to the  */
/* nearest multiple of its bf16 spacing, 2^(e-7) for 2^e <= |x| < 2^(e+1)     */
/* (2^-133 below 2^-126), ties to the even multiple; results of magnitude    */
/* 2^128 or more become infinities.  Computed in double, where every step is */
/* exact.                                                                    */
/* ------------------------------------------------------------------------- */
float oracle_round_bf16(float x)
{
    if (isnan(x) || isinf(x) || x == 0.0f) return x;
    const double ax = fabs((double)x);
    int e;
    (void)frexp(ax, &e);             /* ax = m 2^e, 0.5 <= m < 1: 2^(e-1) <= ax < 2^e */
    int lo = e - 1;                  /* the binade's exponent */
    if (lo < -126) lo = -126;        /* subnormal bf16: fixed spacing */
    const double spacing = ldexp(1.0, lo - 7);
    const double q = nearbyint(ax / spacing);    /* default rounding: to nearest, ties to even */
    double r = q * spacing;
    if (r >= ldexp(1.0, 128)) r = INFINITY;
    return (float)(x < 0.0f ? -r : r);
}

/* ------------------------------------------------------------------------- */
/* Row-local drop / regrow: every row keeps its number of entries.  [PCSR    */
/* 8.3]: SparseLab's SET and RigL keep each row's nnz fixed (adaptive-density */
/* variants change it); [PCSR 4.3]: drop a fraction of the live entries and   */
/* grow as many.  Row i with n_i entries drops d_i = floor(n_i * num / den)   */
/* of them -- the smallest |v| in the row, ties by slot -- and grows d_i      */
/* cells of the same row, empty after the row's drop, value +0.0:             */
/*  mode 0 (SET):  candidate t of row i is column high64(u_t * K), u_t the    */
/*                 SplitMix64 output of s_i + (t + 1) * gamma, where s_i =    */
/*                 mix64(seed ^ mix64(epoch * 2^32 + i)); a candidate is      */
/*                 accepted when its column is neither kept nor accepted at   */
/*                 a smaller t; candidates t < 64 K + 4096 are tried, and     */
/*                 grows still missing after them take the smallest empty     */
/*                 columns in order;                                          */
/*  mode 1 (RigL): the d_i empty columns of largest |dY^T X| score (the key   */
/*                 of oracle_grow_key), ties by smaller column.               */
/* ------------------------------------------------------------------------- */
static uint64_t row_stream_base(uint64_t seed, uint64_t epoch, int32_t row)
{
    return oracle_splitmix64_mix(seed ^ oracle_splitmix64_mix((epoch << 32) + (uint64_t)(uint32_t)row));
}

int32_t oracle_row_candidate(uint64_t seed, uint64_t epoch, int32_t row, uint64_t t, int32_t K)
{
    const uint64_t x = row_stream_base(seed, epoch, row) + (t + 1ULL) * 0x9E3779B97F4A7C15ULL;
    const uint64_t u = oracle_splitmix64_mix(x);
    return (int32_t)(((unsigned __int128)u * (unsigned __int128)(uint64_t)K) >> 64);
}

int oracle_prune_regrow_rows(int32_t M, int32_t K, int64_t nnz,
                             const int32_t* rows, const int32_t* cols, const float* vals,
                             int64_t num, int64_t den, int mode, uint64_t seed, uint64_t epoch,
                             int32_t B, const float* X, const float* dY,
                             int32_t* o_rows, int32_t* o_cols, float* o_vals)
{
    if (num < 0 || den < 1 || num > den || (mode != 0 && mode != 1)) return OR_INVALID;
    if (mode == 1 && (B < 1 || !X || !dY)) return OR_INVALID;
    unsigned char* kept = (unsigned char*)malloc((size_t)(K > 0 ? K : 1));
    unsigned char* grown = (unsigned char*)malloc((size_t)(K > 0 ? K : 1));
    dropkey_t* d = (dropkey_t*)malloc(sizeof(dropkey_t) * (size_t)(nnz > 0 ? nnz : 1));
    growkey_t* cand = (growkey_t*)malloc(sizeof(growkey_t) * (size_t)(K > 0 ? K : 1));
    float* kv = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
    if (!kept || !grown || !d || !cand || !kv) {
        free(kept); free(grown); free(d); free(cand); free(kv);
        return OR_NOMEM;
    }
    int64_t p0 = 0, o = 0;
    for (int32_t i = 0; i < M; ++i) {
        int64_t p1 = p0;
        while (p1 < nnz && rows[p1] == i) ++p1;
        const int64_t n = p1 - p0;
        const int64_t drop = n * num / den;
        /* drop: the row's smallest |v|, ties by slot */
        for (int64_t k = 0; k < n; ++k) {
            float a = fabsf(vals[p0 + k]);
            uint32_t bits;
            memcpy(&bits, &a, sizeof bits);
            d[k].mag = bits;
            d[k].slot = p0 + k;
        }
        qsort(d, (size_t)n, sizeof(dropkey_t), cmp_dropkey);
        memset(kept, 0, (size_t)K);
        memset(grown, 0, (size_t)K);
        for (int64_t k = drop; k < n; ++k) {
            kept[cols[d[k].slot]] = 1;
            kv[cols[d[k].slot]] = vals[d[k].slot];
        }
        /* grow inside the row */
        int64_t need = drop;
        if (mode == 0) {
            const uint64_t tmax = 64ULL * (uint64_t)K + 4096ULL;
            for (uint64_t t = 0; t < tmax && need > 0; ++t) {
                const int32_t c = oracle_row_candidate(seed, epoch, i, t, K);
                if (kept[c] || grown[c]) continue;
                grown[c] = 1;
                --need;
            }
            for (int32_t c = 0; c < K && need > 0; ++c) {
                if (kept[c] || grown[c]) continue;
                grown[c] = 1;
                --need;
            }
        } else {
            int64_t e = 0;
            for (int32_t c = 0; c < K; ++c) {
                if (kept[c]) continue;
                cand[e].key = oracle_grow_key(M, K, B, X, dY, i, c);
                cand[e].pos = c;
                ++e;
            }
            qsort(cand, (size_t)e, sizeof(growkey_t), cmp_growkey);
            for (int64_t g = 0; g < need; ++g) grown[cand[g].pos] = 1;
            need = 0;
        }
        /* the row, ascending by column */
        for (int32_t c = 0; c < K; ++c) {
            if (!kept[c] && !grown[c]) continue;
            o_rows[o] = i;
            o_cols[o] = c;
            o_vals[o] = kept[c] ? kv[c] : 0.0f;
            ++o;
        }
        p0 = p1;
    }
    free(kept); free(grown); free(d); free(cand); free(kv);
    return o == nnz ? OR_OK : OR_INVALID;
}
