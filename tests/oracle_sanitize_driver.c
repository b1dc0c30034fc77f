/*
 * oracle_sanitize_driver.c -- drives every entry point of oracle/snack_oracle.c
 * on small inputs (including the degenerate ones: no entries, one row, one
 * column, a full matrix, n_drop = 0 and n_drop = nnz, ties, +-0 and NaN) so
 * that a build with AddressSanitizer and UndefinedBehaviorSanitizer checks the
 * oracle's memory accesses and integer arithmetic.  Test infrastructure only:
 * tests/test_oracle_sanitize.py compiles it together with the oracle and runs
 * it; exit status 0 means every call returned and no sanitizer fired.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_canonicalize(int32_t M, int32_t K, int64_t nnz, const int32_t* rows, const int32_t* cols,
                        const float* vals, int32_t* c_rows, int32_t* c_cols, float* c_vals, int32_t* row_ptr,
                        int32_t* perm, int32_t* rows_t, int32_t* col_ptr);
void oracle_forward(int32_t M, int32_t K, int64_t nnz, const int32_t* rows, const int32_t* cols, const float* vals,
                    int32_t B, const float* X, double* Y, double* Yabs);
void oracle_backward_dx(int32_t M, int32_t K, int64_t nnz, const int32_t* rows, const int32_t* cols,
                        const float* vals, int32_t B, const float* dY, double* dX, double* dXabs);
void oracle_backward_dw(int32_t M, int32_t K, int64_t nnz, const int32_t* rows, const int32_t* cols, int32_t B,
                        const float* X, const float* dY, double* dW, double* dWabs);
void oracle_mse_grad(int64_t n, const float* Y, const float* T, double* dY);
void oracle_gelu_fwd(int64_t n, const float* X, double* Y);
void oracle_gelu_bwd(int64_t n, const float* X, const float* dY, double* dX);
void oracle_sgd(int64_t n, const float* v, const float* g, double lr, double* out);
uint64_t oracle_regrow_candidate(uint64_t seed, uint64_t epoch, uint64_t t, uint64_t N);
float oracle_round_bf16(float x);
uint32_t oracle_grow_key(int32_t M, int32_t K, int32_t B, const float* X, const float* dY, int32_t r, int32_t c);
int oracle_prune_regrow_grad(int32_t M, int32_t K, int64_t nnz, const int32_t* rows, const int32_t* cols,
                             const float* vals, int64_t n_drop, int32_t B, const float* X, const float* dY,
                             int32_t* o_rows, int32_t* o_cols, float* o_vals);
int oracle_prune_regrow_rows(int32_t M, int32_t K, int64_t nnz, const int32_t* rows, const int32_t* cols,
                             const float* vals, int64_t num, int64_t den, int mode, uint64_t seed, uint64_t epoch,
                             int32_t B, const float* X, const float* dY, int32_t* o_rows, int32_t* o_cols,
                             float* o_vals);
int32_t oracle_row_candidate(uint64_t seed, uint64_t epoch, int32_t row, uint64_t t, int32_t K);
int oracle_prune_regrow(int32_t M, int32_t K, int64_t nnz, const int32_t* rows, const int32_t* cols,
                        const float* vals, int64_t n_drop, uint64_t seed, uint64_t epoch, int32_t* o_rows,
                        int32_t* o_cols, float* o_vals, uint64_t* candidates_used);

static uint64_t rng_state = 12345;
static uint64_t next_u64(void)
{
    /* xorshift64: only a source of test data */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}
static float next_f(void) { return (float)((double)(next_u64() >> 11) / 9007199254740992.0 * 2.0 - 1.0); }

/* exact-size heap copies, so any read past the end is an ASan report */
static void* dup_exact(const void* src, size_t bytes)
{
    void* p = malloc(bytes ? bytes : 1);
    if (bytes) memcpy(p, src, bytes);
    return p;
}

static int run_case(int32_t M, int32_t K, int64_t nnz, int32_t B, int special)
{
    const int64_t N = (int64_t)M * K;
    /* distinct positions: a shuffled prefix of all cells */
    int64_t* cells = malloc(sizeof(int64_t) * (size_t)N);
    for (int64_t i = 0; i < N; ++i) cells[i] = i;
    for (int64_t i = N - 1; i > 0; --i) {
        const int64_t j = (int64_t)(next_u64() % (uint64_t)(i + 1));
        const int64_t t = cells[i];
        cells[i] = cells[j];
        cells[j] = t;
    }
    int32_t* rows = malloc(sizeof(int32_t) * (size_t)(nnz ? nnz : 1));
    int32_t* cols = malloc(sizeof(int32_t) * (size_t)(nnz ? nnz : 1));
    float* vals = malloc(sizeof(float) * (size_t)(nnz ? nnz : 1));
    for (int64_t k = 0; k < nnz; ++k) {
        rows[k] = (int32_t)(cells[k] / K);
        cols[k] = (int32_t)(cells[k] % K);
        vals[k] = next_f();
        if (special && k % 5 == 0) vals[k] = 0.25f;            /* ties */
        if (special && k % 7 == 1) vals[k] = -0.0f;            /* -0 ties +0 */
        if (special && k % 11 == 2) vals[k] = nanf("");        /* NaN sorts last */
    }
    free(cells);
    int32_t* r = dup_exact(rows, sizeof(int32_t) * (size_t)nnz);
    int32_t* c = dup_exact(cols, sizeof(int32_t) * (size_t)nnz);
    float* v = dup_exact(vals, sizeof(float) * (size_t)nnz);
    free(rows);
    free(cols);
    free(vals);

    int32_t* cr = malloc(sizeof(int32_t) * (size_t)(nnz ? nnz : 1));
    int32_t* cc = malloc(sizeof(int32_t) * (size_t)(nnz ? nnz : 1));
    float* cv = malloc(sizeof(float) * (size_t)(nnz ? nnz : 1));
    int32_t* rp = malloc(sizeof(int32_t) * (size_t)(M + 1));
    int32_t* pm = malloc(sizeof(int32_t) * (size_t)(nnz ? nnz : 1));
    int32_t* rt = malloc(sizeof(int32_t) * (size_t)(nnz ? nnz : 1));
    int32_t* cp = malloc(sizeof(int32_t) * (size_t)(K + 1));
    if (oracle_canonicalize(M, K, nnz, r, c, v, cr, cc, cv, rp, pm, rt, cp) != 0) return 1;

    float* X = malloc(sizeof(float) * (size_t)B * K);
    float* dY = malloc(sizeof(float) * (size_t)B * M);
    for (int64_t i = 0; i < (int64_t)B * K; ++i) X[i] = next_f();
    for (int64_t i = 0; i < (int64_t)B * M; ++i) dY[i] = next_f();
    double* Y = malloc(sizeof(double) * (size_t)B * M);
    double* Ya = malloc(sizeof(double) * (size_t)B * M);
    double* dX = malloc(sizeof(double) * (size_t)B * K);
    double* dXa = malloc(sizeof(double) * (size_t)B * K);
    double* dW = malloc(sizeof(double) * (size_t)(nnz ? nnz : 1));
    double* dWa = malloc(sizeof(double) * (size_t)(nnz ? nnz : 1));
    oracle_forward(M, K, nnz, cr, cc, cv, B, X, Y, Ya);
    oracle_forward(M, K, nnz, cr, cc, cv, B, X, Y, NULL);
    oracle_backward_dx(M, K, nnz, cr, cc, cv, B, dY, dX, dXa);
    oracle_backward_dw(M, K, nnz, cr, cc, B, X, dY, dW, dWa);

    float* Yf = malloc(sizeof(float) * (size_t)B * M);
    for (int64_t i = 0; i < (int64_t)B * M; ++i) Yf[i] = (float)Y[i];
    double* g = malloc(sizeof(double) * (size_t)B * M);
    oracle_mse_grad((int64_t)B * M, Yf, dY, g);
    oracle_gelu_fwd((int64_t)B * M, Yf, g);
    oracle_gelu_bwd((int64_t)B * M, Yf, dY, g);
    float* dWf = malloc(sizeof(float) * (size_t)(nnz ? nnz : 1));
    for (int64_t k = 0; k < nnz; ++k) dWf[k] = (float)dW[k];
    double* sv = malloc(sizeof(double) * (size_t)(nnz ? nnz : 1));
    oracle_sgd(nnz, cv, dWf, 0.01, sv);

    const int64_t drops[3] = {0, nnz * 3 / 10, nnz};
    for (int d = 0; d < 3; ++d) {
        /* growing needs that many empty cells after the drop: always true, since the dropped cells are empty */
        int32_t* orow = malloc(sizeof(int32_t) * (size_t)(nnz ? nnz : 1));
        int32_t* ocol = malloc(sizeof(int32_t) * (size_t)(nnz ? nnz : 1));
        float* oval = malloc(sizeof(float) * (size_t)(nnz ? nnz : 1));
        uint64_t used = 0;
        if (oracle_prune_regrow(M, K, nnz, cr, cc, cv, drops[d], 99, (uint64_t)d, orow, ocol, oval, &used) != 0)
            return 2;
        if (oracle_prune_regrow_grad(M, K, nnz, cr, cc, cv, drops[d], B, X, dY, orow, ocol, oval) != 0) return 5;
        /* row-local: the same three fractions of every row (0, 3/10, all) */
        const int64_t num = d == 0 ? 0 : (d == 1 ? 3 : 1), den = d == 1 ? 10 : 1;
        if (oracle_prune_regrow_rows(M, K, nnz, cr, cc, cv, num, den, 0, 99, (uint64_t)d, 0, NULL, NULL, orow, ocol,
                                     oval) != 0)
            return 6;
        if (oracle_prune_regrow_rows(M, K, nnz, cr, cc, cv, num, den, 1, 0, 0, B, X, dY, orow, ocol, oval) != 0)
            return 7;
        free(orow);
        free(ocol);
        free(oval);
    }
    (void)oracle_regrow_candidate(~0ULL, (1ULL << 23) - 1, (1ULL << 40) - 1, (uint64_t)N);
    (void)oracle_grow_key(M, K, B, X, dY, M - 1, K - 1);
    (void)oracle_row_candidate(~0ULL, 0xFFFFFFFFULL, M - 1, (uint64_t)64 * K + 4095, K);
    for (int64_t k = 0; k < nnz; ++k) (void)oracle_round_bf16(cv[k]);
    (void)oracle_round_bf16(3.4028235e38f);
    (void)oracle_round_bf16(1e-45f);

    free(r); free(c); free(v); free(cr); free(cc); free(cv); free(rp); free(pm); free(rt); free(cp);
    free(X); free(dY); free(Y); free(Ya); free(dX); free(dXa); free(dW); free(dWa); free(Yf); free(g);
    free(dWf); free(sv);
    return 0;
}

int main(void)
{
    /* (M, K, nnz, B, special values) */
    const int64_t cases[][5] = {
        {1, 1, 0, 1, 0},   {1, 1, 1, 1, 0},    {1, 9, 5, 3, 1},    {9, 1, 5, 2, 1},   {6, 5, 30, 4, 1},
        {6, 5, 12, 1, 1},  {17, 23, 97, 5, 1}, {40, 33, 660, 7, 0}, {64, 64, 4096, 2, 1}, {3, 200, 37, 9, 0},
    };
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
        const int rc = run_case((int32_t)cases[i][0], (int32_t)cases[i][1], cases[i][2], (int32_t)cases[i][3],
                                (int)cases[i][4]);
        if (rc != 0) {
            fprintf(stderr, "case %zu failed with %d\n", i, rc);
            return rc;
        }
    }
    /* bad input: range and duplicate errors return without touching outputs past nnz */
    {
        const int32_t r[2] = {0, 3}, c[2] = {0, 0};
        const float v[2] = {1, 1};
        if (oracle_canonicalize(3, 3, 2, r, c, v, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != 2) return 3;
        const int32_t r2[2] = {1, 1}, c2[2] = {2, 2};
        if (oracle_canonicalize(3, 3, 2, r2, c2, v, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != 3) return 4;
    }
    printf("oracle sanitize driver: all cases ran\n");
    return 0;
}
