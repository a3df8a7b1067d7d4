/*
 * oracle.c -- plain fp64 CPU oracle for the fused LoRA linear layer and for the
 * merge of a LoRA adapter into a pristine copy of the base weight.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code, header, table or
 * helper with the GPU library; it is the plain definition, written out.
 *
 * Sources (page titles as published):
 *   "fastaf: Minimal LoRA fine-tuning with hand-written Triton kernels",
 *     section "FWD kernel speedup": the forward of one LoRA layer is
 *     out = X W^T + ((X A^T) B^T) * scale, with scale = alpha / r;
 *     section "BWD kernel speedup": its backward yields dA, dB and dX.
 *   unsloth commit log for scripts/benchmarks/qwen3_flex_inference.py, entry
 *     "Replace the copy+merge_adapter pair ...": the refresh writes
 *     W_inf = pristine + scaling * (B A) in one addmm, accumulated in fp32,
 *     and the pristine copy is never written.
 *
 * Layouts (nn.Linear convention, all row-major, unit inner stride):
 *   X[M,K] tokens x d_in, W[N,K] d_out x d_in, A[r,K], B[N,r], Y[M,N].
 * Element types: ORC_F32 (float) or ORC_BF16 (uint16 bit patterns of bf16).
 * Every input value is widened exactly to double; every sum runs in ascending
 * index order in double; the forward result is not rounded.
 *
 * Pins (tests/test_oracle_pins.py; no function here is left unpinned):
 * oracle_fwd_rows against hand-worked values, a literal quadruple loop on
 * tiny shapes (bitwise), B = 0 / scale = 0 / W = 0 reductions, linearity in
 * the scale, the merged-weight form, exact integer cases and numpy float64;
 * oracle_fwd_entries bitwise against oracle_fwd_rows; oracle_merge_rows
 * against hand-worked values, its special cases and numpy float64;
 * oracle_round_bf16 against torch's float32 -> bf16 conversion and against
 * ties and double-rounding cases; oracle_bwd against the forward through the
 * adjoint identities <dY, Y(X)> = <dX, X> and their A and B counterparts,
 * a literal loop on tiny shapes (bitwise), B = 0 / A = 0 / scale = 0
 * reductions and numpy float64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

enum { ORC_F32 = 0, ORC_BF16 = 1 };

static double widen(int dt, const void *p, int64_t i)
{
    if (dt == ORC_F32)
        return (double)((const float *)p)[i];
    uint32_t u = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Widen rows [r0, r1) of a row-major [rows, cols] matrix into a dense double
 * buffer. */
static void widen_rows(int dt, const void *p, int64_t cols, int64_t r0, int64_t r1,
                       double *out)
{
    for (int64_t i = r0; i < r1; ++i)
        for (int64_t c = 0; c < cols; ++c)
            out[(i - r0) * cols + c] = widen(dt, p, i * cols + c);
}

static int g_threads = 0;

void oracle_set_threads(int n) { g_threads = n; }

int oracle_get_threads(void)
{
    return g_threads > 0 ? g_threads : omp_get_max_threads();
}

/*
 * Forward, rows [m0, m1) of the output, all N columns, into Y[(m - m0) * N + n]:
 *   T[m,j]  = sum_k X[m,k] A[j,k]          (down-projection)
 *   Yb[m,n] = sum_k X[m,k] W[n,k]          (base product)
 *   L[m,n]  = sum_j T[m,j] B[n,j]          (up-projection)
 *   Y[m,n]  = Yb[m,n] + scale * L[m,n]     (scale, then add onto the base)
 * "scale" is the caller's float widened to double.  Returns 0, or -1 when a
 * work buffer cannot be allocated.
 */
int oracle_fwd_rows(int dt, int64_t m0, int64_t m1, int64_t N, int64_t K, int64_t r,
                    const void *X, const void *W, const void *A, const void *B,
                    float scale, double *Y)
{
    if (m1 <= m0 || N <= 0)
        return 0;
    double *Wd = (double *)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
    double *Ad = (double *)malloc(sizeof(double) * (size_t)(r * K > 0 ? r * K : 1));
    double *Bd = (double *)malloc(sizeof(double) * (size_t)(N * r > 0 ? N * r : 1));
    int err = (Wd == NULL || Ad == NULL || Bd == NULL);
    if (!err) {
        widen_rows(dt, W, K, 0, N, Wd);
        widen_rows(dt, A, K, 0, r, Ad);
        widen_rows(dt, B, r, 0, N, Bd);
    }
    const double s = (double)scale;
    if (!err)
#pragma omp parallel num_threads(oracle_get_threads())
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double *t = (double *)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
        if (x == NULL || t == NULL) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t m = m0; m < m1; ++m) {
                widen_rows(dt, X, K, m, m + 1, x);
                for (int64_t j = 0; j < r; ++j) {
                    double acc = 0.0;
                    for (int64_t k = 0; k < K; ++k)
                        acc += x[k] * Ad[j * K + k];
                    t[j] = acc;
                }
                for (int64_t n = 0; n < N; ++n) {
                    double yb = 0.0;
                    for (int64_t k = 0; k < K; ++k)
                        yb += x[k] * Wd[n * K + k];
                    double l = 0.0;
                    for (int64_t j = 0; j < r; ++j)
                        l += t[j] * Bd[n * r + j];
                    Y[(m - m0) * N + n] = yb + s * l;
                }
            }
        }
        free(x);
        free(t);
    }
    free(Wd);
    free(Ad);
    free(Bd);
    return err ? -1 : 0;
}

/*
 * Forward at chosen output positions (ms[i], ns[i]), i < count, into Y[i].
 * Same definition as oracle_fwd_rows, evaluated one element at a time, so that
 * shapes too large for the full product can still be checked.
 */
int oracle_fwd_entries(int dt, int64_t N, int64_t K, int64_t r,
                       const void *X, const void *W, const void *A, const void *B,
                       float scale, int64_t count, const int64_t *ms, const int64_t *ns,
                       double *Y)
{
    (void)N;
    const double s = (double)scale;
#pragma omp parallel for num_threads(oracle_get_threads()) schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i) {
        const int64_t m = ms[i], n = ns[i];
        double yb = 0.0;
        for (int64_t k = 0; k < K; ++k)
            yb += widen(dt, X, m * K + k) * widen(dt, W, n * K + k);
        double l = 0.0;
        for (int64_t j = 0; j < r; ++j) {
            double t = 0.0;
            for (int64_t k = 0; k < K; ++k)
                t += widen(dt, X, m * K + k) * widen(dt, A, j * K + k);
            l += t * widen(dt, B, n * r + j);
        }
        Y[i] = yb + s * l;
    }
    return 0;
}

/*
 * Round a double to the nearest bf16 value, ties to even, once (no detour
 * through float).  bf16 keeps 8 significant bits, the float exponent range
 * and float's subnormal spacing 2^-133.  Returns the bf16 bit pattern.
 */
uint16_t oracle_round_bf16(double x)
{
    if (isnan(x))
        return (uint16_t)0x7FC0;
    const int neg = signbit(x) != 0;
    double ax = fabs(x);
    double q;
    if (isinf(ax)) {
        q = INFINITY;
    } else if (ax == 0.0) {
        q = 0.0;
    } else {
        int e2;
        (void)frexp(ax, &e2);          /* ax = f * 2^e2, f in [0.5, 1) */
        int e = e2 - 1;                /* ax in [2^e, 2^(e+1)) */
        if (e < -126)
            e = -126;                  /* subnormal range: fixed spacing */
        const double ulp = ldexp(1.0, e - 7);
        q = rint(ax / ulp) * ulp;      /* rint: nearest, ties to even */
        if (q >= ldexp(1.0, 128))
            q = INFINITY;
    }
    float f = (float)q;                /* exact: q is a bf16 value or inf */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t b = (uint16_t)(u >> 16);
    if (neg)
        b |= (uint16_t)0x8000;
    return b;
}

/* oracle_round_bf16 applied to n values, x[i] -> out[i]. */
void oracle_round_bf16_n(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_round_bf16(x[i]);
}

/*
 * Merge from pristine, rows [n0, n1) of the [N, K] result:
 *   Wref[n,k] = W0[n,k] + scale * sum_j B[n,j] A[j,k]
 * written as double into Wd[(n - n0) * K + k] when Wd is not NULL, and
 * rounded once to bf16 into Wb[...] when Wb is not NULL.  W0 is only read.
 */
int oracle_merge_rows(int dt, int64_t n0, int64_t n1, int64_t K, int64_t r,
                      const void *W0, const void *B, const void *A, float scale,
                      double *Wd, uint16_t *Wb)
{
    if (n1 <= n0 || K <= 0)
        return 0;
    double *Ad = (double *)malloc(sizeof(double) * (size_t)(r * K > 0 ? r * K : 1));
    if (Ad == NULL)
        return -1;
    widen_rows(dt, A, K, 0, r, Ad);
    const double s = (double)scale;
#pragma omp parallel for num_threads(oracle_get_threads()) schedule(dynamic, 1)
    for (int64_t n = n0; n < n1; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            double p = 0.0;
            for (int64_t j = 0; j < r; ++j)
                p += widen(dt, B, n * r + j) * Ad[j * K + k];
            const double w = widen(dt, W0, n * K + k) + s * p;
            if (Wd != NULL)
                Wd[(n - n0) * K + k] = w;
            if (Wb != NULL)
                Wb[(n - n0) * K + k] = oracle_round_bf16(w);
        }
    }
    free(Ad);
    return 0;
}

/*
 * Backward of the layer with the base weight frozen, "fastaf: Minimal LoRA
 * fine-tuning with hand-written Triton kernels", section "BWD kernel speedup"
 * (the three gradients dA, dB, dX of out = X W^T + ((X A^T) B^T) * scale):
 *   T[m,j]  = sum_k X[m,k] A[j,k]             (the forward's intermediate)
 *   G[m,j]  = sum_n dY[m,n] B[n,j]            (the output gradient in rank space)
 *   dX[m,k] = sum_n dY[m,n] W[n,k] + scale * sum_j G[m,j] A[j,k]
 *   dA[j,k] = scale * sum_m G[m,j] X[m,k]
 *   dB[n,j] = scale * sum_m dY[m,n] T[m,j]
 * All in double, ascending sums.  dX is written for rows [dx0, dx1) only
 * (into dX[(m - dx0) * K + k]; dX may be NULL), so that large shapes can be
 * checked on sampled rows; dA ([r, K]) and dB ([N, r]) are always complete.
 * Returns 0, or -1 when a work buffer cannot be allocated.
 */
int oracle_bwd(int dt, int64_t M, int64_t N, int64_t K, int64_t r,
               const void *X, const void *W, const void *A, const void *B, const void *dY,
               float scale, int64_t dx0, int64_t dx1, double *dX, double *dA, double *dB)
{
    const double s = (double)scale;
    double *T = (double *)malloc(sizeof(double) * (size_t)(M * r > 0 ? M * r : 1));
    double *G = (double *)malloc(sizeof(double) * (size_t)(M * r > 0 ? M * r : 1));
    if (T == NULL || G == NULL) {
        free(T);
        free(G);
        return -1;
    }
#pragma omp parallel for num_threads(oracle_get_threads()) schedule(dynamic, 4)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j = 0; j < r; ++j) {
            double t = 0.0, g = 0.0;
            for (int64_t k = 0; k < K; ++k)
                t += widen(dt, X, m * K + k) * widen(dt, A, j * K + k);
            for (int64_t n = 0; n < N; ++n)
                g += widen(dt, dY, m * N + n) * widen(dt, B, n * r + j);
            T[m * r + j] = t;
            G[m * r + j] = g;
        }
    }
    if (dX != NULL) {
#pragma omp parallel for num_threads(oracle_get_threads()) schedule(dynamic, 1)
        for (int64_t m = dx0; m < dx1; ++m) {
            for (int64_t k = 0; k < K; ++k) {
                double base = 0.0, lora = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    base += widen(dt, dY, m * N + n) * widen(dt, W, n * K + k);
                for (int64_t j = 0; j < r; ++j)
                    lora += G[m * r + j] * widen(dt, A, j * K + k);
                dX[(m - dx0) * K + k] = base + s * lora;
            }
        }
    }
#pragma omp parallel for num_threads(oracle_get_threads()) schedule(dynamic, 4)
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t j = 0; j < r; ++j) {
            double a = 0.0;
            for (int64_t m = 0; m < M; ++m)
                a += G[m * r + j] * widen(dt, X, m * K + k);
            dA[j * K + k] = s * a;
        }
    }
#pragma omp parallel for num_threads(oracle_get_threads()) schedule(dynamic, 4)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < r; ++j) {
            double b = 0.0;
            for (int64_t m = 0; m < M; ++m)
                b += widen(dt, dY, m * N + n) * T[m * r + j];
            dB[n * r + j] = s * b;
        }
    }
    free(T);
    free(G);
    return 0;
}
