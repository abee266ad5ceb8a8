/*
 * oracle_gemm.c -- plain CPU reference for dense GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity oracle: it is used by
 * tests/, by __graft_entry__.smoke() and by the cpu_baseline leg of bench.py,
 * and by nothing else.  It shares no source, header, table or helper with the
 * HIP library under dense_gemm_tiled_amd/ and never calls it.
 *
 * What it computes, for every batch element z, row i < M and column j < N:
 *
 *   opA(i,k) = transpose_a ? A[k*lda + i] : A[i*lda + k]
 *   opB(k,j) = transpose_b ? B[j*ldb + k] : B[k*ldb + j]
 *   S(i,j)   = sum over k = 0 .. K-1, in ascending k, of opA(i,k)*opB(k,j)
 *   C(i,j)   = round_c( alpha*S(i,j) + (beta != 0 ? beta*C_in(i,j) : 0) )
 *
 * and, on request, the magnitude sum
 *
 *   T(i,j)   = sum over k = 0 .. K-1, in ascending k, of |opA(i,k)*opB(k,j)|
 *
 * which scales the a-priori error bound of a floating-point dot product of
 * length K (|computed - exact| <= gamma_K * T, gamma_K = K*u / (1 - K*u) for
 * unit roundoff u; tessl "Architecture", section "Reductions and Numerical
 * Safety", bounds its row sums the same way, by a multiple of eps * n times
 * the term magnitudes).
 *
 * Sources (web pages, cited by title and section):
 *  - tensorcore "GEMM", section "Surface": the descriptor, the BLAS row-major
 *    definition C = alpha*A@B + beta*C, and leading dims that default to
 *    contiguous when 0.
 *  - tensorcore "GEMM", section "Transposes": a transposed operand is the same
 *    storage read with swapped strides (the opA/opB above).
 *  - tensorcore "GEMM", section "Numerical guarantees": the reference is fp64;
 *    int8 accumulates exactly in integers.
 *  - Phobos "Matrix products", kernels sgemm/hgemm: alpha*acc + beta*c_old
 *    epilogue; f16 inputs with an f32 (here: wider) accumulator; matmul_t is
 *    the NT form (B stored [N,K]).
 *  - tessl "Architecture", section "Integer GEMM": int8 x int8 sums are exact
 *    integers.
 *  - tessl "Architecture", section "Fused Epilogue": C is read only when
 *    beta != 0.
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes): round_c is a single round-to-nearest-even from the fp64 value (no
 * fp32 intermediate); alpha == 0 follows BLAS (C = beta*C, A and B unread);
 * the int8 path has alpha == 1, beta == 0 and writes the exact int64 sum as
 * int32 (callers keep K small enough that it cannot wrap).
 *
 * Arithmetic: products of two bf16/fp16/fp32 values are exact in fp64 (at most
 * 24+24 significand bits), so the only fp64 rounding is in the additions,
 * which run in ascending k.  Build with -ffp-contract=off so that no fused
 * multiply-add changes that.  int8 products and sums are exact in int64.
 *
 * The row loop is parallel (OpenMP) over output rows; every output element is
 * still the same ascending-k sum, so the result does not depend on threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype codes of this oracle (its own numbering). */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_I8 = 3, OR_I32 = 4 };

/* ------------------------------------------------------------------------ */
/* Decoding stored bit patterns to fp64.                                     */
/* ------------------------------------------------------------------------ */

/* bfloat16: the high half of an IEEE binary32. */
double oracle_decode_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24);                 /* zero and subnormals */
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + m), e - 25);     /* (1.m) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Rounding fp64 to a narrower binary format, round-to-nearest-even.         */
/* p = significand bits including the hidden bit; emin = exponent of the     */
/* smallest normal; emax = exponent of the largest finite binade.            */
/* Returns the rounded value as a double (exactly representable), with       */
/* overflow to +-inf and gradual underflow.                                  */
/* ------------------------------------------------------------------------ */
static double round_to_format(double x, int p, int emin, int emax) {
    if (isnan(x) || isinf(x) || x == 0.0) return x;
    double a = fabs(x);
    int E;
    (void)frexp(a, &E);            /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                 /* a in [2^e, 2^(e+1)) */
    int qexp = (e < emin ? emin : e) - (p - 1);   /* exponent of one ulp */
    double r = ldexp(a, -qexp);    /* exact: scaling by a power of two */
    double fl = floor(r);
    double diff = r - fl;          /* exact */
    double n;
    if (diff > 0.5) {
        n = fl + 1.0;
    } else if (diff < 0.5) {
        n = fl;
    } else {
        n = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;   /* tie: to even */
    }
    double v = ldexp(n, qexp);
    double maxfinite = ldexp(ldexp(1.0, p) - 1.0, emax - (p - 1));
    if (v > maxfinite) v = INFINITY;
    return x < 0 ? -v : v;
}

double oracle_round_f32(double x) { return round_to_format(x, 24, -126, 127); }
double oracle_round_bf16(double x) { return round_to_format(x, 8, -126, 127); }
double oracle_round_f16(double x) { return round_to_format(x, 11, -14, 15); }

/* Encoders take a value that is already exactly representable. */
uint16_t oracle_encode_bf16(double x) {
    double v = oracle_round_bf16(x);
    if (isnan(v)) return (uint16_t)(signbit(x) ? 0xFFC0 : 0x7FC0);
    float f = (float)v;            /* exact: v has 8 significand bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

uint16_t oracle_encode_f16(double x) {
    double v = oracle_round_f16(x);
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return (uint16_t)(sign | 0x7E00);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7C00);
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -14)) {                      /* subnormal */
        return (uint16_t)(sign | (uint16_t)ldexp(a, 24));
    }
    int E;
    (void)frexp(a, &E);
    int e = E - 1;
    int m = (int)(ldexp(a, 10 - e) - 1024.0);      /* exact fraction */
    return (uint16_t)(sign | ((e + 15) << 10) | m);
}

float oracle_encode_f32(double x) {
    return (float)oracle_round_f32(x);             /* exact once rounded */
}

/* ------------------------------------------------------------------------ */
/* Element access.                                                           */
/* ------------------------------------------------------------------------ */
static double load_float(const void *p, int dtype, int64_t idx) {
    switch (dtype) {
    case OR_F32: return (double)((const float *)p)[idx];
    case OR_F16: return oracle_decode_f16(((const uint16_t *)p)[idx]);
    case OR_BF16: return oracle_decode_bf16(((const uint16_t *)p)[idx]);
    default: return NAN;
    }
}

static void store_rounded(void *p, int dtype, int64_t idx, double v) {
    switch (dtype) {
    case OR_F32: ((float *)p)[idx] = oracle_encode_f32(v); break;
    case OR_F16: ((uint16_t *)p)[idx] = oracle_encode_f16(v); break;
    case OR_BF16: ((uint16_t *)p)[idx] = oracle_encode_bf16(v); break;
    default: break;
    }
}

static int64_t opa_index(int64_t i, int64_t k, int transpose_a, int64_t lda) {
    return transpose_a ? k * lda + i : i * lda + k;
}

static int64_t opb_index(int64_t k, int64_t j, int transpose_b, int64_t ldb) {
    return transpose_b ? j * ldb + k : k * ldb + j;
}

/* Argument check shared by the two entry points.  Returns 0 if usable. */
static int check_args(int64_t M, int64_t N, int64_t K, int a_dtype,
                      int c_dtype, double alpha, double beta, int64_t batch) {
    if (M < 1 || N < 1 || K < 1 || batch < 1) return -1;
    if (a_dtype == OR_I8) {
        if (c_dtype != OR_I32 || alpha != 1.0 || beta != 0.0) return -2;
    } else if (a_dtype == OR_F32 || a_dtype == OR_F16 || a_dtype == OR_BF16) {
        if (c_dtype != OR_F32 && c_dtype != a_dtype) return -2;
    } else {
        return -2;
    }
    return 0;
}

/*
 * Full product.  A, B, C_in hold the stored bit patterns (fp32 / binary16 /
 * bfloat16 / int8 for A and B; c_dtype for C).  The b operand has the same
 * dtype as a.  Batch element z starts at z*stride_a, z*stride_b, z*stride_c
 * elements.
 *
 * C_out (same layout as C_in, ldc) receives round_c(value) at every (i, j)
 * inside the M x N extent and is left untouched elsewhere.
 * value_out, if non-NULL, receives the unrounded fp64 value
 * alpha*S + beta*C_in, densely as [batch][M][N].  abs_out, if non-NULL,
 * receives T (the sum of |products|, exact for int8), densely likewise.
 * C_in may be NULL when beta == 0 (it is never read then).
 *
 * Returns 0 on success, a negative code on bad arguments.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K, int a_dtype, int c_dtype,
                int transpose_a, int transpose_b, double alpha, double beta,
                const void *A, int64_t lda, const void *B, int64_t ldb,
                const void *C_in, int64_t ldc, void *C_out, double *value_out,
                int64_t batch, int64_t stride_a, int64_t stride_b,
                int64_t stride_c, double *abs_out) {
    int rc = check_args(M, N, K, a_dtype, c_dtype, alpha, beta, batch);
    if (rc) return rc;
    if (beta != 0.0 && C_in == NULL) return -3;
    const int is_int = (a_dtype == OR_I8);

#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)N);
        double *tacc = (double *)malloc(sizeof(double) * (size_t)N);
        int64_t *iacc = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
        int64_t *itacc = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
#pragma omp for schedule(dynamic)
        for (int64_t zi = 0; zi < batch * M; ++zi) {
            int64_t z = zi / M, i = zi % M;
            const char *Az = (const char *)A;
            const char *Bz = (const char *)B;
            int64_t a_off = z * stride_a, b_off = z * stride_b;
            int64_t c_off = z * stride_c;
            if (is_int) {
                const int8_t *a8 = (const int8_t *)Az + a_off;
                const int8_t *b8 = (const int8_t *)Bz + b_off;
                for (int64_t j = 0; j < N; ++j) iacc[j] = itacc[j] = 0;
                for (int64_t k = 0; k < K; ++k) {
                    int64_t a = a8[opa_index(i, k, transpose_a, lda)];
                    if (abs_out) {
                        for (int64_t j = 0; j < N; ++j) {
                            int64_t t = a * (int64_t)b8[opb_index(k, j, transpose_b, ldb)];
                            iacc[j] += t;
                            itacc[j] += t < 0 ? -t : t;
                        }
                    } else {
                        for (int64_t j = 0; j < N; ++j)
                            iacc[j] += a * (int64_t)b8[opb_index(k, j, transpose_b, ldb)];
                    }
                }
                for (int64_t j = 0; j < N; ++j) {
                    ((int32_t *)C_out)[c_off + i * ldc + j] = (int32_t)iacc[j];
                    if (value_out) value_out[(z * M + i) * N + j] = (double)iacc[j];
                    if (abs_out) abs_out[(z * M + i) * N + j] = (double)itacc[j];
                }
            } else {
                for (int64_t j = 0; j < N; ++j) acc[j] = tacc[j] = 0.0;
                if (alpha != 0.0) {
                    for (int64_t k = 0; k < K; ++k) {
                        double a = load_float(A, a_dtype,
                                              a_off + opa_index(i, k, transpose_a, lda));
                        if (abs_out) {
                            for (int64_t j = 0; j < N; ++j) {
                                double t = a * load_float(B, a_dtype,
                                                          b_off + opb_index(k, j, transpose_b, ldb));
                                acc[j] += t;
                                tacc[j] += fabs(t);
                            }
                        } else {
                            for (int64_t j = 0; j < N; ++j)
                                acc[j] += a * load_float(B, a_dtype,
                                                         b_off + opb_index(k, j, transpose_b, ldb));
                        }
                    }
                }
                for (int64_t j = 0; j < N; ++j) {
                    double v = (alpha != 0.0) ? alpha * acc[j] : 0.0;
                    if (beta != 0.0)
                        v += beta * load_float(C_in, c_dtype, c_off + i * ldc + j);
                    store_rounded(C_out, c_dtype, c_off + i * ldc + j, v);
                    if (value_out) value_out[(z * M + i) * N + j] = v;
                    if (abs_out) abs_out[(z * M + i) * N + j] = tacc[j];
                }
            }
        }
        free(acc);
        free(tacc);
        free(iacc);
        free(itacc);
    }
    return 0;
}

/*
 * The same definition evaluated at npts chosen outputs (z[p], i[p], j[p]),
 * one by one, for full-size shapes where the whole product is too slow.
 * value_out[p] receives the unrounded fp64 value (the exact sum for int8);
 * rounded_out (c_dtype elements, npts of them), if non-NULL, its rounding;
 * abs_out[p], if non-NULL, the magnitude sum T at that output.
 */
int oracle_gemm_points(int64_t M, int64_t N, int64_t K, int a_dtype,
                       int c_dtype, int transpose_a, int transpose_b,
                       double alpha, double beta, const void *A, int64_t lda,
                       const void *B, int64_t ldb, const void *C_in,
                       int64_t ldc, int64_t stride_a, int64_t stride_b,
                       int64_t stride_c, int64_t npts, const int64_t *zs,
                       const int64_t *is, const int64_t *js, double *value_out,
                       void *rounded_out, double *abs_out) {
    int rc = check_args(M, N, K, a_dtype, c_dtype, alpha, beta, 1);
    if (rc) return rc;
    if (beta != 0.0 && C_in == NULL) return -3;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npts; ++p) {
        int64_t z = zs[p], i = is[p], j = js[p];
        int64_t a_off = z * stride_a, b_off = z * stride_b, c_off = z * stride_c;
        if (a_dtype == OR_I8) {
            const int8_t *a8 = (const int8_t *)A + a_off;
            const int8_t *b8 = (const int8_t *)B + b_off;
            int64_t s = 0, sa = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t t = (int64_t)a8[opa_index(i, k, transpose_a, lda)] *
                            (int64_t)b8[opb_index(k, j, transpose_b, ldb)];
                s += t;
                sa += t < 0 ? -t : t;
            }
            value_out[p] = (double)s;
            if (rounded_out) ((int32_t *)rounded_out)[p] = (int32_t)s;
            if (abs_out) abs_out[p] = (double)sa;
        } else {
            double s = 0.0, sa = 0.0;
            if (alpha != 0.0)
                for (int64_t k = 0; k < K; ++k) {
                    double t = load_float(A, a_dtype, a_off + opa_index(i, k, transpose_a, lda)) *
                               load_float(B, a_dtype, b_off + opb_index(k, j, transpose_b, ldb));
                    s += t;
                    sa += fabs(t);
                }
            double v = (alpha != 0.0) ? alpha * s : 0.0;
            if (beta != 0.0) v += beta * load_float(C_in, c_dtype, c_off + i * ldc + j);
            value_out[p] = v;
            if (rounded_out) store_rounded(rounded_out, c_dtype, p, v);
            if (abs_out) abs_out[p] = sa;
        }
    }
    return 0;
}

/* Array forms of the codecs (n elements, dense). */
void oracle_decode_array(const void *bits, int dtype, int64_t n, double *out) {
    for (int64_t t = 0; t < n; ++t) {
        switch (dtype) {
        case OR_I8: out[t] = (double)((const int8_t *)bits)[t]; break;
        case OR_I32: out[t] = (double)((const int32_t *)bits)[t]; break;
        default: out[t] = load_float(bits, dtype, t); break;
        }
    }
}

void oracle_encode_array(const double *values, int dtype, int64_t n, void *bits) {
    for (int64_t t = 0; t < n; ++t) store_rounded(bits, dtype, t, values[t]);
}

/* Number of threads the OpenMP runtime will use (for reporting). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
