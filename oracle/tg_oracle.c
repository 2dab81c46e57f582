/*
 * tg_oracle.c -- CPU oracle for the tiled half-precision GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library; the GEMM library never does, and the
 * two share no code, header, table or constant.
 *
 * What it computes is the plain definition of the matrix product that the
 * TileLang pages build their tiled kernel around ("TileLang: writing LLM GPU
 * kernels by thinking in tiles", section 2 "The basic idea: a GPU should reuse
 * data": C[i,j] is the sum over k of A[i,k]*B[k,j], with A of size MxK, B of
 * size KxN and C of size MxN), followed by the epilogue the fourth page
 * ("Designing high-performance GPU kernels with TileLang", part 3 "Epilogue
 * fusion") describes as GELU(MatMul + Bias).  It is written out directly:
 *
 *   1. decode every 16-bit input (IEEE binary16, or bfloat16 = the upper half
 *      of IEEE binary32) to double, exactly, by the format definitions;
 *   2. for each requested row i and each column j, sum a_ik * b_kj in double
 *      in ascending k (each product of two 16-bit values is exact in double);
 *   3. add bias[j] in double, then apply GELU in its tanh form,
 *      0.5*y*(1 + tanh(sqrt(2/pi)*(y + 0.044715*y^3))), in double;
 *   4. return the double result and its round-to-nearest-even 16-bit pattern.
 *
 * Rows are distributed over OpenMP threads; every output element is still a
 * single ascending-k sum, so results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F16 0
#define OR_BF16 1
#define OR_EPI_NONE 0
#define OR_EPI_BIAS 1
#define OR_EPI_BIAS_GELU_TANH 2

#define OR_OK 0
#define OR_BAD_ARG 1
#define OR_NO_MEMORY 2

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero or subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25);      /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
static double decode_bf16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                /* zero or subnormal: f * 2^-133 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 128), e - 134);      /* (1 + f/2^7) * 2^(e-127) */
    return sign ? -v : v;
}

static double decode(int dtype, uint16_t h)
{
    return dtype == OR_F16 ? decode_f16(h) : decode_bf16(h);
}

/*
 * Round a double to the nearest value of a binary format with `fbits`
 * fraction bits and `ebits` exponent bits, ties to even; overflow gives
 * infinity, NaN gives the positive quiet NaN.
 */
static uint16_t encode_format(double x, int fbits, int ebits)
{
    const int bias = (1 << (ebits - 1)) - 1;
    const int emin = 1 - bias;
    const uint16_t sign = signbit(x) ? (uint16_t)0x8000 : (uint16_t)0;
    const uint16_t exp_all_ones = (uint16_t)(((1 << ebits) - 1) << fbits);
    if (isnan(x))
        return (uint16_t)(exp_all_ones | (1 << (fbits - 1)));
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | exp_all_ones);
    if (a == 0.0)
        return sign;
    int e2;
    (void)frexp(a, &e2);            /* a = m * 2^e2 with m in [0.5, 1) */
    int E = e2 - 1;                 /* 2^E <= a < 2^(E+1) */
    if (E < emin)
        E = emin;                   /* subnormals share the smallest binade's spacing */
    /* Representable values near a are n * 2^(E - fbits) for integer n. */
    double n = nearbyint(ldexp(a, fbits - E));   /* exact scaling; rounds to nearest even */
    if (n >= ldexp(1.0, fbits + 1)) {            /* rounded up into the next binade */
        n = ldexp(n, -1);
        E += 1;
    }
    if (E > bias)
        return (uint16_t)(sign | exp_all_ones);  /* overflow */
    uint32_t ni = (uint32_t)n;
    if (ni < (1u << fbits))
        return (uint16_t)(sign | ni);            /* subnormal: exponent field 0 */
    return (uint16_t)(sign | ((uint32_t)(E + bias) << fbits) | (ni - (1u << fbits)));
}

static uint16_t encode(int dtype, double x)
{
    return dtype == OR_F16 ? encode_format(x, 10, 5) : encode_format(x, 7, 8);
}

/* GELU, tanh form, in double. */
static double gelu_tanh(double y)
{
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * y * (1.0 + tanh(c * (y + 0.044715 * y * y * y)));
}

int tg_oracle_decode(int dtype, const uint16_t *bits, double *out, int64_t n)
{
    if ((dtype != OR_F16 && dtype != OR_BF16) || n < 0 || (n > 0 && (!bits || !out)))
        return OR_BAD_ARG;
    for (int64_t i = 0; i < n; ++i)
        out[i] = decode(dtype, bits[i]);
    return OR_OK;
}

int tg_oracle_encode(int dtype, const double *values, uint16_t *out, int64_t n)
{
    if ((dtype != OR_F16 && dtype != OR_BF16) || n < 0 || (n > 0 && (!values || !out)))
        return OR_BAD_ARG;
    for (int64_t i = 0; i < n; ++i)
        out[i] = encode(dtype, values[i]);
    return OR_OK;
}

int tg_oracle_gelu_tanh(const double *x, double *out, int64_t n)
{
    if (n < 0 || (n > 0 && (!x || !out)))
        return OR_BAD_ARG;
    for (int64_t i = 0; i < n; ++i)
        out[i] = gelu_tanh(x[i]);
    return OR_OK;
}

int tg_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Steps 2-4 on decoded operands: C rows `rows[0..nrows)` (or all M rows when
 * rows == NULL) of epilogue(A*B [+ bias]) with B given as doubles Bd (KxN)
 * and the bias as doubles biasd (N entries).
 */
static void gemm_decoded(int64_t M, int64_t N, int64_t K, int dtype, const uint16_t *A, const double *Bd,
                         const double *biasd, int epilogue, const int64_t *rows, int64_t nrows,
                         double *out64, uint16_t *outq)
{
    (void)M;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        double *acc = out64 + r * N;
        /* Step 2: acc[j] = sum over ascending k of a_ik * b_kj. */
        for (int64_t j = 0; j < N; ++j)
            acc[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = decode(dtype, A[i * K + k]);
            const double *brow = Bd + k * N;
            for (int64_t j = 0; j < N; ++j)
                acc[j] += a * brow[j];
        }
        /* Steps 3 and 4: epilogue in double, then round to the 16-bit format. */
        for (int64_t j = 0; j < N; ++j) {
            double y = acc[j];
            if (epilogue != OR_EPI_NONE)
                y = y + biasd[j];
            if (epilogue == OR_EPI_BIAS_GELU_TANH)
                y = gelu_tanh(y);
            acc[j] = y;
            outq[r * N + j] = encode(dtype, y);
        }
    }
}

static int check_common(int64_t M, int64_t N, int64_t K, int dtype, int epilogue, const int64_t *rows,
                        int64_t nrows)
{
    if (M < 0 || N < 0 || K < 0 || nrows < 0)
        return OR_BAD_ARG;
    if (dtype != OR_F16 && dtype != OR_BF16)
        return OR_BAD_ARG;
    if (epilogue != OR_EPI_NONE && epilogue != OR_EPI_BIAS && epilogue != OR_EPI_BIAS_GELU_TANH)
        return OR_BAD_ARG;
    if (rows == NULL && nrows != M)
        return OR_BAD_ARG;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M)
            return OR_BAD_ARG;
    return OR_OK;
}

/*
 * C rows `rows[0..nrows)` (or all M rows when rows == NULL, nrows == M) of
 * epilogue(A*B [+ bias]).  A is MxK, B is KxN, bias has N entries, all
 * row-major 16-bit patterns of `dtype`.  out64 and outq are nrows x N,
 * row r holding C row rows[r].
 */
int tg_oracle_gemm(int64_t M, int64_t N, int64_t K, int dtype,
                   const uint16_t *A, const uint16_t *B, const uint16_t *bias, int epilogue,
                   const int64_t *rows, int64_t nrows, double *out64, uint16_t *outq)
{
    int rc = check_common(M, N, K, dtype, epilogue, rows, nrows);
    if (rc != OR_OK)
        return rc;
    if (nrows == 0 || N == 0)
        return OR_OK;
    if (!out64 || !outq || (epilogue != OR_EPI_NONE && !bias) || (K > 0 && (!A || !B)))
        return OR_BAD_ARG;

    /* Step 1: decode B and bias once. */
    double *Bd = (double *)malloc((size_t)(K > 0 ? K : 1) * (size_t)N * sizeof(double));
    double *biasd = (double *)malloc((size_t)N * sizeof(double));
    if (!Bd || !biasd) {
        free(Bd);
        free(biasd);
        return OR_NO_MEMORY;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            Bd[k * N + j] = decode(dtype, B[k * N + j]);
    for (int64_t j = 0; j < N; ++j)
        biasd[j] = (epilogue != OR_EPI_NONE) ? decode(dtype, bias[j]) : 0.0;

    gemm_decoded(M, N, K, dtype, A, Bd, biasd, epilogue, rows, nrows, out64, outq);
    free(Bd);
    free(biasd);
    return OR_OK;
}

/*
 * The same product with B held as 4-bit weights, the weight-only quantized
 * GEMM of LLM inference that the first TileLang page ("TileLang: writing LLM
 * GPU kernels by thinking in tiles", section 5, "Quantized LLM inference")
 * describes: packed integer weights are turned back into 16-bit values and
 * fed to the matrix product.  Here that turning back is written out as its
 * definition, for every weight:
 *
 *   b_kj = (q_kj - 8) * s_gj,   g = k / group,
 *
 * with q_kj in 0..15 (one value per byte of Q, KxN row-major), and s the
 * scales (K/group x N row-major 16-bit patterns of `dtype`), decoded exactly.
 * The product (q - 8) * s is exact in double.  Then steps 2-4 as above.
 */
int tg_oracle_gemm_w4(int64_t M, int64_t N, int64_t K, int dtype, const uint16_t *A, const uint8_t *Q,
                      const uint16_t *scales, int64_t group, const uint16_t *bias, int epilogue,
                      const int64_t *rows, int64_t nrows, double *out64, uint16_t *outq)
{
    int rc = check_common(M, N, K, dtype, epilogue, rows, nrows);
    if (rc != OR_OK)
        return rc;
    if (group <= 0 || K % group != 0)
        return OR_BAD_ARG;
    if (nrows == 0 || N == 0)
        return OR_OK;
    if (!out64 || !outq || (epilogue != OR_EPI_NONE && !bias) || (K > 0 && (!A || !Q || !scales)))
        return OR_BAD_ARG;
    for (int64_t i = 0; i < K * N; ++i)
        if (Q[i] > 15)
            return OR_BAD_ARG;

    double *Bd = (double *)malloc((size_t)(K > 0 ? K : 1) * (size_t)N * sizeof(double));
    double *biasd = (double *)malloc((size_t)N * sizeof(double));
    if (!Bd || !biasd) {
        free(Bd);
        free(biasd);
        return OR_NO_MEMORY;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            Bd[k * N + j] = ((double)Q[k * N + j] - 8.0) * decode(dtype, scales[(k / group) * N + j]);
    for (int64_t j = 0; j < N; ++j)
        biasd[j] = (epilogue != OR_EPI_NONE) ? decode(dtype, bias[j]) : 0.0;

    gemm_decoded(M, N, K, dtype, A, Bd, biasd, epilogue, rows, nrows, out64, outq);
    free(Bd);
    free(biasd);
    return OR_OK;
}

/*
 * Attention forward, written out from its definition as the first TileLang
 * page states it ("TileLang: writing LLM GPU kernels by thinking in tiles",
 * section 5, "FlashAttention": S = Q K^T / sqrt(d), P = softmax(S), O = P V),
 * which FlashAttention computes blockwise with an online softmax and reaches
 * up to rounding.  Layout BSHD as in the second page's listing ("TileLang: you
 * write the dataflow, the compiler owns the schedule", "FlashAttention, in
 * tiles"): Q is [batch][Sq][heads][D] row-major, K and V [batch][Sk][heads][D],
 * O like Q.  For each requested query (b, i, h), in double:
 *
 *   s_j = scale * sum_d Q[b][i][h][d] * K[b][j][h][d]   for the allowed keys j,
 *   m   = max_j s_j,   p_j = exp(s_j - m),   l = sum_j p_j,
 *   O[b][i][h][d] = (sum_j p_j * V[b][j][h][d]) / l,
 *
 * where the allowed keys are all j < Sk, or with `causal` (Sq == Sk) the keys
 * j <= i.  Sums run in ascending j (and d).  `queries` lists (b, i, h)
 * triples; out64 and outq are nq x D.
 */
int tg_oracle_attention(int64_t Bn, int64_t Sq, int64_t Sk, int64_t H, int64_t D, int dtype, const uint16_t *Q,
                        const uint16_t *K, const uint16_t *V, int causal, double scale, const int64_t *queries,
                        int64_t nq, double *out64, uint16_t *outq)
{
    if (Bn < 0 || Sq < 0 || Sk < 0 || H < 0 || D < 0 || nq < 0)
        return OR_BAD_ARG;
    if (dtype != OR_F16 && dtype != OR_BF16)
        return OR_BAD_ARG;
    if (causal && Sq != Sk)
        return OR_BAD_ARG;
    if (nq == 0 || D == 0)
        return OR_OK;
    if (!queries || !out64 || !outq || !Q || (Sk > 0 && (!K || !V)))
        return OR_BAD_ARG;
    for (int64_t r = 0; r < nq; ++r) {
        const int64_t *t = queries + 3 * r;
        if (t[0] < 0 || t[0] >= Bn || t[1] < 0 || t[1] >= Sq || t[2] < 0 || t[2] >= H)
            return OR_BAD_ARG;
    }
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nq; ++r) {
        const int64_t b = queries[3 * r], i = queries[3 * r + 1], h = queries[3 * r + 2];
        const int64_t nk = causal ? i + 1 : Sk;
        double *o = out64 + r * D;
        double *s = (double *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(double));
        double *q = (double *)malloc((size_t)D * sizeof(double));
        if (!s || !q) {
            free(s);
            free(q);
            #pragma omp atomic write
            bad = 1;
            continue;
        }
        for (int64_t d = 0; d < D; ++d)
            q[d] = decode(dtype, Q[((b * Sq + i) * H + h) * D + d]);
        double m = -INFINITY;
        for (int64_t j = 0; j < nk; ++j) {
            double acc = 0.0;
            const uint16_t *krow = K + ((b * Sk + j) * H + h) * D;
            for (int64_t d = 0; d < D; ++d)
                acc += q[d] * decode(dtype, krow[d]);
            s[j] = scale * acc;
            if (s[j] > m)
                m = s[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < nk; ++j) {
            s[j] = exp(s[j] - m);
            l += s[j];
        }
        for (int64_t d = 0; d < D; ++d)
            o[d] = 0.0;
        for (int64_t j = 0; j < nk; ++j) {
            const uint16_t *vrow = V + ((b * Sk + j) * H + h) * D;
            for (int64_t d = 0; d < D; ++d)
                o[d] += s[j] * decode(dtype, vrow[d]);
        }
        for (int64_t d = 0; d < D; ++d) {
            o[d] = nk > 0 ? o[d] / l : 0.0;
            outq[r * D + d] = encode(dtype, o[d]);
        }
        free(s);
        free(q);
    }
    return bad ? OR_NO_MEMORY : OR_OK;
}
