/*
 * softmax_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU reference for the numerically stable row
 * softmax, computed in double precision.  It exists to check the GPU library;
 * it is not part of the product.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no source, header,
 * table or helper with the HIP library, and includes no HIP header.
 *
 * What it computes (the plain definition, written out):
 *   for every row i:   m_i  = max_j x_ij
 *                      y_ij = exp(x_ij - m_i) / sum_k exp(x_ik - m_i)
 * Sources:
 *   - "I Wrote My First GPU Kernel", section "What Fusion Actually Does":
 *     subtract the row max before exponentiating so that large entries
 *     (the page's example is 100) cannot overflow; then normalise by the sum.
 *   - "fused-softmax-roofline" (henryhe.ai), the row-softmax fragment:
 *     shift by the row max, exponentiate, divide by the sum.
 *   - "GPU Kernels - Implementing and optimizing Softmax", section
 *     "Baseline & Triton Softmax kernel": max, subtract, exp, sum, divide,
 *     and the remark that exp(-inf) = 0 so masked columns add nothing.
 *   - "Dissecting Memory Bandwidth & SRAM Tiling in Triton", section
 *     "The Mathematical Remedy: Online Softmax Tiling": the two-pass form
 *     m = max x, l = sum exp(x - m), p = exp(x - m) / l.
 *
 * Readings where the pages are silent (each is listed with the design notes):
 *   - a row whose entries are all -inf has no finite maximum; its outputs
 *     are all +0 (the pages' masking rule, under which a masked column
 *     contributes and receives zero, applied to every column);
 *   - +inf and NaN inputs are outside the contract and are not special-cased;
 *   - fp16 and bf16 inputs are decoded exactly from their bit patterns by
 *     the two decoders below (IEEE 754 binary16, and bfloat16 = the upper 16
 *     bits of an IEEE 754 binary32).
 *
 * Precision: every step runs in double.  The sum is a plain left-to-right
 * double sum; its relative error is at most cols * 2^-53 (about 2e-12 at
 * 16384 columns), far below any tolerance the GPU path is held to.
 *
 * Build: gcc -O2 -std=c11 -shared -fPIC, never with -ffast-math (the -inf
 * handling relies on IEEE semantics).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);               /* subnormal: frac * 2^-14 / 2^10 */
    } else if (expo == 31) {
        v = (frac == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/2^10) * 2^(expo-15) */
    }
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_decode_bf16(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int expo = (b >> 7) & 0xff;
    int frac = b & 0x7f;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -133);              /* subnormal: frac * 2^-126 / 2^7 */
    } else if (expo == 255) {
        v = (frac == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(128 + frac), expo - 134); /* (1 + frac/2^7) * 2^(expo-127) */
    }
    return sign ? -v : v;
}

/* Element (i, j) of the input, exactly as a double. */
static double load_element(const void *in, int dtype, int64_t index)
{
    if (dtype == ORACLE_F32) {
        float f;
        memcpy(&f, (const char *)in + index * 4, 4);
        return (double)f;
    } else {
        uint16_t bits;
        memcpy(&bits, (const char *)in + index * 2, 2);
        return dtype == ORACLE_F16 ? oracle_decode_f16(bits) : oracle_decode_bf16(bits);
    }
}

/*
 * Row softmax of a rows x cols matrix stored row-major with a row stride of
 * row_stride elements.  out receives rows * cols doubles, dense (row i at
 * out + i * cols).  Returns 0 on success, -1 on a bad argument.
 */
int oracle_softmax(const void *in, int dtype, int64_t rows, int64_t cols,
                   int64_t row_stride, double *out)
{
    if (rows < 0 || cols < 0 || row_stride < cols) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    if (rows == 0 || cols == 0) return 0;
    if (in == NULL || out == NULL) return -1;

    for (int64_t i = 0; i < rows; ++i) {
        double *y = out + i * cols;

        /* Decode the row once; y doubles as storage for x and then e. */
        for (int64_t j = 0; j < cols; ++j)
            y[j] = load_element(in, dtype, i * row_stride + j);

        /* Row maximum, seeded with -inf. */
        double m = -INFINITY;
        for (int64_t j = 0; j < cols; ++j)
            if (y[j] > m) m = y[j];

        /* All entries -inf: no finite maximum, every output is +0. */
        if (m == -INFINITY) {
            for (int64_t j = 0; j < cols; ++j) y[j] = 0.0;
            continue;
        }

        /* Shifted exponentials and their sum; exp(-inf) is exactly +0. */
        double s = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            y[j] = exp(y[j] - m);
            s += y[j];
        }

        /* Normalise with a true division. */
        for (int64_t j = 0; j < cols; ++j)
            y[j] = y[j] / s;
    }
    return 0;
}

/*
 * oracle_softmax_mt -- the same oracle over `threads` contiguous row ranges,
 * one POSIX thread each, for timing the CPU baseline on all of a host's
 * cores.  Each range is one unchanged call of oracle_softmax on its rows, so
 * the result is bit-identical to the single-threaded call.  threads must be
 * 1 ... 256 (fewer are used when there are fewer rows).
 */
struct oracle_range {
    const void *in;
    int dtype;
    int64_t rows, cols, row_stride;
    double *out;
    int rc;
};

static void *oracle_range_run(void *arg)
{
    struct oracle_range *r = (struct oracle_range *)arg;
    r->rc = oracle_softmax(r->in, r->dtype, r->rows, r->cols, r->row_stride, r->out);
    return NULL;
}

int oracle_softmax_mt(const void *in, int dtype, int64_t rows, int64_t cols,
                      int64_t row_stride, double *out, int threads)
{
    if (threads < 1 || threads > 256) return -1;
    if (rows < 0 || cols < 0 || row_stride < cols) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    if (rows == 0 || cols == 0) return 0;
    if (in == NULL || out == NULL) return -1;
    if (threads > rows) threads = (int)rows;
    const int64_t esz = dtype == ORACLE_F32 ? 4 : 2;
    struct oracle_range r[256];
    pthread_t tid[256];
    int started[256] = {0};
    for (int k = 0; k < threads; ++k) {
        const int64_t r0 = rows * k / threads, r1 = rows * (k + 1) / threads;
        r[k].in = (const char *)in + r0 * row_stride * esz;
        r[k].dtype = dtype;
        r[k].rows = r1 - r0;
        r[k].cols = cols;
        r[k].row_stride = row_stride;
        r[k].out = out + r0 * cols;
        r[k].rc = 0;
    }
    for (int k = 1; k < threads; ++k)
        started[k] = pthread_create(&tid[k], NULL, oracle_range_run, &r[k]) == 0;
    oracle_range_run(&r[0]);
    int rc = r[0].rc;
    for (int k = 1; k < threads; ++k) {
        if (started[k]) pthread_join(tid[k], NULL);
        else oracle_range_run(&r[k]); /* no thread: run the range here */
        if (rc == 0) rc = r[k].rc;
    }
    return rc;
}

/*
 * Scaled, causally masked row softmax ("Dissecting Memory Bandwidth & SRAM
 * Tiling in Triton", section "Writing the Kernel in OpenAI Triton": scores
 * scaled by 1/sqrt(d), entries with column > row set to -inf before the
 * softmax).  For row i, column j is kept when j <= i + diag; for the kept
 * columns  z_j = scale * x_ij  and
 *     y_ij = exp(z_j - max_kept z) / sum_kept exp(z_k - max_kept z),
 * and every masked column gets +0.  A row with no kept column, or whose kept
 * entries are all -inf, is all +0.  `scale` must be finite and > 0.
 * Masked inputs are never read.  Returns 0, or -1 on a bad argument.
 */
int oracle_softmax_causal(const void *in, int dtype, int64_t rows, int64_t cols,
                          int64_t row_stride, double scale, int64_t diag, double *out)
{
    if (rows < 0 || cols < 0 || row_stride < cols) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    if (!(scale > 0.0) || isinf(scale)) return -1;
    if (rows == 0 || cols == 0) return 0;
    if (in == NULL || out == NULL) return -1;

    for (int64_t i = 0; i < rows; ++i) {
        double *y = out + i * cols;
        /* Number of kept columns: j = 0 .. i + diag, clipped to [0, cols]
           (written so that no sum can overflow for any diag). */
        int64_t kept;
        if (diag >= cols) {
            kept = cols;
        } else if (diag < -i) {
            kept = 0;
        } else {
            kept = i + diag + 1;
            if (kept > cols) kept = cols;
        }

        for (int64_t j = 0; j < cols; ++j) y[j] = 0.0;
        for (int64_t j = 0; j < kept; ++j)
            y[j] = scale * load_element(in, dtype, i * row_stride + j);

        double m = -INFINITY;
        for (int64_t j = 0; j < kept; ++j)
            if (y[j] > m) m = y[j];
        if (m == -INFINITY) {
            for (int64_t j = 0; j < kept; ++j) y[j] = 0.0;
            continue;
        }

        double s = 0.0;
        for (int64_t j = 0; j < kept; ++j) {
            y[j] = exp(y[j] - m);
            s += y[j];
        }
        for (int64_t j = 0; j < kept; ++j)
            y[j] = y[j] / s;
    }
    return 0;
}

/*
 * Attention forward with the softmax in the middle ("Dissecting Memory
 * Bandwidth & SRAM Tiling in Triton", section "Memory Hierarchy: Why Standard
 * Attention Collapses": O = softmax(Q K^T / sqrt(d)) V, and section "Writing
 * the Kernel in OpenAI Triton": the causal mask).  Computed the plain way, in
 * double: for every batch b, head h and query i,
 *     s_j = scale * sum_d q[i][d] k[j][d]           for every kept key j,
 *     p_j = exp(s_j - max s) / sum exp(s - max s),
 *     o[i][d] = sum_j p_j v[j][d].
 * With `causal`, key j is kept for query i when j <= i + (nk - nq) (the mask
 * aligned to the last query, as for a query block appended to a key cache);
 * a query with no kept key gets o = 0.  q is [b][h][nq][d], k and v are
 * [b][h][nk][d], out is [b][h][nq][d] doubles, all dense.  dtype is that of
 * q, k and v (ORACLE_F16 or ORACLE_BF16 for the MFMA path; ORACLE_F32 works
 * too).  Returns 0, or -1 on a bad argument.
 */
int oracle_attention_fwd(const void *q, const void *k, const void *v, int dtype,
                         int64_t batch, int64_t heads, int64_t nq, int64_t nk, int64_t d,
                         double scale, int causal, double *out)
{
    if (batch < 0 || heads < 0 || nq < 0 || nk < 0 || d <= 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    if (!(scale > 0.0) || isinf(scale)) return -1;
    if (batch == 0 || heads == 0 || nq == 0) return 0;
    if (q == NULL || k == NULL || v == NULL || out == NULL) return -1;

    double *s = (double *)malloc((size_t)(nk > 0 ? nk : 1) * sizeof(double));
    if (s == NULL) return -1;
    for (int64_t bh = 0; bh < batch * heads; ++bh) {
        const int64_t qb = bh * nq * d, kb = bh * nk * d;
        for (int64_t i = 0; i < nq; ++i) {
            double *o = out + qb + i * d;
            for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
            int64_t kept = nk;
            if (causal) {
                kept = i + (nk - nq) + 1;
                if (kept < 0) kept = 0;
                if (kept > nk) kept = nk;
            }
            if (kept == 0) continue;

            double m = -INFINITY;
            for (int64_t j = 0; j < kept; ++j) {
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    dot += load_element(q, dtype, qb + i * d + c) * load_element(k, dtype, kb + j * d + c);
                s[j] = scale * dot;
                if (s[j] > m) m = s[j];
            }
            double sum = 0.0;
            for (int64_t j = 0; j < kept; ++j) {
                s[j] = exp(s[j] - m);
                sum += s[j];
            }
            for (int64_t j = 0; j < kept; ++j) {
                const double p = s[j] / sum;
                for (int64_t c = 0; c < d; ++c)
                    o[c] += p * load_element(v, dtype, kb + j * d + c);
            }
        }
    }
    free(s);
    return 0;
}
