/*
 * oracle.c -- plain, slow, single-threaded CPU reference for the W4A16
 * group-affine quantized product.  TEST INFRASTRUCTURE ONLY: the tests, the
 * smoke check and the benchmark's CPU-baseline leg load this file's library;
 * the product path never does.  It shares no code, header or constant with
 * the HIP library.
 *
 * What it computes (N = output rows, K = the reduction length):
 *
 *   y[m,n] = sum_k x[m,k] * w[n,k],   w[n,k] = q[n,k]*scale[n,g] + bias[n,g],
 *   g = floor(k / G)
 *
 * Sources on the pages:
 *   - "Week 2 Day 2: Keep W4 Packed" (tiny-llm), section "Group-Wise Affine
 *     Quantization" and "Reconstruct a Stored Group" (the equation w = q s + b,
 *     unsigned code, signed scale used as stored);
 *   - same page, "Packed Storage Layout" (8 codes per uint32, first code in the
 *     lowest nibble; codes [rows, K/8] u32, scales/biases [rows, K/G]);
 *   - same page, "Quantized Matrix Multiplication" / "Mathematical
 *     Formulation" (C = A B^T with B dequantized per group) and
 *     "Computation Flow" (groups -> packed words -> nibbles, output cast to
 *     bf16);
 *   - RESMP-DEV Gemma-4 megakernel page, "Usage" (group size 64) and "What it
 *     does" (a 4-bit LM head with an in-kernel argmax);
 *   - hy4-preview-metal page, kernel table (mul_mv_id: routed-expert matvec)
 *     and "Results" (a float64 reference as the correctness yardstick).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - the dequantized weight is ONE fp32 fused multiply-add fmaf(s, q, b);
 *   - products and sums are formed in fp64 (a bf16 x fp32 product is exact
 *     in fp64), summed in ascending k;
 *   - bf16 output = round-to-nearest-even of the fp64 sum (one rounding);
 *   - argmax scans n ascending with strict '>', so ties keep the lowest index;
 *   - routed form: y[m,j,:] = W[ids[m,j]] . x[m]  (or x[m,j] when each slot
 *     carries its own input row).
 *
 * Parity pins: every function here is pinned by tests that do not re-type
 * its arithmetic (printed worked example, closed forms, exact rational brute
 * force, library conversions, invariants).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL -1

/* ---- bf16 <-> wider floats ------------------------------------------------ */

/* A bf16 value is the upper half of an IEEE-754 binary32 pattern. */
float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round an fp64 value to bf16 (1 sign, 8 exponent bits with bias 127, 7
 * stored significand bits, subnormals), nearest, ties to even, in one step. */
uint16_t orc_f64_to_bf16(double v)
{
    if (isnan(v))
        return (uint16_t)0x7FC0;
    uint16_t sign = signbit(v) ? (uint16_t)0x8000 : (uint16_t)0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80);

    int e2;
    (void)frexp(a, &e2);        /* a = f * 2^e2, f in [0.5, 1) */
    int u = e2 - 1;             /* a in [2^u, 2^(u+1)) */
    double units;               /* a measured in units of the bf16 spacing */
    int subnormal = 0;
    if (u >= -126) {
        units = ldexp(a, 7 - u);        /* in [128, 256) */
    } else {
        units = ldexp(a, 133);          /* spacing 2^-133 below 2^-126 */
        subnormal = 1;
    }
    double fl = floor(units);
    double frac = units - fl;           /* exact: units has few integer bits */
    double r = fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0))
        r = fl + 1.0;

    uint32_t bits;
    if (subnormal) {
        bits = (uint32_t)r;             /* r == 128 lands on the smallest normal */
    } else {
        if (r == 256.0) {
            r = 128.0;
            u += 1;
        }
        if (u > 127)
            return (uint16_t)(sign | 0x7F80);
        bits = ((uint32_t)(u + 127) << 7) | ((uint32_t)r - 128u);
    }
    return (uint16_t)(sign | bits);
}

void orc_round_bf16(const double *y, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_f64_to_bf16(y[i]);
}

/* ---- packing ---------------------------------------------------------------- */

/* Eight 4-bit codes a..h -> one word, a in bits 0-3, h in bits 28-31. */
uint32_t orc_pack8(const uint8_t *c)
{
    uint32_t w = 0;
    for (int i = 0; i < 8; i++)
        w |= ((uint32_t)(c[i] & 0xFu)) << (4 * i);
    return w;
}

/* Code i (0..7) of a packed word. */
int orc_unpack(uint32_t w, int i)
{
    return (int)((w >> (4 * i)) & 0xFu);
}

/* codes[N][K] (one code per byte) -> qw[N][K/8]. */
int orc_pack_rows(const uint8_t *codes, int64_t N, int64_t K, uint32_t *qw)
{
    if (!codes || !qw || N < 0 || K < 0 || K % 8)
        return ORC_EINVAL;
    for (int64_t n = 0; n < N; n++)
        for (int64_t j = 0; j < K / 8; j++)
            qw[n * (K / 8) + j] = orc_pack8(codes + n * K + 8 * j);
    return ORC_OK;
}

int orc_unpack_rows(const uint32_t *qw, int64_t N, int64_t K, uint8_t *codes)
{
    if (!codes || !qw || N < 0 || K < 0 || K % 8)
        return ORC_EINVAL;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            codes[n * K + k] = (uint8_t)orc_unpack(qw[n * (K / 8) + k / 8], (int)(k % 8));
    return ORC_OK;
}

/* ---- dequantization ------------------------------------------------------- */

/* w = q * s + b as one fp32 fused multiply-add (s, b given as bf16 bits). */
float orc_dequant(uint16_t s_bits, uint16_t b_bits, int q)
{
    return fmaf(orc_bf16_to_f32(s_bits), (float)q, orc_bf16_to_f32(b_bits));
}

/* Weight (n, k) of one quantized matrix. */
static float weight_at(const uint32_t *qw, const uint16_t *scales, const uint16_t *biases,
                       int64_t K, int64_t G, int64_t n, int64_t k)
{
    int q = orc_unpack(qw[n * (K / 8) + k / 8], (int)(k % 8));
    int64_t g = k / G;
    return orc_dequant(scales[n * (K / G) + g], biases[n * (K / G) + g], q);
}

/* out[r][k] = w[rows[r], k]; rows == NULL means rows 0..N-1 (R = N). */
int orc_dequant_rows(const uint32_t *qw, const uint16_t *scales, const uint16_t *biases,
                     int64_t N, int64_t K, int64_t G, const int32_t *rows, int64_t R, float *out)
{
    if (!qw || !scales || !biases || !out || N < 0 || K <= 0 || G <= 0 || K % G || K % 8)
        return ORC_EINVAL;
    if (!rows)
        R = N;
    for (int64_t r = 0; r < R; r++) {
        int64_t n = rows ? rows[r] : r;
        if (n < 0 || n >= N)
            return ORC_EINVAL;
        for (int64_t k = 0; k < K; k++)
            out[r * K + k] = weight_at(qw, scales, biases, K, G, n, k);
    }
    return ORC_OK;
}

/* ---- the product -------------------------------------------------------------- */

/*
 * y[m][r] = sum_k x[m][k] * w[rows[r]][k] in fp64, ascending k; also
 * absy[m][r] = sum_k |x[m][k] * w[rows[r]][k]| (the scale of the error bound).
 * x is [M][K] bf16 bits.  rows == NULL: all N rows (R = N).  absy may be NULL.
 * Each weight is dequantized once per (n, k) and used for all M rows.
 */
int orc_qmm(const uint16_t *x, const uint32_t *qw, const uint16_t *scales, const uint16_t *biases,
            int64_t M, int64_t N, int64_t K, int64_t G, const int32_t *rows, int64_t R,
            double *y, double *absy)
{
    if (!x || !qw || !scales || !biases || !y || M <= 0 || N < 0 || K <= 0 || G <= 0 ||
        K % G || K % 8 || M > 4096)
        return ORC_EINVAL;
    if (!rows)
        R = N;
    double acc[4096];
    double aacc[4096];
    for (int64_t r = 0; r < R; r++) {
        int64_t n = rows ? rows[r] : r;
        if (n < 0 || n >= N)
            return ORC_EINVAL;
        for (int64_t m = 0; m < M; m++) {
            acc[m] = 0.0;
            aacc[m] = 0.0;
        }
        for (int64_t k = 0; k < K; k++) {
            double w = (double)weight_at(qw, scales, biases, K, G, n, k);
            for (int64_t m = 0; m < M; m++) {
                double p = (double)orc_bf16_to_f32(x[m * K + k]) * w;
                acc[m] += p;
                aacc[m] += fabs(p);
            }
        }
        for (int64_t m = 0; m < M; m++) {
            y[m * R + r] = acc[m];
            if (absy)
                absy[m * R + r] = aacc[m];
        }
    }
    return ORC_OK;
}

/*
 * Routed (expert-gathered) product.  Expert e owns rows [e*N, (e+1)*N) of the
 * stacked qw/scales/biases.  For token m and slot j:
 *   y[m][j][n] = sum_k xin[k] * W_{ids[m][j]}[n][k]
 * with xin = x[m] (x_per_slot == 0, x is [M][K]) or x[m][j] (x_per_slot != 0,
 * x is [M][top_k][K]).  An id outside [0, E) is an error.
 */
int orc_qmm_id(const uint16_t *x, int x_per_slot, const uint32_t *qw, const uint16_t *scales,
               const uint16_t *biases, const int32_t *ids, int64_t M, int64_t top_k, int64_t E,
               int64_t N, int64_t K, int64_t G, double *y, double *absy)
{
    if (!x || !qw || !scales || !biases || !ids || !y || M <= 0 || top_k <= 0 || E <= 0 ||
        N < 0 || K <= 0 || G <= 0 || K % G || K % 8)
        return ORC_EINVAL;
    for (int64_t m = 0; m < M; m++) {
        for (int64_t j = 0; j < top_k; j++) {
            int64_t e = ids[m * top_k + j];
            if (e < 0 || e >= E)
                return ORC_EINVAL;
            const uint16_t *xin = x_per_slot ? x + (m * top_k + j) * K : x + m * K;
            const uint32_t *qe = qw + e * N * (K / 8);
            const uint16_t *se = scales + e * N * (K / G);
            const uint16_t *be = biases + e * N * (K / G);
            double *yo = y + (m * top_k + j) * N;
            double *ao = absy ? absy + (m * top_k + j) * N : NULL;
            int rc = orc_qmm(xin, qe, se, be, 1, N, K, G, NULL, N, yo, ao);
            if (rc != ORC_OK)
                return rc;
        }
    }
    return ORC_OK;
}

/*
 * Argmax of y[0..N-1]: ascending scan, strict '>', so the lowest index wins a
 * tie.  *gap = y[best] - (largest value at any other index), or +inf if N == 1.
 */
int orc_argmax(const double *y, int64_t N, int64_t *best, double *gap)
{
    if (!y || !best || N <= 0)
        return ORC_EINVAL;
    int64_t b = 0;
    for (int64_t n = 1; n < N; n++)
        if (y[n] > y[b])
            b = n;
    double second = -INFINITY;
    for (int64_t n = 0; n < N; n++)
        if (n != b && y[n] > second)
            second = y[n];
    *best = b;
    if (gap)
        *gap = (N == 1) ? INFINITY : y[b] - second;
    return ORC_OK;
}

/*
 * GeGLU feed-forward activation (Gemma-4 E4B megakernel page, "What it does":
 * the MLP is GeGLU).  The pages name the activation only, so the definition
 * taken is the exact one: GELU(g) = g * Phi(g), Phi the standard normal CDF,
 * Phi(g) = (1 + erf(g / sqrt 2)) / 2, and the gated output h = GELU(gate) * up,
 * all in fp64.  gate[i], up[i] -> h[i] for i < n.
 */
int orc_geglu(const double *gate, const double *up, int64_t n, double *h)
{
    if (!gate || !up || !h || n < 0)
        return ORC_EINVAL;
    for (int64_t i = 0; i < n; i++) {
        double g = gate[i];
        double gelu = 0.5 * g * (1.0 + erf(g / sqrt(2.0)));
        h[i] = gelu * up[i];
    }
    return ORC_OK;
}
