/*
 * CPU oracle for the multi-token block-quantized mat-vec  y[t] = W . x[t].
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library; it decodes the packed bytes with its own
 * decoders, written from the IEEE-754 binary16 and bfloat16 bit definitions.
 *
 * What it computes (the plain definition, in fp64, one sequential k loop per
 * output):
 *
 *   y[t][r]     = sum_{k < cols} w[r][k] * x[t][k]
 *   bound[t][r] = sum_{k < cols} |w[r][k] * x[t][k]|
 *
 * with w the dequantised weight:
 *   Q8_0  w = d * c,        c the signed int8 code, d the block's fp16 scale
 *   Q4_0  w = d * (c - 8),  c the 4-bit code
 *   BF16  w = the bfloat16 value
 *
 * Sources: the mat-vec whose cost the pages measure as weight bytes / time
 * ("Where the time goes on an M2 Max", the 8192x2560 mat-vec table); ntok
 * activation vectors sharing one pass over the weights (M5 multi-token audit,
 * section 1 item 1 and the section 2.1 tile sweep); grouping tokens by expert
 * id (same audit, section 1 item 2); each token's sum being independent of the
 * token count (opus-mtp-turbo report, finding 3).  The block byte layouts are
 * the ggml Q8_0/Q4_0 ones that the pages' format names refer to: fp16 scale
 * first, then the codes; Q4_0 byte j holds code j in its low nibble and code
 * j + 16 in its high nibble.
 *
 * The file ends with the quantizers that make those blocks from fp32 values
 * (see the comment there for what they compute and why).
 *
 * Every function returns 0 on success, or a negative number for bad arguments
 * (the oracle raises where the library would return a status code).
 *
 * ORACLE_MUTANT (compile-time only, never set in the shipped build) plants
 * one deliberate mistake so the tests can show that the pins catch it.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

enum { ORACLE_Q8_0 = 0, ORACLE_Q4_0 = 1, ORACLE_BF16 = 2 };

/* ---------------------------------------------------------------- scalars */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0 -> subnormal  (-1)^s * f * 2^-24
 * exponent 31 -> inf / nan
 * otherwise   -> (-1)^s * (1024 + f) * 2^(e - 25)                            */
double oracle_fp16_to_f64(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    double v;
#if ORACLE_MUTANT == 6
    if (e == 0) v = 0.0; /* flush subnormals to zero */
#else
    if (e == 0) v = ldexp((double)f, -24);
#endif
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - 25);
    return s ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 * exponent 0 -> subnormal (-1)^s * f * 2^-133
 * exponent 255 -> inf / nan
 * otherwise  -> (-1)^s * (128 + f) * 2^(e - 134)                             */
double oracle_bf16_to_f64(uint16_t b)
{
    int s = b >> 15, e = (b >> 7) & 255, f = b & 127;
    double v;
    if (e == 0) v = ldexp((double)f, -133);
    else if (e == 255) v = f ? NAN : INFINITY;
    else v = ldexp((double)(128 + f), e - 134);
    return s ? -v : v;
}

static uint16_t le16(const uint8_t* p)
{
#if ORACLE_MUTANT == 7
    return (uint16_t)(p[1] | (p[0] << 8)); /* big-endian read */
#else
    return (uint16_t)(p[0] | (p[1] << 8));
#endif
}

/* ------------------------------------------------------------------ sizes */

/* Packed bytes per row: 34 B per 32 weights (Q8_0), 18 B per 32 (Q4_0), 2 B
 * per weight (BF16).  Returns -1 when cols is not a whole number of blocks. */
int64_t oracle_row_bytes(int fmt, int64_t cols)
{
    if (cols <= 0) return -1;
    switch (fmt) {
    case ORACLE_Q8_0: return cols % 32 ? -1 : cols / 32 * 34;
    case ORACLE_Q4_0: return cols % 32 ? -1 : cols / 32 * 18;
    case ORACLE_BF16: return cols * 2;
    }
    return -1;
}

int64_t oracle_packed_bytes(int fmt, int64_t rows, int64_t cols)
{
    int64_t rb = oracle_row_bytes(fmt, cols);
    return (rb < 0 || rows < 0) ? -1 : rb * rows;
}

/* ------------------------------------------------------------ dequantise */

/* Weight k of one row, from that row's packed bytes. */
static double weight_at(int fmt, const uint8_t* row, int64_t k)
{
    if (fmt == ORACLE_Q8_0) {
        int64_t b = k / 32, j = k % 32;
#if ORACLE_MUTANT == 4
        const uint8_t* blk = row + b * 34;
        double d = oracle_fp16_to_f64(le16(row)); /* every block takes block 0's scale */
#else
        const uint8_t* blk = row + b * 34;
        double d = oracle_fp16_to_f64(le16(blk));
#endif
        return d * (double)(int8_t)blk[2 + j];
    }
    if (fmt == ORACLE_Q4_0) {
        int64_t b = k / 32, j = k % 32;
        const uint8_t* blk = row + b * 18;
        double d = oracle_fp16_to_f64(le16(blk));
        int c;
#if ORACLE_MUTANT == 3
        c = (j % 2 == 0) ? (blk[2 + j / 2] & 15) : (blk[2 + j / 2] >> 4); /* pairwise nibble order */
#else
        c = (j < 16) ? (blk[2 + j] & 15) : (blk[2 + j - 16] >> 4);
#endif
#if ORACLE_MUTANT == 2
        return d * (double)(c + 8);
#else
        return d * (double)(c - 8);
#endif
    }
    return oracle_bf16_to_f64(le16(row + 2 * k));
}

/* out[r][k] = w[r][k] for the whole matrix (fp64, row-major). */
int oracle_dequant(int fmt, int64_t rows, int64_t cols, const uint8_t* W, double* out)
{
    int64_t rb = oracle_row_bytes(fmt, cols);
    if (rb < 0 || rows < 0 || !W || !out) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k)
            out[r * cols + k] = weight_at(fmt, W + r * rb, k);
    return 0;
}

/* The stored fields of each block: scale bits and codes (Q4_0 codes 0..15). */
int oracle_unpack(int fmt, int64_t rows, int64_t cols, const uint8_t* W, uint16_t* d_bits, int32_t* codes)
{
    int64_t rb = oracle_row_bytes(fmt, cols);
    if (rb < 0 || fmt == ORACLE_BF16 || !W || !d_bits || !codes) return -1;
    int64_t nb = cols / 32, bb = fmt == ORACLE_Q8_0 ? 34 : 18;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = W + r * rb + b * bb;
            d_bits[r * nb + b] = le16(blk);
            for (int j = 0; j < 32; ++j) {
                int c;
                if (fmt == ORACLE_Q8_0) c = (int8_t)blk[2 + j];
                else c = j < 16 ? (blk[2 + j] & 15) : (blk[2 + j - 16] >> 4);
                codes[r * cols + b * 32 + j] = c;
            }
        }
    return 0;
}

/* ------------------------------------------------------------- mat-vec */

/* One output: a sequential fp64 k loop over the dequantised row. */
static void dot_row(int fmt, const uint8_t* row, int64_t cols, const float* xt, double* y, double* bound)
{
    double s = 0.0, a = 0.0;
#if ORACLE_MUTANT == 1
    int64_t kend = cols - 32; /* drops the last block */
#else
    int64_t kend = cols;
#endif
    for (int64_t k = 0; k < kend; ++k) {
        double p = weight_at(fmt, row, k) * (double)xt[k];
        s += p;
        a += fabs(p);
    }
    *y = s;
    *bound = a;
}

/*
 * y[t][i], bound[t][i] for t < T and the selected rows sel[i] (i < nsel); if
 * sel is NULL, every row (nsel must equal rows).  x is [T][cols] fp32,
 * W the packed [rows] x [row bytes] matrix.
 */
int oracle_gemv(int fmt, int64_t rows, int64_t cols, int T, const uint8_t* W, const float* x,
                int64_t nsel, const int64_t* sel, double* y, double* bound)
{
    int64_t rb = oracle_row_bytes(fmt, cols);
    if (rb < 0 || rows <= 0 || T < 1 || !W || !x || !y || !bound) return -1;
    if (!sel && nsel != rows) return -1;
    for (int64_t i = 0; sel && i < nsel; ++i)
        if (sel[i] < 0 || sel[i] >= rows) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nsel; ++i) {
        int64_t r = sel ? sel[i] : i;
        for (int t = 0; t < T; ++t) {
#if ORACLE_MUTANT == 5
            const float* xt = x + (int64_t)(T - 1 - t) * cols; /* tokens reversed */
#else
            const float* xt = x + (int64_t)t * cols;
#endif
            dot_row(fmt, W + r * rb, cols, xt, &y[(int64_t)t * nsel + i], &bound[(int64_t)t * nsel + i]);
        }
    }
    return 0;
}

/*
 * Grouped experts: y[t][j][r] = W_{ids[t][j]} . x[t] for every slot (t, j),
 * written out slot by slot (no grouping: that the grouped kernel streams each
 * distinct expert once is a property of the kernel, not of the result).
 * W holds n_experts matrices of [rows][cols] back to back.  An id outside
 * [0, n_experts) is an error (-2).
 */
int oracle_grouped(int fmt, int64_t n_experts, int64_t rows, int64_t cols, int T, int topk,
                   const int32_t* ids, const uint8_t* W, const float* x, double* y, double* bound)
{
    int64_t rb = oracle_row_bytes(fmt, cols);
    if (rb < 0 || n_experts < 1 || rows <= 0 || T < 1 || topk < 1 || !ids || !W || !x || !y || !bound)
        return -1;
    for (int i = 0; i < T * topk; ++i)
        if (ids[i] < 0 || ids[i] >= n_experts) return -2;
    int64_t nslot = (int64_t)T * topk;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < nslot * rows; ++q) {
        int64_t slot = q / rows, r = q % rows;
        int t = (int)(slot / topk);
        const uint8_t* row = W + ((int64_t)ids[slot] * rows + r) * rb;
        dot_row(fmt, row, cols, x + (int64_t)t * cols, &y[q], &bound[q]);
    }
    return 0;
}

/*
 * The down projection of the routed experts: y[t][j][r] = W_{ids[t][j]}[r] . h[t][j],
 * one input row h[t][j] (cols values) per slot, written out slot by slot (M5
 * multi-token audit, section 1 item 2: the down projection applied to each
 * (token, expert) pair).  An id outside [0, n_experts) is an error (-2).
 */
int oracle_grouped_per_slot(int fmt, int64_t n_experts, int64_t rows, int64_t cols, int T, int topk,
                            const int32_t* ids, const uint8_t* W, const float* h, double* y, double* bound)
{
    int64_t rb = oracle_row_bytes(fmt, cols);
    if (rb < 0 || n_experts < 1 || rows <= 0 || T < 1 || topk < 1 || !ids || !W || !h || !y || !bound)
        return -1;
    for (int i = 0; i < T * topk; ++i)
        if (ids[i] < 0 || ids[i] >= n_experts) return -2;
    int64_t nslot = (int64_t)T * topk;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < nslot * rows; ++q) {
        int64_t slot = q / rows, r = q % rows;
        const uint8_t* row = W + ((int64_t)ids[slot] * rows + r) * rb;
#if ORACLE_MUTANT == 13
        dot_row(fmt, row, cols, h + (slot / topk) * cols, &y[q], &bound[q]); /* input of the token's first slot */
#else
        dot_row(fmt, row, cols, h + slot * cols, &y[q], &bound[q]);
#endif
    }
    return 0;
}

/* ------------------------------------------------------------ quantizers */
/*
 * The quantizers that produce the packed blocks on the device (opus-mtp-turbo:
 * Track 1 report, item 3 "Q4_0 / Q5_0 draft weights": Q4_0 draft weights made by
 * the "Lloyd" quantizer of the hyper-connection loader; "Where the time goes"
 * (meld-turbo-performance), the re-encoding of dense projections to Q8_0).  The
 * pages name the quantizers but print no procedure, so these are the plainest
 * readings: symmetric absmax rounding for Q8_0, the absmax rule that maps the
 * block's signed extreme to code 0 for Q4_0, and for "Lloyd" alternating
 * least-squares fits of the scale with nearest-level assignments of the codes,
 * started from the absmax rule.  Every decision that turns a float into a code
 * is taken in fp32, one operation at a time in the order written (no fused
 * multiply-add), because a code is an integer the two sides must agree on.
 */

/* fp32 -> binary16, round to nearest, ties to even, from the bit definition:
 * a finite |f| >= 65520 (the midpoint of 65504 and 2^16) overflows to inf;
 * below 2^-14 the value is an integer multiple of 2^-24 (subnormal, or the
 * smallest normal when it rounds up to 1024); otherwise 1024..2047 units of
 * 2^(e-10) for 2^e <= |f| < 2^(e+1).                                        */
uint16_t oracle_f32_to_fp16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if ((u & 0x7F800000u) == 0x7F800000u) return (u & 0x007FFFFFu) ? (uint16_t)(sign | 0x7E00u) : (uint16_t)(sign | 0x7C00u);
    double a = fabs((double)f); /* exact */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    if (a < ldexp(1.0, -14)) {
#if ORACLE_MUTANT == 12
        double n = floor(ldexp(a, 24)); /* truncates instead of rounding */
#else
        double n = nearbyint(ldexp(a, 24)); /* default rounding mode: nearest, ties to even */
#endif
        return (uint16_t)(sign | (uint16_t)n);
    }
    int e2;
    frexp(a, &e2); /* a = m * 2^e2, 0.5 <= m < 1, so 2^(e2-1) <= a < 2^e2 */
    int e = e2 - 1;
#if ORACLE_MUTANT == 12
    double n = floor(ldexp(a, 10 - e));
#else
    double n = nearbyint(ldexp(a, 10 - e)); /* 1024 <= n <= 2048 */
#endif
    if (n == 2048.0) {
        n = 1024.0;
        e += 1;
    }
    if (e + 15 >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(n - 1024.0));
}

void oracle_f32_to_fp16_array(int64_t n, const float* src, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_fp16(src[i]);
}

static void put_le16(uint8_t* p, uint16_t v)
{
    p[0] = (uint8_t)(v & 0xFF);
    p[1] = (uint8_t)(v >> 8);
}

/*
 * Q8_0: per block of 32, d = max|v| / 127 and code = round(v / d), computed as
 * v * (1/d) and rounded half away from zero; the block stores fp16(d).  A block
 * whose d rounds to a zero fp16 (max|v| below about 127 * 2^-25, all-zero blocks
 * included) decodes to zeros whatever its codes, and is stored with d = +0 and
 * codes 0.  Inputs must be finite (else -2).  out: rows * cols/32 blocks of 34
 * bytes.
 */
int oracle_quantize_q8_0(int64_t rows, int64_t cols, const float* src, uint8_t* out)
{
    if (rows <= 0 || cols <= 0 || cols % 32 || !src || !out) return -1;
    int64_t nblk = rows * (cols / 32);
    for (int64_t i = 0; i < nblk * 32; ++i)
        if (!isfinite(src[i])) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
        const float* v = src + b * 32;
        uint8_t* o = out + b * 34;
        float amax = 0.0f;
        for (int j = 0; j < 32; ++j) {
            float a = fabsf(v[j]);
            if (a > amax) amax = a;
        }
#if ORACLE_MUTANT == 8
        float d = amax / 128.0f; /* wrong level count */
#else
        float d = amax / 127.0f;
#endif
        uint16_t dh = oracle_f32_to_fp16(d);
        float id = 1.0f / d;
        if ((dh & 0x7FFF) == 0) {
            dh = 0;
            id = 0.0f;
        }
        put_le16(o, dh);
        for (int j = 0; j < 32; ++j) {
            float q = v[j] * id;
#if ORACLE_MUTANT == 9
            o[2 + j] = (uint8_t)(int8_t)(int)q; /* truncates */
#else
            o[2 + j] = (uint8_t)(int8_t)(int)roundf(q);
#endif
        }
    }
    return 0;
}

/* The Q4_0 absmax rule on one block: the element of largest magnitude (the
 * first one on ties), with its sign, is mapped to code 0, d = that value / -8,
 * code = min(15, trunc(v * (1/d) + 8.5)).  Returns d.  A block whose d rounds
 * to a zero fp16 is the zero block: d = +0, codes 8.                        */
static float q4_absmax(const float* v, int* c)
{
    float amax = 0.0f, vmax = 0.0f;
    for (int j = 0; j < 32; ++j)
        if (amax < fabsf(v[j])) {
            amax = fabsf(v[j]);
            vmax = v[j];
        }
#if ORACLE_MUTANT == 10
    (void)vmax;
    float d = amax / -8.0f; /* sign of the extreme dropped */
#else
    float d = vmax / -8.0f;
#endif
    float id = 1.0f / d;
    if ((oracle_f32_to_fp16(d) & 0x7FFF) == 0) {
        d = 0.0f;
        id = 0.0f;
    }
    for (int j = 0; j < 32; ++j) {
        float t = v[j] * id;
        t = t + 8.5f;
        int q = (int)t;
        c[j] = q < 15 ? q : 15;
    }
    return d;
}

/* "Lloyd": fit d to the codes by least squares, d = sum v*q / sum q*q with
 * q = code - 8 (the sums in index order), re-assign every code to the nearest
 * level for that d, clamp(floor(v * (1/d) + 8.5), 0, 15), and repeat until the
 * codes stop changing; at most ORACLE_LLOYD_ROUNDS fits.  The stored scale is
 * the last fit, so it is the least-squares scale of the stored codes.  The zero
 * block of the absmax rule (all codes 8) is kept as it is.  (Each term v*q has
 * the sign of d, and the fit is a weighted mean of v/q, so |d| <= max|v| keeps
 * the extreme's |q| >= 1: every fitted |d| is at least max|v| / 2048, a normal
 * fp32 whenever the start is not the zero block.)                           */
#define ORACLE_LLOYD_ROUNDS 8
static float q4_lloyd(const float* v, int* c)
{
    float d = q4_absmax(v, c);
#if ORACLE_MUTANT == 11
    return d; /* no refinement */
#endif
    for (int it = 0; it < ORACLE_LLOYD_ROUNDS; ++it) {
        float s1 = 0.0f;
        int s2 = 0;
        for (int j = 0; j < 32; ++j) {
            int q = c[j] - 8;
            s1 = s1 + v[j] * (float)q;
            s2 += q * q;
        }
        if (s2 == 0) break;
        d = s1 / (float)s2;
        if (it == ORACLE_LLOYD_ROUNDS - 1 || d == 0.0f) break;
        float id = 1.0f / d;
        int changed = 0;
        for (int j = 0; j < 32; ++j) {
            float t = v[j] * id;
            t = t + 8.5f;
            t = floorf(t);
            int q = t < 0.0f ? 0 : t > 15.0f ? 15 : (int)t;
            changed |= q != c[j];
            c[j] = q;
        }
        if (!changed) break;
    }
    return d;
}

/*
 * Q4_0: method 0 the absmax rule, method 1 the Lloyd refinement above.  Byte j
 * of a block's 16 code bytes holds code j in its low nibble and code j + 16 in
 * its high nibble.  out: rows * cols/32 blocks of 18 bytes.
 */
int oracle_quantize_q4_0(int64_t rows, int64_t cols, int method, const float* src, uint8_t* out)
{
    if (rows <= 0 || cols <= 0 || cols % 32 || !src || !out || (method != 0 && method != 1)) return -1;
    int64_t nblk = rows * (cols / 32);
    for (int64_t i = 0; i < nblk * 32; ++i)
        if (!isfinite(src[i])) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
        int c[32];
        float d = method ? q4_lloyd(src + b * 32, c) : q4_absmax(src + b * 32, c);
        uint8_t* o = out + b * 18;
        put_le16(o, oracle_f32_to_fp16(d));
        for (int j = 0; j < 16; ++j) o[2 + j] = (uint8_t)(c[j] | (c[j + 16] << 4));
    }
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the next calls use (the host's logical cores by default); timing only,
 * the results do not depend on it. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
