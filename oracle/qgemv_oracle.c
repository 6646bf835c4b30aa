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
 * Every function returns 0 on success, or a negative number for bad arguments
 * (the oracle raises where the library would return a status code).
 *
 * ORACLE_MUTANT (compile-time only, never set in the shipped build) plants
 * one deliberate mistake so the tests can show that the pins catch it.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

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

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
