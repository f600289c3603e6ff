/*
 * CPU oracle for the last-axis ArgMax / ArgMin reduction.
 *
 * TEST INFRASTRUCTURE ONLY. This library exists to check the HIP library, and is
 * loaded only by tests/, by __graft_entry__.smoke() and by the cpu_baseline leg of
 * bench.py. It shares no source, header, table or constant with the HIP path, and the
 * HIP path never loads it.
 *
 * What it computes (the definition, written out):
 *   For every row r of a contiguous row-major [rows, cols] tensor, the index that the
 *   sequential one-thread-per-row kernel returns. The ONNX Runtime pages define the
 *   result through that kernel: "[CUDA] Parallelize ArgMax/ArgMin over wide last axes"
 *   (Description, "Semantics": the parallel kernel must return, bit for bit, what the
 *   serial scan returns, for every input; ties go to the lowest index, i.e.
 *   select_last_index == 0; a leading NaN gives index 0; rows made only of -inf, +inf or
 *   NaN give index 0), and "[CUDA] Parallelize ArgMax/ArgMin over the reduction axis"
 *   (Semantics: element 0 is the starting candidate of the scan).
 *
 *   The scan: the running best starts as element 0 with index 0. Columns 1 .. cols-1
 *   are visited in increasing order; a column replaces the running best only when it
 *   compares strictly greater (ArgMax) or strictly less (ArgMin) under IEEE-754
 *   comparison, which is false whenever either operand is NaN. The index of the final
 *   running best is the result, stored as int64.
 *
 *   Last-index variants (ONNX's select_last_index = 1, which the first page names in its
 *   Semantics section and leaves to the CPU): the same scan with the non-strict comparison
 *   (greater-or-equal / less-or-equal), so that a later equal element replaces the
 *   running best. The pages define no more than that; this is the plain reading.
 *
 *   Elements are widened to double before they are compared. For f16, bf16 and f32 the
 *   widening is exact and order-preserving, NaN stays NaN and -0 / +0 keep comparing
 *   equal, so a comparison of two widened elements has the same outcome as the same
 *   comparison carried out in the element's own format. f16 and bf16 are decoded from
 *   their bit patterns below (IEEE-754 binary16; bfloat16 = the upper half of a binary32).
 *
 * Build: plain C, -O2, no fast-math, no flush-to-zero (oracle/__init__.py builds it).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* Element formats, numbered as the Python wrapper of this file numbers them. */
#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2
#define ORACLE_F64 3

#define ORACLE_ARGMAX 0
#define ORACLE_ARGMIN 1
#define ORACLE_ARGMAX_LAST 2
#define ORACLE_ARGMIN_LAST 3

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double mag;
    if (expo == 0x1f) {
        mag = frac ? NAN : INFINITY;
    } else if (expo == 0) {
        /* subnormal (or zero): frac * 2^-24 */
        mag = ldexp((double)frac, -24);
    } else {
        /* normal: (1024 + frac) * 2^(expo - 15 - 10) */
        mag = ldexp((double)(1024 + frac), expo - 25);
    }
    return sign ? -mag : mag;
}

/* bfloat16: the 16 most significant bits of an IEEE-754 binary32. */
static double decode_bf16(uint16_t b)
{
    const uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Element k (flat, row-major) of the tensor at x, widened to double. */
static double element(const void *x, int dtype, int64_t k)
{
    switch (dtype) {
    case ORACLE_F32: {
        float f;
        memcpy(&f, (const char *)x + k * 4, 4);
        return (double)f;
    }
    case ORACLE_F16: {
        uint16_t h;
        memcpy(&h, (const char *)x + k * 2, 2);
        return decode_f16(h);
    }
    case ORACLE_BF16: {
        uint16_t b;
        memcpy(&b, (const char *)x + k * 2, 2);
        return decode_bf16(b);
    }
    default: {
        double d;
        memcpy(&d, (const char *)x + k * 8, 8);
        return d;
    }
    }
}

/* Whether the scan moves from the running best to element a (IEEE comparisons: false
 * whenever either operand is NaN). */
static int moves(int op, double a, double best)
{
    int better;
    switch (op) {
    case ORACLE_ARGMAX: better = a > best; break;
    case ORACLE_ARGMIN: better = a < best; break;
    case ORACLE_ARGMAX_LAST: better = a >= best; break;
    default: better = a <= best; break;
    }
    return better;
}

/*
 * out[r] = index chosen by the sequential strict-compare scan of row r.
 * Returns 0 on success, -1 on an argument the definition does not cover
 * (cols < 1: an empty row has no index; unknown dtype or op).
 */
int oracle_argreduce_lastaxis(const void *x, int dtype, int64_t rows, int64_t cols,
                              int op, int64_t *out)
{
    if (rows < 0 || cols < 1 || dtype < ORACLE_F32 || dtype > ORACLE_F64 ||
        op < ORACLE_ARGMAX || op > ORACLE_ARGMIN_LAST)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t row0 = r * cols;
        double best = element(x, dtype, row0);
        int64_t idx = 0;
        for (int64_t j = 1; j < cols; ++j) {
            const double a = element(x, dtype, row0 + j);
            if (moves(op, a, best)) {
                best = a;
                idx = j;
            }
        }
        out[r] = idx;
    }
    return 0;
}

/*
 * Reduction over the middle axis of a contiguous [outer, len, inner] tensor:
 * out[o * inner + i] = index chosen by the same sequential scan over r = 0 .. len-1 of
 * the elements x[o][r][i] (flat position (o * len + r) * inner + i). With inner == 1 this
 * is the last-axis reduction above. ONNX Runtime's CUDA provider leaves this case to its
 * fallback ("[CUDA] Parallelize ArgMax/ArgMin over wide last axes", Semantics).
 */
int oracle_argreduce_axis(const void *x, int dtype, int64_t outer, int64_t len, int64_t inner,
                          int op, int64_t *out)
{
    if (outer < 0 || len < 1 || inner < 1 || dtype < ORACLE_F32 || dtype > ORACLE_F64 ||
        op < ORACLE_ARGMAX || op > ORACLE_ARGMIN_LAST)
        return -1;
    for (int64_t o = 0; o < outer; ++o) {
        for (int64_t i = 0; i < inner; ++i) {
            const int64_t base = o * len * inner + i;
            double best = element(x, dtype, base);
            int64_t idx = 0;
            for (int64_t r = 1; r < len; ++r) {
                const double a = element(x, dtype, base + r * inner);
                if (moves(op, a, best)) {
                    best = a;
                    idx = r;
                }
            }
            out[o * inner + i] = idx;
        }
    }
    return 0;
}

/* Every element of a flat array of n elements as the scan sees it (widened to double),
 * exported so that the decoders can be checked on their own. */
int oracle_widen(const void *x, int dtype, int64_t n, double *out)
{
    if (n < 0 || dtype < ORACLE_F32 || dtype > ORACLE_F64)
        return -1;
    for (int64_t k = 0; k < n; ++k)
        out[k] = element(x, dtype, k);
    return 0;
}
