/*
 * CPU oracle for the last-axis ArgMax / ArgMin reduction, its middle-axis form, and the
 * cumulative (running) extremum with indices at the end of this file.
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

/* Element formats, numbered as the Python wrapper of this file numbers them. The integer
 * formats are read only by the cumulative scan at the end of this file. */
#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2
#define ORACLE_F64 3
#define ORACLE_I32 4
#define ORACLE_I64 5

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

/* ---------------------------------------------------------------------------------------
 * Cumulative maximum / minimum with indices along the last axis (the PaddlePaddle issue on
 * the cummax/cummin CUDA kernel: "[Performance] cummax/cummin ... dim3(16,32)": the scan
 * returns, for every position, the running extremum and its index; its fix proposals
 * describe the reduce operator as ArgMax semantics with ties going to the earlier index).
 *
 * Definition written out: for every row and every position j, the result at j is what the
 * sequential ArgMax (cummax) / ArgMin (cummin) scan above returns for the prefix of
 * elements 0 .. j: the running best starts as element 0 with index 0 and moves only to a
 * strictly greater (smaller) element, so ties keep the earlier index, a NaN never becomes
 * the running best except as element 0, and a leading NaN stays the running best for the
 * whole row. out_idx[r][j] is that index; out_val[r][j] is a copy of the storage bytes of
 * the element at that index (so a leading NaN is reported with its own bit pattern).
 *
 * The running best is kept as an index, and every comparison reads both elements in their
 * own format: floating-point elements widened to double as above (exact), integers as
 * int64_t (exact; a double would round integers beyond 2^53).
 * --------------------------------------------------------------------------------------- */

static int elem_size(int dtype)
{
    switch (dtype) {
    case ORACLE_F32: return 4;
    case ORACLE_F16: return 2;
    case ORACLE_BF16: return 2;
    case ORACLE_F64: return 8;
    case ORACLE_I32: return 4;
    case ORACLE_I64: return 8;
    default: return 0;
    }
}

static int64_t int_element(const void *x, int dtype, int64_t k)
{
    if (dtype == ORACLE_I32) {
        int32_t v;
        memcpy(&v, (const char *)x + k * 4, 4);
        return v;
    }
    int64_t v;
    memcpy(&v, (const char *)x + k * 8, 8);
    return v;
}

/* Whether element ka of x moves the scan from its running best, element kb. */
static int scan_moves(const void *x, int dtype, int op, int64_t ka, int64_t kb)
{
    if (dtype == ORACLE_I32 || dtype == ORACLE_I64) {
        const int64_t a = int_element(x, dtype, ka), b = int_element(x, dtype, kb);
        return op == ORACLE_ARGMAX ? a > b : a < b;
    }
    return moves(op, element(x, dtype, ka), element(x, dtype, kb));
}

/*
 * out_val (same format as x) and out_idx (int64), both [rows, cols], as defined above.
 * op: ORACLE_ARGMAX = cummax, ORACLE_ARGMIN = cummin. Returns 0, or -1 for arguments the
 * definition does not cover (cols < 1, unknown format, other ops).
 */
int oracle_cumulative(const void *x, int dtype, int64_t rows, int64_t cols, int op,
                      void *out_val, int64_t *out_idx)
{
    const int size = elem_size(dtype);
    if (rows < 0 || cols < 1 || size == 0 || (op != ORACLE_ARGMAX && op != ORACLE_ARGMIN))
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t row0 = r * cols;
        int64_t best = 0; /* index of the running best within the row */
        for (int64_t j = 0; j < cols; ++j) {
            if (j > 0 && scan_moves(x, dtype, op, row0 + j, row0 + best))
                best = j;
            out_idx[row0 + j] = best;
            memcpy((char *)out_val + (row0 + j) * size, (const char *)x + (row0 + best) * size,
                   (size_t)size);
        }
    }
    return 0;
}
