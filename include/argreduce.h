/*
 * argreduce.h -- C ABI of the MI355X (gfx950) last-axis ArgMax / ArgMin library.
 *
 * One operation: for every row of a contiguous row-major [rows, cols] tensor, the int64
 * index of its maximum (ArgMax) or minimum (ArgMin). The result is defined by the
 * sequential one-thread-per-row scan described in "[CUDA] Parallelize ArgMax/ArgMin over
 * wide last axes" (ONNX Runtime pull request 32092), Description / Semantics:
 *   - the result equals, for every input, that of a scan that starts with element 0 as the
 *     running best and moves to a later element only when it compares strictly greater
 *     (ArgMax) or strictly less (ArgMin);
 *   - hence ties resolve to the lowest index (select_last_index == 0);
 *   - a NaN at index 0 yields 0, a NaN elsewhere is never selected (IEEE comparisons with
 *     NaN are false);
 *   - rows made only of -inf, +inf or NaN yield 0; -inf / +inf are ordinary values, which
 *     is why the parallel merge uses them, not the lowest / highest finite value, as the
 *     identity of an empty partial result.
 * Element formats are IEEE binary32 (f32), binary16 (f16), bfloat16 (bf16) and binary64
 * (f64); comparisons are exact (f16 and bf16 are widened exactly to binary32), subnormals
 * included.
 *
 * Threading, memory and streams (same page, Description / Approach and Testing):
 *   - every pointer argument is a DEVICE pointer owned by the caller; the library never
 *     allocates, frees or prints, and only argreduce_wait_timeouts (a diagnostic read of
 *     a device counter) synchronises;
 *   - all work is enqueued on the caller's HIP stream (`stream` is a hipStream_t, NULL for
 *     the default stream), so a call may be captured into a HIP graph and replayed;
 *   - functions are safe to call from several host threads; calls that share one scratch
 *     buffer must be ordered on one stream.
 *
 * Status codes: 0 on success, a negative ARGREDUCE_ERR_* value otherwise. On every error
 * except ARGREDUCE_ERR_HIP nothing has been enqueued and out_idx is untouched. One
 * device-side condition cannot be returned by the call, which returns before the kernels
 * run: should a workgroup of a split row never publish its result (not expected: those
 * workgroups wait on nothing), the row's finalizing workgroup gives up after a bounded
 * wait, stores -1 in out_idx[r] and adds one to the device's timeout count, which
 * argreduce_wait_timeouts reads.
 */
#ifndef ARGREDUCE_H
#define ARGREDUCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ARGREDUCE_F32 = 0,  /* IEEE binary32, 4-byte aligned */
    ARGREDUCE_F16 = 1,  /* IEEE binary16, 2-byte aligned */
    ARGREDUCE_BF16 = 2, /* bfloat16 (upper half of a binary32), 2-byte aligned */
    ARGREDUCE_F64 = 3,  /* IEEE binary64, 8-byte aligned */
    /* Integer formats: accepted by argreduce_scan_lastaxis only (the other entry points
     * return ARGREDUCE_ERR_UNSUPPORTED_DTYPE); compared exactly. */
    ARGREDUCE_I32 = 4,  /* int32, 4-byte aligned */
    ARGREDUCE_I64 = 5   /* int64, 8-byte aligned */
} argreduce_dtype_t;

typedef enum {
    ARGREDUCE_MAX = 0,      /* ArgMax, ties to the lowest index */
    ARGREDUCE_MIN = 1,      /* ArgMin, ties to the lowest index */
    /* Ties to the HIGHEST index: ONNX's select_last_index = 1, which the first page's
     * Semantics section names and leaves to the CPU. Defined here as the same sequential
     * scan with the non-strict comparison (>= / <=): a later equal element replaces the
     * running best, NaN is still never selected, a NaN at index 0 still yields 0, and a row
     * of all -inf (ArgMax) yields its last index. */
    ARGREDUCE_MAX_LAST = 2,
    ARGREDUCE_MIN_LAST = 3
} argreduce_op_t;

enum {
    ARGREDUCE_OK = 0,
    ARGREDUCE_ERR_INVALID_ARG = -1,      /* null pointer with rows > 0, rows < 0, cols < 1,
                                            bad op, misaligned x or out_idx */
    ARGREDUCE_ERR_UNSUPPORTED_DTYPE = -2,
    ARGREDUCE_ERR_TOO_WIDE = -3,         /* a reduced axis the entry point does not admit:
                                            len > INT32_MAX (argreduce_axis with inner > 1),
                                            cols > INT32_MAX (argreduce_scan_lastaxis), or
                                            more workgroups than a grid holds */
    ARGREDUCE_ERR_SCRATCH_TOO_SMALL = -4,/* scratch_bytes below argreduce_scratch_bytes() */
    ARGREDUCE_ERR_HIP = -5,              /* a HIP call or kernel launch failed */
    ARGREDUCE_ERR_NO_DEVICE = -6         /* no current HIP device to plan for */
};

/*
 * Bytes of scratch that argreduce_lastaxis needs for this shape on the CURRENT device
 * ("[CUDA] Parallelize ArgMax/ArgMin over wide last axes", Description / Approach: the
 * caller allocates the intermediate buffer; its size is bounded by the device's thread
 * capacity, so it stays in the low kilobytes for any shape).
 *
 * Returns 0 when the chosen launch needs no scratch, else 16 bytes (32 for F64) per
 * (row, workgroup) of a split row, or 16 bytes per (row, window) of a row wider than
 * INT32_MAX, plus 15 bytes of slack, so the buffer may start at any byte address. Returns
 * SIZE_MAX on an invalid argument (rows < 0, cols < 1, bad dtype) or when there is no
 * current device.
 */
size_t argreduce_scratch_bytes(int64_t rows, int64_t cols, argreduce_dtype_t dtype);

/*
 * out_idx[r] = ArgMax / ArgMin of row r of x, for r in [0, rows).
 *
 *   x             device pointer to rows * cols elements of `dtype`, row-major, rows
 *                 contiguous (row r starts at element r * cols); aligned to the element
 *                 size. Read only. rows * cols * element size must fit in int64.
 *   rows          >= 0; rows == 0 is a no-op that returns ARGREDUCE_OK.
 *   cols          >= 1 (an empty row has no index). rows * cols may exceed 2^31. Rows wider
 *                 than INT32_MAX are cut into windows of at most 2^30 elements (positions
 *                 stay 32-bit inside a window; "[CUDA] Parallelize ArgMax/ArgMin over wide
 *                 last axes", "Why not int64 positions"); each window's candidate carries
 *                 its 64-bit index to a merge kernel (ARGREDUCE_PATH_WIDE, two dispatches).
 *   out_idx       device pointer to `rows` int64 values, 8-byte aligned. Written only on
 *                 success; each value lies in [0, cols).
 *   scratch       device pointer to at least argreduce_scratch_bytes(rows, cols, dtype)
 *                 bytes, at any byte alignment, with any contents on entry: a row split
 *                 over several workgroups publishes two 8-byte words per workgroup (three
 *                 for F64), each tagged with a per-call nonce, and the call ignores words
 *                 that do not carry its own nonce and an in-range index (arbitrary
 *                 contents pass that filter with probability below 2^-32 per word). May be
 *                 NULL when that figure is 0. The call leaves the words it used zeroed.
 *                 Calls that can run at the same time (on different streams) need
 *                 separate scratch buffers.
 *   scratch_bytes size of the scratch buffer in bytes.
 *   stream        hipStream_t on which all work is enqueued (NULL = default stream).
 *
 * The call returns after enqueuing; results are ready when the stream reaches that point.
 */
int argreduce_lastaxis(const void *x, argreduce_dtype_t dtype, int64_t rows, int64_t cols,
                       argreduce_op_t op, int64_t *out_idx, void *scratch,
                       size_t scratch_bytes, void *stream);

/* ----------------------------------------------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph capture that must
 * not call hipMalloc, tight serving loops, harnesses that forbid allocation.
 *
 * argreduce_lastaxis without the scratch arguments: the scratch is a buffer the library
 * holds, a device array of ARGREDUCE_NOALLOC_SCRATCH_BYTES bytes, one copy per device,
 * located on the first call on that device and kept until the process ends. Same
 * arguments otherwise, same results, kernels and status codes; the call allocates and
 * frees nothing. Returns ARGREDUCE_ERR_SCRATCH_TOO_SMALL, before enqueuing anything, when
 * argreduce_scratch_bytes(rows, cols, dtype) exceeds ARGREDUCE_NOALLOC_SCRATCH_BYTES (on
 * MI355X no shape does: the split path needs at most 32 bytes per resident workgroup,
 * 65,551 bytes in all, and rows wider than INT32_MAX a few tens of KiB at any size that
 * fits in memory); ARGREDUCE_ERR_HIP when the buffer cannot be located.
 *
 * Every call on one device shares that device's buffer, which keeps the last call's
 * contents (the next call needs nothing cleared: its words carry a per-call nonce). Calls
 * that can overlap on one device (several streams, several host threads) race on the
 * buffer and may return wrong indices: the caller must order them, e.g. on one stream.
 */
#define ARGREDUCE_NOALLOC_SCRATCH_BYTES (128u * 1024u)
int argreduce_lastaxis_noalloc(const void *x, argreduce_dtype_t dtype, int64_t rows,
                               int64_t cols, argreduce_op_t op, int64_t *out_idx, void *stream);

/* ----------------------------------------------------------------------------------------
 * Launch plan and test hooks. The pages' tests force every dispatch path and simulate
 * devices of several thread capacities ("[CUDA] Parallelize ArgMax/ArgMin over wide last
 * axes", Description / Testing); these entry points expose the same controls.
 */

typedef enum {
    ARGREDUCE_PATH_AUTO = -1,
    ARGREDUCE_PATH_SUBWAVE = 0, /* a group of 1..64 lanes of one wavefront per row */
    ARGREDUCE_PATH_BLOCK = 1,   /* one workgroup per row, rows looped over the grid */
    ARGREDUCE_PATH_SPLIT = 2,   /* several workgroups per row; the highest-id one merges */
    ARGREDUCE_PATH_AXIS = 3,    /* middle-axis reduction: a tile of consecutive outputs per
                                   workgroup, thread rows along the axis (argreduce_axis) */
    ARGREDUCE_PATH_SCAN = 4,    /* cumulative scan: a tile of a row per workgroup, tiles of
                                   a row chained by look-back (argreduce_scan_lastaxis) */
    ARGREDUCE_PATH_WIDE = 5,    /* rows wider than INT32_MAX: windows of <= 2^30 elements,
                                   one workgroup each, merged by a second dispatch */
    ARGREDUCE_PATH_THREAD = 6   /* forced only, never chosen: one lane scans each row alone,
                                   the pages' serial thread-per-row kernel, for a "before"
                                   timing from the same library ("[CUDA] Parallelize
                                   ArgMax/ArgMin over wide last axes", Verification log);
                                   its plan reads as ARGREDUCE_PATH_SUBWAVE with one lane */
} argreduce_path_t;

typedef struct {
    int32_t path;             /* argreduce_path_t */
    int32_t lanes_per_row;    /* lanes that scan one row */
    int32_t blocks_per_row;   /* workgroups per row (1 unless SPLIT) */
    int32_t block_threads;    /* threads per workgroup */
    int64_t grid_blocks;      /* workgroups launched */
    int64_t grid_rows;        /* rows in flight at once (rows beyond are looped over) */
    int32_t unroll;           /* loads each lane keeps in flight per step */
    int32_t outputs_per_block;/* outputs one workgroup produces at a time */
    int64_t device_threads;   /* thread capacity the plan was made for */
    size_t scratch_bytes;     /* == argreduce_scratch_bytes() for the same arguments */
    int32_t load_bytes;       /* bytes of one lane load in the body of the scan: 16, or the
                                 element size for an AXIS plan whose `inner` row is not a
                                 multiple of 16 bytes */
    int32_t dispatches;       /* kernels one call launches: 1, or 2 for an AXIS or WIDE plan
                                 whose workgroups store partials that a second kernel merges */
    int64_t window;           /* WIDE: elements per window (one workgroup each); else 0 */
} argreduce_plan_t;

/* The plan argreduce_lastaxis would use for these arguments on the current device. */
int argreduce_plan(int64_t rows, int64_t cols, argreduce_dtype_t dtype, argreduce_plan_t *plan);

/* Plan as if the device held `threads` resident threads (0 = the real device). Process-wide.
 * Lets tests reach the row-loop and split paths of devices of other sizes, and lets
 * argreduce_plan / argreduce_scratch_bytes run without a GPU. */
int argreduce_debug_set_capacity(int64_t threads);

/* Force one path (ARGREDUCE_PATH_AUTO restores the automatic choice). Process-wide.
 * A forced path keeps its own geometry rules; a forced SPLIT uses at least two workgroups
 * per row, however short the row; a forced WIDE cuts every row into windows (of the size
 * set below, else the automatic one). SUBWAVE, BLOCK, SPLIT, WIDE and THREAD can be
 * forced (THREAD: 16-byte loads, one in flight per lane, so milliseconds per call on rows
 * of 10^5 elements). */
int argreduce_debug_force_path(int path);

/* Force the split path's geometry for every last-axis plan: blocks_per_row workgroups per
 * row (2 .. the plan's maximum, 1024) and unroll 16-byte loads per lane per step (1, 2, 4 or
 * 8); rows longer than one step take several. blocks_per_row = 0 restores the automatic
 * plans. Process-wide; for measuring plan alternatives (a forced grid may exceed what is
 * resident at once, and then relies on the in-order start of workgroups). Returns
 * ARGREDUCE_ERR_INVALID_ARG for other values. */
int argreduce_debug_force_split(int64_t blocks_per_row, int unroll);

/* Window size of the WIDE path in elements, 1 .. 2^30 (0 = automatic). Process-wide. Lets
 * tests run the windowed path on rows small enough for the CPU oracle. */
int argreduce_debug_set_window(int64_t elements);

/* ----------------------------------------------------------------------------------------
 * Reduction over a middle axis.
 *
 * out_idx[o * inner + i] = ArgMax / ArgMin over r in [0, len) of x[o][r][i], for a contiguous
 * row-major [outer, len, inner] tensor (flat position (o * len + r) * inner + i): ONNX's
 * ArgMax/ArgMin over any axis after collapsing the dimensions before it into `outer` and
 * those after it into `inner`. The first page (Semantics) notes that its CUDA provider
 * sends non-last axes to a fallback; the semantics here are exactly those of
 * argreduce_lastaxis applied to each (o, i) column, for every op. inner == 1 IS
 * argreduce_lastaxis (rows = outer, cols = len), with the same scratch and plan.
 *
 *   outer >= 0 (0 is a no-op), 1 <= len <= INT32_MAX, inner >= 1. Pointers, alignment,
 *   scratch, stream and status codes as for argreduce_lastaxis; out_idx holds
 *   outer * inner int64 values.
 *
 *   When few outputs leave the device idle, the axis is split over several workgroups per
 *   tile of outputs: each stores a (value, index) partial per output in scratch, and a
 *   second kernel, enqueued on the same stream, merges them (the plan's `dispatches` is
 *   then 2; nothing waits on another workgroup, so no output is ever -1). 16-byte loads
 *   are used when inner * element size is a multiple of 16 and x is 16-byte aligned; the
 *   scratch size returned covers both cases.
 */
size_t argreduce_axis_scratch_bytes(int64_t outer, int64_t len, int64_t inner,
                                    argreduce_dtype_t dtype);
int argreduce_axis(const void *x, argreduce_dtype_t dtype, int64_t outer, int64_t len,
                   int64_t inner, argreduce_op_t op, int64_t *out_idx, void *scratch,
                   size_t scratch_bytes, void *stream);
/* The plan argreduce_axis would use for a 16-byte aligned x (path ARGREDUCE_PATH_AXIS
 * unless inner == 1). */
int argreduce_axis_plan(int64_t outer, int64_t len, int64_t inner, argreduce_dtype_t dtype,
                        argreduce_plan_t *plan);

/* ----------------------------------------------------------------------------------------
 * Cumulative extremum with indices along the last axis: cummax / cummin.
 *
 * The PaddlePaddle issue on the cummax/cummin CUDA kernel (its reproduction scans the last
 * axis of [rows, cols] tensors; its fix proposals describe the operator as a (value,
 * index) reduce with ArgMax semantics, ties to the earlier index). For every row r and
 * position j:
 *   out_idx[r*cols + j]    = the index the ArgMax (op ARGREDUCE_MAX: cummax) / ArgMin
 *                            (ARGREDUCE_MIN: cummin) scan of x[r][0..j] returns, with the
 *                            semantics of argreduce_lastaxis: ties keep the earlier index,
 *                            a NaN after position 0 is never taken, a NaN at position 0
 *                            holds for the whole row (index 0);
 *   out_values[r*cols + j] = a copy of the element x[r][out_idx[r*cols + j]] (same format
 *                            and bits as x; a leading NaN keeps its own bit pattern).
 *
 *   Formats: F32, F16, BF16, F64, I32, I64 (integers compared exactly). Ops: ARGREDUCE_MAX
 *   and ARGREDUCE_MIN only. 1 <= cols <= INT32_MAX, rows >= 0 (0 is a no-op). x and
 *   out_values aligned to the element size, out_idx to 8 bytes; 16-byte aligned rows
 *   (x, out_values and out_idx 16-byte aligned and cols * element size a multiple of 16)
 *   move as 16-byte vectors. out_values and out_idx hold rows * cols elements each and must
 *   not overlap x.
 *
 *   Scratch: rows longer than one tile (argreduce_scan_plan's outputs_per_block elements)
 *   chain their tiles through per-tile state words in scratch (any contents on entry);
 *   argreduce_scan_scratch_bytes gives the size (0 when every row fits in one tile;
 *   SIZE_MAX for invalid arguments). One dispatch per call; when `stream` is being
 *   captured into a HIP graph, a small kernel that clears the state words is enqueued
 *   before it, so that graph replays stay correct. Calls that can run at the same time
 *   need separate scratch buffers. Status codes as argreduce_lastaxis;
 *   ARGREDUCE_ERR_TOO_WIDE also when rows * tiles per row exceeds 2^32 - 1.
 */
size_t argreduce_scan_scratch_bytes(int64_t rows, int64_t cols, argreduce_dtype_t dtype);
int argreduce_scan_lastaxis(const void *x, argreduce_dtype_t dtype, int64_t rows, int64_t cols,
                            argreduce_op_t op, void *out_values, int64_t *out_idx,
                            void *scratch, size_t scratch_bytes, void *stream);
/* The plan argreduce_scan_lastaxis would use for 16-byte aligned buffers (path
 * ARGREDUCE_PATH_SCAN; blocks_per_row = tiles per row, outputs_per_block = elements per
 * tile). */
int argreduce_scan_plan(int64_t rows, int64_t cols, argreduce_dtype_t dtype,
                        argreduce_plan_t *plan);

/* Measurement hook: the launch floor. Enqueues one empty kernel (one workgroup of 64
 * threads) on `stream`, the same way argreduce_lastaxis enqueues its kernels, so that a
 * benchmark can time bare launch latency in the same harness ("[CUDA] Parallelize
 * ArgMax/ArgMin over wide last axes", Description / Results: per-call times include the
 * launch). Returns ARGREDUCE_OK or ARGREDUCE_ERR_HIP. */
int argreduce_debug_launch_empty(void *stream);

/* Measurement hook: the floor of a call that delivers a result. Enqueues one workgroup of
 * a kernel that takes one pointer argument and stores one int64 (0) at `out` (8-byte
 * aligned device memory) — the same launch and kernel-argument cost as every entry point,
 * with no data read. Returns ARGREDUCE_OK, ARGREDUCE_ERR_INVALID_ARG or ARGREDUCE_ERR_HIP. */
int argreduce_debug_launch_store(int64_t *out, void *stream);

/* Measurement hook: the practical read roofline. Enqueues on `stream` a plain streaming
 * read of `bytes` (a non-zero multiple of 16) at `x` (16-byte aligned device memory) by
 * `grid` workgroups of 256 threads (1 .. 65536): grid-stride 16-byte nontemporal loads, four
 * in flight per lane, folded with XOR. `out` (device memory of `grid` uint32 words, 4-byte
 * aligned) is written only when a workgroup's XOR equals one fixed 32-bit pattern, so in
 * practice nothing is written; the kernel does none of the reduction's work. Returns
 * ARGREDUCE_OK, ARGREDUCE_ERR_INVALID_ARG or ARGREDUCE_ERR_HIP. */
int argreduce_debug_launch_read(const void *x, size_t bytes, uint32_t *out, int64_t grid,
                                void *stream);

/* Test hook for the bounded waits (the split ArgMax path's finalizing workgroup, the scan's
 * look-back): polls of one published word before the wait gives up, the affected outputs
 * become -1 and argreduce_wait_timeouts counts it (0 restores the default, 2^20 polls). Process-wide. With a tiny limit
 * a wait can give up although nothing is wrong; this lets tests drive the time-out path
 * from the host while every kernel still ends normally. */
int argreduce_debug_set_spin_limit(uint32_t polls);

/* Bounded waits that gave up on the CURRENT device since the library was loaded. Two kinds
 * of workgroup wait for results that other workgroups of the same launch publish: the
 * finalizing workgroup of a split row (argreduce_lastaxis, "[CUDA] Parallelize ArgMax/ArgMin
 * over wide last axes", Description / Approach: the last block merges the partials) and a
 * tile of a long cumulative-scan row (argreduce_scan_lastaxis). Each stops after a bounded
 * number of polls (argreduce_debug_set_spin_limit); its outputs then hold -1 and the count
 * goes up by one per row (split) or per tile (scan). No wait is expected to give up unless a
 * test forces a tiny limit; a caller that must rule it out compares the count before and
 * after its calls. Copies the device's counter to *count synchronously, after the work
 * already enqueued on the default stream (call it off the hot path). Returns ARGREDUCE_OK,
 * ARGREDUCE_ERR_INVALID_ARG (count NULL), ARGREDUCE_ERR_NO_DEVICE or ARGREDUCE_ERR_HIP. */
int argreduce_wait_timeouts(uint64_t *count);

/* Measurement hook: when both are non-NULL, every later call launches its main kernel
 * (not a merge or clear kernel) with `start` recorded just before and
 * `stop` just after it on the same stream (hipEvent_t values created by the caller with
 * timing enabled); NULL, NULL turns this off. Process-wide; for benchmarks only. */
int argreduce_debug_set_kernel_events(void *start, void *stop);

#ifdef __cplusplus
}
#endif

#endif /* ARGREDUCE_H */
