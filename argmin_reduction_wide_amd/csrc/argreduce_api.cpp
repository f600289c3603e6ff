// C ABI of the last-axis ArgMax / ArgMin library: argument checks, launch planning, scratch
// sizing, and the test hooks. Declarations and the contract are in include/argreduce.h.
//
// Launch planning follows the geometry rule of "[CUDA] Parallelize ArgMax/ArgMin over wide
// last axes" (Description / Approach): aim at about one wave of resident threads over the
// device, give every lane a minimum amount of the row, and split a row over several
// workgroups only when there are too few rows to fill the device, so that the scratch
// holding the partials stays bounded by the device's thread capacity. The thresholds are
// re-derived for gfx950: 64-lane wavefronts, 256 CUs of 2048 resident threads, and 16-byte
// vector loads as the unit of work of a lane.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <limits>

#include "argreduce.h"
#include "argreduce_internal.hpp"

#define ARGREDUCE_EXPORT extern "C" __attribute__((visibility("default")))

namespace argreduce {
namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kBlock = 256;
constexpr int64_t kWave = 64;
// Rows of up to this many 16-byte vectors (4 KiB) are scanned by one wavefront; rows of up
// to kBlockRowMaxVec (32 KiB) by one workgroup with all of a lane's loads in one step.
constexpr int64_t kWaveRowMaxVec = 256;
// Middle axis: at most one wavefront of lanes along `inner` per tile.
constexpr int64_t kAxisMaxLanes = 64;
constexpr int64_t kBlockRowMaxVec = 2048;
constexpr int64_t kMaxBlocksPerRow = 1024;
// Rows too wide for one step of loads (or too many to split in one device wave) use at most
// 1/kSplitFillDiv of a device wave of workgroups: there the call is bandwidth-bound, and
// fewer workgroups per row (fewer partials to merge) measured faster than filling the device.
constexpr int64_t kSplitFillDiv = 4;
// Grids hold at most this many device-fulls of workgroups; further rows are looped over.
// Many-row shapes run fastest with every row's team launched at once (the dispatcher keeps
// the CUs fed), so the cap only bounds pathological row counts.
constexpr int64_t kOversubscribe = 64;
// 16-byte loads in flight per lane: more costs registers (and with them occupancy);
// 8-byte elements need twice the registers per loaded vector.
constexpr int64_t kMaxUnrollWave = 8;
constexpr int64_t kMaxUnrollWaveF64 = 4;
constexpr int64_t kMaxUnrollBlocks = 8;

std::atomic<int64_t> g_device_threads[kMaxDevices];
std::atomic<int64_t> g_capacity_override{0};
std::atomic<int> g_force_path{ARGREDUCE_PATH_AUTO};
// Forced split geometry (debug hook): workgroups per row (0 = automatic) and loads per lane.
std::atomic<int64_t> g_force_split_b{0};
std::atomic<int> g_force_split_u{0};
std::atomic<int64_t> g_window{0};
constexpr int64_t kMaxWindow = int64_t{1} << 30;
// Workgroups of the streaming-read measurement kernel.
constexpr int64_t kMaxReadGrid = 65536;

int64_t elem_size(int dtype) {
    switch (dtype) {
        case ARGREDUCE_F32: return 4;
        case ARGREDUCE_F16: return 2;
        case ARGREDUCE_BF16: return 2;
        case ARGREDUCE_F64: return 8;
        default: return 0;
    }
}

int device_threads(int64_t* threads) {
    const int64_t forced = g_capacity_override.load(std::memory_order_relaxed);
    if (forced > 0) {
        *threads = forced;
        return ARGREDUCE_OK;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ARGREDUCE_ERR_NO_DEVICE;
    if (dev < kMaxDevices) {
        const int64_t cached = g_device_threads[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *threads = cached;
            return ARGREDUCE_OK;
        }
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxThreadsPerMultiProcessor, dev) !=
            hipSuccess ||
        cus <= 0 || per_cu <= 0)
        return ARGREDUCE_ERR_NO_DEVICE;
    const int64_t t = static_cast<int64_t>(cus) * per_cu;
    if (dev < kMaxDevices) g_device_threads[dev].store(t, std::memory_order_relaxed);
    *threads = t;
    return ARGREDUCE_OK;
}

int64_t next_pow2(int64_t v) {
    int64_t p = 1;
    while (p < v) p <<= 1;
    return p;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// 16-byte vectors from the one holding a row's first byte to the one holding its last, for
// the worst row of a 16-byte aligned tensor: row r starts r * row_bytes bytes in, so its
// misalignment is at most 16 - g, where g is the largest power of two (at most 16) dividing
// row_bytes (0 for a single row).
int64_t span_vecs(int64_t rows, int64_t row_bytes) {
    const int64_t g = row_bytes % 16 == 0 ? 16 : (row_bytes & -row_bytes);
    return ceil_div((rows <= 1 ? 0 : 16 - g) + row_bytes, 16);
}

int check_shape(int64_t rows, int64_t cols, int dtype) {
    if (elem_size(dtype) == 0) return ARGREDUCE_ERR_UNSUPPORTED_DTYPE;
    if (rows < 0 || cols < 1) return ARGREDUCE_ERR_INVALID_ARG;
    // rows * cols * element size must fit in int64 (cols * 8 cannot overflow first)
    if (cols > std::numeric_limits<int64_t>::max() / 8 ||
        rows > std::numeric_limits<int64_t>::max() / (cols * elem_size(dtype)))
        return ARGREDUCE_ERR_INVALID_ARG;
    return ARGREDUCE_OK;
}

// Window plan of rows wider than INT32_MAX (or of any row when the path is forced).
int make_wide_plan(int64_t rows, int64_t cols, int dtype, int64_t cap, Plan* p) {
    const int64_t cap_blocks = cap / kBlock > 0 ? cap / kBlock : 1;
    const int64_t rows1 = rows > 0 ? rows : 1;
    int64_t W = g_window.load(std::memory_order_relaxed);
    if (W <= 0) {
        // about one resident workgroup per window over the device, in whole 4096-element
        // blocks, at most 2^30 elements (positions inside a window stay 32-bit)
        const int64_t per_row = cap_blocks / rows1 > 0 ? cap_blocks / rows1 : 1;
        W = ceil_div(ceil_div(cols, per_row), 4096) * 4096;
        W = W < kMaxWindow ? W : kMaxWindow;
    }
    const int64_t G = ceil_div(cols, W);
    if (rows1 > static_cast<int64_t>(std::numeric_limits<uint32_t>::max()) / G)
        return ARGREDUCE_ERR_TOO_WIDE;
    *p = Plan{};
    p->path = ARGREDUCE_PATH_WIDE;
    p->block_threads = static_cast<int>(kBlock);
    p->device_threads = cap;
    p->window = W;
    p->windows = G;
    p->blocks_per_row = static_cast<int>(G < std::numeric_limits<int>::max() ? G : std::numeric_limits<int>::max());
    p->lanes_per_row = static_cast<int>(std::min<int64_t>(G * kBlock, std::numeric_limits<int>::max()));
    // 8 vectors per lane per step once a window spans many steps of 256 lanes
    p->unroll = W * elem_size(dtype) >= kBlock * 16 * 8 ? 8 : 2;
    p->grid_rows = rows1;
    p->grid_blocks = rows1 * G;
    p->entry_bytes = wide_partial_bytes(dtype);
    p->scratch_bytes = 15 + static_cast<size_t>(rows1) * static_cast<size_t>(G) * p->entry_bytes;
    return ARGREDUCE_OK;
}

int make_plan(int64_t rows, int64_t cols, int dtype, Plan* p) {
    int rc = check_shape(rows, cols, dtype);
    if (rc != ARGREDUCE_OK) return rc;
    int64_t cap = 0;
    rc = device_threads(&cap);
    if (rc != ARGREDUCE_OK) return rc;

    if (cols > std::numeric_limits<int32_t>::max() ||
        g_force_path.load(std::memory_order_relaxed) == ARGREDUCE_PATH_WIDE)
        return make_wide_plan(rows, cols, dtype, cap, p);

    const int64_t vec_row = ceil_div(cols * elem_size(dtype), 16);  // 16-byte vectors per row
    const int64_t cap_blocks = cap / kBlock > 0 ? cap / kBlock : 1;
    const int64_t rows1 = rows > 0 ? rows : 1;
    // Split rows: the fewest 16-byte loads per lane (U) for which one step of
    // B = ceil(vec_row / (256 U)) workgroups per row covers the row, with the workgroups of
    // every row in one device wave. First with U <= 4 and B <= 65, so that the row's
    // finalizing workgroup receives at most one published candidate per lane of one
    // wavefront, which then polls and merges them alone; then with U <= 8 and B <= 256 (at
    // most one candidate per thread of the finalizer: a second costs a second round trip).
    // Measured per call on MI355X: [1,202048] fp32 3.58 us with B = 198, U = 1, against
    // 3.24-3.28 with U = 2 or 4 (B = 99, 50) and 3.60 with U = 8; [8,202048] fp32 4.39 (U =
    // 1), 4.24 (U = 4); [32,202048] fp16 5.26 (U = 2, B = 50), 5.80 (U = 8); [1,2^20] fp32
    // 3.96 (U = 4, B = 256), 4.08 (U = 8). Failing both, 8 loads per lane and a share of the
    // device's workgroups per row; the row then takes several steps.
    int64_t split_b = 0;
    for (int tier = 0; tier < 2 && split_b == 0; ++tier) {
        const int64_t max_b = tier == 0 ? kWave + 1 : kBlock;
        const int64_t max_u = tier == 0 ? 4 : kMaxUnrollBlocks;
        for (int64_t u = 1; u <= max_u; u *= 2) {
            const int64_t b = ceil_div(vec_row, kBlock * u);
            if (b <= max_b && b * rows1 <= cap_blocks) {
                split_b = b;
                break;
            }
        }
    }
    if (split_b == 0) {
        split_b = cap_blocks / kSplitFillDiv / rows1;
        split_b = split_b < kMaxBlocksPerRow ? split_b : kMaxBlocksPerRow;
    }

    int path = g_force_path.load(std::memory_order_relaxed);
    int64_t group = 64, blocks_per_row = 1;
    if (path == ARGREDUCE_PATH_AUTO) {
        if (vec_row <= 32) {
            path = ARGREDUCE_PATH_SUBWAVE;
            group = next_pow2(vec_row);
        } else if (vec_row <= kWaveRowMaxVec) {
            path = ARGREDUCE_PATH_SUBWAVE;
            group = 64;
        } else if (vec_row <= kBlockRowMaxVec) {
            // one workgroup per row, every load of a lane issued at once: measured faster
            // than a wavefront per row from 4 KiB rows up, and than splitting up to 32 KiB
            path = ARGREDUCE_PATH_BLOCK;
        } else if (split_b >= 2) {
            path = ARGREDUCE_PATH_SPLIT;
            blocks_per_row = split_b;
        } else {
            path = ARGREDUCE_PATH_BLOCK;
        }
    } else if (path == ARGREDUCE_PATH_SUBWAVE) {
        group = next_pow2(vec_row) < 64 ? next_pow2(vec_row) : 64;
    } else if (path == ARGREDUCE_PATH_THREAD) {
        path = ARGREDUCE_PATH_SUBWAVE;  // a group of one lane, one load in flight
        group = 1;
    } else if (path == ARGREDUCE_PATH_SPLIT) {
        blocks_per_row = split_b > 2 ? split_b : 2;
    }
    const int64_t forced_b = g_force_split_b.load(std::memory_order_relaxed);
    if (forced_b > 0) {
        path = ARGREDUCE_PATH_SPLIT;
        blocks_per_row = forced_b;
    }

    *p = Plan{};
    p->path = path;
    p->block_threads = static_cast<int>(kBlock);
    p->device_threads = cap;
    const int64_t max_grid = cap_blocks * kOversubscribe;
    if (path == ARGREDUCE_PATH_SUBWAVE) {
        // enough 16-byte loads in flight per lane to cover the row in one step (narrow
        // groups already hold at most one vector per lane)
        int64_t unroll = 1;
        if (group == 64) {
            const int64_t cap_u = dtype == ARGREDUCE_F64 ? kMaxUnrollWaveF64 : kMaxUnrollWave;
            unroll = next_pow2(ceil_div(vec_row, 64));
            unroll = unroll < cap_u ? unroll : cap_u;
        }
        const int64_t rows_per_block = kBlock / group;
        const int64_t need = ceil_div(rows1, rows_per_block);
        // Groups narrower than a wavefront on rows of whole 16-byte vectors, or on rows whose
        // span of vectors the group covers (in a 16-byte aligned tensor): at most one device
        // wave of workgroups, each group looping over rows. A workgroup per 256 / G rows
        // measured 10-22% slower wherever that exceeded the wave (the dispatch of the extra
        // workgroups): [65536,100] fp32 8.16 -> 6.76 us, [200000,40] fp32 10.57 -> 8.24,
        // [65536,96] fp16 5.50 -> 4.67, [131072,24] fp64 8.30 -> 6.88. Rows that the general
        // scan takes (head and tail loads) gained nothing (bf16 [65536,250] 12.35 us, 12.97
        // capped) and keep a group per row.
        const int64_t row_bytes = cols * elem_size(dtype);
        const bool covered = row_bytes % 16 == 0 || span_vecs(rows, row_bytes) <= group;
        const int64_t grid_cap = (group < 64 && covered) ? cap_blocks : max_grid;
        p->lanes_per_row = static_cast<int>(group);
        p->blocks_per_row = 1;
        p->unroll = static_cast<int>(unroll);
        p->grid_blocks = need < grid_cap ? need : grid_cap;
        p->grid_rows = p->grid_blocks * rows_per_block;
    } else {
        int64_t unroll = next_pow2(ceil_div(vec_row, blocks_per_row * kBlock));
        unroll = unroll < kMaxUnrollBlocks ? unroll : kMaxUnrollBlocks;
        if (forced_b > 0) unroll = g_force_split_u.load(std::memory_order_relaxed);
        int64_t grid_rows = max_grid / blocks_per_row;
        grid_rows = grid_rows > 0 ? grid_rows : 1;
        grid_rows = rows1 < grid_rows ? rows1 : grid_rows;
        if (blocks_per_row > 1) {
            // a split row's workgroups wait on each other: every row's team is launched at
            // once (the split kernel has no row loop)
            if (rows1 > static_cast<int64_t>(std::numeric_limits<uint32_t>::max()) / blocks_per_row)
                return ARGREDUCE_ERR_TOO_WIDE;
            grid_rows = rows1;
        }
        p->lanes_per_row = static_cast<int>(blocks_per_row * kBlock);
        p->blocks_per_row = static_cast<int>(blocks_per_row);
        p->unroll = static_cast<int>(unroll);
        p->grid_rows = grid_rows;
        p->grid_blocks = grid_rows * blocks_per_row;
    }
    if (blocks_per_row > 1) {
        // the published words of every (row, workgroup), plus slack to align the pointer
        p->entry_bytes = partial_entry_bytes(dtype);
        p->scratch_bytes = 15 + static_cast<size_t>(rows1) * static_cast<size_t>(blocks_per_row) *
                                    p->entry_bytes;
    }
    return ARGREDUCE_OK;
}

int check_axis_shape(int64_t outer, int64_t len, int64_t inner, int dtype) {
    if (elem_size(dtype) == 0) return ARGREDUCE_ERR_UNSUPPORTED_DTYPE;
    if (outer < 0 || len < 1 || inner < 1) return ARGREDUCE_ERR_INVALID_ARG;
    if (len > std::numeric_limits<int32_t>::max()) return ARGREDUCE_ERR_TOO_WIDE;
    const int64_t lim = std::numeric_limits<int64_t>::max() / elem_size(dtype);
    if (inner > lim / len || (outer > 0 && outer > lim / (len * inner)))
        return ARGREDUCE_ERR_INVALID_ARG;
    return ARGREDUCE_OK;
}

// Plan of a middle-axis reduction with inner > 1.
int make_axis_plan(int64_t outer, int64_t len, int64_t inner, int dtype, uintptr_t x_addr,
                   AxisPlan* p) {
    int rc = check_axis_shape(outer, len, inner, dtype);
    if (rc != ARGREDUCE_OK) return rc;
    int64_t cap = 0;
    rc = device_threads(&cap);
    if (rc != ARGREDUCE_OK) return rc;
    const int64_t cap_blocks = cap / kBlock > 0 ? cap / kBlock : 1;
    const int64_t esize = elem_size(dtype);
    const int64_t vw = 16 / esize;
    *p = AxisPlan{};
    p->outer = outer;
    p->len = len;
    p->inner = inner;
    // 16-byte vectors when every (o, r) row of the tensor starts 16-byte aligned
    p->vec = (inner % vw == 0 && x_addr % 16 == 0) ? 1 : 0;
    // lanes along `inner`: the next power of two of the vectors (or elements) per row, <= 64
    const int64_t units = p->vec ? inner / vw : inner;
    const int64_t lanes = units < kAxisMaxLanes ? next_pow2(units) : kAxisMaxLanes;
    p->lanes = static_cast<int>(lanes);
    const int64_t tile = p->vec ? lanes * vw : lanes;
    const int64_t rows_per_tile = kBlock / lanes;  // thread rows along the axis (TR)
    p->tile = static_cast<int>(tile);
    p->tiles_per_o = ceil_div(inner, tile);
    p->tiles = outer * p->tiles_per_o;
    const int64_t tiles1 = p->tiles > 0 ? p->tiles : 1;
    // positions per thread and step: the kernel's unroll (16-byte loads: 8, or 4 for 8-byte
    // elements; element loads: 64 bytes per lane, 32 / 16 / 8 elements of 2 / 4 / 8 bytes)
    p->unroll = p->vec ? (vw == 2 ? 4 : 8) : 64 / esize;
    // Split the axis over workgroups while the tiles leave a quarter of a device wave of
    // workgroups unfilled, but not beyond one step (unroll positions) per thread. Filling the
    // whole wave measured 2-22% slower (more partials, and the 100-register kernel runs only
    // four workgroups per CU): [1,1048576,32] fp32 29.5 -> 27.7 us, [1,4096,4096] 20.3 -> 15.9.
    const int64_t fill = cap_blocks / kSplitFillDiv / tiles1;
    const int64_t want = ceil_div(len, rows_per_tile * p->unroll);
    // One step per thread when that takes at most 1.5 times the fill: a ragged second step
    // costs more than the extra partials ([1,600000,8] and [1,150000,32] fp32 10.8 -> 9.7 us,
    // 512 -> 586 workgroups; [1,1200000,8] bf16 -6%); nearer twice the fill it measured
    // no faster (977 and 782 workgroups: +0.6-1.1%).
    int64_t b = 2 * want <= 3 * fill ? want : fill;
    b = b < kMaxBlocksPerRow ? b : kMaxBlocksPerRow;
    // With 16-byte loads, two workgroups per tile do not pay for the merge dispatch they
    // need: one per tile, with twice the steps, measured faster ([256,1024,256] fp32 44.8 ->
    // 41.6 us per call). With element loads (fewer bytes in flight per wave) one per tile
    // left the device short of loads, and two measured faster: [48,4096,300] fp16 41.4 ->
    // 29.4 us, [200,2048,63] fp32 30.4 -> 22.9, [64,4096,255] fp32 60.4 -> 47.8,
    // [64,2048,255] fp64 55.9 -> 47.9, [256,1024,63] fp32 17.7 -> 16.3 (four per tile: 3-16%
    // slower than two); one short axis slower, [256,512,33] fp32 9.19 -> 9.68.
    b = b > 2 ? b : ((p->vec || b < 2) ? 1 : b);
    const int forced = g_force_path.load(std::memory_order_relaxed);
    if (forced == ARGREDUCE_PATH_SPLIT) b = b > 2 ? b : 2;
    if (forced == ARGREDUCE_PATH_BLOCK) b = 1;
    p->blocks_per_tile = static_cast<int>(b);
    const int64_t max_grid = cap_blocks * kOversubscribe;
    int64_t grid_tiles = max_grid / b;
    grid_tiles = grid_tiles > 0 ? grid_tiles : 1;
    grid_tiles = tiles1 < grid_tiles ? tiles1 : grid_tiles;
    p->grid_tiles = grid_tiles;
    p->grid_blocks = grid_tiles * b;
    p->device_threads = cap;
    p->scratch_bytes = b > 1 ? 15 + static_cast<size_t>(tiles1) * static_cast<size_t>(b) *
                                        static_cast<size_t>(tile) * axis_partial_bytes(dtype)
                             : 0;
    return ARGREDUCE_OK;
}

void fill_plan(const Plan& p, argreduce_plan_t* out) {
    out->path = p.path;
    out->lanes_per_row = p.lanes_per_row;
    out->blocks_per_row = p.blocks_per_row;
    out->block_threads = p.block_threads;
    out->grid_blocks = p.grid_blocks;
    out->grid_rows = p.grid_rows;
    out->unroll = p.unroll;
    out->outputs_per_block = p.path == ARGREDUCE_PATH_SUBWAVE ? p.block_threads / p.lanes_per_row : 1;
    out->device_threads = p.device_threads;
    out->scratch_bytes = p.scratch_bytes;
    out->load_bytes = 16;
    out->dispatches = p.path == ARGREDUCE_PATH_WIDE ? 2 : 1;
    out->window = p.path == ARGREDUCE_PATH_WIDE ? p.window : 0;
}

// Cumulative scan: every format, integers included.
int64_t scan_elem_size(int dtype) {
    switch (dtype) {
        case ARGREDUCE_I32: return 4;
        case ARGREDUCE_I64: return 8;
        default: return elem_size(dtype);
    }
}

int make_scan_plan(int64_t rows, int64_t cols, int dtype, bool aligned, ScanPlan* p) {
    const int64_t es = scan_elem_size(dtype);
    if (es == 0) return ARGREDUCE_ERR_UNSUPPORTED_DTYPE;
    if (rows < 0 || cols < 1) return ARGREDUCE_ERR_INVALID_ARG;
    if (cols > std::numeric_limits<int32_t>::max()) return ARGREDUCE_ERR_TOO_WIDE;
    if (rows > std::numeric_limits<int64_t>::max() / (cols * 8)) return ARGREDUCE_ERR_INVALID_ARG;
    int64_t cap = 0;
    const int rc = device_threads(&cap);
    if (rc != ARGREDUCE_OK) return rc;
    *p = ScanPlan{};
    p->rows = rows;
    p->cols = cols;
    // Tile size (U 16-byte chunks per lane). A row that fits one tile of U <= 2 takes the
    // smallest tile that holds it whole (no look-back: a second tile costs a handoff). A
    // longer row takes U = 1 while it needs at most 64 such tiles and the grid stays within
    // one device wave of workgroups (more, smaller tiles: more loads in flight, the
    // look-back still one round), else U = 2 under the same 64-tile bound (a bound of two
    // device waves measured 14-29% slower between one and two: [512,5000] fp32 11.57 ->
    // 9.24 us with U = 2, [512,3000] int64 11.07 -> 7.86, [600,7000] bf16 14.0 -> 11.6,
    // [800,1500] fp64 9.69 -> 7.74). Measured against
    // U = 4 for every short row: [1,65536] int64 5.9 -> 5.35 us, fp32 6.0 -> 4.1, [64,1024]
    // int64 4.0 -> 3.2, [1024,64] int64 4.4 -> 3.0, [4096,1024] fp32 15.5 -> 12.7,
    // [4096,4096] fp32 48.9 -> 45.5 (U = 2, two tiles per row; U = 1 with four: 52.7).
    // Longer rows take the smallest of U = 2, 4, 8 whose grid is at most a quarter of a
    // device wave of workgroups (one or two tiles per CU), else U = 8: fewer tiles leave CUs
    // idle, and more than fit at once wait for one another. Measured, U = 8 / 4 / 2: [1,2^18]
    // fp32 8.30 / 6.65 / 6.31 us; [1,2^20] 9.83 / 8.52 / 7.99; [1,2^21] 10.40 / 10.14 /
    // 10.12; [1,2^22] 15.15 / 15.17 / 16.82; [1,2^24] 50.2 / 54.6 / -; [1,2^21] fp16 12.48 /
    // 9.63 / 8.81; [1,2^20] int64 9.47 / 9.25 / 11.09; [1,2^22] int64 20.9 / 28.7 / -;
    // [8,2^18] fp32 9.76 / 9.44 / 9.48. The rule is within 4% of the best on every one.
    const int64_t vec_elems = 16 / es;
    const int64_t cap_blocks = cap / kBlock > 0 ? cap / kBlock : 1;
    const auto tiles_of = [&](int64_t u) { return ceil_div(cols, kBlock * u * vec_elems); };
    const int64_t t1 = tiles_of(kScanUnrollTiny), t2 = tiles_of(kScanUnrollShort);
    const bool vecio = aligned && (cols * es) % 16 == 0;
    const int64_t tile2 = kBlock * kScanUnrollShort * vec_elems, rem2 = cols % tile2;
    if (t2 == 1)
        p->unroll = t1 == 1 ? kScanUnrollTiny : kScanUnrollShort;
    else if ((!vecio || (rem2 != 0 && 2 * rem2 <= tile2)) && tiles_of(kScanUnrollMid) == 1 &&
             rows >= cap_blocks / 2)
        // many rows that one tile of 4 chunks per lane holds: that tile rather than two or
        // three chained ones, for element I/O, and for 16-byte I/O when the last of two
        // tiles would be at most half full ([2048,2049] fp32, element I/O, 21.3 -> 16.3 us;
        // [1024,4099] fp16 15.2 -> 13.1; [2048,2560] fp32 19.5 -> 14.5; [2048,1028] fp64
        // 15.1 -> 11.4; [2048,3000] fp32 21.1 -> 20.0; with a full second tile, [4096,4096]
        // fp32, 8% slower)
        p->unroll = kScanUnrollMid;
    else if (t1 <= 64 && rows <= cap_blocks / t1)
        p->unroll = kScanUnrollTiny;
    else if (t2 <= 64)
        p->unroll = kScanUnrollShort;
    else if (rows <= cap_blocks / kSplitFillDiv / t2)
        p->unroll = kScanUnrollShort;
    else if (rows <= cap_blocks / kSplitFillDiv / tiles_of(kScanUnrollMid))
        p->unroll = kScanUnrollMid;
    else
        p->unroll = kScanUnrollLong;
    p->tile_elems = kBlock * p->unroll * (16 / es);
    p->tiles_per_row = ceil_div(cols, p->tile_elems);
    if (rows > 0 && rows > static_cast<int64_t>(std::numeric_limits<uint32_t>::max()) / p->tiles_per_row)
        return ARGREDUCE_ERR_TOO_WIDE;
    p->grid_blocks = rows * p->tiles_per_row;
    p->vecio = vecio ? 1 : 0;
    p->device_threads = cap;
    if (p->tiles_per_row > 1) {
        p->state_words = static_cast<size_t>(rows) * static_cast<size_t>(p->tiles_per_row) *
                         scan_state_words(dtype);
        p->scratch_bytes = 15 + p->state_words * sizeof(uint64_t);
    }
    return ARGREDUCE_OK;
}

}  // namespace
}  // namespace argreduce

using argreduce::AxisPlan;
using argreduce::Plan;
using argreduce::ScanPlan;

ARGREDUCE_EXPORT size_t argreduce_scratch_bytes(int64_t rows, int64_t cols,
                                                argreduce_dtype_t dtype) {
    Plan p;
    if (argreduce::make_plan(rows, cols, dtype, &p) != ARGREDUCE_OK)
        return std::numeric_limits<size_t>::max();
    return p.scratch_bytes;
}

ARGREDUCE_EXPORT int argreduce_plan(int64_t rows, int64_t cols, argreduce_dtype_t dtype,
                                    argreduce_plan_t* out) {
    if (out == nullptr) return ARGREDUCE_ERR_INVALID_ARG;
    Plan p;
    const int rc = argreduce::make_plan(rows, cols, dtype, &p);
    if (rc != ARGREDUCE_OK) return rc;
    argreduce::fill_plan(p, out);
    return ARGREDUCE_OK;
}

namespace argreduce {
namespace {
// Argument checks and plan of a last-axis call; *noop is set when there is nothing to do.
int lastaxis_plan(const void* x, int dtype, int64_t rows, int64_t cols, int op,
                  const int64_t* out_idx, Plan* p, bool* noop) {
    *noop = false;
    int rc = check_shape(rows, cols, dtype);
    if (rc != ARGREDUCE_OK) return rc;
    if (op != ARGREDUCE_MAX && op != ARGREDUCE_MIN && op != ARGREDUCE_MAX_LAST &&
        op != ARGREDUCE_MIN_LAST)
        return ARGREDUCE_ERR_INVALID_ARG;
    if (rows == 0) {
        *noop = true;
        return ARGREDUCE_OK;
    }
    if (x == nullptr || out_idx == nullptr) return ARGREDUCE_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(x) % elem_size(dtype) != 0 ||
        reinterpret_cast<uintptr_t>(out_idx) % 8 != 0)
        return ARGREDUCE_ERR_INVALID_ARG;
    return make_plan(rows, cols, dtype, p);
}
}  // namespace
}  // namespace argreduce

ARGREDUCE_EXPORT int argreduce_lastaxis(const void* x, argreduce_dtype_t dtype, int64_t rows,
                                        int64_t cols, argreduce_op_t op, int64_t* out_idx,
                                        void* scratch, size_t scratch_bytes, void* stream) {
    Plan p;
    bool noop = false;
    const int rc = argreduce::lastaxis_plan(x, dtype, rows, cols, op, out_idx, &p, &noop);
    if (rc != ARGREDUCE_OK || noop) return rc;
    uint8_t* scratch16 = nullptr;
    if (p.scratch_bytes > 0) {
        if (scratch == nullptr || scratch_bytes < p.scratch_bytes)
            return ARGREDUCE_ERR_SCRATCH_TOO_SMALL;
        scratch16 = reinterpret_cast<uint8_t*>((reinterpret_cast<uintptr_t>(scratch) + 15u) &
                                               ~static_cast<uintptr_t>(15u));
    }
    const hipError_t err = argreduce::launch(p, x, dtype, op, rows, cols, out_idx, scratch16,
                                             static_cast<hipStream_t>(stream));
    return err == hipSuccess ? ARGREDUCE_OK : ARGREDUCE_ERR_HIP;
}

ARGREDUCE_EXPORT int argreduce_lastaxis_noalloc(const void* x, argreduce_dtype_t dtype,
                                                int64_t rows, int64_t cols, argreduce_op_t op,
                                                int64_t* out_idx, void* stream) {
    Plan p;
    bool noop = false;
    const int rc = argreduce::lastaxis_plan(x, dtype, rows, cols, op, out_idx, &p, &noop);
    if (rc != ARGREDUCE_OK || noop) return rc;
    uint8_t* scratch16 = nullptr;
    if (p.scratch_bytes > 0) {
        if (p.scratch_bytes > ARGREDUCE_NOALLOC_SCRATCH_BYTES) return ARGREDUCE_ERR_SCRATCH_TOO_SMALL;
        scratch16 = argreduce::noalloc_scratch();  // 256-byte aligned
        if (scratch16 == nullptr) return ARGREDUCE_ERR_HIP;
    }
    const hipError_t err = argreduce::launch(p, x, dtype, op, rows, cols, out_idx, scratch16,
                                             static_cast<hipStream_t>(stream));
    return err == hipSuccess ? ARGREDUCE_OK : ARGREDUCE_ERR_HIP;
}

ARGREDUCE_EXPORT int argreduce_debug_set_capacity(int64_t threads) {
    if (threads < 0) return ARGREDUCE_ERR_INVALID_ARG;
    argreduce::g_capacity_override.store(threads, std::memory_order_relaxed);
    return ARGREDUCE_OK;
}

ARGREDUCE_EXPORT int argreduce_debug_set_window(int64_t elements) {
    if (elements < 0 || elements > argreduce::kMaxWindow) return ARGREDUCE_ERR_INVALID_ARG;
    argreduce::g_window.store(elements, std::memory_order_relaxed);
    return ARGREDUCE_OK;
}

ARGREDUCE_EXPORT int argreduce_debug_force_split(int64_t blocks_per_row, int unroll) {
    if (blocks_per_row == 0) {
        argreduce::g_force_split_b.store(0, std::memory_order_relaxed);
        return ARGREDUCE_OK;
    }
    if (blocks_per_row < 2 || blocks_per_row > argreduce::kMaxBlocksPerRow ||
        (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8))
        return ARGREDUCE_ERR_INVALID_ARG;
    argreduce::g_force_split_u.store(unroll, std::memory_order_relaxed);
    argreduce::g_force_split_b.store(blocks_per_row, std::memory_order_relaxed);
    return ARGREDUCE_OK;
}

ARGREDUCE_EXPORT int argreduce_debug_force_path(int path) {
    if (path < ARGREDUCE_PATH_AUTO ||
        (path > ARGREDUCE_PATH_SPLIT && path != ARGREDUCE_PATH_WIDE && path != ARGREDUCE_PATH_THREAD))
        return ARGREDUCE_ERR_INVALID_ARG;
    argreduce::g_force_path.store(path, std::memory_order_relaxed);
    return ARGREDUCE_OK;
}

ARGREDUCE_EXPORT int argreduce_debug_launch_store(int64_t* out, void* stream) {
    if (out == nullptr || reinterpret_cast<uintptr_t>(out) % 8 != 0) return ARGREDUCE_ERR_INVALID_ARG;
    return argreduce::launch_store_floor(out, static_cast<hipStream_t>(stream)) == hipSuccess
               ? ARGREDUCE_OK
               : ARGREDUCE_ERR_HIP;
}

ARGREDUCE_EXPORT int argreduce_debug_launch_read(const void* x, size_t bytes, uint32_t* out,
                                                 int64_t grid, void* stream) {
    if (x == nullptr || out == nullptr || bytes == 0 || bytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(x) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 4 != 0 ||
        grid < 1 || grid > argreduce::kMaxReadGrid)
        return ARGREDUCE_ERR_INVALID_ARG;
    return argreduce::launch_read_floor(x, bytes, out, static_cast<uint32_t>(grid),
                                        static_cast<hipStream_t>(stream)) == hipSuccess
               ? ARGREDUCE_OK
               : ARGREDUCE_ERR_HIP;
}

ARGREDUCE_EXPORT int argreduce_debug_set_spin_limit(uint32_t polls) {
    argreduce::set_spin_limit(polls);
    return ARGREDUCE_OK;
}

ARGREDUCE_EXPORT int argreduce_wait_timeouts(uint64_t* count) {
    if (count == nullptr) return ARGREDUCE_ERR_INVALID_ARG;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ARGREDUCE_ERR_NO_DEVICE;
    unsigned long long c = 0;
    if (argreduce::read_wait_timeouts(&c) != hipSuccess) return ARGREDUCE_ERR_HIP;
    *count = static_cast<uint64_t>(c);
    return ARGREDUCE_OK;
}

ARGREDUCE_EXPORT int argreduce_debug_launch_empty(void* stream) {
    return argreduce::launch_empty(static_cast<hipStream_t>(stream)) == hipSuccess
               ? ARGREDUCE_OK
               : ARGREDUCE_ERR_HIP;
}

ARGREDUCE_EXPORT int argreduce_debug_set_kernel_events(void* start, void* stop) {
    argreduce::set_kernel_events(static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop));
    return ARGREDUCE_OK;
}

ARGREDUCE_EXPORT size_t argreduce_axis_scratch_bytes(int64_t outer, int64_t len, int64_t inner,
                                                     argreduce_dtype_t dtype) {
    if (inner == 1) return argreduce_scratch_bytes(outer, len, dtype);
    // The plan (and scratch) differ between 16-byte aligned tensors and others; size for
    // the larger of the two.
    AxisPlan p, q;
    if (argreduce::make_axis_plan(outer, len, inner, dtype, 0, &p) != ARGREDUCE_OK ||
        argreduce::make_axis_plan(outer, len, inner, dtype, 1, &q) != ARGREDUCE_OK)
        return std::numeric_limits<size_t>::max();
    return p.scratch_bytes > q.scratch_bytes ? p.scratch_bytes : q.scratch_bytes;
}

ARGREDUCE_EXPORT int argreduce_axis_plan(int64_t outer, int64_t len, int64_t inner,
                                         argreduce_dtype_t dtype, argreduce_plan_t* out) {
    if (out == nullptr) return ARGREDUCE_ERR_INVALID_ARG;
    if (inner == 1) return argreduce_plan(outer, len, dtype, out);
    AxisPlan p;
    const int rc = argreduce::make_axis_plan(outer, len, inner, dtype, 0, &p);
    if (rc != ARGREDUCE_OK) return rc;
    out->path = ARGREDUCE_PATH_AXIS;
    out->lanes_per_row = static_cast<int32_t>(p.blocks_per_tile * (argreduce::kBlock / p.lanes));
    out->blocks_per_row = p.blocks_per_tile;
    out->block_threads = static_cast<int32_t>(argreduce::kBlock);
    out->grid_blocks = p.grid_blocks;
    out->grid_rows = p.grid_tiles;
    out->unroll = p.unroll;
    out->outputs_per_block = p.tile;
    out->device_threads = p.device_threads;
    out->scratch_bytes = p.scratch_bytes;
    out->load_bytes = p.vec ? 16 : static_cast<int32_t>(argreduce::elem_size(dtype));
    out->dispatches = p.blocks_per_tile > 1 ? 2 : 1;
    out->window = 0;
    return ARGREDUCE_OK;
}

ARGREDUCE_EXPORT int argreduce_axis(const void* x, argreduce_dtype_t dtype, int64_t outer,
                                    int64_t len, int64_t inner, argreduce_op_t op,
                                    int64_t* out_idx, void* scratch, size_t scratch_bytes,
                                    void* stream) {
    if (inner == 1)
        return argreduce_lastaxis(x, dtype, outer, len, op, out_idx, scratch, scratch_bytes,
                                  stream);
    int rc = argreduce::check_axis_shape(outer, len, inner, dtype);
    if (rc != ARGREDUCE_OK) return rc;
    if (op != ARGREDUCE_MAX && op != ARGREDUCE_MIN && op != ARGREDUCE_MAX_LAST &&
        op != ARGREDUCE_MIN_LAST)
        return ARGREDUCE_ERR_INVALID_ARG;
    if (outer == 0) return ARGREDUCE_OK;
    if (x == nullptr || out_idx == nullptr) return ARGREDUCE_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(x) % argreduce::elem_size(dtype) != 0 ||
        reinterpret_cast<uintptr_t>(out_idx) % 8 != 0)
        return ARGREDUCE_ERR_INVALID_ARG;
    AxisPlan p;
    rc = argreduce::make_axis_plan(outer, len, inner, dtype, reinterpret_cast<uintptr_t>(x), &p);
    if (rc != ARGREDUCE_OK) return rc;
    uint8_t* scratch16 = nullptr;
    if (p.scratch_bytes > 0) {
        if (scratch == nullptr || scratch_bytes < p.scratch_bytes)
            return ARGREDUCE_ERR_SCRATCH_TOO_SMALL;
        scratch16 = reinterpret_cast<uint8_t*>((reinterpret_cast<uintptr_t>(scratch) + 15u) &
                                               ~static_cast<uintptr_t>(15u));
    }
    const hipError_t err = argreduce::launch_axis(p, x, dtype, op, out_idx, scratch16,
                                                  static_cast<hipStream_t>(stream));
    return err == hipSuccess ? ARGREDUCE_OK : ARGREDUCE_ERR_HIP;
}

ARGREDUCE_EXPORT size_t argreduce_scan_scratch_bytes(int64_t rows, int64_t cols,
                                                     argreduce_dtype_t dtype) {
    ScanPlan p;
    if (argreduce::make_scan_plan(rows, cols, dtype, true, &p) != ARGREDUCE_OK)
        return std::numeric_limits<size_t>::max();
    return p.scratch_bytes;  // the same for aligned and unaligned buffers
}

ARGREDUCE_EXPORT int argreduce_scan_plan(int64_t rows, int64_t cols, argreduce_dtype_t dtype,
                                         argreduce_plan_t* out) {
    if (out == nullptr) return ARGREDUCE_ERR_INVALID_ARG;
    ScanPlan p;
    const int rc = argreduce::make_scan_plan(rows, cols, dtype, true, &p);
    if (rc != ARGREDUCE_OK) return rc;
    out->path = ARGREDUCE_PATH_SCAN;
    out->lanes_per_row = static_cast<int32_t>(p.tiles_per_row * argreduce::kBlock);
    out->blocks_per_row = static_cast<int32_t>(p.tiles_per_row);
    out->block_threads = static_cast<int32_t>(argreduce::kBlock);
    out->grid_blocks = p.grid_blocks;
    out->grid_rows = rows;
    out->unroll = p.unroll;
    out->outputs_per_block = static_cast<int32_t>(p.tile_elems);
    out->device_threads = p.device_threads;
    out->scratch_bytes = p.scratch_bytes;
    out->load_bytes = p.vecio ? 16 : static_cast<int32_t>(argreduce::scan_elem_size(dtype));
    out->dispatches = 1;
    out->window = 0;
    return ARGREDUCE_OK;
}

ARGREDUCE_EXPORT int argreduce_scan_lastaxis(const void* x, argreduce_dtype_t dtype, int64_t rows,
                                             int64_t cols, argreduce_op_t op, void* out_values,
                                             int64_t* out_idx, void* scratch,
                                             size_t scratch_bytes, void* stream) {
    const int64_t es = argreduce::scan_elem_size(dtype);
    if (es == 0) return ARGREDUCE_ERR_UNSUPPORTED_DTYPE;
    if (op != ARGREDUCE_MAX && op != ARGREDUCE_MIN) return ARGREDUCE_ERR_INVALID_ARG;
    if (rows < 0 || cols < 1) return ARGREDUCE_ERR_INVALID_ARG;
    if (cols > std::numeric_limits<int32_t>::max()) return ARGREDUCE_ERR_TOO_WIDE;
    if (rows == 0) return ARGREDUCE_OK;
    if (x == nullptr || out_values == nullptr || out_idx == nullptr) return ARGREDUCE_ERR_INVALID_ARG;
    const uintptr_t xa = reinterpret_cast<uintptr_t>(x);
    const uintptr_t va = reinterpret_cast<uintptr_t>(out_values);
    const uintptr_t ia = reinterpret_cast<uintptr_t>(out_idx);
    if (xa % es != 0 || va % es != 0 || ia % 8 != 0) return ARGREDUCE_ERR_INVALID_ARG;
    if (rows > std::numeric_limits<int64_t>::max() / (cols * 8)) return ARGREDUCE_ERR_INVALID_ARG;
    // the outputs must not overlap the input
    const uintptr_t n = static_cast<uintptr_t>(rows) * static_cast<uintptr_t>(cols);
    const auto overlap = [](uintptr_t a, uintptr_t an, uintptr_t b, uintptr_t bn) {
        return a < b + bn && b < a + an;
    };
    if (overlap(xa, n * es, va, n * es) || overlap(xa, n * es, ia, n * 8) ||
        overlap(va, n * es, ia, n * 8))
        return ARGREDUCE_ERR_INVALID_ARG;
    const bool aligned = xa % 16 == 0 && va % 16 == 0 && ia % 16 == 0;
    ScanPlan p;
    const int rc = argreduce::make_scan_plan(rows, cols, dtype, aligned, &p);
    if (rc != ARGREDUCE_OK) return rc;
    uint8_t* scratch16 = nullptr;
    if (p.scratch_bytes > 0) {
        if (scratch == nullptr || scratch_bytes < p.scratch_bytes)
            return ARGREDUCE_ERR_SCRATCH_TOO_SMALL;
        scratch16 = reinterpret_cast<uint8_t*>((reinterpret_cast<uintptr_t>(scratch) + 15u) &
                                               ~static_cast<uintptr_t>(15u));
    }
    const hipError_t err = argreduce::launch_cum(p, x, dtype, op, out_values, out_idx, scratch16,
                                                 static_cast<hipStream_t>(stream));
    return err == hipSuccess ? ARGREDUCE_OK : ARGREDUCE_ERR_HIP;
}
