// Host-side declarations shared by the C ABI (argreduce_api.cpp) and the kernel
// launchers (argreduce_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "argreduce.h"

namespace argreduce {

struct Plan {
    int path;                // argreduce_path_t
    int lanes_per_row;       // SUBWAVE: group size G (1..64); BLOCK/SPLIT: blocks * 256
    int blocks_per_row;      // B
    int block_threads;       // 256
    int64_t grid_blocks;
    int64_t grid_rows;
    int unroll;
    int64_t device_threads;
    size_t scratch_bytes;    // including 15 bytes of alignment slack; 0 if none needed
    size_t entry_bytes;      // split path: bytes per published (nonce, index) slot
    int64_t window;          // WIDE: elements per window
    int64_t windows;         // WIDE: windows per row (G)
};

// Launch plan of a reduction over the middle axis of [outer, len, inner], inner > 1.
struct AxisPlan {
    int64_t outer, len, inner;
    int vec;                 // 1: each lane owns VW outputs loaded as one 16-byte vector
    int lanes;               // lanes along `inner` per workgroup (TL)
    int tile;                // outputs per workgroup tile (TL, times VW with vec)
    int64_t tiles_per_o;     // tiles per outer index
    int64_t tiles;           // outer * tiles_per_o
    int blocks_per_tile;     // B (> 1: partials, merged by a second dispatch)
    int64_t grid_blocks;
    int64_t grid_tiles;      // tiles in flight at once (further tiles are looped over)
    int unroll;              // loads in flight per thread along the axis
    int64_t device_threads;
    size_t scratch_bytes;    // including 15 bytes of alignment slack; 0 if none needed
};

// Cumulative extremum with indices (cummax / cummin) along the last axis.
// 16-byte chunks per lane per tile: 1 or 2 while a row needs at most 64 tiles of that size;
// for longer rows 2, 4 or 8, the smallest whose grid fits a quarter of a device wave. The
// choice between them is the scan plan's.
constexpr int kScanUnrollTiny = 1;
constexpr int kScanUnrollShort = 2;
constexpr int kScanUnrollMid = 4;
constexpr int kScanUnrollLong = 8;

struct ScanPlan {
    int64_t rows, cols;
    int64_t tiles_per_row;   // T; > 1: tiles chained by look-back through scratch
    int unroll;              // chunks per lane per tile (U)
    int64_t tile_elems;      // 256 * U * VW
    int64_t grid_blocks;     // rows * T
    int vecio;               // 16-byte loads and stores of full chunks
    size_t state_words;      // 64-bit scratch words of all tile states (0 if T == 1)
    int64_t device_threads;
    size_t scratch_bytes;    // including 15 bytes of alignment slack; 0 if none needed
};

// Enqueues the cumulative scan of `plan` on `stream` (and, when the stream is being
// captured into a graph, a clear of the tile states before it).
hipError_t launch_cum(const ScanPlan& plan, const void* x, int dtype, int op, void* out_val,
                      int64_t* out_idx, uint8_t* scratch16, hipStream_t stream);

// 64-bit scratch words of one tile's states (aggregate + inclusive prefix).
size_t scan_state_words(int dtype);

// Enqueues the middle-axis kernel of `plan` on `stream`.
hipError_t launch_axis(const AxisPlan& plan, const void* x, int dtype, int op, int64_t* out,
                       uint8_t* scratch16, hipStream_t stream);

// Enqueues the kernels of `plan` on `stream`. `scratch16` is the caller's scratch aligned
// up to 16 bytes (or null when plan.scratch_bytes == 0). Returns a hipError_t.
hipError_t launch(const Plan& plan, const void* x, int dtype, int op, int64_t rows, int64_t cols,
                  int64_t* out, uint8_t* scratch16, hipStream_t stream);

// Launches one empty kernel (the launch floor of the measurement hooks).
hipError_t launch_empty(hipStream_t stream);
hipError_t launch_store_floor(int64_t* out, hipStream_t stream);
// A plain streaming read of `bytes` (a multiple of 16) at `x` (16-byte aligned) with `grid`
// workgroups; `out` holds `grid` words (written only for one improbable XOR of the data).
hipError_t launch_read_floor(const void* x, size_t bytes, uint32_t* out, uint32_t grid,
                             hipStream_t stream);
void set_spin_limit(uint32_t polls);

// The current device's copy of the library-held scratch of argreduce_lastaxis_noalloc
// (ARGREDUCE_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned), located on the first call per
// device; null when it cannot be located.
uint8_t* noalloc_scratch();

// Copies the current device's count of bounded waits that gave up to *count (synchronous).
hipError_t read_wait_timeouts(unsigned long long* count);

// Events recorded around the row-scanning kernel of every launch when both are set.
void set_kernel_events(hipEvent_t start, hipEvent_t stop);

// Bytes of one (value, 64-bit index) window candidate of a row wider than INT32_MAX.
size_t wide_partial_bytes(int dtype);

// Bytes of one (value, index) partial of a two-dispatch middle-axis reduction.
size_t axis_partial_bytes(int dtype);

// Bytes of one published slot of the split path.
size_t partial_entry_bytes(int dtype);

}  // namespace argreduce
