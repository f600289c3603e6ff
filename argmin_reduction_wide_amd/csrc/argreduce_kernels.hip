// gfx950 kernels of the last-axis ArgMax / ArgMin library and their launchers.
//
// Three launch shapes, after the dispatch paths of "[CUDA] Parallelize ArgMax/ArgMin over
// wide last axes" (Description / Approach and Testing: narrow rows, one block per row,
// several blocks per row, more rows than grid rows), re-cut for 64-lane wavefronts:
//
//   k_subwave  a group of G lanes (G = 1..64, a power of two) of one wavefront per row;
//              G = 64 is a wavefront per row. Rows beyond the grid are looped over.
//              Narrow rows use the group idea of TVM's shared-memory reduction page
//              ("reduction -> shared", Algorithm: group size from the reduction length,
//              xor-shuffle tree within the group).
//   k_blocks   B workgroups of 256 threads per row. B == 1: the workgroup's merged result
//              is the row's. B > 1: each workgroup publishes a (value, index) partial to
//              scratch and increments the row's counter with an agent-scope
//              acquire-release atomic (the partial store is released before it); the
//              workgroup that brings the counter to B acquires and merges the B partials.
//              This is the page's partial write -> device-wide fence -> per-row atomic
//              completion order, in the gfx950 memory model: blocks of one row run on
//              different XCDs, whose L2 caches are not coherent with each other, so the
//              reader acquires at agent scope as well.
//   k_clear    zeroes the per-row counters before a k_blocks launch with B > 1 (a kernel,
//              not a memset, so the sequence can be captured into a HIP graph).
#include <hip/hip_ext.h>

#include <atomic>

#include "argreduce_device.hpp"
#include "argreduce_internal.hpp"

namespace argreduce {

template <typename C>
struct Partial {
    C v;
    uint32_t i;
};

template <typename Fmt, int OP, int G, int U>
__global__ __launch_bounds__(kBlockThreads) void k_subwave(const uint8_t* __restrict__ x,
                                                           uint32_t cols, int64_t rows,
                                                           int64_t* __restrict__ out) {
    const uint32_t lane = threadIdx.x % G;
    const int64_t first = (static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x) / G;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * (kBlockThreads / G);
    const size_t row_bytes = static_cast<size_t>(cols) * Fmt::kSize;
    for (int64_t r = first; r < rows; r += stride) {
        Cand<typename Fmt::C, OP> c;
        scan_row<Fmt, OP, U>(x + static_cast<size_t>(r) * row_bytes, cols, lane, G, c);
        group_merge<G>(c);
        if (lane == 0) out[r] = static_cast<int64_t>(c.i);
    }
}

template <typename Fmt, int OP, int U>
__global__ __launch_bounds__(kBlockThreads) void k_blocks(const uint8_t* __restrict__ x,
                                                          uint32_t cols, int64_t rows,
                                                          uint32_t B, int64_t grid_rows,
                                                          int64_t* __restrict__ out,
                                                          uint32_t* __restrict__ counters,
                                                          uint8_t* __restrict__ partials) {
    using C = typename Fmt::C;
    __shared__ int s_last;
    const uint32_t b = blockIdx.x % B;
    const int64_t slot = blockIdx.x / B;
    const uint32_t team = B * kBlockThreads;
    const uint32_t lane = b * kBlockThreads + threadIdx.x;
    const size_t row_bytes = static_cast<size_t>(cols) * Fmt::kSize;
    for (int64_t r = slot; r < rows; r += grid_rows) {
        Cand<C, OP> c;
        scan_row<Fmt, OP, U>(x + static_cast<size_t>(r) * row_bytes, cols, lane, team, c);
        block_merge(c);
        if (B == 1) {
            if (threadIdx.x == 0) out[r] = static_cast<int64_t>(c.i);
            continue;
        }
        Partial<C>* part = reinterpret_cast<Partial<C>*>(partials) + static_cast<size_t>(r) * B;
        if (threadIdx.x == 0) {
            part[b].v = c.v;
            part[b].i = c.i;
            const uint32_t prev = __hip_atomic_fetch_add(&counters[r], 1u, __ATOMIC_ACQ_REL,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            s_last = (prev == B - 1);
        }
        __syncthreads();
        if (s_last) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            Cand<C, OP> m;
            m.init();
            for (uint32_t k = threadIdx.x; k < B; k += kBlockThreads) m.merge(part[k].v, part[k].i);
            block_merge(m);
            if (threadIdx.x == 0) {
                out[r] = static_cast<int64_t>(m.i);
                counters[r] = 0u;
            }
        }
        __syncthreads();  // s_last is rewritten for the next row
    }
}

__global__ __launch_bounds__(kBlockThreads) void k_clear(uint32_t* __restrict__ p, int64_t n) {
    for (int64_t k = static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x; k < n;
         k += static_cast<int64_t>(gridDim.x) * kBlockThreads)
        p[k] = 0u;
}

__global__ void k_empty() {}

namespace {

constexpr int kUnroll = 4;

std::atomic<hipEvent_t> g_ev_start{nullptr};
std::atomic<hipEvent_t> g_ev_stop{nullptr};

// Launch of a row-scanning kernel; with the measurement events set, the HIP extension
// launch records them around the kernel on the same stream.
template <typename... KArgs, typename... Args>
void launch_scan(void (*kernel)(KArgs...), dim3 grid, hipStream_t s, Args... args) {
    hipEvent_t e0 = g_ev_start.load(std::memory_order_relaxed);
    hipEvent_t e1 = g_ev_stop.load(std::memory_order_relaxed);
    if (e0 != nullptr && e1 != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, dim3(kBlockThreads), 0, s, e0, e1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, dim3(kBlockThreads), 0, s, args...);
}

template <typename Fmt, int OP, int G>
void launch_subwave(const Plan& p, const uint8_t* x, uint32_t cols, int64_t rows, int64_t* out,
                    hipStream_t s) {
    launch_scan(k_subwave<Fmt, OP, G, kUnroll>, dim3(static_cast<uint32_t>(p.grid_blocks)), s, x,
                cols, rows, out);
}

template <typename Fmt, int OP>
hipError_t launch_fmt(const Plan& p, const void* xv, int64_t rows, int64_t cols, int64_t* out,
                      uint8_t* scratch16, hipStream_t s) {
    const uint8_t* x = static_cast<const uint8_t*>(xv);
    const uint32_t c32 = static_cast<uint32_t>(cols);
    if (p.path == ARGREDUCE_PATH_SUBWAVE) {
        switch (p.lanes_per_row) {
            case 1: launch_subwave<Fmt, OP, 1>(p, x, c32, rows, out, s); break;
            case 2: launch_subwave<Fmt, OP, 2>(p, x, c32, rows, out, s); break;
            case 4: launch_subwave<Fmt, OP, 4>(p, x, c32, rows, out, s); break;
            case 8: launch_subwave<Fmt, OP, 8>(p, x, c32, rows, out, s); break;
            case 16: launch_subwave<Fmt, OP, 16>(p, x, c32, rows, out, s); break;
            case 32: launch_subwave<Fmt, OP, 32>(p, x, c32, rows, out, s); break;
            case 64: launch_subwave<Fmt, OP, 64>(p, x, c32, rows, out, s); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    uint32_t* counters = nullptr;
    uint8_t* partials = nullptr;
    if (p.blocks_per_row > 1) {
        counters = reinterpret_cast<uint32_t*>(scratch16);
        partials = scratch16 + p.counters_bytes;
        const int64_t clear_blocks = rows / kBlockThreads + 1 < 1024 ? rows / kBlockThreads + 1 : 1024;
        hipLaunchKernelGGL(k_clear, dim3(static_cast<uint32_t>(clear_blocks)), dim3(kBlockThreads), 0, s,
                           counters, rows);
    }
    launch_scan(k_blocks<Fmt, OP, kUnroll>, dim3(static_cast<uint32_t>(p.grid_blocks)), s, x, c32,
                rows, static_cast<uint32_t>(p.blocks_per_row), p.grid_rows, out, counters,
                partials);
    return hipGetLastError();
}

template <typename Fmt>
hipError_t launch_op(const Plan& p, const void* x, int op, int64_t rows, int64_t cols, int64_t* out,
                     uint8_t* scratch16, hipStream_t s) {
    return op == ARGREDUCE_MAX ? launch_fmt<Fmt, kMax>(p, x, rows, cols, out, scratch16, s)
                               : launch_fmt<Fmt, kMin>(p, x, rows, cols, out, scratch16, s);
}

}  // namespace

hipError_t launch(const Plan& p, const void* x, int dtype, int op, int64_t rows, int64_t cols,
                  int64_t* out, uint8_t* scratch16, hipStream_t s) {
    switch (dtype) {
        case ARGREDUCE_F32: return launch_op<F32>(p, x, op, rows, cols, out, scratch16, s);
        case ARGREDUCE_F16: return launch_op<F16>(p, x, op, rows, cols, out, scratch16, s);
        case ARGREDUCE_BF16: return launch_op<BF16>(p, x, op, rows, cols, out, scratch16, s);
        case ARGREDUCE_F64: return launch_op<F64>(p, x, op, rows, cols, out, scratch16, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_empty(hipStream_t s) {
    hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, s);
    return hipGetLastError();
}

void set_kernel_events(hipEvent_t start, hipEvent_t stop) {
    g_ev_start.store(start, std::memory_order_relaxed);
    g_ev_stop.store(stop, std::memory_order_relaxed);
}

size_t partial_entry_bytes(int dtype) {
    return dtype == ARGREDUCE_F64 ? sizeof(Partial<double>) : sizeof(Partial<float>);
}

}  // namespace argreduce
