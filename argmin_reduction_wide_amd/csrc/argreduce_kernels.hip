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
//   k_blocks   B workgroups of 256 threads per row; B == 1 is a workgroup per row.
//
// Merging a row split over B > 1 workgroups. The page merges partials through a small
// global buffer reduced by the last block to arrive, ordered as partial write, device-wide
// fence, per-row atomic completion counter that the caller's memset clears every call.
// On gfx950 that order costs a full L2 write-back per workgroup (the release fence, since
// the eight XCDs' L2 caches are not coherent with each other) and a second dispatch for the
// clear. This library instead uses one single-location handshake per workgroup:
//
//   * workgroup b of row r publishes its candidate as 64-bit agent-scope atomic stores of
//     words (nonce << 32) | payload, where the nonce is a per-call value and the payloads
//     are the index and the 32-bit halves of the value: 2 words for f32/f16/bf16 (value
//     widened to f32), 3 for f64;
//   * the row's workgroup with the highest id (dispatched after the others) polls the
//     words of the other B-1 workgroups with agent-scope atomic loads until every word
//     carries this call's nonce, merges, writes out[r], and resets the words to 0 so that
//     a replayed HIP graph, whose nonce is fixed, starts from clean words.
//
// Every word is written once and validated on its own, so no cross-location ordering (and
// no release fence) is needed; stale or arbitrary scratch contents are ignored unless a
// word equals this call's nonce in its upper half (and, for the index word, holds an
// in-range index). The poll is bounded: should a word never arrive, out[r] = -1 (never
// expected: the other workgroups of the row wait on nothing, and have lower ids).
#include <hip/hip_ext.h>

#include <atomic>

#include "argreduce_device.hpp"
#include "argreduce_internal.hpp"

namespace argreduce {

constexpr uint32_t kSpinLimit = 1u << 20;  // polls of one slot before giving up (~1 s)

// Payload words of one published candidate: the index, then the value's 32-bit halves.
template <typename C>
struct Words;
template <>
struct Words<float> {
    static constexpr int kWords = 2;
    static constexpr int kStride = 2;
    __device__ static void pack(float v, uint32_t i, uint32_t (&p)[2]) {
        p[0] = i;
        p[1] = __float_as_uint(v);
    }
    __device__ static void unpack(const uint32_t (&p)[2], float& v, uint32_t& i) {
        i = p[0];
        v = __uint_as_float(p[1]);
    }
};
template <>
struct Words<double> {
    static constexpr int kWords = 3;
    static constexpr int kStride = 4;
    __device__ static void pack(double v, uint32_t i, uint32_t (&p)[3]) {
        const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
        p[0] = i;
        p[1] = static_cast<uint32_t>(b);
        p[2] = static_cast<uint32_t>(b >> 32);
    }
    __device__ static void unpack(const uint32_t (&p)[3], double& v, uint32_t& i) {
        i = p[0];
        v = __longlong_as_double(
            static_cast<long long>((static_cast<uint64_t>(p[2]) << 32) | p[1]));
    }
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
        if (lane == G - 1) out[r] = Cand<typename Fmt::C, OP>::result(c.i);
    }
}

template <typename Fmt, int OP, int U>
__global__ __launch_bounds__(kBlockThreads) void k_blocks(const uint8_t* __restrict__ x,
                                                          uint32_t cols, int64_t rows,
                                                          uint32_t B, int64_t grid_rows,
                                                          int64_t* __restrict__ out,
                                                          uint64_t* __restrict__ slots,
                                                          uint32_t nonce) {
    using C = typename Fmt::C;
    __shared__ int s_timeout;
    const uint32_t b = blockIdx.x % B;
    const int64_t slot = blockIdx.x / B;
    const uint32_t team = B * kBlockThreads;
    const uint32_t lane = b * kBlockThreads + threadIdx.x;
    const size_t row_bytes = static_cast<size_t>(cols) * Fmt::kSize;
    if (threadIdx.x == 0) s_timeout = 0;
    for (int64_t r = slot; r < rows; r += grid_rows) {
        const uint8_t* row = x + static_cast<size_t>(r) * row_bytes;
        Cand<C, OP> c;
        scan_row<Fmt, OP, U>(row, cols, lane, team, c);
        block_merge(c);
        if (B == 1) {
            if (threadIdx.x == 0) out[r] = Cand<C, OP>::result(c.i);
            continue;
        }
        uint64_t* rs = slots + static_cast<size_t>(r) * B * Words<C>::kStride;
        const uint64_t tag = static_cast<uint64_t>(nonce) << 32;
        if (b != B - 1) {
            if (threadIdx.x == 0) {
                uint64_t* e = rs + static_cast<size_t>(b) * Words<C>::kStride;
                uint32_t pay[Words<C>::kWords];
                Words<C>::pack(c.v, c.i, pay);
#pragma unroll
                for (int w = 0; w < Words<C>::kWords; ++w)
                    __hip_atomic_store(&e[w], tag | pay[w], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            continue;
        }
        // The row's finalizing workgroup.
        Cand<C, OP> m;
        if (threadIdx.x == 0) {
            m = c;
        } else {
            m.init();
        }
        for (uint32_t k = threadIdx.x; k + 1 < B; k += kBlockThreads) {
            uint64_t* e = rs + static_cast<size_t>(k) * Words<C>::kStride;
            uint32_t pay[Words<C>::kWords];
            uint32_t spins = 0;
            bool ok = false;
            while (!ok) {
                uint64_t w[Words<C>::kWords];
#pragma unroll
                for (int j = 0; j < Words<C>::kWords; ++j)
                    w[j] = __hip_atomic_load(&e[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = true;
#pragma unroll
                for (int j = 0; j < Words<C>::kWords; ++j) {
                    ok = ok && (w[j] & 0xffffffff00000000ull) == tag;
                    pay[j] = static_cast<uint32_t>(w[j]);
                }
                ok = ok && Cand<C, OP>::valid_index(pay[0], cols);
                if (!ok) {
                    if (++spins > kSpinLimit) {
                        s_timeout = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            if (ok) {
                C v;
                uint32_t idx;
                Words<C>::unpack(pay, v, idx);
                m.merge(v, idx);
            }
#pragma unroll
            for (int j = 0; j < Words<C>::kWords; ++j)
                __hip_atomic_store(&e[j], uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        block_merge(m);
        if (threadIdx.x == 0) out[r] = s_timeout ? int64_t{-1} : Cand<C, OP>::result(m.i);
    }
}

__global__ void k_empty() {}

namespace {

std::atomic<uint32_t> g_nonce{0};

// A fresh per-call nonce; never 0 (the value slots are reset to) nor 0xffffffff.
uint32_t next_nonce() {
    uint32_t n;
    do {
        n = g_nonce.fetch_add(1u, std::memory_order_relaxed) + 1u;
    } while (n == 0u || n == 0xffffffffu);
    return n;
}

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

template <typename Fmt, int OP, int G, int U>
void launch_subwave(const Plan& p, const uint8_t* x, uint32_t cols, int64_t rows, int64_t* out,
                    hipStream_t s) {
    launch_scan(k_subwave<Fmt, OP, G, U>, dim3(static_cast<uint32_t>(p.grid_blocks)), s, x,
                cols, rows, out);
}

template <typename Fmt, int OP, int U>
void launch_blocks(const Plan& p, const uint8_t* x, uint32_t cols, int64_t rows, int64_t* out,
                   uint64_t* slots, hipStream_t s) {
    launch_scan(k_blocks<Fmt, OP, U>, dim3(static_cast<uint32_t>(p.grid_blocks)), s, x, cols,
                rows, static_cast<uint32_t>(p.blocks_per_row), p.grid_rows, out, slots,
                p.blocks_per_row > 1 ? next_nonce() : 0u);
}

template <typename Fmt, int OP>
hipError_t launch_fmt(const Plan& p, const void* xv, int64_t rows, int64_t cols, int64_t* out,
                      uint8_t* scratch16, hipStream_t s) {
    const uint8_t* x = static_cast<const uint8_t*>(xv);
    const uint32_t c32 = static_cast<uint32_t>(cols);
    if (p.path == ARGREDUCE_PATH_SUBWAVE) {
        // Narrow groups cover their row with one vector per lane; a wavefront per row keeps
        // up to 8 vectors per lane in flight.
        switch (p.lanes_per_row * 100 + p.unroll) {
            case 101: launch_subwave<Fmt, OP, 1, 1>(p, x, c32, rows, out, s); break;
            case 201: launch_subwave<Fmt, OP, 2, 1>(p, x, c32, rows, out, s); break;
            case 401: launch_subwave<Fmt, OP, 4, 1>(p, x, c32, rows, out, s); break;
            case 801: launch_subwave<Fmt, OP, 8, 1>(p, x, c32, rows, out, s); break;
            case 1601: launch_subwave<Fmt, OP, 16, 1>(p, x, c32, rows, out, s); break;
            case 3201: launch_subwave<Fmt, OP, 32, 1>(p, x, c32, rows, out, s); break;
            case 6401: launch_subwave<Fmt, OP, 64, 1>(p, x, c32, rows, out, s); break;
            case 6402: launch_subwave<Fmt, OP, 64, 2>(p, x, c32, rows, out, s); break;
            case 6404: launch_subwave<Fmt, OP, 64, 4>(p, x, c32, rows, out, s); break;
            case 6408: launch_subwave<Fmt, OP, 64, 8>(p, x, c32, rows, out, s); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    uint64_t* slots = p.blocks_per_row > 1 ? reinterpret_cast<uint64_t*>(scratch16) : nullptr;
    switch (p.unroll) {
        case 1: launch_blocks<Fmt, OP, 1>(p, x, c32, rows, out, slots, s); break;
        case 2: launch_blocks<Fmt, OP, 2>(p, x, c32, rows, out, slots, s); break;
        case 4: launch_blocks<Fmt, OP, 4>(p, x, c32, rows, out, slots, s); break;
        case 8: launch_blocks<Fmt, OP, 8>(p, x, c32, rows, out, slots, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename Fmt>
hipError_t launch_op(const Plan& p, const void* x, int op, int64_t rows, int64_t cols, int64_t* out,
                     uint8_t* scratch16, hipStream_t s) {
    switch (op) {
        case ARGREDUCE_MAX: return launch_fmt<Fmt, kMax>(p, x, rows, cols, out, scratch16, s);
        case ARGREDUCE_MIN: return launch_fmt<Fmt, kMin>(p, x, rows, cols, out, scratch16, s);
        case ARGREDUCE_MAX_LAST: return launch_fmt<Fmt, kMaxLast>(p, x, rows, cols, out, scratch16, s);
        case ARGREDUCE_MIN_LAST: return launch_fmt<Fmt, kMinLast>(p, x, rows, cols, out, scratch16, s);
        default: return hipErrorInvalidValue;
    }
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
    return sizeof(uint64_t) * (dtype == ARGREDUCE_F64 ? Words<double>::kStride : Words<float>::kStride);
}

}  // namespace argreduce
