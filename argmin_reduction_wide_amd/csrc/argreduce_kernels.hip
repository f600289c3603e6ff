// gfx950 kernels of the last-axis ArgMax / ArgMin library and their launchers.
//
// The last-axis launch shapes follow the dispatch paths of "[CUDA] Parallelize
// ArgMax/ArgMin over wide last axes" (Description / Approach and Testing: narrow rows, one
// block per row, several blocks per row, more rows than grid rows), re-cut for 64-lane
// wavefronts:
//
//   k_narrow   rows of at most 32 whole 16-byte vectors starting 16-byte aligned: a group
//              of G lanes (G = 1..32, a power of two) per row, one vector per lane.
//   k_subwave  a group of G lanes (G = 1..64, a power of two) of one wavefront per row, any
//              alignment; G = 64 is a wavefront per row. Rows beyond the grid are looped over.
//              Modes as for k_blocks: aligned (16-byte aligned whole vectors one step of the
//              group covers), span (other rows whose 16-byte vectors one step covers), general.
//              Narrow rows use the group idea of TVM's shared-memory reduction page
//              ("reduction -> shared", Algorithm: group size from the reduction length,
//              a tree within the group; here on the DPP crossbar).
//   k_blocks   a workgroup of 256 threads per row; rows beyond the grid are looped over.
//   k_split    B > 1 workgroups per row, every row's team launched at once.
//              Both have an aligned variant for rows of 16-byte aligned whole vectors that
//              one step of the team covers (scan_row_aligned: no head, tail or seed load),
//              and a span variant for other rows one step covers (scan_row_span: aligned
//              vector loads, the elements outside the row masked).
//   k_wide     rows wider than INT32_MAX: one workgroup per window of at most 2^30
//              elements (32-bit positions inside it), k_wide_merge as a second dispatch.
//
// A reduction over a middle axis uses k_axis (a tile of outputs per workgroup, the axis
// split over B workgroups when tiles are few) with k_axis_merge as its second dispatch when
// B > 1. k_empty, k_store_floor and k_read_floor are the measurement hooks' kernels.
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
//   * the row's workgroup with the highest id polls the
//     words of the other B-1 workgroups with agent-scope atomic loads until every word
//     carries this call's nonce, merges, writes out[r], and resets the words to 0 so that
//     a replayed HIP graph, whose nonce is fixed, starts from clean words.
//
// Every word is written once and validated on its own, so no cross-location ordering (and
// no release fence) is needed; stale or arbitrary scratch contents are ignored unless a
// word equals this call's nonce in its upper half (and, for the index word, holds an
// in-range index). Only finalizers wait, and only on lower-numbered workgroups, which wait
// on nothing. The automatic plans launch at most one device wave of workgroups (CUs * 2048
// threads / 256), and k_split is compiled for eight waves per SIMD, so on an otherwise idle
// device every workgroup is resident at once. Larger grids (forced plans), or a device
// shared with other work, rely on each XCD starting the workgroups it is given in id order,
// which makes every wait end by induction on the id. The poll is bounded all the same:
// should a word never arrive, out[r] = -1 and the device's timeout counter g_wait_timeouts
// (argreduce_wait_timeouts) goes up by one (never observed outside tests that force it).
#include <hip/hip_ext.h>

#include <atomic>
#include <type_traits>

#include "argreduce_device.hpp"
#include "argreduce_internal.hpp"
#include "argreduce_launch.hpp"

namespace argreduce {

// Bounded waits of the split kernel that gave up, one copy per device (read by
// argreduce_wait_timeouts). The kernel names it directly rather than taking its address as
// an argument: its arguments (14 dwords) then all fit the SGPRs preloaded at wave launch,
// and a fifteenth would be read from kernel-argument memory, on the host, by every wave.
__device__ unsigned long long g_wait_timeouts;

template <typename Fmt, int OP, int G, int U, int MODE>
__global__ __launch_bounds__(kBlockThreads) void k_subwave(const uint8_t* __restrict__ x,
                                                           uint32_t cols, int64_t rows,
                                                           int64_t* __restrict__ out) {
    const uint32_t lane = threadIdx.x % G;
    const int64_t first = (static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x) / G;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * (kBlockThreads / G);
    const size_t row_bytes = static_cast<size_t>(cols) * Fmt::kSize;
    for (int64_t r = first; r < rows; r += stride) {
        Cand<typename Fmt::C, OP> c;
        if constexpr (MODE == 1)
            scan_row_aligned<Fmt, OP, U>(x + static_cast<size_t>(r) * row_bytes, cols / Fmt::VW, lane, G, c);
        else if constexpr (MODE == 2)
            scan_row_span<Fmt, OP, U>(x + static_cast<size_t>(r) * row_bytes, cols, lane, G, c);
        else
            scan_row<Fmt, OP, U>(x + static_cast<size_t>(r) * row_bytes, cols, lane, G, c);
        group_merge<G>(c);
        if (lane == G - 1) out[r] = Cand<typename Fmt::C, OP>::result(c.i);
    }
}

// Narrow rows that start 16-byte aligned and are a whole number nvec <= G of 16-byte
// vectors (the common case of the narrow path, e.g. [65536, 64] fp16: 8 vectors): a group
// of G lanes per row, one vector per lane, no head or tail, and position 0 taken from lane
// 0's own vector (no separate seed load). Each lane keeps one candidate for its VW
// elements with the step-slot trick of scan_step, the group merges on the DPP crossbar,
// and the group's last lane stores the index. Lanes past nvec hold all-ones bits (NaN in
// every format), which no comparison takes. One row per group while the grid covers the
// rows; beyond that the groups loop over rows.
template <typename Fmt, int OP, int G>
__global__ __launch_bounds__(kBlockThreads) void k_narrow(const uint8_t* __restrict__ x,
                                                          uint32_t nvec, int64_t rows,
                                                          int64_t* __restrict__ out) {
    using C = typename Fmt::C;
    using Vec = typename Fmt::Vec;
    using K = Cand<C, OP>;
    constexpr int VW = Fmt::VW;
    constexpr uint32_t kNoSlot = 0xffffffffu;
    const uint32_t lane = threadIdx.x % G;
    const int64_t first = (static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x) / G;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * (kBlockThreads / G);
    const size_t row_bytes = static_cast<size_t>(nvec) * 16u;
    const bool has = lane < nvec;
    const uint32_t dl = has ? lane : nvec - 1;  // a lane past the row re-reads its last vector
    for (int64_t r = first; r < rows; r += stride) {
        Vec q = __builtin_nontemporal_load(
            reinterpret_cast<const Vec*>(x + static_cast<size_t>(r) * row_bytes + dl * 16u));
        u32x4 w = __builtin_bit_cast(u32x4, q);
        w.x = has ? w.x : 0xffffffffu;
        w.y = has ? w.y : 0xffffffffu;
        w.z = has ? w.z : 0xffffffffu;
        w.w = has ? w.w : 0xffffffffu;
        C e[VW];
        Fmt::unpack(__builtin_bit_cast(Vec, w), e);
        C lv = K::identity();
        uint32_t ls = kNoSlot;
#pragma unroll
        for (int k = 0; k < VW; ++k) {
            const bool t = K::kLast ? (K::better(e[k], lv) | (e[k] == lv)) : K::better(e[k], lv);
            lv = t ? e[k] : lv;
            ls = t ? static_cast<uint32_t>(k) : ls;
        }
        K c;
        c.init();
        c.merge(lv, ls == kNoSlot ? K::kNone : lane * VW + ls);
        if (lane == 0) {  // position 0 as its own candidate (fix(x0), 0)
            K f;
            f.take_first(e[0]);
            c.merge(f.v, f.i);
        }
        group_merge<G>(c);
        if (lane == G - 1) out[r] = K::result(c.i);
    }
}

// One published candidate of a split row: polls its words (agent-scope atomic loads) until
// each carries this call's nonce and the index is one a lane's scan can produce, at most
// about spin_limit polls. The polls are unrolled four at a time with the bound checked once
// per four: a loop that tested the bound and the words' validity on separate branches every
// poll measured 0.1-0.15 us slower per call on split rows. One sleep unit (64 cycles)
// between polls measured 0.03-0.05 us faster than two, and no faster than none.
template <typename C, int OP>
__device__ inline bool poll_candidate(const uint64_t* e, uint64_t tag, uint32_t cols,
                                      uint32_t spin_limit, C& v, uint32_t& idx) {
    constexpr int kW = Words<C>::kWords;
    for (uint32_t spins = 0;; spins += 4) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint64_t w[kW];
#pragma unroll
            for (int j = 0; j < kW; ++j)
                w[j] = __hip_atomic_load(&e[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            uint32_t pay[kW];
            bool tags = true;
#pragma unroll
            for (int j = 0; j < kW; ++j) {
                tags = tags & ((w[j] & 0xffffffff00000000ull) == tag);
                pay[j] = static_cast<uint32_t>(w[j]);
            }
            if (tags & Cand<C, OP>::valid_index(pay[0], cols)) {
                Words<C>::unpack(pay, v, idx);
                return true;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (spins >= spin_limit) return false;
    }
}

template <typename C>
__device__ inline void clear_candidate(uint64_t* e) {
#pragma unroll
    for (int j = 0; j < Words<C>::kWords; ++j)
        __hip_atomic_store(&e[j], uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup per row; rows beyond the grid are looped over. MODE as for k_split below:
// 0 the general scan, 1 every row 16-byte aligned whole vectors, at most 256 * U of them
// (one step: scan_row_aligned), 2 every row's span of vectors within one step.
template <typename Fmt, int OP, int U, int MODE>
__global__ __launch_bounds__(kBlockThreads) void k_blocks(const uint8_t* __restrict__ x,
                                                          int64_t rows,
                                                          int64_t* __restrict__ out,
                                                          uint32_t cols) {
    using K = Cand<typename Fmt::C, OP>;
    const size_t row_bytes = static_cast<size_t>(cols) * Fmt::kSize;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        K c;
        const uint8_t* row = x + static_cast<size_t>(r) * row_bytes;
        if constexpr (MODE == 1)
            scan_row_aligned<Fmt, OP, U>(row, cols / Fmt::VW, threadIdx.x, kBlockThreads, c);
        else if constexpr (MODE == 2)
            scan_row_span<Fmt, OP, U>(row, cols, threadIdx.x, kBlockThreads, c);
        else
            scan_row<Fmt, OP, U>(row, cols, threadIdx.x, kBlockThreads, c);
        block_merge(c);
        if (threadIdx.x == 0) out[r] = K::result(c.i);
    }
}

// A row split over B > 1 workgroups: workgroup b of row r = blockIdx / B scans the row's
// lanes b * 256 .. b * 256 + 255 of a team of B * 256 lanes (one row per team, every row's
// team launched at once). Workgroups b < B - 1 publish their candidate; workgroup B - 1
// finalizes the row. MODE: 0 the general scan (scan_row); 1 as ALIGNED for k_blocks (one
// step of B * 256 lanes); 2 rows whose 16-byte vectors, counted from the one holding the
// row's first byte, one step covers (scan_row_span; at most 32 elements per lane).
//
// Eight waves per SIMD (at most 64 VGPRs): eight workgroups of 256 threads per CU, so a
// grid of up to (CUs * 2048 / 256) workgroups, the most an automatic split plan launches,
// is resident at once on an otherwise idle device, whatever the format and unroll. (A row
// loop here cost registers: values the compiler hoisted out of it stayed live through the
// scan and pushed the U = 8 instances past 64 VGPRs.)
template <typename Fmt, int OP, int U, int MODE>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void k_split(const uint8_t* __restrict__ x, int64_t* __restrict__ out,
             uint64_t* __restrict__ slots, uint32_t cols, uint32_t B, uint32_t nonce,
             uint32_t spin_limit) {
    using C = typename Fmt::C;
    using K = Cand<C, OP>;
    __shared__ int s_timeout;
    const uint32_t b = blockIdx.x % B;
    const uint32_t r = blockIdx.x / B;
    if (threadIdx.x == 0) s_timeout = 0;  // read after the barriers of the last merge
    K c;
    const uint8_t* row = x + static_cast<size_t>(r) * cols * Fmt::kSize;
    if constexpr (MODE == 1)
        scan_row_aligned<Fmt, OP, U>(row, cols / Fmt::VW, b * kBlockThreads + threadIdx.x,
                                     B * kBlockThreads, c);
    else if constexpr (MODE == 2)
        scan_row_span<Fmt, OP, U>(row, cols, b * kBlockThreads + threadIdx.x, B * kBlockThreads, c);
    else
        scan_row<Fmt, OP, U>(row, cols, b * kBlockThreads + threadIdx.x, B * kBlockThreads, c);
    block_merge(c);
    uint64_t* rs = slots + static_cast<size_t>(r) * B * Words<C>::kStride;
    const uint64_t tag = static_cast<uint64_t>(nonce) << 32;
    if (b != B - 1) {
        if (threadIdx.x == 0) {
            uint64_t* e = rs + static_cast<size_t>(b) * Words<C>::kStride;
            uint32_t pay[Words<C>::kWords];
            Words<C>::pack(c.v, c.i, pay);
#pragma unroll
            for (int w = 0; w < Words<C>::kWords; ++w)
                __hip_atomic_store(&e[w], tag | pay[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    // The row's finalizing workgroup. Its index goes out as an agent-scope store (written
    // through, like the published words), which measured 0.06 us faster per call on
    // [32, 202048] than a plain store.
    if (B - 1 <= static_cast<uint32_t>(kWave)) {
        // At most one published candidate per lane of wavefront 0: it polls and merges them
        // alone (no LDS round, no barrier); its lane 0 holds this workgroup's own candidate.
        if (threadIdx.x >= static_cast<uint32_t>(kWave)) return;
        K m;
        if (threadIdx.x == 0) {
            m = c;
        } else {
            m.init();
        }
        bool ok = true;
        if (threadIdx.x + 1 < B) {
            uint64_t* e = rs + static_cast<size_t>(threadIdx.x) * Words<C>::kStride;
            C v;
            uint32_t idx;
            ok = poll_candidate<C, OP>(e, tag, cols, spin_limit, v, idx);
            if (ok) m.merge(v, idx);
            clear_candidate<C>(e);
        }
        const bool gave_up = __ballot(!ok) != 0;
        group_merge<kWave>(m);
        if (threadIdx.x == kWave - 1) {
            __hip_atomic_store(&out[r], gave_up ? int64_t{-1} : K::result(m.i), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            if (gave_up)
                __hip_atomic_fetch_add(&g_wait_timeouts, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    K m;
    if (threadIdx.x == 0) {
        m = c;
    } else {
        m.init();
    }
    for (uint32_t k = threadIdx.x; k + 1 < B; k += kBlockThreads) {
        uint64_t* e = rs + static_cast<size_t>(k) * Words<C>::kStride;
        C v;
        uint32_t idx;
        if (poll_candidate<C, OP>(e, tag, cols, spin_limit, v, idx))
            m.merge(v, idx);
        else
            s_timeout = 1;
        clear_candidate<C>(e);
    }
    block_merge(m);
    if (threadIdx.x == 0) {
        __hip_atomic_store(&out[r], s_timeout ? int64_t{-1} : K::result(m.i), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (s_timeout)
            __hip_atomic_fetch_add(&g_wait_timeouts, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Tree merge of the TR = 256 / TL thread rows of a workgroup (TL lanes each, EPL candidates
// per lane) through LDS: the result lands in thread row 0. Ends with a barrier, so the
// arrays may be rewritten right after.
template <int TL, int EPL, typename Cand, typename C>
__device__ void merge_rows(Cand (&c)[EPL], C (*s_v)[kBlockThreads], uint32_t (*s_i)[kBlockThreads]) {
    constexpr int TR = kBlockThreads / TL;
    const uint32_t tl = threadIdx.x % TL;
    const uint32_t tr = threadIdx.x / TL;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
        s_v[k][threadIdx.x] = c[k].v;
        s_i[k][threadIdx.x] = c[k].i;
    }
    __syncthreads();
#pragma unroll
    for (int h = TR / 2; h > 0; h >>= 1) {
        // rows [0, h) take rows [h, 2h): no row is read and written in the same round
        if (tr < static_cast<uint32_t>(h)) {
#pragma unroll
            for (int k = 0; k < EPL; ++k) {
                c[k].merge(s_v[k][(tr + h) * TL + tl], s_i[k][(tr + h) * TL + tl]);
                s_v[k][threadIdx.x] = c[k].v;
                s_i[k][threadIdx.x] = c[k].i;
            }
        }
        __syncthreads();
    }
}

// Workgroup id with the 8 XCDs in mind: workgroups are handed to the XCDs round-robin
// (XCD = blockIdx % 8); this maps the ones XCD k receives onto one contiguous range of ids,
// so that each XCD streams its own contiguous part of the tensor.
__device__ inline uint32_t xcd_contiguous_id(uint32_t g) {
    const uint32_t q = g / 8, r = g % 8, k = blockIdx.x % 8;
    return k * q + (k < r ? k : r) + blockIdx.x / 8;
}

// Word 3 of a gfx9 buffer resource for raw byte-addressed loads: DATA_FORMAT (bits 15-18) =
// 4, 32-bit; no swizzle, no index stride, NUM_FORMAT 0.
constexpr int kRawBufferWord3 = 0x00020000;

template <typename C>
struct Partial {
    C v;
    uint32_t i;
};

// Reduction over the middle axis of a contiguous [outer, len, inner] tensor (inner > 1),
// laid out like the column kernel of AcceleratedKernels.jl's pull request on reductions of
// wide matrices along dims (Wide matrices: a column kernel): a workgroup takes a tile of
// consecutive outputs of one outer index, TL lanes along `inner`, so that every load of a
// wavefront reads consecutive memory. LD = 1: each lane owns VW consecutive outputs and
// loads them as one 16-byte vector (inner * sizeof(T) a multiple of 16, x 16-byte aligned).
// Otherwise one output and one element per lane: LD = 2 through a buffer resource over the
// tile (a lane's fixed 32-bit offset plus a uniform offset per load, so U loads in flight
// hold one address register, not U 64-bit addresses), when every offset of the tile fits in
// 32 bits; LD = 0 with 64-bit addresses. The TR = 256 / TL thread rows split the reduced axis
// (thread row tr takes positions tr, tr + TR, ..., U loads in flight) and tree-merge in LDS.
//
// With B > 1 the axis is also split over B workgroups per tile (few outputs, long axis):
// each stores a plain (value, index) partial per output and k_axis_merge, the second
// dispatch, merges them; the kernel boundary orders the two, so nothing waits.
template <typename Fmt, int OP, int TL, int LD, int U>
__global__ __launch_bounds__(kBlockThreads) void k_axis(const uint8_t* __restrict__ x,
                                                        int64_t inner, int64_t tiles,
                                                        int64_t* __restrict__ out,
                                                        Partial<typename Fmt::C>* __restrict__ part,
                                                        uint32_t len, uint32_t B, uint32_t grid) {
    using C = typename Fmt::C;
    using L = typename std::conditional<LD == 1, typename Fmt::Vec, C>::type;
    constexpr int TR = kBlockThreads / TL;
    constexpr int EPL = LD == 1 ? Fmt::VW : 1;  // outputs per lane
    constexpr int TO = TL * EPL;            // outputs per tile
    __shared__ C s_v[EPL][kBlockThreads];
    __shared__ uint32_t s_i[EPL][kBlockThreads];
    const uint32_t tl = threadIdx.x % TL;
    const uint32_t tr = threadIdx.x / TL;
    const int64_t tiles_per_o = (inner + TO - 1) / TO;
    const int64_t grid_tiles = grid / B;
    const uint32_t id = xcd_contiguous_id(grid);
    const uint32_t b = id % B;
    const int64_t slot = id / B;
    const uint32_t rteam = B * TR;  // thread rows sharing one tile
    const uint32_t rlane = b * TR + tr;
    const uint32_t step = rteam * U;
    const size_t rstride = static_cast<size_t>(inner) * Fmt::kSize;
    for (int64_t t = slot; t < tiles; t += grid_tiles) {
        const int64_t o = t / tiles_per_o;
        const int64_t i0 = (t - o * tiles_per_o) * TO + static_cast<int64_t>(tl) * EPL;
        const bool active = i0 < inner;  // with LD = 1 all EPL outputs of a lane exist together
        Cand<C, OP> c[EPL];
#pragma unroll
        for (int k = 0; k < EPL; ++k) c[k].init();
        if (active) {
            const uint8_t* col =
                x + (static_cast<size_t>(o) * len * static_cast<size_t>(inner) + i0) * Fmt::kSize;
            // One step: U loads per lane (positions base + rlane + u * rteam), issued back to
            // back, then the compares. No load sits under a lane condition (that would make
            // it a branch, and the loads of the step would wait on each other): in the last,
            // partial step a lane past the end re-reads the last position, and visiting a
            // real element again, with its own position and after every smaller position of
            // the lane, changes no result.
            // LD = 2 loads through a buffer resource that starts at the tile's first output
            // at position 0 and ends with the tensor: a lane's element at position d is at
            // lane_off + d * rstride, below 2^32 (the launcher checks the tile's largest
            // offset). The resource is built in every mode (the others leave it unused) from
            // uniform values passed through readfirstlane, so that it sits in scalar
            // registers: a resource the compiler took for per-lane made every load a loop
            // over the lanes' distinct resources.
            const uint64_t tfirst = static_cast<uint64_t>(o) * len * static_cast<uint64_t>(inner) +
                                    static_cast<uint64_t>(t - o * tiles_per_o) * TO;
            const uint64_t toff = tfirst * Fmt::kSize;
            const uint64_t total = static_cast<uint64_t>(tiles / tiles_per_o) * len *
                                   static_cast<uint64_t>(inner) * Fmt::kSize;
            const uint64_t left = total - toff;
            const uintptr_t ta = reinterpret_cast<uintptr_t>(x) + toff;
            const uint32_t ta_lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(ta));
            const uint32_t ta_hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(ta >> 32));
            const int nrec = __builtin_amdgcn_readfirstlane(left < 0xffffffffull ? static_cast<int>(left) : -1);
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                reinterpret_cast<void*>((static_cast<uintptr_t>(ta_hi) << 32) | ta_lo), 0, nrec,
                kRawBufferWord3);
            const uint32_t lane_off = static_cast<uint32_t>(rlane * rstride + tl * Fmt::kSize);
            // A full step of element loads: the lane's positions p0 + u * rteam, u < U, in
            // increasing order. The step keeps its best value with the slot u it came from
            // (an inline constant) and merges (value, p0 + slot * rteam) into the lane's
            // candidate once, which equals updating it position by position (the merge
            // keeps the earlier index on ties, or the later one for the last-index ops, and
            // an empty step merges nothing). Updating position by position, the compiler
            // formed all U positions ahead of the compares and kept them live.
            auto step_merge = [&](Cand<C, OP>& cc, const auto& q, uint32_t p0) {
                if constexpr (LD != 1) {  // element values only
                    using K = Cand<C, OP>;
                    C lv = K::identity();
                    uint32_t ls = 0xffffffffu;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const bool tk = K::kLast ? (K::better(q[u], lv) | (q[u] == lv)) : K::better(q[u], lv);
                        lv = tk ? q[u] : lv;
                        ls = tk ? static_cast<uint32_t>(u) : ls;
                    }
                    cc.merge(lv, ls == 0xffffffffu ? K::kNone : p0 + ls * rteam);
                }
            };
            auto scan = [&](uint32_t base, auto guard) {
                constexpr bool kGuard = decltype(guard)::value;
                const uint32_t rem = len - base;
                if constexpr (LD == 2) {
                    if constexpr (!kGuard) {
                        C q[U];
#pragma unroll
                        for (int u = 0; u < U; ++u)
                            q[u] = buffer_load1<Fmt>(rsrc, lane_off,
                                                     (base + static_cast<uint32_t>(u) * rteam) * static_cast<uint32_t>(rstride));
                        __builtin_amdgcn_sched_barrier(0);
                        step_merge(c[0], q, base + rlane);
                    } else {
                        // the last, partial step at clamped positions (a lane past the end
                        // re-reads the last position, as below), every load issued at once:
                        // each offset is needed only until its load issues
                        uint32_t dd[U];
                        C q[U];
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            const uint32_t d = rlane + static_cast<uint32_t>(u) * rteam;
                            dd[u] = d < rem ? d : rem - 1;
                            q[u] = buffer_load1<Fmt>(rsrc, tl * Fmt::kSize + (base + dd[u]) * static_cast<uint32_t>(rstride), 0);
                        }
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int u = 0; u < U; ++u) c[0].update(q[u], base + dd[u]);
                    }
                    return;
                }
                uint32_t dd[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t d = rlane + static_cast<uint32_t>(u) * rteam;
                    dd[u] = (!kGuard || d < rem) ? d : rem - 1;
                }
                L q[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint8_t* a = col + static_cast<size_t>(base + dd[u]) * rstride;
                    if constexpr (LD == 1)
                        q[u] = __builtin_nontemporal_load(reinterpret_cast<const L*>(a));
                    else
                        q[u] = Fmt::load1(a);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if constexpr (LD == 1) {
                        C e[Fmt::VW];
                        Fmt::unpack(q[u], e);
#pragma unroll
                        for (int k = 0; k < EPL; ++k) c[k].update(e[k], base + dd[u]);
                    } else if constexpr (kGuard) {
                        c[0].update(q[u], base + dd[u]);
                    }
                }
                if constexpr (LD == 0 && !kGuard) step_merge(c[0], q, base + rlane);
            };
            // Position 0 enters as its own candidate (fix(x0), 0), merged into the scan's
            // result at the end: the merge is commutative, so this equals taking it first.
            // The scan's plain visit of position 0 is then harmless (a NaN moves nothing;
            // any other value makes the same candidate). Its load is issued here and only
            // waited for after the scan.
            L seed;
            if (rlane == 0) {
                if constexpr (LD == 1)
                    seed = *reinterpret_cast<const L*>(col);
                else
                    seed = Fmt::load1(col);
            }
            // step <= 1024 * 256 * 32 (B * TR * U), so base + step cannot wrap below
            // len <= INT32_MAX
            const uint32_t full = len - len % step;
            for (uint32_t base = 0; base < full; base += step) scan(base, std::false_type{});
            if (full < len) scan(full, std::true_type{});
            if (rlane == 0) {
                C e[EPL];
                if constexpr (LD == 1) {
                    Fmt::unpack(seed, e);
                } else {
                    e[0] = seed;
                }
#pragma unroll
                for (int k = 0; k < EPL; ++k) {
                    Cand<C, OP> f;
                    f.take_first(e[k]);
                    c[k].merge(f.v, f.i);
                }
            }
        }
        merge_rows<TL>(c, s_v, s_i);  // the tile's candidates, in thread row 0
        if (tr == 0 && active) {
            if (B == 1) {
#pragma unroll
                for (int k = 0; k < EPL; ++k) out[o * inner + i0 + k] = Cand<C, OP>::result(c[k].i);
            } else {
                // part[(t * B + b) * TO + output]: one workgroup's partials are contiguous
                Partial<C>* pp = part + (static_cast<size_t>(t) * B + b) * TO + tl * EPL;
#pragma unroll
                for (int k = 0; k < EPL; ++k) {
                    pp[k].v = c[k].v;
                    pp[k].i = c[k].i;
                }
            }
        }
    }
}

// Second dispatch of a split middle-axis reduction. Workgroup g takes ML consecutive
// outputs of one tile (g = tile * groups + group): lane ml owns an output, the 256 / ML
// thread rows share out its B partials (coalesced: the partials of one first-dispatch
// workgroup are contiguous), then the thread rows tree-merge through LDS (with one output
// per workgroup, ML = 1, the workgroup merge instead: DPP within each wavefront, then the
// four wavefronts' keys).
template <typename Fmt, int OP, int ML>
__global__ __launch_bounds__(kBlockThreads) void k_axis_merge(
    const Partial<typename Fmt::C>* __restrict__ part, int64_t* __restrict__ out, int64_t inner,
    int64_t tiles_per_o, int64_t tiles, uint32_t B, int to, uint32_t grid) {
    using C = typename Fmt::C;
    constexpr int MR = kBlockThreads / ML;
    constexpr int kBatch = 8;
    __shared__ C s_v[1][kBlockThreads];
    __shared__ uint32_t s_i[1][kBlockThreads];
    const uint32_t ml = threadIdx.x % ML;
    const uint32_t mr = threadIdx.x / ML;
    const int64_t groups = (to + ML - 1) / ML;
    for (int64_t g = blockIdx.x; g < tiles * groups; g += grid) {
        const int64_t t = g / groups;
        const int64_t j = (g - t * groups) * ML + ml;  // output within the tile
        const int64_t o = t / tiles_per_o;
        const int64_t i = (t - o * tiles_per_o) * to + j;
        const bool active = j < to && i < inner;
        Cand<C, OP> m[1];
        m[0].init();
        if (active) {
            const Partial<C>* col = part + static_cast<size_t>(t) * B * to + j;
            uint32_t b = mr;
            // batches of kBatch independent loads, then the remainder one by one
            for (; b + (kBatch - 1) * MR < B; b += kBatch * MR) {
                Partial<C> e[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) e[u] = col[static_cast<size_t>(b + u * MR) * to];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) m[0].merge(e[u].v, e[u].i);
            }
            for (; b < B; b += MR) {
                const Partial<C> e = col[static_cast<size_t>(b) * to];
                m[0].merge(e.v, e.i);
            }
        }
        if constexpr (ML == 1) {
            block_merge(m[0]);  // one output per workgroup: wavefront DPP, then four keys in LDS
        } else {
            merge_rows<ML>(m, s_v, s_i);
        }
        if (mr == 0 && active) out[o * inner + i] = Cand<C, OP>::result(m[0].i);
    }
}

// Rows wider than INT32_MAX (and any row, when a window size is forced for testing): each
// row is cut into G windows of at most W <= 2^30 elements. Workgroup (row, w) scans window w
// with the ordinary 32-bit positions of scan_row, relative to the window's start (the
// positions stay 32-bit, the overflow fix's reasoning in "[CUDA] Parallelize ArgMax/ArgMin
// over wide last axes": no per-element 64-bit positions), and stores the window's candidate
// with its 64-bit global index; a second dispatch merges the G candidates of each row. Only
// window 0 holds the row's position 0 (a leading NaN or the first element's seed).
template <typename C>
struct Wide {
    C v;
    int64_t i;  // global index; kWideEmpty: no candidate; kWideNaN0: last-index leading NaN
};
constexpr int64_t kWideNaN0 = -2;

template <typename C, int OP>
__device__ inline int64_t wide_empty() {
    // loses every tie: the highest index for first-index ops, -1 for last-index ones
    return op_is_last(OP) ? int64_t{-1} : INT64_MAX;
}

template <typename C, int OP>
__device__ inline void wide_merge(C& av, int64_t& ai, C bv, int64_t bi) {
    using K = Cand<C, OP>;
    constexpr bool kLast = op_is_last(OP);
    const bool a_nan0 = kLast ? (ai == kWideNaN0) : false;
    const bool b_nan0 = kLast ? (bi == kWideNaN0) : false;
    const bool tie = kLast ? (bi > ai) : (bi < ai);
    const bool t = b_nan0 | (!a_nan0 & (K::better(bv, av) | ((bv == av) & tie)));
    av = t ? bv : av;
    ai = t ? bi : ai;
}

template <typename Fmt, int OP, int U>
__global__ __launch_bounds__(kBlockThreads) void k_wide(const uint8_t* __restrict__ x, int64_t cols,
                                                        uint32_t W, uint32_t G,
                                                        Wide<typename Fmt::C>* __restrict__ part) {
    using C = typename Fmt::C;
    using K = Cand<C, OP>;
    const uint32_t g = blockIdx.x;
    const uint32_t r = g / G;
    const uint32_t w = g - r * G;
    const int64_t start = static_cast<int64_t>(w) * W;
    const int64_t left = cols - start;
    const uint32_t len = left < static_cast<int64_t>(W) ? static_cast<uint32_t>(left) : W;
    const uint8_t* win = x + (static_cast<size_t>(r) * static_cast<size_t>(cols) + static_cast<size_t>(start)) * Fmt::kSize;
    K c;
    scan_row<Fmt, OP, U>(win, len, threadIdx.x, kBlockThreads, c, w == 0);
    block_merge(c);
    if (threadIdx.x == 0) {
        int64_t gi;
        if (c.i == K::kNone)
            gi = wide_empty<C, OP>();
        else if (op_is_last(OP) && c.i == kNaN0Last && w == 0)
            gi = kWideNaN0;
        else
            gi = start + static_cast<int64_t>(c.i);
        part[g].v = c.v;
        part[g].i = gi;
    }
}

// One workgroup per row (rows looped): merges the row's G window candidates.
template <typename Fmt, int OP>
__global__ __launch_bounds__(kBlockThreads) void k_wide_merge(const Wide<typename Fmt::C>* __restrict__ part,
                                                              uint32_t G, int64_t rows,
                                                              int64_t* __restrict__ out) {
    using C = typename Fmt::C;
    __shared__ C s_v[kBlockThreads];
    __shared__ int64_t s_i[kBlockThreads];
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        C v = Cand<C, OP>::identity();
        int64_t i = wide_empty<C, OP>();
        for (uint32_t k = threadIdx.x; k < G; k += kBlockThreads) {
            const Wide<C> e = part[static_cast<size_t>(r) * G + k];
            wide_merge<C, OP>(v, i, e.v, e.i);
        }
        s_v[threadIdx.x] = v;
        s_i[threadIdx.x] = i;
        __syncthreads();
        for (int h = kBlockThreads / 2; h > 0; h >>= 1) {
            if (threadIdx.x < static_cast<uint32_t>(h)) {
                wide_merge<C, OP>(v, i, s_v[threadIdx.x + h], s_i[threadIdx.x + h]);
                s_v[threadIdx.x] = v;
                s_i[threadIdx.x] = i;
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) out[r] = i == kWideNaN0 ? int64_t{0} : i;
        __syncthreads();  // s_v / s_i are rewritten for the next row
    }
}

__global__ void k_empty() {}

// The floor of any call that delivers a result: one workgroup, one argument, one store.
__global__ void k_store_floor(int64_t* __restrict__ out) {
    if (threadIdx.x == 0) out[0] = 0;
}

// The practical read roofline: a plain grid-stride stream of 16-byte nontemporal loads
// (four in flight per lane) folded with XOR. The store is taken only for one bit pattern,
// so the loads cannot be removed and nothing is written in practice.
__global__ __launch_bounds__(kBlockThreads) void k_read_floor(const u32x4* __restrict__ x,
                                                              size_t nvec,
                                                              uint32_t* __restrict__ out) {
    constexpr int U = 4;
    const size_t stride = static_cast<size_t>(gridDim.x) * kBlockThreads;
    size_t i = static_cast<size_t>(blockIdx.x) * kBlockThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < nvec; i += U * stride) {
        u32x4 q[U];
#pragma unroll
        for (int u = 0; u < U; ++u) q[u] = __builtin_nontemporal_load(x + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= q[u].x ^ q[u].y ^ q[u].z ^ q[u].w;
    }
    for (; i < nvec; i += stride) {
        const u32x4 q = __builtin_nontemporal_load(x + i);
        acc ^= q.x ^ q.y ^ q.z ^ q.w;
    }
    if (acc == 0x9e3779b9u) out[blockIdx.x] = acc;
}

std::atomic<uint32_t> g_nonce{0};

uint32_t next_nonce() {
    uint32_t n;
    do {
        n = g_nonce.fetch_add(1u, std::memory_order_relaxed) + 1u;
    } while (n == 0u || n == 0xffffffffu);
    return n;
}

std::atomic<uint32_t> g_spin_limit{1u << 20};

uint32_t spin_limit() { return g_spin_limit.load(std::memory_order_relaxed); }

void set_spin_limit(uint32_t polls) {
    g_spin_limit.store(polls == 0 ? (1u << 20) : polls, std::memory_order_relaxed);
}

std::atomic<hipEvent_t> g_ev_start{nullptr};
std::atomic<hipEvent_t> g_ev_stop{nullptr};

namespace {
constexpr int kMaxSymbolDevices = 64;
std::atomic<unsigned long long*> g_timeouts_addr[kMaxSymbolDevices];
}  // namespace

// Scratch of argreduce_lastaxis_noalloc: a file-scope device array, one copy per device,
// held until the process ends. Host code never passes its name (on the host that is a
// stand-in, not a device address); noalloc_scratch() returns the device's own address.
static __device__ __align__(256) uint8_t noalloc_scratch_buf[ARGREDUCE_NOALLOC_SCRATCH_BYTES];

namespace {
std::atomic<uint8_t*> g_noalloc_addr[kMaxSymbolDevices];
}  // namespace

uint8_t* noalloc_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSymbolDevices) return nullptr;
    uint8_t* p = g_noalloc_addr[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    // once per device, with that device current
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(noalloc_scratch_buf)) != hipSuccess || addr == nullptr)
        return nullptr;
    p = static_cast<uint8_t*>(addr);
    g_noalloc_addr[dev].store(p, std::memory_order_release);
    return p;
}

hipError_t read_wait_timeouts(unsigned long long* count) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSymbolDevices)
        return hipErrorInvalidDevice;
    unsigned long long* p = g_timeouts_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // the device's own copy of the counter: host code never passes the variable's name
        void* addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(g_wait_timeouts)) != hipSuccess || addr == nullptr)
            return hipErrorInvalidSymbol;
        p = static_cast<unsigned long long*>(addr);
        g_timeouts_addr[dev].store(p, std::memory_order_release);
    }
    unsigned long long split = 0, scan = 0;
    hipError_t e = hipMemcpy(&split, p, sizeof(split), hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = read_scan_wait_timeouts(&scan);
    if (e == hipSuccess) *count = split + scan;
    return e;
}

namespace {

// 16-byte vectors of the longest row counted from the one holding its first byte. Row r
// starts at byte x + r * row_bytes, 16-byte misaligned by (x + r * row_bytes) mod 16: at
// most 16 - g + (x mod g) over the rows, where g is the largest power of two (at most 16)
// dividing row_bytes, and exactly x mod 16 when there is one row.
uint64_t span_vectors(const uint8_t* x, uint64_t row_bytes, int64_t rows) {
    const uint64_t xm = reinterpret_cast<uintptr_t>(x) & 15u;
    const uint64_t g = row_bytes % 16 == 0 ? 16 : (row_bytes & (~row_bytes + 1));
    const uint64_t mis = (rows <= 1 || g == 16) ? xm : 16 - g + (xm & (g - 1));
    return (mis + row_bytes + 15) / 16;
}

// The aligned scan for rows of 16-byte aligned whole vectors that one step of the group
// covers; else the span scan when one step covers every row's vectors and a lane holds at
// most 32 elements; else the general scan.
template <typename Fmt, int OP, int G, int U>
void launch_subwave(const Plan& p, const uint8_t* x, uint32_t cols, int64_t rows, int64_t* out,
                    hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(p.grid_blocks));
    const uint64_t row_bytes = static_cast<uint64_t>(cols) * Fmt::kSize;
    if (row_bytes % 16 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
        row_bytes / 16 <= static_cast<uint64_t>(G) * U) {
        launch_scan(k_subwave<Fmt, OP, G, U, 1>, grid, s, x, cols, rows, out);
        return;
    }
    if constexpr (U * Fmt::VW <= 32) {
        if (span_vectors(x, row_bytes, rows) <= static_cast<uint64_t>(G) * U) {
            launch_scan(k_subwave<Fmt, OP, G, U, 2>, grid, s, x, cols, rows, out);
            return;
        }
    }
    launch_scan(k_subwave<Fmt, OP, G, U, 0>, grid, s, x, cols, rows, out);
}

template <typename Fmt, int OP, int U, int MODE>
void launch_split(const Plan& p, const uint8_t* x, uint32_t cols, int64_t* out, uint64_t* slots,
                  hipStream_t s) {
    launch_scan(k_split<Fmt, OP, U, MODE>, dim3(static_cast<uint32_t>(p.grid_blocks)), s, x, out,
                slots, cols, static_cast<uint32_t>(p.blocks_per_row), next_nonce(), spin_limit());
}

template <typename Fmt, int OP, int U, int MODE>
void launch_rows(const Plan& p, const uint8_t* x, uint32_t cols, int64_t rows, int64_t* out,
                 uint64_t* slots, hipStream_t s) {
    if (p.blocks_per_row <= 1)
        launch_scan(k_blocks<Fmt, OP, U, MODE>, dim3(static_cast<uint32_t>(p.grid_blocks)), s, x,
                    rows, out, cols);
    else
        launch_split<Fmt, OP, U, MODE>(p, x, cols, out, slots, s);
}

// The one-step aligned kernels when the rows are 16-byte aligned whole vectors that one step
// of the team's lanes covers. Otherwise a row takes the span scan when one step covers every
// row's vectors and a lane holds at most 32 elements (a workgroup per row: at most 4 vectors
// per lane; with 8 the span scan measured slower, [4096,4097] fp32 12.8 -> 13.7 us), and
// every other row the general scan.
template <typename Fmt, int OP, int U>
void launch_blocks(const Plan& p, const uint8_t* x, uint32_t cols, int64_t rows, int64_t* out,
                   uint64_t* slots, hipStream_t s) {
    const uint64_t row_bytes = static_cast<uint64_t>(cols) * Fmt::kSize;
    const uint64_t xm = reinterpret_cast<uintptr_t>(x) & 15u;
    const uint64_t step = static_cast<uint64_t>(p.blocks_per_row) * kBlockThreads * U;
    if (row_bytes % 16 == 0 && xm == 0 && row_bytes / 16 <= step) {
        launch_rows<Fmt, OP, U, 1>(p, x, cols, rows, out, slots, s);
        return;
    }
    if constexpr (U * Fmt::VW <= 32) {
        if ((p.blocks_per_row > 1 || U <= 4) && span_vectors(x, row_bytes, rows) <= step) {
            launch_rows<Fmt, OP, U, 2>(p, x, cols, rows, out, slots, s);
            return;
        }
    }
    launch_rows<Fmt, OP, U, 0>(p, x, cols, rows, out, slots, s);
}

template <typename Fmt, int OP>
hipError_t launch_fmt(const Plan& p, const void* xv, int64_t rows, int64_t cols, int64_t* out,
                      uint8_t* scratch16, hipStream_t s) {
    const uint8_t* x = static_cast<const uint8_t*>(xv);
    const uint32_t c32 = static_cast<uint32_t>(cols);
    if (p.path == ARGREDUCE_PATH_SUBWAVE) {
        // Rows of whole 16-byte vectors starting 16-byte aligned, at most one per lane of
        // the group (at most 32): the narrow kernel (one vector per lane, no head, tail or
        // seed load).
        const size_t row_bytes = static_cast<size_t>(cols) * Fmt::kSize;
        if (p.lanes_per_row <= 32 && p.unroll == 1 && row_bytes % 16 == 0 &&
            row_bytes / 16 <= static_cast<size_t>(p.lanes_per_row) &&
            reinterpret_cast<uintptr_t>(x) % 16 == 0) {
            const uint32_t nvec = static_cast<uint32_t>(row_bytes / 16);
            const dim3 grid(static_cast<uint32_t>(p.grid_blocks));
            switch (p.lanes_per_row) {
                case 1: launch_scan(k_narrow<Fmt, OP, 1>, grid, s, x, nvec, rows, out); break;
                case 2: launch_scan(k_narrow<Fmt, OP, 2>, grid, s, x, nvec, rows, out); break;
                case 4: launch_scan(k_narrow<Fmt, OP, 4>, grid, s, x, nvec, rows, out); break;
                case 8: launch_scan(k_narrow<Fmt, OP, 8>, grid, s, x, nvec, rows, out); break;
                case 16: launch_scan(k_narrow<Fmt, OP, 16>, grid, s, x, nvec, rows, out); break;
                case 32: launch_scan(k_narrow<Fmt, OP, 32>, grid, s, x, nvec, rows, out); break;
                default: return hipErrorInvalidValue;
            }
            return hipGetLastError();
        }
        // Other narrow rows: groups cover their row with one vector per lane; a wavefront per
        // row keeps up to 8 vectors per lane in flight.
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
    if (p.path == ARGREDUCE_PATH_WIDE) {
        using Wd = Wide<typename Fmt::C>;
        Wd* part = reinterpret_cast<Wd*>(scratch16);
        const uint32_t W = static_cast<uint32_t>(p.window);
        const uint32_t G = static_cast<uint32_t>(p.windows);
        const dim3 grid(static_cast<uint32_t>(rows * p.windows));
        switch (p.unroll) {
            case 2: launch_scan(k_wide<Fmt, OP, 2>, grid, s, x, cols, W, G, part); break;
            case 8: launch_scan(k_wide<Fmt, OP, 8>, grid, s, x, cols, W, G, part); break;
            default: return hipErrorInvalidValue;
        }
        const int64_t mgrid = rows < 65536 ? rows : 65536;
        hipLaunchKernelGGL((k_wide_merge<Fmt, OP>), dim3(static_cast<uint32_t>(mgrid)),
                           dim3(kBlockThreads), 0, s, static_cast<const Wd*>(part), G, rows, out);
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

template <typename Fmt, int OP, int TL, int LD, int U>
void launch_axis_tl(const AxisPlan& p, const uint8_t* x, int64_t* out, uint8_t* scratch16,
                    hipStream_t s) {
    using P = Partial<typename Fmt::C>;
    P* part = reinterpret_cast<P*>(scratch16);
    const uint32_t B = static_cast<uint32_t>(p.blocks_per_tile);
    launch_scan(k_axis<Fmt, OP, TL, LD, U>, dim3(static_cast<uint32_t>(p.grid_blocks)), s, x,
                p.inner, p.tiles, out, B > 1 ? part : nullptr, static_cast<uint32_t>(p.len), B,
                static_cast<uint32_t>(p.grid_blocks));
    if (B == 1) return;
    // lanes per output group: fewer (more thread rows) as B grows, so that every thread
    // loads at most 8 partials
    const int ml = B <= 32 ? 64 : (B <= 256 ? 8 : 1);
    const int64_t groups = (p.tile + ml - 1) / ml;
    const int64_t work = p.tiles * groups;
    const dim3 grid(static_cast<uint32_t>(work < (int64_t{1} << 20) ? work : (int64_t{1} << 20)));
    const P* cpart = part;
    if (ml == 64)
        hipLaunchKernelGGL((k_axis_merge<Fmt, OP, 64>), grid, dim3(kBlockThreads), 0, s, cpart, out,
                           p.inner, p.tiles_per_o, p.tiles, B, static_cast<int>(p.tile), grid.x);
    else if (ml == 8)
        hipLaunchKernelGGL((k_axis_merge<Fmt, OP, 8>), grid, dim3(kBlockThreads), 0, s, cpart, out,
                           p.inner, p.tiles_per_o, p.tiles, B, static_cast<int>(p.tile), grid.x);
    else
        hipLaunchKernelGGL((k_axis_merge<Fmt, OP, 1>), grid, dim3(kBlockThreads), 0, s, cpart, out,
                           p.inner, p.tiles_per_o, p.tiles, B, static_cast<int>(p.tile), grid.x);
}

template <typename Fmt, int OP>
hipError_t launch_axis_fmt(const AxisPlan& p, const void* xv, int64_t* out, uint8_t* scratch16,
                           hipStream_t s) {
    const uint8_t* x = static_cast<const uint8_t*>(xv);
    // 16-byte loads: U = 8 (4 for 8-byte elements, whose vectors need twice the registers
    // per output). Element loads: 64 bytes in flight per lane, U = 32 / 16 / 8 for 2- / 4- /
    // 8-byte elements; with U = 8 for every size, a lane of 2-byte elements had 16 bytes in
    // flight and the calls ran 3.7-6.3 times longer ([1,100000,1100] fp16 327.7 -> 51.9 us,
    // [256,2048,5] fp16 25.6 -> 5.2 us), 4-byte ones 16-32% longer. Element loads have
    // inner >= 2, so at least 2 lanes.
    constexpr int UV = Fmt::VW == 2 ? 4 : 8;
    constexpr int UE = Fmt::kSize == 2 ? 32 : (Fmt::kSize == 4 ? 16 : 8);
    // element loads through a buffer resource when every offset from a tile's first output
    // at position 0 fits in 32 bits: positions up to len + one step, columns up to a tile
    const uint64_t rstride = static_cast<uint64_t>(p.inner) * Fmt::kSize;
    const uint64_t step = static_cast<uint64_t>(p.blocks_per_tile) * (kBlockThreads / p.lanes) * UE;
    const bool buf = !p.vec && (static_cast<uint64_t>(p.len) + step) * rstride +
                                   static_cast<uint64_t>(p.tile) * Fmt::kSize < (uint64_t{1} << 32);
    switch (p.vec * 1000 + (buf ? 2000 : 0) + p.lanes) {
        case 2: launch_axis_tl<Fmt, OP, 2, 0, UE>(p, x, out, scratch16, s); break;
        case 2002: launch_axis_tl<Fmt, OP, 2, 2, UE>(p, x, out, scratch16, s); break;
        case 4: launch_axis_tl<Fmt, OP, 4, 0, UE>(p, x, out, scratch16, s); break;
        case 2004: launch_axis_tl<Fmt, OP, 4, 2, UE>(p, x, out, scratch16, s); break;
        case 8: launch_axis_tl<Fmt, OP, 8, 0, UE>(p, x, out, scratch16, s); break;
        case 2008: launch_axis_tl<Fmt, OP, 8, 2, UE>(p, x, out, scratch16, s); break;
        case 16: launch_axis_tl<Fmt, OP, 16, 0, UE>(p, x, out, scratch16, s); break;
        case 2016: launch_axis_tl<Fmt, OP, 16, 2, UE>(p, x, out, scratch16, s); break;
        case 32: launch_axis_tl<Fmt, OP, 32, 0, UE>(p, x, out, scratch16, s); break;
        case 2032: launch_axis_tl<Fmt, OP, 32, 2, UE>(p, x, out, scratch16, s); break;
        case 64: launch_axis_tl<Fmt, OP, 64, 0, UE>(p, x, out, scratch16, s); break;
        case 2064: launch_axis_tl<Fmt, OP, 64, 2, UE>(p, x, out, scratch16, s); break;
        case 1001: launch_axis_tl<Fmt, OP, 1, 1, UV>(p, x, out, scratch16, s); break;
        case 1002: launch_axis_tl<Fmt, OP, 2, 1, UV>(p, x, out, scratch16, s); break;
        case 1004: launch_axis_tl<Fmt, OP, 4, 1, UV>(p, x, out, scratch16, s); break;
        case 1008: launch_axis_tl<Fmt, OP, 8, 1, UV>(p, x, out, scratch16, s); break;
        case 1016: launch_axis_tl<Fmt, OP, 16, 1, UV>(p, x, out, scratch16, s); break;
        case 1032: launch_axis_tl<Fmt, OP, 32, 1, UV>(p, x, out, scratch16, s); break;
        case 1064: launch_axis_tl<Fmt, OP, 64, 1, UV>(p, x, out, scratch16, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename Fmt>
hipError_t launch_axis_op(const AxisPlan& p, const void* x, int op, int64_t* out,
                          uint8_t* scratch16, hipStream_t s) {
    switch (op) {
        case ARGREDUCE_MAX: return launch_axis_fmt<Fmt, kMax>(p, x, out, scratch16, s);
        case ARGREDUCE_MIN: return launch_axis_fmt<Fmt, kMin>(p, x, out, scratch16, s);
        case ARGREDUCE_MAX_LAST: return launch_axis_fmt<Fmt, kMaxLast>(p, x, out, scratch16, s);
        case ARGREDUCE_MIN_LAST: return launch_axis_fmt<Fmt, kMinLast>(p, x, out, scratch16, s);
        default: return hipErrorInvalidValue;
    }
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

hipError_t launch_axis(const AxisPlan& p, const void* x, int dtype, int op, int64_t* out,
                       uint8_t* scratch16, hipStream_t s) {
    switch (dtype) {
        case ARGREDUCE_F32: return launch_axis_op<F32>(p, x, op, out, scratch16, s);
        case ARGREDUCE_F16: return launch_axis_op<F16>(p, x, op, out, scratch16, s);
        case ARGREDUCE_BF16: return launch_axis_op<BF16>(p, x, op, out, scratch16, s);
        case ARGREDUCE_F64: return launch_axis_op<F64>(p, x, op, out, scratch16, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_empty(hipStream_t s) {
    hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, s);
    return hipGetLastError();
}

hipError_t launch_store_floor(int64_t* out, hipStream_t s) {
    hipLaunchKernelGGL(k_store_floor, dim3(1), dim3(64), 0, s, out);
    return hipGetLastError();
}

hipError_t launch_read_floor(const void* x, size_t bytes, uint32_t* out, uint32_t grid,
                             hipStream_t s) {
    hipLaunchKernelGGL(k_read_floor, dim3(grid), dim3(kBlockThreads), 0, s,
                       static_cast<const u32x4*>(x), bytes / 16, out);
    return hipGetLastError();
}

void set_kernel_events(hipEvent_t start, hipEvent_t stop) {
    g_ev_start.store(start, std::memory_order_relaxed);
    g_ev_stop.store(stop, std::memory_order_relaxed);
}

size_t wide_partial_bytes(int dtype) {
    return dtype == ARGREDUCE_F64 ? sizeof(Wide<double>) : sizeof(Wide<float>);
}

size_t axis_partial_bytes(int dtype) {
    return dtype == ARGREDUCE_F64 ? sizeof(Partial<double>) : sizeof(Partial<float>);
}

size_t partial_entry_bytes(int dtype) {
    return sizeof(uint64_t) * (dtype == ARGREDUCE_F64 ? Words<double>::kStride : Words<float>::kStride);
}

}  // namespace argreduce
