// Device-side building blocks of the gfx950 last-axis ArgMax / ArgMin kernels.
//
// The semantics being parallelised ("[CUDA] Parallelize ArgMax/ArgMin over wide last
// axes", Description / Semantics) are those of a sequential scan seeded with element 0
// that moves only on a strictly better element. Its result is the first position of the
// extremum of the non-NaN elements, or 0 when element 0 is NaN. That closed form is what
// makes a parallel merge possible:
//
//   * each lane scans its share of the row in increasing position order with the same
//     strict comparison, starting from an empty candidate (value -inf for ArgMax / +inf
//     for ArgMin, index SENTINEL > any position): the identity the page prescribes;
//   * candidates of different lanes, waves and workgroups are merged with a commutative,
//     associative rule: the better value wins, equal values go to the lower index;
//   * the lane that owns the row's first element is seeded with (fix(x[0]), 0), where
//     fix(NaN) is the op's absorbing value (+inf for ArgMax, -inf for ArgMin) and
//     fix(v) = v otherwise. A NaN at position 0 then beats every other candidate, which
//     gives the page's "leading NaN yields index 0"; a -inf (ArgMax) at position 0 is kept
//     as a real candidate, which gives "a row of -inf returns 0".
//
// NaN elsewhere never enters a candidate (every comparison with NaN is false). -0 and +0
// compare equal, so the index decides. No fast-math, no flush-to-zero: subnormals compare
// exactly. Values travel only through compare-and-select, never through min/max
// instructions, whose NaN and signed-zero rules differ.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace argreduce {

constexpr int kBlockThreads = 256;  // threads per workgroup of every kernel
constexpr int kWave = 64;           // gfx950 wavefront
constexpr uint32_t kSentinel = 0x7fffffffu;  // > every position (cols <= INT32_MAX)

enum Op { kMax = 0, kMin = 1 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// Element formats. VW = elements per 16-byte vector; C = the (exact) comparison type.

struct F32 {
    using C = float;
    static constexpr int kSize = 4;
    static constexpr int VW = 4;
    __device__ static C load1(const uint8_t* p) { return *reinterpret_cast<const float*>(p); }
    __device__ static void unpack(const u32x4 q, C (&e)[VW]) {
        e[0] = __uint_as_float(q.x);
        e[1] = __uint_as_float(q.y);
        e[2] = __uint_as_float(q.z);
        e[3] = __uint_as_float(q.w);
    }
};

struct F16 {
    using C = float;
    static constexpr int kSize = 2;
    static constexpr int VW = 8;
    __device__ static C lo(uint32_t w) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
    }
    __device__ static C hi(uint32_t w) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
    }
    __device__ static C load1(const uint8_t* p) {
        return static_cast<float>(*reinterpret_cast<const _Float16*>(p));
    }
    __device__ static void unpack(const u32x4 q, C (&e)[VW]) {
        e[0] = lo(q.x); e[1] = hi(q.x);
        e[2] = lo(q.y); e[3] = hi(q.y);
        e[4] = lo(q.z); e[5] = hi(q.z);
        e[6] = lo(q.w); e[7] = hi(q.w);
    }
};

struct BF16 {
    using C = float;
    static constexpr int kSize = 2;
    static constexpr int VW = 8;
    // bfloat16 is the upper half of a binary32: widening is a shift (exact).
    __device__ static C lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ static C hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
    __device__ static C load1(const uint8_t* p) {
        return __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(p)) << 16);
    }
    __device__ static void unpack(const u32x4 q, C (&e)[VW]) {
        e[0] = lo(q.x); e[1] = hi(q.x);
        e[2] = lo(q.y); e[3] = hi(q.y);
        e[4] = lo(q.z); e[5] = hi(q.z);
        e[6] = lo(q.w); e[7] = hi(q.w);
    }
};

struct F64 {
    using C = double;
    static constexpr int kSize = 8;
    static constexpr int VW = 2;
    __device__ static C load1(const uint8_t* p) { return *reinterpret_cast<const double*>(p); }
    __device__ static void unpack(const u32x4 q, C (&e)[VW]) {
        e[0] = __hiloint2double(static_cast<int>(q.y), static_cast<int>(q.x));
        e[1] = __hiloint2double(static_cast<int>(q.w), static_cast<int>(q.z));
    }
};

// ---------------------------------------------------------------------------------------
// (value, index) candidate.

template <typename C, int OP>
struct Cand {
    C v;
    uint32_t i;

    __device__ static constexpr C identity() {
        return OP == kMax ? -__builtin_huge_val() : __builtin_huge_val();
    }
    __device__ static constexpr C absorbing() {
        return OP == kMax ? __builtin_huge_val() : -__builtin_huge_val();
    }
    __device__ static bool better(C a, C b) { return OP == kMax ? (a > b) : (a < b); }

    __device__ void init() {
        v = identity();
        i = kSentinel;
    }
    // Position 0 of the row: taken unconditionally, with NaN replaced by the absorbing value.
    __device__ void seed(C x0) {
        v = (x0 != x0) ? absorbing() : x0;
        i = 0;
    }
    // Strict update, for positions visited in increasing order by one lane.
    __device__ void update(C e, uint32_t pos) {
        const bool t = better(e, v);
        v = t ? e : v;
        i = t ? pos : i;
    }
    // Merge with another lane's candidate: better value wins, equal values -> lower index.
    __device__ void merge(C ov, uint32_t oi) {
        const bool t = better(ov, v) || (ov == v && oi < i);
        v = t ? ov : v;
        i = t ? oi : i;
    }
};

// ---------------------------------------------------------------------------------------
// Cross-lane merges.

template <typename C>
__device__ inline C shfl_xor(C v, int mask, int width) {
    return __shfl_xor(v, mask, width);
}

// Butterfly over aligned groups of G lanes (G a power of two <= 64): every lane of the
// group ends with the group's merged candidate.
template <int G, typename C, int OP>
__device__ inline void group_merge(Cand<C, OP>& c) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) {
        const C ov = shfl_xor(c.v, m, G);
        const uint32_t oi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(c.i), m, G));
        c.merge(ov, oi);
    }
}

// Merge over the whole workgroup; the result is valid in thread 0. Uses LDS and two
// barriers; every thread of the block must call it.
template <typename C, int OP>
__device__ inline void block_merge(Cand<C, OP>& c) {
    constexpr int kWaves = kBlockThreads / kWave;
    __shared__ C s_v[kWaves];
    __shared__ uint32_t s_i[kWaves];
    group_merge<kWave>(c);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (lane == 0) {
        s_v[wave] = c.v;
        s_i[wave] = c.i;
    }
    __syncthreads();
    if (wave == 0) {
        if (lane < kWaves) {
            c.v = s_v[lane];
            c.i = s_i[lane];
        } else {
            c.init();
        }
        group_merge<kWaves>(c);
    }
    __syncthreads();  // s_v / s_i may be reused by the caller's next call
}

// ---------------------------------------------------------------------------------------
// Per-lane scan of one row.
//
// A team of `team` lanes scans row `row` (cols elements, starting at any address aligned
// to the element size). The row is cut into a head of up to VW-1 elements before the first
// 16-byte boundary, a body of nvec 16-byte vectors, and a tail of up to VW-1 elements.
// Lane `lane` takes head/tail elements lane, lane+team, ... and body vectors lane,
// lane+team, ... in increasing order, U vectors in flight per step. Positions are 32-bit
// and formed only after the bounds check: the remaining count (nvec - base) is compared,
// never a sum that could pass INT32_MAX. Byte offsets are 64-bit.

template <typename Fmt, int OP, int U, bool kGuard>
__device__ inline void scan_step(const uint8_t* __restrict__ body, uint32_t base, uint32_t rem,
                                 uint32_t lane, uint32_t team, uint32_t head,
                                 Cand<typename Fmt::C, OP>& c) {
    u32x4 q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t d = lane + static_cast<uint32_t>(u) * team;
        if (!kGuard || d < rem)
            q[u] = *reinterpret_cast<const u32x4*>(body + static_cast<size_t>(base + d) * 16u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t d = lane + static_cast<uint32_t>(u) * team;
        if (!kGuard || d < rem) {
            typename Fmt::C e[Fmt::VW];
            Fmt::unpack(q[u], e);
            const uint32_t pos = head + (base + d) * Fmt::VW;
#pragma unroll
            for (int k = 0; k < Fmt::VW; ++k) c.update(e[k], pos + k);
        }
    }
}

template <typename Fmt, int OP, int U>
__device__ inline void scan_row(const uint8_t* __restrict__ row, uint32_t cols, uint32_t lane,
                                uint32_t team, Cand<typename Fmt::C, OP>& c) {
    c.init();
    const uint32_t misalign = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(row) & 15u);
    uint32_t head = ((16u - misalign) & 15u) / Fmt::kSize;
    head = head < cols ? head : cols;
    const uint32_t nvec = (cols - head) / Fmt::VW;
    const uint32_t tail0 = head + nvec * Fmt::VW;

    if (lane == 0) c.seed(Fmt::load1(row));
    for (uint32_t k = lane; k < head; k += team)
        c.update(Fmt::load1(row + static_cast<size_t>(k) * Fmt::kSize), k);

    const uint8_t* body = row + static_cast<size_t>(head) * Fmt::kSize;  // 16-byte aligned
    const uint32_t step = team * U;
    for (uint32_t base = 0; base < nvec; base += step) {
        const uint32_t rem = nvec - base;
        if (rem >= step) {
            scan_step<Fmt, OP, U, false>(body, base, rem, lane, team, head, c);
        } else {
            scan_step<Fmt, OP, U, true>(body, base, rem, lane, team, head, c);
            break;
        }
        if (rem == step) break;
    }

    for (uint32_t k = tail0 + lane; k < cols; k += team)
        c.update(Fmt::load1(row + static_cast<size_t>(k) * Fmt::kSize), k);
}

}  // namespace argreduce
