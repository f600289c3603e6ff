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
//   * position 0 also enters as a candidate of its own, (fix(x[0]), 0), merged like any
//     other (the merge is commutative, so this equals seeding the scan with it), where
//     fix(NaN) is the op's absorbing
//     value (+inf for ArgMax, -inf for ArgMin) and fix(v) = v otherwise. A NaN at
//     position 0 then beats every other candidate, which gives the page's "leading NaN
//     yields index 0"; a -inf (ArgMax) at position 0 is kept as a real candidate, which
//     gives "a row of -inf returns 0".
//
// The last-index ops (ONNX's select_last_index = 1: the same scan with a non-strict
// comparison) mirror the tie rule: a lane moves to equal later elements, equal values go
// to the HIGHER index, and the empty candidate's index is -1. A NaN at position 0 enters
// as (NaN, INT32_MAX): no comparison can displace a NaN value inside a lane, merges give
// that index priority explicitly, and the result maps it back to 0.
//
// NaN elsewhere never enters a candidate (every comparison with NaN is false). -0 and +0
// compare equal, so the index decides. No fast-math, no flush-to-zero: subnormals compare
// exactly. Values travel only through compare-and-select, never through min/max
// instructions, whose NaN and signed-zero rules differ.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace argreduce {

constexpr int kBlockThreads = 256;  // threads per workgroup of every kernel
constexpr int kWave = 64;           // gfx950 wavefront
constexpr uint32_t kSentinel = 0x7fffffffu;  // > every position (cols <= INT32_MAX)
constexpr uint32_t kNoneLast = 0xffffffffu;  // -1 as int32: < every position
constexpr uint32_t kNaN0Last = 0x7fffffffu;  // leading NaN under the last-index ops

// Values match argreduce_op_t.
enum Op { kMax = 0, kMin = 1, kMaxLast = 2, kMinLast = 3 };
__host__ __device__ constexpr bool op_is_max(int op) { return op == kMax || op == kMaxLast; }
__host__ __device__ constexpr bool op_is_last(int op) { return op == kMaxLast || op == kMinLast; }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// Element formats. VW = elements per 16-byte vector; C = the (exact) comparison type;
// Vec = the 16-byte vector type the body is loaded as. Loading each format as its own
// vector type keeps the compiler from re-reading parts of a vector through narrower loads.

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct F32 {
    using C = float;
    using Vec = f32x4;
    static constexpr int kSize = 4;
    static constexpr int VW = 4;
    using Bits = uint32_t;
    __device__ static C from_bits(Bits b) { return __uint_as_float(b); }
    __device__ static C load1(const uint8_t* p) { return *reinterpret_cast<const float*>(p); }
    __device__ static void unpack(const Vec q, C (&e)[VW]) {
        e[0] = q.x;
        e[1] = q.y;
        e[2] = q.z;
        e[3] = q.w;
    }
};

struct F16 {
    using C = float;
    using Vec = f16x8;
    static constexpr int kSize = 2;
    static constexpr int VW = 8;
    using Bits = uint16_t;
    __device__ static C from_bits(Bits b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }
    __device__ static C load1(const uint8_t* p) {
        return static_cast<float>(*reinterpret_cast<const _Float16*>(p));
    }
    __device__ static void unpack(const Vec q, C (&e)[VW]) {
#pragma unroll
        for (int k = 0; k < VW; ++k) e[k] = static_cast<float>(q[k]);
    }
};

struct BF16 {
    using C = float;
    using Vec = u32x4;
    static constexpr int kSize = 2;
    static constexpr int VW = 8;
    // bfloat16 is the upper half of a binary32: widening is a shift (exact).
    __device__ static C lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ static C hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
    using Bits = uint16_t;
    __device__ static C from_bits(Bits b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }
    __device__ static C load1(const uint8_t* p) {
        return from_bits(*reinterpret_cast<const uint16_t*>(p));
    }
    __device__ static void unpack(const Vec q, C (&e)[VW]) {
        e[0] = lo(q.x); e[1] = hi(q.x);
        e[2] = lo(q.y); e[3] = hi(q.y);
        e[4] = lo(q.z); e[5] = hi(q.z);
        e[6] = lo(q.w); e[7] = hi(q.w);
    }
};

struct F64 {
    using C = double;
    using Vec = f64x2;
    static constexpr int kSize = 8;
    static constexpr int VW = 2;
    using Bits = uint64_t;
    __device__ static C from_bits(Bits b) { return __longlong_as_double(static_cast<long long>(b)); }
    __device__ static C load1(const uint8_t* p) { return *reinterpret_cast<const double*>(p); }
    __device__ static void unpack(const Vec q, C (&e)[VW]) {
        e[0] = q.x;
        e[1] = q.y;
    }
};

// One element of a floating-point format through a buffer resource (raw buffer load at
// byte offset voff + soff; soff is uniform across the wavefront).
template <typename Fmt>
__device__ inline typename Fmt::C buffer_load1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (Fmt::kSize == 2) {
        const unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(voff), static_cast<int>(soff), 0);
        return Fmt::from_bits(h);
    } else if constexpr (Fmt::kSize == 4) {
        const unsigned int w = __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff), static_cast<int>(soff), 0);
        return Fmt::from_bits(w);
    } else {
        const auto w = __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(voff), static_cast<int>(soff), 0);
        return Fmt::from_bits(static_cast<uint64_t>(w[0]) | (static_cast<uint64_t>(w[1]) << 32));
    }
}

// Integer formats (the cumulative scan): compared exactly in their own type.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef long i64x2 __attribute__((ext_vector_type(2)));

struct I32 {
    using C = int32_t;
    using Vec = i32x4;
    static constexpr int kSize = 4;
    static constexpr int VW = 4;
    __device__ static C load1(const uint8_t* p) { return *reinterpret_cast<const int32_t*>(p); }
    __device__ static void unpack(const Vec q, C (&e)[VW]) {
        e[0] = q.x;
        e[1] = q.y;
        e[2] = q.z;
        e[3] = q.w;
    }
};

struct I64 {
    using C = int64_t;
    using Vec = i64x2;
    static constexpr int kSize = 8;
    static constexpr int VW = 2;
    __device__ static C load1(const uint8_t* p) { return *reinterpret_cast<const int64_t*>(p); }
    __device__ static void unpack(const Vec q, C (&e)[VW]) {
        e[0] = q.x;
        e[1] = q.y;
    }
};

// ---------------------------------------------------------------------------------------
// (value, index) candidate.

template <typename C, int OP>
struct Cand {
    C v;
    uint32_t i;

    static constexpr bool kMaxOp = op_is_max(OP);
    static constexpr bool kLast = op_is_last(OP);
    static constexpr uint32_t kNone = kLast ? kNoneLast : kSentinel;  // empty candidate

    __device__ static constexpr C identity() {
        return kMaxOp ? -__builtin_huge_val() : __builtin_huge_val();
    }
    __device__ static constexpr C absorbing() {
        return kMaxOp ? __builtin_huge_val() : -__builtin_huge_val();
    }
    __device__ static bool better(C a, C b) { return kMaxOp ? (a > b) : (a < b); }
    // Tie preference between two indices: lower wins, or higher for the last-index ops
    // (compared as signed, so the empty candidate's -1 loses).
    __device__ static bool tie_wins(uint32_t a, uint32_t b) {
        return kLast ? static_cast<int32_t>(a) > static_cast<int32_t>(b) : a < b;
    }
    // Whether an index can come out of a lane's scan of a row of `cols` elements.
    __device__ static bool valid_index(uint32_t a, uint32_t cols) {
        return a < cols || a == kNone || (kLast && a == kNaN0Last);
    }
    // The row's result from the merged candidate's index.
    __device__ static int64_t result(uint32_t a) {
        return (kLast && a == kNaN0Last) ? int64_t{0} : static_cast<int64_t>(a);
    }

    __device__ void init() {
        v = identity();
        i = kNone;
    }
    // Value under which position 0 enters: NaN becomes the absorbing value.
    __device__ static C fix(C x0) { return (x0 != x0) ? absorbing() : x0; }
    // The candidate of position 0: (fix(e), 0); under the last-index ops a NaN there
    // enters as (NaN, INT32_MAX), which no element can replace (every comparison with NaN
    // is false) and merges give priority.
    __device__ void take_first(C e) {
        const bool nan = (e != e);
        if constexpr (kLast) {
            v = e;
            i = nan ? kNaN0Last : 0u;
        } else {
            v = nan ? absorbing() : e;
            i = 0u;
        }
    }
    // Update for positions visited in increasing order by one lane: strict comparison, or
    // non-strict for the last-index ops (false for NaN either way).
    // (Bitwise, not short-circuit, operators here and in merge: each comparison becomes a
    // lane mask combined on the scalar unit, with no branches.)
    __device__ void update(C e, uint32_t pos) {
        const bool t = kLast ? (better(e, v) | (e == v)) : better(e, v);
        v = t ? e : v;
        i = t ? pos : i;
    }
    // Merge with another lane's candidate: better value wins, equal values -> tie rule;
    // under the last-index ops a leading NaN (index INT32_MAX) wins outright.
    __device__ void merge(C ov, uint32_t oi) {
        const bool nan0 = kLast ? (oi == kNaN0Last) : false;
        const bool t = nan0 | better(ov, v) | ((ov == v) & tie_wins(oi, i));
        v = t ? ov : v;
        i = t ? oi : i;
    }
};

// ---------------------------------------------------------------------------------------
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

// ---------------------------------------------------------------------------------------
// Cross-lane merges, on the DPP crossbar (no LDS round trip).
//
// update_dpp keeps a lane's own value where the pattern gives it no source (row_mask),
// and merging a candidate with itself changes nothing, so every step is safe in all lanes.

template <int CTRL, int ROW_MASK>
__device__ inline uint32_t dpp_u32(uint32_t v) {
    // With every row enabled each pattern used here gives every lane a source, so no
    // "old" value (and no copy of it) is needed.
    if constexpr (ROW_MASK == 0xf)
        return static_cast<uint32_t>(
            __builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, ROW_MASK, 0xf, false));
    else
        return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
            static_cast<int>(v), static_cast<int>(v), CTRL, ROW_MASK, 0xf, false));
}
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_val(float v) {
    return __uint_as_float(dpp_u32<CTRL, ROW_MASK>(__float_as_uint(v)));
}
template <int CTRL, int ROW_MASK>
__device__ inline double dpp_val(double v) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint32_t lo = dpp_u32<CTRL, ROW_MASK>(static_cast<uint32_t>(b));
    const uint32_t hi = dpp_u32<CTRL, ROW_MASK>(static_cast<uint32_t>(b >> 32));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
template <int CTRL, int ROW_MASK, typename C, int OP>
__device__ inline void dpp_merge(Cand<C, OP>& c) {
    const C ov = dpp_val<CTRL, ROW_MASK>(c.v);
    const uint32_t oi = dpp_u32<CTRL, ROW_MASK>(c.i);
    c.merge(ov, oi);
}

// A 32-bit candidate as one 64-bit key whose unsigned order is the merge rule: the value,
// mapped to an unsigned integer in its order (sign-magnitude to offset binary; reversed for
// the min ops; -0 first made +0, since the two compare equal), above the index arranged so
// that the preferred index of a tie is the larger (its complement for the first-index ops,
// index + 1 for the last-index ones, whose empty index -1 then loses every tie). A
// last-index leading NaN, which wins outright, is the all-ones key (no other key reaches
// it: the largest value key is that of +inf). A merge step is then one 64-bit compare and
// two selects. Only the value's order survives the round trip (-0 returns as +0), which is
// all a merge or a result uses.
template <int OP>
struct Key32 {
    static constexpr bool kMaxOp = op_is_max(OP);
    static constexpr bool kLast = op_is_last(OP);
    __device__ static uint64_t make(float v, uint32_t i) {
        const uint32_t u = __float_as_uint(v + 0.0f);  // -0 -> +0 (never folded: no fast-math)
        uint32_t hi = (u >> 31) ? ~u : (u | 0x80000000u);
        hi = kMaxOp ? hi : ~hi;
        const uint32_t lo = kLast ? i + 1u : ~i;
        const uint64_t k = (static_cast<uint64_t>(hi) << 32) | lo;
        return (kLast && i == kNaN0Last) ? ~uint64_t{0} : k;
    }
    __device__ static void split(uint64_t k, float& v, uint32_t& i) {
        uint32_t hi = static_cast<uint32_t>(k >> 32);
        const uint32_t lo = static_cast<uint32_t>(k);
        hi = kMaxOp ? hi : ~hi;
        v = __uint_as_float((hi >> 31) ? (hi & 0x7fffffffu) : ~hi);
        i = kLast ? lo - 1u : ~lo;
        if (kLast && k == ~uint64_t{0}) {
            v = __builtin_nanf("");
            i = kNaN0Last;
        }
    }
};

// One step of an unsigned 32-bit maximum over the DPP pattern CTRL: a lane without a
// source (bound_ctrl) or outside ROW_MASK takes 0, the identity, so the compiler folds the
// move into one v_max_u32 with a DPP operand.
template <int CTRL, int ROW_MASK>
__device__ inline uint32_t dpp_max_u32(uint32_t h) {
    const uint32_t o = static_cast<uint32_t>(
        ROW_MASK == 0xf
            ? __builtin_amdgcn_mov_dpp(static_cast<int>(h), CTRL, ROW_MASK, 0xf, true)
            : __builtin_amdgcn_update_dpp(0, static_cast<int>(h), CTRL, ROW_MASK, 0xf, false));
    return o > h ? o : h;
}
// Unsigned maximum over the 64 lanes of a wavefront, in lane 63 (the six patterns of
// group_merge), then read out as a wave-uniform value.
__device__ inline uint32_t wave_max_u32(uint32_t h) {
    h = dpp_max_u32<0xB1, 0xf>(h);
    h = dpp_max_u32<0x4E, 0xf>(h);
    h = dpp_max_u32<0x141, 0xf>(h);
    h = dpp_max_u32<0x140, 0xf>(h);
    h = dpp_max_u32<0x142, 0xa>(h);
    h = dpp_max_u32<0x143, 0xc>(h);
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(h), 63));
}
// The largest 64-bit key of a wavefront, in two 32-bit passes: the largest upper half,
// then the largest lower half among the lanes that hold it. Each pass is six single
// instructions (v_max_u32 with a DPP operand) instead of six 64-bit compare-and-select
// steps, and the result is uniform across the wavefront.
__device__ inline uint64_t wave_max_key(uint64_t k) {
    const uint32_t hi = static_cast<uint32_t>(k >> 32);
    const uint32_t top = wave_max_u32(hi);
    const uint32_t lo = wave_max_u32(hi == top ? static_cast<uint32_t>(k) : 0u);
    return (static_cast<uint64_t>(top) << 32) | lo;
}

template <int CTRL, int ROW_MASK>
__device__ inline uint64_t dpp_max_key(uint64_t k) {
    const uint32_t lo = dpp_u32<CTRL, ROW_MASK>(static_cast<uint32_t>(k));
    const uint32_t hi = dpp_u32<CTRL, ROW_MASK>(static_cast<uint32_t>(k >> 32));
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    return o > k ? o : k;
}

// Merge over aligned groups of G lanes (G a power of two <= 64). Afterwards the group's
// last lane (lane % G == G - 1) holds the group's merged candidate; for G <= 16 every lane
// of the group does. Steps: swap neighbours, swap pairs (quad permutes), mirror within 8,
// mirror within 16, broadcast lane 15 of each 16-lane row into the next row (rows 1, 3),
// broadcast lane 31 into rows 2 and 3. 32-bit values merge as 64-bit keys (Key32); a whole
// wavefront of them in two 32-bit passes (wave_max_key), which leaves the result in every
// lane.
template <int G, typename C, int OP>
__device__ inline void group_merge(Cand<C, OP>& c) {
    if constexpr (std::is_same<C, float>::value && G == 64) {
        Key32<OP>::split(wave_max_key(Key32<OP>::make(c.v, c.i)), c.v, c.i);
    } else if constexpr (std::is_same<C, float>::value) {
        uint64_t k = Key32<OP>::make(c.v, c.i);
        if constexpr (G >= 2) k = dpp_max_key<0xB1, 0xf>(k);   // quad_perm [1,0,3,2]
        if constexpr (G >= 4) k = dpp_max_key<0x4E, 0xf>(k);   // quad_perm [2,3,0,1]
        if constexpr (G >= 8) k = dpp_max_key<0x141, 0xf>(k);  // row_half_mirror
        if constexpr (G >= 16) k = dpp_max_key<0x140, 0xf>(k); // row_mirror
        if constexpr (G >= 32) k = dpp_max_key<0x142, 0xa>(k); // row_bcast:15
        if constexpr (G >= 64) k = dpp_max_key<0x143, 0xc>(k); // row_bcast:31
        Key32<OP>::split(k, c.v, c.i);
    } else {
        if constexpr (G >= 2) dpp_merge<0xB1, 0xf>(c);
        if constexpr (G >= 4) dpp_merge<0x4E, 0xf>(c);
        if constexpr (G >= 8) dpp_merge<0x141, 0xf>(c);
        if constexpr (G >= 16) dpp_merge<0x140, 0xf>(c);
        if constexpr (G >= 32) dpp_merge<0x142, 0xa>(c);
        if constexpr (G >= 64) dpp_merge<0x143, 0xc>(c);
    }
}

// Merge over the whole workgroup; the result is valid in thread 0. Uses LDS and two
// barriers; every thread of the block must call it.
template <typename C, int OP>
__device__ inline void block_merge(Cand<C, OP>& c) {
    constexpr int kWaves = kBlockThreads / kWave;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if constexpr (std::is_same<C, float>::value) {
        // the wavefronts' keys through LDS, merged by thread 0 as three 64-bit maxima
        __shared__ uint64_t s_k[kWaves];
        const uint64_t k = wave_max_key(Key32<OP>::make(c.v, c.i));
        if (lane == 0) s_k[wave] = k;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint64_t m = s_k[0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) m = s_k[w] > m ? s_k[w] : m;
            Key32<OP>::split(m, c.v, c.i);
        }
    } else {
        __shared__ C s_v[kWaves];
        __shared__ uint32_t s_i[kWaves];
        group_merge<kWave>(c);
        if (lane == kWave - 1) {
            s_v[wave] = c.v;
            s_i[wave] = c.i;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            c.v = s_v[0];
            c.i = s_i[0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) c.merge(s_v[w], s_i[w]);
        }
    }
    __syncthreads();  // the LDS words may be reused by the caller's next call
}

// ---------------------------------------------------------------------------------------
// Per-lane scan of one row.
//
// A team of `team` lanes scans row `row` (cols elements, starting at any address aligned
// to the element size). The row is cut into a head of up to VW-1 elements before the first
// 16-byte boundary, a body of nvec 16-byte vectors, and a tail of up to VW-1 elements.
// Lane `lane` takes head elements lane, lane+team, ..., then body vectors lane,
// lane+team, ... (U vectors in flight per step, loaded nontemporally: each byte is read
// once), then tail elements; its positions therefore increase.
//
// Per step, each lane keeps one running candidate for the step's U·VW elements, as a value
// and the element's step slot u·VW + k (a compile-time constant, so the index select takes
// an inline constant): one compare and two selects per element, no per-slot candidates to
// merge afterwards. The slot becomes a position once per step and the step's candidate is
// merged into the lane's candidate with the tie rule (every position of a step is greater
// than those visited before it). In the last, partial step a lane past the end loads the
// last vector again (a load under a lane condition would be a branch that makes the step's
// loads wait on each other) and replaces it with all-ones bits, a NaN in every format,
// which no comparison takes. Positions are 32-bit and formed only after the bounds check:
// the remaining count (nvec - base) is compared, never a sum that could pass INT32_MAX.
// Byte offsets are 64-bit.

template <typename Fmt, int OP, int U, bool kGuard>
__device__ inline void scan_step(const uint8_t* __restrict__ body, uint32_t base, uint32_t rem,
                                 uint32_t lane, uint32_t team, uint32_t head,
                                 Cand<typename Fmt::C, OP>& c) {
    using C = typename Fmt::C;
    using Vec = typename Fmt::Vec;
    using K = Cand<C, OP>;
    static_assert(U * Fmt::VW <= 64, "step slots must be inline constants");
    constexpr uint32_t kNoSlot = 0xffffffffu;
    Vec q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t d = lane + static_cast<uint32_t>(u) * team;
        const uint32_t dd = (!kGuard || d < rem) ? d : rem - 1;
        q[u] = __builtin_nontemporal_load(
            reinterpret_cast<const Vec*>(body + static_cast<size_t>(base + dd) * 16u));
    }
    // Issue every load of the step before any arithmetic: the scheduler would otherwise
    // interleave (and, under register pressure, wait on) loads one by one.
    __builtin_amdgcn_sched_barrier(0);
    C lv = K::identity();
    uint32_t ls = kNoSlot;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        Vec qu = q[u];
        if constexpr (kGuard) {
            const bool past = lane + static_cast<uint32_t>(u) * team >= rem;
            u32x4 w = __builtin_bit_cast(u32x4, qu);
            w.x = past ? 0xffffffffu : w.x;
            w.y = past ? 0xffffffffu : w.y;
            w.z = past ? 0xffffffffu : w.z;
            w.w = past ? 0xffffffffu : w.w;
            qu = __builtin_bit_cast(Vec, w);
        }
        C e[Fmt::VW];
        Fmt::unpack(qu, e);
#pragma unroll
        for (int k = 0; k < Fmt::VW; ++k) {
            const uint32_t slot = static_cast<uint32_t>(u * Fmt::VW + k);
            const bool t = K::kLast ? (K::better(e[k], lv) | (e[k] == lv)) : K::better(e[k], lv);
            lv = t ? e[k] : lv;
            ls = t ? slot : ls;
        }
    }
    constexpr uint32_t kShift = Fmt::VW == 8 ? 3 : (Fmt::VW == 4 ? 2 : 1);
    const uint32_t pos = head + (base + lane + (ls >> kShift) * team) * Fmt::VW +
                         (ls & (Fmt::VW - 1));
    c.merge(lv, ls == kNoSlot ? K::kNone : pos);
}

// `origin`: false when `row` is a window of a longer row that does not start at the row's
// position 0 (its first element is then an ordinary element).
//
// Position 0 enters as its own candidate (fix(x0), 0) (for the last-index ops a NaN there
// as (NaN, INT32_MAX)), merged into lane 0's result after the scan: the merge is
// commutative, so this equals taking it first, and the scan's ordinary visit of position 0
// is harmless (a NaN is never taken; any other value gives the same or a tie-losing
// candidate). The other lanes, and every step, carry no position-0 test. Lane 0 issues
// the seed's load (raw bits: a conversion right after it would wait for it) before the
// scan and converts it after. The load is a relaxed wavefront-scope atomic load, which is
// always a vector-memory load: with the row address uniform across the wavefront a plain
// (or nontemporal) load becomes a scalar load, whose value the compiler moves into a vector
// register at once, so the wavefront would wait one memory latency before issuing any load
// of the scan.
template <typename Fmt, int OP, int U>
__device__ inline void scan_row(const uint8_t* __restrict__ row, uint32_t cols, uint32_t lane,
                                uint32_t team, Cand<typename Fmt::C, OP>& c, bool origin = true) {
    using C = typename Fmt::C;
    c.init();
    const bool seeded = origin & (lane == 0);
    typename Fmt::Bits x0 = 0;
    if (seeded)
        x0 = __hip_atomic_load(reinterpret_cast<const typename Fmt::Bits*>(row), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WAVEFRONT);
    const uint32_t misalign = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(row) & 15u);
    uint32_t head = ((16u - misalign) & 15u) / Fmt::kSize;
    head = head < cols ? head : cols;
    const uint32_t nvec = (cols - head) / Fmt::VW;
    const uint32_t tail0 = head + nvec * Fmt::VW;

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

    if (seeded) {
        Cand<C, OP> f;
        asm volatile("" : "+v"(x0));  // keeps the conversion (and its wait) here
        f.take_first(Fmt::from_bits(x0));
        c.merge(f.v, f.i);
    }
}

// One step over a row that starts 16-byte aligned and is a whole number nvec <= team * U of
// 16-byte vectors: lane `lane` of a team of `team` lanes loads vectors lane, lane + team,
// ..., all U at once, with no head, tail or step loop; a lane past the row re-reads the
// last vector and turns it into all-ones bits (a NaN in every format, never taken).
// Position 0 enters as its own candidate (fix(x0), 0) from lane 0's first vector, so no
// separate seed load. Same results as scan_row on such rows; measured 0.15-0.17 us per call
// faster on [32, 202048] fp16 and [8, 202048] fp32 split rows.
template <typename Fmt, int OP, int U>
__device__ inline void scan_row_aligned(const uint8_t* __restrict__ row, uint32_t nvec,
                                        uint32_t lane, uint32_t team, Cand<typename Fmt::C, OP>& c) {
    using C = typename Fmt::C;
    using Vec = typename Fmt::Vec;
    using K = Cand<C, OP>;
    constexpr int VW = Fmt::VW;
    static_assert(U * VW <= 64, "step slots must be inline constants");
    constexpr uint32_t kNoSlot = 0xffffffffu;
    Vec q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t d = lane + static_cast<uint32_t>(u) * team;
        q[u] = __builtin_nontemporal_load(reinterpret_cast<const Vec*>(row) + (d < nvec ? d : nvec - 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    C lv = K::identity();
    uint32_t ls = kNoSlot;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool past = lane + static_cast<uint32_t>(u) * team >= nvec;
        u32x4 w = __builtin_bit_cast(u32x4, q[u]);
        w.x = past ? 0xffffffffu : w.x;
        w.y = past ? 0xffffffffu : w.y;
        w.z = past ? 0xffffffffu : w.z;
        w.w = past ? 0xffffffffu : w.w;
        C e[VW];
        Fmt::unpack(__builtin_bit_cast(Vec, w), e);
#pragma unroll
        for (int k = 0; k < VW; ++k) {
            const uint32_t slot = static_cast<uint32_t>(u * VW + k);
            const bool t = K::kLast ? (K::better(e[k], lv) | (e[k] == lv)) : K::better(e[k], lv);
            lv = t ? e[k] : lv;
            ls = t ? slot : ls;
        }
    }
    constexpr uint32_t kShift = VW == 8 ? 3 : (VW == 4 ? 2 : 1);
    c.init();
    c.merge(lv, ls == kNoSlot ? K::kNone : (lane + (ls >> kShift) * team) * VW + (ls & (VW - 1)));
    if (lane == 0) {
        C e[VW];
        Fmt::unpack(q[0], e);
        K f;
        f.take_first(e[0]);
        c.merge(f.v, f.i);
    }
}

// One step over a row at any element-aligned address whose 16-byte vectors, from the one
// holding the row's first byte to the one holding its last, number nv <= team * U: lane
// `lane` of a team of `team` lanes loads vectors lane, lane + team, ..., all U at once, with
// no head, tail, seed load or step loop. Every vector is read whole from its 16-byte aligned
// address: the bytes of it outside the row lie in the same aligned 16 bytes, so the same
// page, as a byte of the row. The lanes holding the row's first and last vector (a branch
// no other lane takes) turn the elements outside the row into NaN, and a lane past the span
// re-reads the last vector and turns it into all-ones bits (a NaN in every format); a NaN is
// never taken. Position 0 enters as its own candidate (fix(x0), 0) from lane 0's first
// vector. Same results as scan_row; it saves scan_row's element loads of the head and tail
// and its seed load. The split kernel takes it for rows that scan_row_aligned does not
// cover (a start off 16 bytes or a partial last vector): measured per call against
// scan_row, [64,32001] fp32 5.19 -> 4.48 us, [1,32001] fp32 3.23 -> 3.01, [1,50257] fp32
// 3.05 -> 2.90, [32,202047] fp16 5.50 -> 5.27. On aligned whole-vector rows its edge tests
// cost 2-7% against scan_row_aligned, and with one workgroup per row ([4096,4097] fp32,
// [300,4099] bf16) it was 5-8% slower than scan_row.
template <typename Fmt, int OP, int U>
__device__ inline void scan_row_span(const uint8_t* __restrict__ row, uint32_t cols,
                                        uint32_t lane, uint32_t team, Cand<typename Fmt::C, OP>& c) {
    using C = typename Fmt::C;
    using Vec = typename Fmt::Vec;
    using K = Cand<C, OP>;
    constexpr int VW = Fmt::VW;
    static_assert(U * VW <= 64, "step slots must be inline constants");
    constexpr uint32_t kNoSlot = 0xffffffffu;
    // at most 32 elements per lane: with 64 (2-byte formats, U = 8) the edge handling does
    // not fit the split kernel's 64 registers
    static_assert(U * VW <= 32, "edge handling needs registers");
    const uint32_t mis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(row) & 15u);
    const uint8_t* base = row - mis;           // 16-byte aligned
    const uint32_t lead = mis / Fmt::kSize;    // elements of vector 0 before the row
    const uint32_t span = lead + cols;         // elements from `base` to the row's end
    const uint32_t nv = (span + VW - 1) / VW;  // vectors (span <= INT32_MAX + 7: no wrap)
    Vec q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t d = lane + static_cast<uint32_t>(u) * team;
        q[u] = __builtin_nontemporal_load(reinterpret_cast<const Vec*>(base) + (d < nv ? d : nv - 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    C lv = K::identity();
    uint32_t ls = kNoSlot;
    C x0 = lv;  // position 0 (lane 0, vector 0, element `lead`)
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t d = lane + static_cast<uint32_t>(u) * team;
        const bool past = d >= nv;
        u32x4 w = __builtin_bit_cast(u32x4, q[u]);
        w.x = past ? 0xffffffffu : w.x;
        w.y = past ? 0xffffffffu : w.y;
        w.z = past ? 0xffffffffu : w.z;
        w.w = past ? 0xffffffffu : w.w;
        C e[VW];
        Fmt::unpack(__builtin_bit_cast(Vec, w), e);
        if (u == 0) {
            x0 = e[0];
#pragma unroll
            for (int k = 1; k < VW; ++k) x0 = (static_cast<uint32_t>(k) == lead) ? e[k] : x0;
        }
        // the first vector's elements before the row, the last one's after it
        const uint32_t lo = d == 0 ? lead : 0u;
        const uint32_t hi = d + 1 == nv ? span - d * VW : static_cast<uint32_t>(VW);
        if ((lo != 0) | (hi < static_cast<uint32_t>(VW))) {
#pragma unroll
            for (int k = 0; k < VW; ++k) {
                const uint32_t kk = static_cast<uint32_t>(k);
                e[k] = (kk >= lo && kk < hi) ? e[k] : static_cast<C>(__builtin_nan(""));
            }
        }
#pragma unroll
        for (int k = 0; k < VW; ++k) {
            const uint32_t slot = static_cast<uint32_t>(u * VW + k);
            const bool t = K::kLast ? (K::better(e[k], lv) | (e[k] == lv)) : K::better(e[k], lv);
            lv = t ? e[k] : lv;
            ls = t ? slot : ls;
        }
    }
    constexpr uint32_t kShift = VW == 8 ? 3 : (VW == 4 ? 2 : 1);
    c.init();
    c.merge(lv, ls == kNoSlot ? K::kNone
                              : (lane + (ls >> kShift) * team) * VW + (ls & (VW - 1)) - lead);
    if (lane == 0) {
        K f;
        f.take_first(x0);
        c.merge(f.v, f.i);
    }
}

}  // namespace argreduce
