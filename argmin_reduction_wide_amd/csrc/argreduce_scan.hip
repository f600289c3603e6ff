// gfx950 kernels of the cumulative extremum with indices (cummax / cummin) along the last
// axis, and their launchers.
//
// What is computed (the PaddlePaddle issue on the cummax/cummin CUDA kernel: its
// reproduction measures cummax along the last axis, and its fix proposals describe the
// operator as a (value, index) reduce with ArgMax semantics, ties to the earlier index):
// every position j of a row reports the sequential ArgMax (cummax) / ArgMin (cummin) scan
// of the prefix 0 .. j, i.e. the index the running best holds after element j and the
// element stored there.
//
// The scan as an associative operator. Each element becomes a pair (value, position):
// position 0 enters as (fix(x0), 0) with fix(NaN) = the op's absorbing value (+inf for
// cummax) and, for a NaN, the marker index kNaN0, so that a leading NaN holds for the
// whole row; an element that is NaN anywhere else enters with the op's identity value
// (-inf for cummax), so it can never be taken. Two adjacent pieces a (earlier) and b
// (later) combine to b when b's value is strictly better, else to a: the leftmost best
// element, which is the sequential strict-compare scan. A piece with no elements is the
// pair (identity, kEmpty) and combines as the identity.
//
// Layout of one call: a row is cut into tiles of 256 * U 16-byte chunks; workgroup g
// takes tile g % T of row g / T (T tiles per row). Wave w of the workgroup owns U rows of
// 64 consecutive chunks (one 16-byte vector per lane per row of chunks, so every load and
// store of a wavefront is contiguous); it scans each row of chunks across its lanes on the
// DPP crossbar (row shifts 1, 2, 4, 8, then the row broadcasts of lanes 15 and 31), carries
// between its rows of chunks, and the four waves carry through LDS.
//
// Rows longer than one tile chain their tiles in a single pass, in the manner of a
// decoupled look-back (Merrill and Garland's scheme, as cub's DeviceScan implements it),
// with aggregates in two levels instead of a walk back through inclusive prefixes: every
// tile publishes its aggregate; the tiles form groups of 64, and the last tile of each full
// group folds its group's aggregates and publishes the group's aggregate before it waits on
// anything else; a tile's exclusive prefix is then the ordered fold of the earlier groups'
// aggregates (64 per round of polls, one per lane of a wavefront) and of the earlier tiles
// of its own group. No wait sits on a chain of other waits. (The walk back through
// inclusive prefixes advanced one 64-tile window per round of polls, and a long row's tiles
// waited for one another: [1, 2^24] fp32 57.2 -> 50.1 us per call.) The states are the
// same self-checking
// words as the split ArgMax path: 64-bit agent-scope atomic stores of (nonce << 32) |
// payload, one word per 32 bits of (index, value), each word validated on its own, so no
// fence orders them. Every call, eager or captured, takes a nonce of its own from the one
// process-wide counter (each value is issued once, until the 32-bit counter wraps), so the
// words an earlier call or graph replay left behind never carry the nonce of a later call.
// A call captured into a HIP graph keeps its nonce across replays, so it first clears its
// words with a small kernel (a graph node, not a memset). Forward progress: a tile waits
// only on tiles of lower workgroup id, which publish their aggregate without waiting. With
// more tiles than fit on the device at once this relies on each XCD starting the
// workgroups it is given in id order (then every wait ends, by induction on the id), the
// assumption of any look-back scan whose tile ids are workgroup ids. The wait is bounded
// all the same: on a timeout the tile's indices are -1 and the device's timeout counter
// g_scan_wait_timeouts goes up by one (never observed outside tests that force it).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <limits>
#include <type_traits>

#include "argreduce_device.hpp"
#include "argreduce_internal.hpp"
#include "argreduce_launch.hpp"

namespace argreduce {

// Look-back waits that gave up, one copy per device (added into argreduce_wait_timeouts).
// Named directly by the kernel, like the split kernel's counter, so that no argument
// carries its address.
__device__ unsigned long long g_scan_wait_timeouts;

hipError_t read_scan_wait_timeouts(unsigned long long* count) {
    void* addr = nullptr;  // the current device's copy
    hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(g_scan_wait_timeouts));
    if (e != hipSuccess) return e;
    return hipMemcpy(count, addr, sizeof(*count), hipMemcpyDeviceToHost);
}

namespace {

constexpr uint32_t kEmpty = 0xffffffffu;  // index of the empty piece
constexpr uint32_t kNaN0 = 0x7fffffffu;   // index of a leading NaN (reported as 0)
constexpr uint32_t kFail = 0xfffffffeu;   // published by a tile whose look-back timed out

// Storage bits of an output value, per format.
template <typename Fmt>
struct Out;
template <>
struct Out<F32> {
    using S = uint32_t;
    __device__ static S bits(float v) { return __float_as_uint(v); }
};
template <>
struct Out<F16> {
    using S = uint16_t;
    __device__ static S bits(float v) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v)); }
};
template <>
struct Out<BF16> {
    using S = uint16_t;
    // the value was widened from bfloat16, so its low 16 bits are zero
    __device__ static S bits(float v) { return static_cast<uint16_t>(__float_as_uint(v) >> 16); }
};
template <>
struct Out<F64> {
    using S = uint64_t;
    __device__ static S bits(double v) { return static_cast<uint64_t>(__double_as_longlong(v)); }
};
template <>
struct Out<I32> {
    using S = uint32_t;
    __device__ static S bits(int32_t v) { return static_cast<uint32_t>(v); }
};
template <>
struct Out<I64> {
    using S = uint64_t;
    __device__ static S bits(int64_t v) { return static_cast<uint64_t>(v); }
};

// The operator on (value, index) pairs.
template <typename C, int OP>
struct ScanOp {
    static constexpr bool kMaxOp = op_is_max(OP);
    __device__ static C identity() {
        if constexpr (std::is_floating_point<C>::value)
            return kMaxOp ? -__builtin_huge_val() : __builtin_huge_val();
        else
            return kMaxOp ? std::numeric_limits<C>::min() : std::numeric_limits<C>::max();
    }
    __device__ static C absorbing() {
        return kMaxOp ? __builtin_huge_val() : -__builtin_huge_val();
    }
    __device__ static bool is_nan(C a) {
        if constexpr (std::is_floating_point<C>::value)
            return a != a;
        else
            return false;
    }
    __device__ static bool better(C a, C b) { return kMaxOp ? (a > b) : (a < b); }
    // (av, ai) := (av, ai) then (bv, bi): the later piece wins only when strictly better.
    __device__ static void combine(C& av, uint32_t& ai, C bv, uint32_t bi) {
        const bool t = (ai == kEmpty) | better(bv, av);  // bitwise: no branch
        av = t ? bv : av;
        ai = t ? bi : ai;
    }
    // The one-element piece of element e at position p.
    __device__ static void single(C e, uint32_t p, C& v, uint32_t& i) {
        const bool nan = is_nan(e);
        if constexpr (std::is_floating_point<C>::value) {
            v = p == 0 ? (nan ? absorbing() : e) : (nan ? identity() : e);
            i = ((p == 0) & nan) ? kNaN0 : p;
        } else {
            v = e;
            i = p;
        }
    }
};

// 32-bit word access to values for the cross-lane moves.
template <typename C>
__device__ inline uint32_t lo_word(C v) {
    if constexpr (sizeof(C) == 4)
        return __builtin_bit_cast(uint32_t, v);
    else
        return static_cast<uint32_t>(__builtin_bit_cast(uint64_t, v));
}
template <typename C>
__device__ inline uint32_t hi_word(C v) {
    if constexpr (sizeof(C) == 4)
        return 0u;
    else
        return static_cast<uint32_t>(__builtin_bit_cast(uint64_t, v) >> 32);
}
template <typename C>
__device__ inline C from_words(uint32_t lo, uint32_t hi) {
    if constexpr (sizeof(C) == 4)
        return __builtin_bit_cast(C, lo);
    else
        return __builtin_bit_cast(C, (static_cast<uint64_t>(hi) << 32) | lo);
}

// DPP move with an explicit value for lanes that get no source.
template <int CTRL, int ROW_MASK>
__device__ inline uint32_t dpp_or(uint32_t old, uint32_t src) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        static_cast<int>(old), static_cast<int>(src), CTRL, ROW_MASK, 0xf, false));
}

// One step of the wavefront's inclusive scan: take the piece of the source lane (the empty
// piece where there is none) as the earlier operand.
template <int CTRL, int ROW_MASK, typename C, int OP>
__device__ inline void scan_dpp_step(C& v, uint32_t& i) {
    using Op = ScanOp<C, OP>;
    const C id = Op::identity();
    C lv = from_words<C>(dpp_or<CTRL, ROW_MASK>(lo_word(id), lo_word(v)),
                         sizeof(C) == 8 ? dpp_or<CTRL, ROW_MASK>(hi_word(id), hi_word(v)) : 0u);
    uint32_t li = dpp_or<CTRL, ROW_MASK>(kEmpty, i);
    Op::combine(lv, li, v, i);
    v = lv;
    i = li;
}

// Inclusive scan over the 64 lanes of a wavefront, in lane order.
template <typename C, int OP>
__device__ inline void wave_scan(C& v, uint32_t& i) {
    scan_dpp_step<0x111, 0xf, C, OP>(v, i);  // row_shr:1
    scan_dpp_step<0x112, 0xf, C, OP>(v, i);  // row_shr:2
    scan_dpp_step<0x114, 0xf, C, OP>(v, i);  // row_shr:4
    scan_dpp_step<0x118, 0xf, C, OP>(v, i);  // row_shr:8
    scan_dpp_step<0x142, 0xa, C, OP>(v, i);  // row_bcast:15 into rows 1 and 3
    scan_dpp_step<0x143, 0xc, C, OP>(v, i);  // row_bcast:31 into rows 2 and 3
}

template <typename C>
__device__ inline C shfl_val(C v, int src) {
    const uint32_t lo = static_cast<uint32_t>(__shfl(static_cast<int>(lo_word(v)), src));
    const uint32_t hi = sizeof(C) == 8 ? static_cast<uint32_t>(__shfl(static_cast<int>(hi_word(v)), src)) : 0u;
    return from_words<C>(lo, hi);
}
template <typename C>
__device__ inline C readlane_val(C v, int lane) {
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo_word(v)), lane));
    const uint32_t hi = sizeof(C) == 8
                            ? static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(hi_word(v)), lane))
                            : 0u;
    return from_words<C>(lo, hi);
}

// Published tile state: (nonce << 32) | payload words: the index, then the value's 32-bit
// halves. 2 words for 32-bit values, 3 for 64-bit ones (stride 4).
template <typename C>
struct StateWords {
    static constexpr int kWords = sizeof(C) == 8 ? 3 : 2;
    static constexpr int kStride = sizeof(C) == 8 ? 4 : 2;
};

template <typename C>
__device__ inline void publish(uint64_t* w, uint32_t nonce, C v, uint32_t i) {
    const uint64_t tag = static_cast<uint64_t>(nonce) << 32;
    __hip_atomic_store(&w[0], tag | i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&w[1], tag | lo_word(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (sizeof(C) == 8)
        __hip_atomic_store(&w[2], tag | hi_word(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reads a published state; true when every word carries this call's nonce.
template <typename C>
__device__ inline bool read_state(const uint64_t* w, uint32_t nonce, C& v, uint32_t& i) {
    const uint64_t w0 = __hip_atomic_load(&w[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t w1 = __hip_atomic_load(&w[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t w2 = 0;
    if constexpr (sizeof(C) == 8)
        w2 = __hip_atomic_load(&w[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = (w0 >> 32) == nonce && (w1 >> 32) == nonce;
    if constexpr (sizeof(C) == 8) ok = ok && (w2 >> 32) == nonce;
    i = static_cast<uint32_t>(w0);
    v = from_words<C>(static_cast<uint32_t>(w1), static_cast<uint32_t>(w2));
    return ok;
}

// The ordered fold of one piece per lane of the wavefront (lane order is tile order; lanes
// without a piece hold the empty one). The result is uniform.
template <typename C, int OP>
__device__ inline void wave_fold(C v, uint32_t i, C& ov, uint32_t& oi) {
    wave_scan<C, OP>(v, i);
    ov = readlane_val(v, kWave - 1);
    oi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(i), kWave - 1));
}

// Polls one published state per lane (`need`) until every lane has its own; false if the
// round limit passed first. Lanes without a state hold the empty piece.
template <typename C, int OP>
__device__ inline bool poll_states(const uint64_t* w, bool need, uint32_t nonce,
                                   uint32_t spin_limit, C& v, uint32_t& i) {
    v = ScanOp<C, OP>::identity();
    i = kEmpty;
    bool have = !need;
    for (uint32_t spins = 0;; ++spins) {
        if (!have) {
            C rv;
            uint32_t ri;
            if (read_state(w, nonce, rv, ri)) {
                v = rv;
                i = ri;
                have = true;
            }
        }
        if (__ballot(!have) == 0) return true;
        if (spins >= spin_limit) return false;
        __builtin_amdgcn_s_sleep(2);
    }
}

// Exclusive prefix of tile t (>= 1) of a row whose tile states start at `row_states`, in
// two levels. The tiles of a row form groups of 64; every tile has published its aggregate
// (state slot 0); the last tile of each full group folds its group's aggregates and
// publishes the group's aggregate (its slot 1) before it waits on anything else. A tile
// then folds, in order, the aggregates of the earlier groups (64 per round of polls) and of
// the earlier tiles of its own group. No wait is on a chain of other waits, so a tile's
// prefix is a round or two of polls behind the last aggregate it needs (a look-back that
// walks back through the tiles' published inclusive prefixes advances one window per
// round: a long row's tiles waited for one another). By one wavefront; the uniform result
// is in every lane. `own` is the tile's aggregate.
template <typename C, int OP>
__device__ inline bool look_back(uint64_t* row_states, uint32_t t, C own_v, uint32_t own_i,
                                 uint32_t nonce, C& accv, uint32_t& acci, uint32_t spin_limit) {
    using Op = ScanOp<C, OP>;
    using SW = StateWords<C>;
    const uint32_t lane = threadIdx.x % kWave;
    const uint32_t gi = t / kWave;  // this tile's group
    const uint32_t pg = t % kWave;  // its place in the group
    auto slot = [&](uint32_t tile, int which) {
        return row_states + (static_cast<size_t>(tile) * 2 + static_cast<size_t>(which)) * SW::kStride;
    };
    // the earlier tiles of the group: lane l < pg holds tile gi * 64 + l
    C v;
    uint32_t i;
    const bool mine = lane < pg;
    bool ok = poll_states<C, OP>(slot(gi * kWave + (mine ? lane : 0), 0), mine, nonce, spin_limit, v, i);
    C yv;
    uint32_t yi;
    wave_fold<C, OP>(v, i, yv, yi);
    if (pg == kWave - 1 && lane == 0) {  // the group's aggregate, for the later groups
        C gv = yv;
        uint32_t gix = yi;
        Op::combine(gv, gix, own_v, own_i);
        publish(slot(t, 1), nonce, gv, ok ? gix : kFail);
    }
    if (!ok) return false;
    // the earlier groups, 64 per round: lane l holds group g0 + l
    accv = Op::identity();
    acci = kEmpty;
    for (uint32_t g0 = 0; g0 < gi; g0 += kWave) {
        const uint32_t g = g0 + lane;
        const bool need = g < gi;
        if (!poll_states<C, OP>(slot((need ? g : g0) * kWave + kWave - 1, 1), need, nonce,
                                spin_limit, v, i))
            return false;
        // a group whose last tile gave up makes this tile fail too, rather than use it
        if (__ballot(need && i == kFail) != 0) return false;
        C xv;
        uint32_t xi;
        wave_fold<C, OP>(v, i, xv, xi);
        Op::combine(accv, acci, xv, xi);
    }
    Op::combine(accv, acci, yv, yi);
    return true;
}

// One call: workgroup g scans tile g % T of row g / T. VECIO: rows start 16-byte aligned in
// x and out_val (and out_idx), so full chunks move as 16-byte vectors.
template <typename Fmt, int OP, int U, bool VECIO>
__global__ __launch_bounds__(kBlockThreads) void k_cum(const uint8_t* __restrict__ x, uint32_t cols,
                                                       uint32_t T, uint8_t* __restrict__ out_val,
                                                       int64_t* __restrict__ out_idx,
                                                       uint64_t* __restrict__ states, uint32_t nonce,
                                                       uint32_t spin_limit) {
    using C = typename Fmt::C;
    using Op = ScanOp<C, OP>;
    using S = typename Out<Fmt>::S;
    using SW = StateWords<C>;
    constexpr int VW = Fmt::VW;
    constexpr int kWaves = kBlockThreads / kWave;
    constexpr uint32_t kTile = kBlockThreads * U * VW;  // elements per tile
    __shared__ C s_v[kWaves + 1];
    __shared__ uint32_t s_i[kWaves + 1];
    __shared__ int s_fail;
    __shared__ int32_t s_x[kWaves][kWave * VW];  // one wavefront's indices of a row of chunks
    __shared__ S s_io[kWaves][VECIO ? 1 : kWave * VW];  // element I/O: a wavefront's row of chunks

    const uint32_t g = blockIdx.x;
    const uint32_t r = g / T;
    const uint32_t t = g - r * T;
    const uint32_t wave = threadIdx.x / kWave;
    const uint32_t lane = threadIdx.x % kWave;
    const size_t row_off = static_cast<size_t>(r) * cols;
    const uint8_t* row = x + row_off * Fmt::kSize;
    uint8_t* vrow = out_val + row_off * sizeof(S);
    int64_t* irow = out_idx + row_off;
    const uint32_t tile0 = t * kTile;
    // x[0] of the row, for positions that report a leading NaN: loaded with the tile's
    // loads, so that it is not a dependent load after the look-back
    S x0 = 0;
    if constexpr (std::is_floating_point<C>::value) x0 = *reinterpret_cast<const S*>(row);
    // first position of chunk u of this lane
    auto chunk_pos = [&](int u) -> uint32_t {
        return tile0 + ((wave * U + static_cast<uint32_t>(u)) * kWave + lane) * VW;
    };
    if (threadIdx.x == 0) s_fail = 0;

    // load: U chunks of VW elements, kept as raw 16-byte vectors (half the registers of
    // widened values for 2-byte formats) and unpacked where used. No load sits under a lane
    // condition (that would make it a branch, and the loads would wait on each other):
    // positions past the row end read the row's last chunk / element again, and every use
    // of them is guarded.
    using Vec = typename Fmt::Vec;
    Vec q[U];
    if constexpr (VECIO) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t p0 = chunk_pos(u);
            // cols is a multiple of VW: chunks are whole or past the end
            const uint32_t pc = p0 < cols ? p0 : cols - VW;
            q[u] = __builtin_nontemporal_load(
                reinterpret_cast<const Vec*>(row + static_cast<size_t>(pc) * Fmt::kSize));
        }
    } else {
        // Element loads in striped order: load k of a row of chunks reads its 64 consecutive
        // elements k * 64 .. k * 64 + 63 (lane l the element k * 64 + l), so that every load
        // instruction covers one contiguous run; all of them are issued before any is used.
        // The row of chunks then passes through LDS into each lane's VW consecutive
        // elements. (Each lane loading its own VW elements instead made every instruction
        // touch 64 runs 16 bytes apart, and such scans ran 1.7-3.7 times longer.)
        S raw[U][VW];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t ub = chunk_pos(u) - lane * VW;  // first position of the row of chunks
#pragma unroll
            for (int k = 0; k < VW; ++k) {
                const uint32_t pe = ub + static_cast<uint32_t>(k) * kWave + lane;
                raw[u][k] = *reinterpret_cast<const S*>(
                    row + static_cast<size_t>(pe < cols ? pe : cols - 1) * Fmt::kSize);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int k = 0; k < VW; ++k) s_io[wave][k * kWave + lane] = raw[u][k];
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            S mine[VW];
#pragma unroll
            for (int k = 0; k < VW; ++k) mine[k] = s_io[wave][lane * VW + k];
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_memcpy(&q[u], mine, sizeof(Vec));
        }
    }

    // per chunk: the chunk's aggregate, then the wavefront's scan of the aggregates
    C exv[U], cv[U];
    uint32_t exi[U], ci[U];
    C carry_v = Op::identity();
    uint32_t carry_i = kEmpty;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t p0 = chunk_pos(u);
        C av = Op::identity();
        uint32_t ai = kEmpty;
        if (p0 < cols) {
            C e[VW];
            Fmt::unpack(q[u], e);
            Op::single(e[0], p0, av, ai);
#pragma unroll
            for (int k = 1; k < VW; ++k) {
                // strict update: NaN never wins; the padding past the row end is skipped
                const bool b = (p0 + k < cols) & Op::better(e[k], av);
                av = b ? e[k] : av;
                ai = b ? p0 + k : ai;
            }
        }
        C iv = av;
        uint32_t ii = ai;
        wave_scan<C, OP>(iv, ii);
        // exclusive: the inclusive piece of the previous lane
        C pv = shfl_val(iv, static_cast<int>(lane) - 1);
        uint32_t pi = static_cast<uint32_t>(__shfl(static_cast<int>(ii), static_cast<int>(lane) - 1));
        exv[u] = lane == 0 ? Op::identity() : pv;
        exi[u] = lane == 0 ? kEmpty : pi;
        cv[u] = carry_v;  // carry into this row of chunks (uniform)
        ci[u] = carry_i;
        const C tv = readlane_val(iv, kWave - 1);
        const uint32_t ti = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ii), kWave - 1));
        Op::combine(carry_v, carry_i, tv, ti);
    }

    // waves: totals through LDS; s_v[kWaves] receives the tile's exclusive prefix
    if (lane == 0) {
        s_v[wave] = carry_v;
        s_i[wave] = carry_i;
    }
    __syncthreads();
    C wv = Op::identity();  // prefix of the earlier waves
    uint32_t wi = kEmpty;
    for (uint32_t w = 0; w < wave; ++w) Op::combine(wv, wi, s_v[w], s_i[w]);
    if (T > 1 && wave == 0) {
        C av = Op::identity();  // the tile's aggregate
        uint32_t ai = kEmpty;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) Op::combine(av, ai, s_v[w], s_i[w]);
        uint64_t* row_states = states + static_cast<size_t>(r) * T * 2 * SW::kStride;
        uint64_t* mine = row_states + static_cast<size_t>(t) * 2 * SW::kStride;
        C pv = Op::identity();
        uint32_t pi = kEmpty;
        bool ok = true;
        if (lane == 0) publish(mine, nonce, av, ai);  // aggregate
        if (t > 0) ok = look_back<C, OP>(row_states, t, av, ai, nonce, pv, pi, spin_limit);
        if (lane == 0) {
            s_v[kWaves] = pv;
            s_i[kWaves] = pi;
            if (!ok) {
                s_fail = 1;
                __hip_atomic_fetch_add(&g_scan_wait_timeouts, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    __syncthreads();
    C tv = Op::identity();  // the tile's exclusive prefix, then this wave's
    uint32_t ti = kEmpty;
    if (T > 1) {
        tv = s_v[kWaves];
        ti = s_i[kWaves];
    }
    Op::combine(tv, ti, wv, wi);
    const bool fail = s_fail != 0;

    // outputs
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t p0 = chunk_pos(u);
        const uint32_t ubase = p0 - lane * VW;  // first position of this row of chunks
        if (ubase >= cols) continue;            // uniform in the wavefront
        C rv = tv;
        uint32_t ri = ti;
        Op::combine(rv, ri, cv[u], ci[u]);
        Op::combine(rv, ri, exv[u], exi[u]);
        // with the long tiles, an opaque copy keeps the compiler from holding the first
        // pass's widened values live until here (it unpacks again: a few cheap instructions)
        Vec qu = q[u];
        if constexpr (U > kScanUnrollShort) asm volatile("" : "+v"(qu));
        C e[VW];
        Fmt::unpack(qu, e);
        C sv;
        uint32_t si;
        Op::single(e[0], p0, sv, si);
        Op::combine(rv, ri, sv, si);
        S ov[VW];
        int32_t oi[VW];  // positions < 2^31 (or -1)
#pragma unroll
        for (int k = 0; k < VW; ++k) {
            if (k > 0) {
                const bool b = (VECIO || p0 + k < cols) & Op::better(e[k], rv);
                rv = b ? e[k] : rv;
                ri = b ? p0 + k : ri;
            }
            const bool nan0 = ri == kNaN0;
            ov[k] = nan0 ? x0 : Out<Fmt>::bits(rv);
            oi[k] = fail ? -1 : (nan0 ? 0 : static_cast<int32_t>(ri));
        }
        if (VECIO) {
            if (p0 < cols) {  // with VECIO, cols is a multiple of VW: the chunk is whole
                u32x4 w;
                __builtin_memcpy(&w, ov, 16);
                __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(vrow + static_cast<size_t>(p0) * sizeof(S)));
            }
            // Indices: VW * 8 bytes per lane. Stored lane by lane, a wavefront's 16-byte
            // stores would hit memory VW * 8 bytes apart and leave every line partly
            // written per store; so they pass through LDS and leave transposed, each
            // store of the wavefront covering 1 KiB (two consecutive indices per lane).
#pragma unroll
            for (int k = 0; k < VW; ++k) s_x[wave][lane * VW + k] = oi[k];
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
            for (int q = 0; q < VW / 2; ++q) {
                const uint32_t pos = static_cast<uint32_t>(q) * 2 * kWave + 2 * lane;
                if (ubase + pos < cols) {  // cols is even: the pair is whole
                    i64x2 pair;
                    pair.x = s_x[wave][pos];
                    pair.y = s_x[wave][pos + 1];
                    __builtin_nontemporal_store(pair, reinterpret_cast<i64x2*>(irow + ubase + pos));
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        } else {
            // through LDS into striped order, so that every store instruction covers 64
            // consecutive values (and indices), as the loads
#pragma unroll
            for (int k = 0; k < VW; ++k) {
                s_io[wave][lane * VW + k] = ov[k];
                s_x[wave][lane * VW + k] = oi[k];
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
            for (int k = 0; k < VW; ++k) {
                const uint32_t e = static_cast<uint32_t>(k) * kWave + lane;
                if (ubase + e < cols) {
                    reinterpret_cast<S*>(vrow)[ubase + e] = s_io[wave][e];
                    irow[ubase + e] = s_x[wave][e];
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }
    }
}

// Clears the tile states of a call captured into a graph (replays share one nonce).
__global__ __launch_bounds__(kBlockThreads) void k_cum_clear(uint64_t* __restrict__ states,
                                                             size_t words) {
    for (size_t k = static_cast<size_t>(blockIdx.x) * kBlockThreads + threadIdx.x; k < words;
         k += static_cast<size_t>(gridDim.x) * kBlockThreads)
        states[k] = 0;
}

template <typename Fmt, int OP>
hipError_t launch_cum_op(const ScanPlan& p, const void* x, void* out_val, int64_t* out_idx,
                         uint8_t* scratch16, hipStream_t s) {
    uint64_t* states = p.tiles_per_row > 1 ? reinterpret_cast<uint64_t*>(scratch16) : nullptr;
    uint32_t nonce = 0;
    if (states != nullptr) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess) return hipErrorInvalidValue;
        if (cs == hipStreamCaptureStatusActive) {
            // replays of the graph repeat this call's nonce: clear the words before each replay
            const size_t words = p.state_words;
            const size_t blocks = (words + kBlockThreads - 1) / kBlockThreads;
            hipLaunchKernelGGL(k_cum_clear, dim3(static_cast<uint32_t>(blocks < 1024 ? blocks : 1024)),
                               dim3(kBlockThreads), 0, s, states, words);
        }
        nonce = next_nonce();
    }
    const dim3 grid(static_cast<uint32_t>(p.grid_blocks));
    const uint8_t* xb = static_cast<const uint8_t*>(x);
    uint8_t* vb = static_cast<uint8_t*>(out_val);
    const uint32_t cols = static_cast<uint32_t>(p.cols);
    const uint32_t T = static_cast<uint32_t>(p.tiles_per_row);
    constexpr int UT = kScanUnrollTiny, US = kScanUnrollShort, UM = kScanUnrollMid,
                  UL = kScanUnrollLong;
    if (p.unroll == UM && p.vecio)
        launch_scan(k_cum<Fmt, OP, UM, true>, grid, s, xb, cols, T, vb, out_idx, states, nonce, spin_limit());
    else if (p.unroll == UM)
        launch_scan(k_cum<Fmt, OP, UM, false>, grid, s, xb, cols, T, vb, out_idx, states, nonce, spin_limit());
    else if (p.unroll == UT && p.vecio)
        launch_scan(k_cum<Fmt, OP, UT, true>, grid, s, xb, cols, T, vb, out_idx, states, nonce, spin_limit());
    else if (p.unroll == UT)
        launch_scan(k_cum<Fmt, OP, UT, false>, grid, s, xb, cols, T, vb, out_idx, states, nonce, spin_limit());
    else if (p.unroll == US && p.vecio)
        launch_scan(k_cum<Fmt, OP, US, true>, grid, s, xb, cols, T, vb, out_idx, states, nonce, spin_limit());
    else if (p.unroll == US)
        launch_scan(k_cum<Fmt, OP, US, false>, grid, s, xb, cols, T, vb, out_idx, states, nonce, spin_limit());
    else if (p.vecio)
        launch_scan(k_cum<Fmt, OP, UL, true>, grid, s, xb, cols, T, vb, out_idx, states, nonce, spin_limit());
    else
        launch_scan(k_cum<Fmt, OP, UL, false>, grid, s, xb, cols, T, vb, out_idx, states, nonce, spin_limit());
    return hipGetLastError();
}

template <typename Fmt>
hipError_t launch_cum_fmt(const ScanPlan& p, const void* x, int op, void* out_val,
                          int64_t* out_idx, uint8_t* scratch16, hipStream_t s) {
    switch (op) {
        case ARGREDUCE_MAX: return launch_cum_op<Fmt, kMax>(p, x, out_val, out_idx, scratch16, s);
        case ARGREDUCE_MIN: return launch_cum_op<Fmt, kMin>(p, x, out_val, out_idx, scratch16, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_cum(const ScanPlan& p, const void* x, int dtype, int op, void* out_val,
                      int64_t* out_idx, uint8_t* scratch16, hipStream_t s) {
    switch (dtype) {
        case ARGREDUCE_F32: return launch_cum_fmt<F32>(p, x, op, out_val, out_idx, scratch16, s);
        case ARGREDUCE_F16: return launch_cum_fmt<F16>(p, x, op, out_val, out_idx, scratch16, s);
        case ARGREDUCE_BF16: return launch_cum_fmt<BF16>(p, x, op, out_val, out_idx, scratch16, s);
        case ARGREDUCE_F64: return launch_cum_fmt<F64>(p, x, op, out_val, out_idx, scratch16, s);
        case ARGREDUCE_I32: return launch_cum_fmt<I32>(p, x, op, out_val, out_idx, scratch16, s);
        case ARGREDUCE_I64: return launch_cum_fmt<I64>(p, x, op, out_val, out_idx, scratch16, s);
        default: return hipErrorInvalidValue;
    }
}

size_t scan_state_words(int dtype) {
    const bool wide = dtype == ARGREDUCE_F64 || dtype == ARGREDUCE_I64;
    return 2 * static_cast<size_t>(wide ? StateWords<double>::kStride : StateWords<float>::kStride);
}

}  // namespace argreduce
