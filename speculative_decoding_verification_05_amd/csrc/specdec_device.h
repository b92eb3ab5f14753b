// Device helpers of the verify-and-commit kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specdec {

constexpr int kThreads = 256;  // 4 waves of 64 lanes per workgroup
constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;

__device__ __forceinline__ float neg_inf() { return __uint_as_float(0xff800000u); }
__device__ __forceinline__ float pos_inf() { return __uint_as_float(0x7f800000u); }

// ---------------------------------------------------------------- Philox
// Philox4x32-10 of Salmon, Moraes, Dror and Shaw (SC'11): ten rounds, each
// two 32x32->64-bit products with the published multipliers; the key is
// bumped by the published Weyl increments before every round but the first.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
        const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    }
    return c;
}

// A uniform in [0, 1) from the 24 high bits of a word (exact in fp32).
__device__ __forceinline__ float uniform24(uint32_t w) {
    return (float)(w >> 8) * 5.9604644775390625e-08f;  // 2^-24
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <bool BF16>
__device__ __forceinline__ float load_logit(const void* row, int64_t v) {
    if constexpr (BF16) {
        const uint16_t h = static_cast<const uint16_t*>(row)[v];
        return __uint_as_float(static_cast<uint32_t>(h) << 16);
    } else {
        return static_cast<const float*>(row)[v];
    }
}

// Values of one 16-byte vector: 8 bf16 or 4 fp32 logits.
template <bool BF16>
struct Vec {
    static constexpr int N = BF16 ? 8 : 4;
    float x[N];
};

template <bool BF16>
__device__ __forceinline__ Vec<BF16> widen(uint4 w) {
    Vec<BF16> r;
    if constexpr (BF16) {
        r.x[0] = bf16_lo(w.x); r.x[1] = bf16_hi(w.x);
        r.x[2] = bf16_lo(w.y); r.x[3] = bf16_hi(w.y);
        r.x[4] = bf16_lo(w.z); r.x[5] = bf16_hi(w.z);
        r.x[6] = bf16_lo(w.w); r.x[7] = bf16_hi(w.w);
    } else {
        r.x[0] = __uint_as_float(w.x); r.x[1] = __uint_as_float(w.y);
        r.x[2] = __uint_as_float(w.z); r.x[3] = __uint_as_float(w.w);
    }
    return r;
}

// One 16-byte vector of a row (no bounds handling: the caller guarantees it).
template <bool BF16>
__device__ __forceinline__ uint4 load16(const void* row, int e) {
    return *reinterpret_cast<const uint4*>(static_cast<const char*>(row) +
                                           static_cast<size_t>(e) * (BF16 ? 2 : 4));
}

// The same with the nontemporal (streaming) hint: for data read exactly once,
// it keeps the read stream from displacing useful lines and measurably raises
// the achieved HBM read bandwidth on gfx950.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <bool BF16>
__device__ __forceinline__ uint4 load16_stream(const void* row, int e) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
        static_cast<const char*>(row) + static_cast<size_t>(e) * (BF16 ? 2 : 4)));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Elements [e, e+N) of a row clipped to [.., hi), `fill` past hi.  Loads are
// never skipped: the address is clamped into the row and the value replaced,
// so a lane issues all its loads without branching and they stay in flight
// together.  VEC: the row is 16-byte aligned and hi is a multiple of N, so a
// 16-byte vector lies wholly inside [.., hi) or wholly past it (hi >= N).
template <bool BF16, bool VEC>
__device__ __forceinline__ Vec<BF16> load_vec(const void* row, int e, int hi, float fill) {
    constexpr int N = Vec<BF16>::N;
    Vec<BF16> r;
    if constexpr (VEC) {
        const int ec = min(e, hi - N);
        const uint4 w = *reinterpret_cast<const uint4*>(
            static_cast<const char*>(row) + static_cast<size_t>(ec) * (BF16 ? 2 : 4));
        r = widen<BF16>(w);
        if (e >= hi) {
#pragma unroll
            for (int k = 0; k < N; ++k) r.x[k] = fill;
        }
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const float x = load_logit<BF16>(row, min(e + k, hi - 1));
            r.x[k] = (e + k < hi) ? x : fill;
        }
    }
    return r;
}

// ---------------------------------------------------------------- reductions
// Wave-wide scans and reductions with DPP row moves (row_shr 1/2/4/8 inside
// each 16-lane row, then row_bcast 15 and 31 across rows): a handful of
// VALU-latency steps instead of LDS permutes.  Lanes whose source lies
// outside the row (or in a masked row) read the operation's identity.  The
// reduction result is the scan's lane 63, broadcast through an SGPR.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_move(uint32_t identity, uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(identity), static_cast<int>(x),
                                                             CTRL, ROW_MASK, 0xf, false));
}

template <class T>
__device__ __forceinline__ uint32_t to_bits(T v) { return __builtin_bit_cast(uint32_t, v); }
template <class T>
__device__ __forceinline__ T from_bits(uint32_t v) { return __builtin_bit_cast(T, v); }

// Inclusive scan of a 32-bit value under an associative op with identity `id`.
template <class T, class Op>
__device__ __forceinline__ T wave_scan(T x, T id, Op op) {
    const uint32_t i = to_bits(id);
    x = op(x, from_bits<T>(dpp_move<kDppRowShr1>(i, to_bits(x))));
    x = op(x, from_bits<T>(dpp_move<kDppRowShr2>(i, to_bits(x))));
    x = op(x, from_bits<T>(dpp_move<kDppRowShr4>(i, to_bits(x))));
    x = op(x, from_bits<T>(dpp_move<kDppRowShr8>(i, to_bits(x))));
    x = op(x, from_bits<T>(dpp_move<kDppRowBcast15, 0xa>(i, to_bits(x))));
    x = op(x, from_bits<T>(dpp_move<kDppRowBcast31, 0xc>(i, to_bits(x))));
    return x;
}

// x of lane `lane` (wave-uniform) to every lane.
template <class T>
__device__ __forceinline__ T lane_value(T x, int lane) {
    return from_bits<T>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(to_bits(x)), lane)));
}

template <class T>
__device__ __forceinline__ T lane63(T x) {
    return from_bits<T>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(to_bits(x)), 63)));
}

__device__ __forceinline__ float wave_max(float v) {
    return lane63(wave_scan(v, neg_inf(), [](float a, float b) { return fmaxf(a, b); }));
}

__device__ __forceinline__ float wave_sum(float v) {
    return lane63(wave_scan(v, 0.0f, [](float a, float b) { return a + b; }));
}

// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ float wave_prefix_sum(float v) {
    return wave_scan(v, 0.0f, [](float a, float b) { return a + b; });
}

// Exclusive prefix sum (lane 0 gets 0) from an inclusive one: a whole-wave
// shift right by one lane.
__device__ __forceinline__ float wave_shift_right(float incl) {
    return from_bits<float>(dpp_move<0x138>(0u, to_bits(incl)));
}

__device__ __forceinline__ int wave_isum(int v) {
    return lane63(wave_scan(v, 0, [](int a, int b) { return a + b; }));
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
    return lane63(wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a | b; }));
}

// Online-softmax pair (running maximum of the raw logits, sum of
// 2^((x - max) * c)); combining rescales the sum of the smaller maximum.
struct MaxSum {
    float m;
    float s;
};

__device__ __forceinline__ MaxSum combine(MaxSum a, MaxSum b, float c) {
    const float m = fmaxf(a.m, b.m);
    if (m == neg_inf()) return {m, 0.0f};
    const float sa = a.m == neg_inf() ? 0.0f : a.s * exp2f((a.m - m) * c);
    const float sb = b.m == neg_inf() ? 0.0f : b.s * exp2f((b.m - m) * c);
    return {m, sa + sb};
}

// The wave's pair: its maximum first (exact, order-free), then each lane's
// sum rescaled to that maximum once and the rescaled sums added.  One
// exponential per lane, all lanes at once; a chain of six pairwise combines
// took two per step, one after another, and ended every statistics
// workgroup 1.4 us later (measured on the headline's statistics pass).
// Every lane gets the pair.  A lane at +inf (a NaN or +inf in its elements)
// makes the sum NaN, as combine does, so the row is flagged.
__device__ __forceinline__ MaxSum wave_combine(MaxSum v, float c) {
    const float m = wave_max(v.m);
    const float s = v.m == neg_inf() ? 0.0f : v.s * exp2f((v.m - m) * c);
    return {m, wave_sum(s)};
}

// (value, index) of a maximum: larger value wins, the lower index on ties.
struct ArgMax {
    float v;
    int i;
};

__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
    if (a.v > b.v) return a;
    if (b.v > a.v) return b;
    return a.i <= b.i ? a : b;
}

// The pair scan below follows wave_scan's steps, moving both members.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ ArgMax dpp_pair(ArgMax v) {
    return {from_bits<float>(dpp_move<CTRL, ROW_MASK>(to_bits(neg_inf()), to_bits(v.v))),
            static_cast<int>(dpp_move<CTRL, ROW_MASK>(0x7fffffffu, static_cast<uint32_t>(v.i)))};
}

__device__ __forceinline__ ArgMax wave_argmax(ArgMax v) {
    v = better(v, dpp_pair<kDppRowShr1>(v));
    v = better(v, dpp_pair<kDppRowShr2>(v));
    v = better(v, dpp_pair<kDppRowShr4>(v));
    v = better(v, dpp_pair<kDppRowShr8>(v));
    v = better(v, dpp_pair<kDppRowBcast15, 0xa>(v));
    v = better(v, dpp_pair<kDppRowBcast31, 0xc>(v));
    return {lane63(v.v), lane63(v.i)};
}

}  // namespace specdec
