// Streaming helpers of the statistics pass, shared by the statistics kernel
// (stats.hip) and the one-kernel verify paths (verify.hip, tree.hip): one
// chunk of one logits row read once with branch-free 16-byte loads, the
// online softmax pair (max, sum of 2^((z - max) c)) of the softmax of z/T
// (AI-infra KB M013 s.04; "Speculative decoding tutorial" s.7.1) or the
// greedy (max, lowest index) pair (tutorial s.3-4).
#pragma once

#include "verify_internal.h"

namespace specdec {

template <bool BF16, int U>
__device__ __forceinline__ void load_tile(uint4 (&raw)[U], const void* rp, int t0) {
    constexpr int N = Vec<BF16>::N;
#pragma unroll
    for (int u = 0; u < U; ++u)
        raw[u] = load16_stream<BF16>(rp, t0 + (u * kThreads + threadIdx.x) * N);
}

template <bool BF16, int U>
__device__ __forceinline__ void widen_tile(Vec<BF16> (&v)[U], const uint4 (&raw)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = widen<BF16>(raw[u]);
}

// Streams elements [lo, hi) of one row through consume(v, t0) in tiles of
// kThreads lanes x U 16-byte vectors (lane l holds vectors u*kThreads + l).
// Whole tiles use branch-free loads, and the next tile's loads are issued
// before the current tile is consumed; a ragged last tile takes the clipped
// path.  keep() is asked once, after the first tile's loads are in flight;
// false abandons the row (the function then returns false).
template <bool BF16, bool VEC, int U, class F, class K>
__device__ __forceinline__ bool stream_row(const void* rp, int lo, int hi, F&& consume, K&& keep) {
    constexpr int N = Vec<BF16>::N;
    constexpr int TILE = kThreads * N * U;
    const int full_end = VEC ? lo + ((hi - lo) / TILE) * TILE : lo;
    int t0 = lo;
    if (t0 < full_end) {
        uint4 cur[U];
        load_tile<BF16, U>(cur, rp, t0);
        if (!keep()) return false;
        for (; t0 + TILE < full_end; t0 += TILE) {
            uint4 nxt[U];
            load_tile<BF16, U>(nxt, rp, t0 + TILE);
            Vec<BF16> v[U];
            widen_tile<BF16, U>(v, cur);
            consume(v, t0);
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        }
        Vec<BF16> v[U];
        widen_tile<BF16, U>(v, cur);
        consume(v, t0);
        t0 += TILE;
    } else if (!keep()) {
        return false;
    }
    for (; t0 < hi; t0 += TILE) {
        Vec<BF16> v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = load_vec<BF16, VEC>(rp, t0 + (u * kThreads + threadIdx.x) * N, hi, neg_inf());
        consume(v, t0);
    }
    return true;
}

// stream_row's element order with one tile in flight at a time (few
// registers): lane l consumes the same vectors of the same tiles in the same
// order, so a fold over it gives the same bits.  For a decision workgroup
// that computes a missing partial itself.
template <bool BF16, bool VEC, int U, class F>
__device__ __forceinline__ void stream_row_lean(const void* rp, int lo, int hi, F&& consume) {
    constexpr int N = Vec<BF16>::N;
    constexpr int TILE = kThreads * N * U;
    for (int t0 = lo; t0 < hi; t0 += TILE) {
        Vec<BF16> v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = load_vec<BF16, VEC>(rp, t0 + (u * kThreads + threadIdx.x) * N, hi, neg_inf());
        consume(v, t0);
    }
}



// The workgroup's pair (every lane gets it): the waves' pairs meet in LDS,
// then the same as wave_combine over them (the maximum, then each wave's
// sum rescaled to it, added in wave order).
__device__ __forceinline__ MaxSum block_combine(MaxSum v, float c) {
    __shared__ float s_m[kWaves], s_s[kWaves];
    v = wave_combine(v, c);
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    if (l == 0) { s_m[w] = v.m; s_s[w] = v.s; }
    __syncthreads();
    float m = s_m[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) m = fmaxf(m, s_m[k]);
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) s += s_m[k] == neg_inf() ? 0.0f : s_s[k] * exp2f((s_m[k] - m) * c);
    return {m, s};
}

__device__ __forceinline__ ArgMax block_argmax(ArgMax v) {
    __shared__ float s_v[kWaves];
    __shared__ int s_i[kWaves];
    v = wave_argmax(v);
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    if (l == 0) { s_v[w] = v.v; s_i[w] = v.i; }
    __syncthreads();
    ArgMax r{s_v[0], s_i[0]};
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r = better(r, ArgMax{s_v[k], s_i[k]});
    return r;
}

// (max, sum of 2^((z - max) c)) of elements [lo, hi) of row rp, combined
// over the workgroup (every lane gets the pair).  keep() as in stream_row;
// returns false if the row was abandoned.
template <bool BF16, bool VEC, class K, bool LEAN = false>
__device__ __forceinline__ bool chunk_maxsum(const void* rp, int lo, int hi, float c, K&& keep,
                                             MaxSum* out) {
    constexpr int N = Vec<BF16>::N;
    float m = neg_inf(), sum = 0.0f;
    auto consume = [&](const Vec<BF16> (&v)[kUnroll], int) {
        float tm = neg_inf();
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int k = 0; k < N; ++k) tm = fmaxf(tm, v[u].x[k]);
        const float mn = fmaxf(m, tm);
        if (mn == neg_inf()) {
            // nothing finite yet in this lane (fmaxf skips NaNs): a NaN here
            // still marks the row non-finite, as a +inf does (max +inf)
            bool nan = false;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int k = 0; k < N; ++k) nan |= v[u].x[k] != v[u].x[k];
            if (nan) m = pos_inf();
            return;
        }
        float part = 0.0f;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float q = 0.0f;
#pragma unroll
            for (int k = 0; k < N; ++k) q += __builtin_amdgcn_exp2f((v[u].x[k] - mn) * c);
            part += q;
        }
        sum = (m == neg_inf() ? 0.0f : sum * exp2f((m - mn) * c)) + part;
        m = mn;
    };
    if constexpr (LEAN) stream_row_lean<BF16, VEC, kUnroll>(rp, lo, hi, consume);
    else if (!stream_row<BF16, VEC, kUnroll>(rp, lo, hi, consume, keep)) return false;
    *out = block_combine(MaxSum{m, sum}, c);
    return true;
}

// Element j of a raw 16-byte vector as fp32 (exact).
template <bool BF16>
__device__ __forceinline__ float raw_elem(const uint4& w, int j) {
    if constexpr (BF16) {
        const uint32_t x = j < 2 ? w.x : j < 4 ? w.y : j < 6 ? w.z : w.w;
        return (j & 1) ? bf16_hi(x) : bf16_lo(x);
    } else {
        return __uint_as_float(j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w);
    }
}

// chunk_maxsum's (max, sum) of [lo, hi) for 16-byte aligned rows, read one
// tile at a time and folded from the raw vectors (widened twice, in the
// maximum pass and the sum pass) with fold_vectors' operations in its order:
// the same bits with few registers, for a decision workgroup that computes a
// missing partial itself.
template <bool BF16>
__device__ MaxSum chunk_maxsum_lean(const void* rp, int lo, int hi, float c) {
    constexpr int N = Vec<BF16>::N;
    constexpr int TILE = kThreads * N * kUnroll;
    float m = neg_inf(), sum = 0.0f;
    for (int t0 = lo; t0 < hi; t0 += TILE) {
        uint4 r[kUnroll];
        bool ok[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int e = t0 + (u * kThreads + threadIdx.x) * N;
            ok[u] = e < hi;
            r[u] = load16<BF16>(rp, min(e, hi - N));
        }
        float tm = neg_inf();
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int k = 0; k < N; ++k) tm = fmaxf(tm, ok[u] ? raw_elem<BF16>(r[u], k) : neg_inf());
        // (the sum pass widens the raw vectors again)
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __asm__ volatile("" : "+v"(r[u].x), "+v"(r[u].y), "+v"(r[u].z), "+v"(r[u].w));
        const float mn = fmaxf(m, tm);
        if (mn == neg_inf()) {
            bool nan = false;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int k = 0; k < N; ++k) {
                    const float x = raw_elem<BF16>(r[u], k);
                    nan |= ok[u] && x != x;
                }
            if (nan) m = pos_inf();
            continue;
        }
        float part = 0.0f;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float q = 0.0f;
#pragma unroll
            for (int k = 0; k < N; ++k)
                q += __builtin_amdgcn_exp2f(((ok[u] ? raw_elem<BF16>(r[u], k) : neg_inf()) - mn) * c);
            part += q;
        }
        sum = (m == neg_inf() ? 0.0f : sum * exp2f((m - mn) * c)) + part;
        m = mn;
    }
    return block_combine(MaxSum{m, sum}, c);
}

// (max, lowest index) of elements [lo, hi) of row rp, combined over the
// workgroup (every lane gets the pair), and whether a NaN was seen.  Each
// lane visits its elements in ascending index order, so a strict ">" keeps
// the lowest index among equal maxima.  keep() as in stream_row; returns
// false if the row was abandoned.
template <bool BF16, bool VEC, class K, bool LEAN = false>
__device__ __forceinline__ bool chunk_argmax(const void* rp, int lo, int hi, K&& keep, ArgMax* out,
                                             bool* any_nan) {
    constexpr int N = Vec<BF16>::N;
    ArgMax best{neg_inf(), 0x7fffffff};
    bool nan = false;
    auto consume = [&](const Vec<BF16> (&v)[kUnroll], int t0) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int e = t0 + (u * kThreads + threadIdx.x) * N;
#pragma unroll
            for (int k = 0; k < N; ++k) {
                const float x = v[u].x[k];
                nan |= (x != x);
                const bool first = best.i == 0x7fffffff && e + k < hi;
                if (x > best.v || first) { best.v = x; best.i = e + k; }
            }
        }
    };
    if constexpr (LEAN) stream_row_lean<BF16, VEC, kUnroll>(rp, lo, hi, consume);
    else if (!stream_row<BF16, VEC, kUnroll>(rp, lo, hi, consume, keep)) return false;
    *out = block_argmax(best);
    *any_nan = __syncthreads_or(nan);
    return true;
}

// Greedy partials as the decision kernels stage them: x = the chunk's
// maximum, y = the bits of its lowest index with bit 31 set if a NaN was seen.
__device__ __forceinline__ float4 greedy_partial(const ArgMax& r, bool nan) {
    return make_float4(r.v, __uint_as_float(static_cast<uint32_t>(r.i) | (nan ? 0x80000000u : 0u)),
                       0.0f, 0.0f);
}

// One-kernel greedy paths: the same partial as one 64-bit word, maximum bits
// low, index bits high with bit 30 set as the published mark (indices are
// below 2^24), so a published word is never zero.
__device__ __forceinline__ unsigned long long greedy_word(const ArgMax& r, bool nan) {
    const uint32_t hi = static_cast<uint32_t>(r.i) | 0x40000000u | (nan ? 0x80000000u : 0u);
    return (static_cast<unsigned long long>(hi) << 32) | __float_as_uint(r.v);
}

// The decision workgroup of request b in a one-kernel greedy path, the only
// reader of the request's words: every word of a used row (used(s)) is taken
// by a lane of its own with an exchange with zero (so it is cleared for the
// next call as it is read), polled with sleeps until published, within
// P.wait_ticks of the 100 MHz constant clock, and staged in s_part as
// greedy_partial stores it.  A word that has not come by then is computed
// here from the row itself, with the statistics workgroup's arithmetic (so
// the result is the same), and its late exchange is then awaited (and taken)
// within the fixed 20 ms bound, so that no word stays set for the next call.
// Returns true (to every lane) if a wait gave up.
template <bool BF16, bool VEC, class U>
__device__ bool collect_greedy(const VerifyParams& P, int b, U&& used, float4* s_part) {
    const int n = P.rows * P.nc;
    unsigned long long* w = reinterpret_cast<unsigned long long*>(P.ready) + static_cast<size_t>(b) * n;
    const uint64_t t0 = wall_clock64();
    bool late = false;
    for (int t = threadIdx.x; t < n; t += kThreads) {
        if (!used(t / P.nc)) continue;
        unsigned long long v;
        while ((v = atomicExch(w + t, 0ull)) == 0ull) {
            if (wall_clock64() - t0 > P.wait_ticks) { late = true; break; }
            __builtin_amdgcn_s_sleep(16);
        }
        const uint32_t hi = static_cast<uint32_t>(v >> 32) & ~0x40000000u;
        // (w = 1 marks a partial that did not come)
        s_part[t] = make_float4(__uint_as_float(static_cast<uint32_t>(v)), __uint_as_float(hi), 0.0f,
                                v == 0ull ? 1.0f : 0.0f);
    }
    if (!__syncthreads_or(late)) return false;
    // the missing partials, computed here
    for (int t = 0; t < n; ++t) {
        if (!used(t / P.nc) || s_part[t].w == 0.0f) continue;
        const int row = t / P.nc, ci = t % P.nc;
        const int lo = ci * P.chunk, hi = min(P.V, lo + P.chunk);
        ArgMax r;
        bool nan;
        auto all = []() { return true; };
        chunk_argmax<BF16, VEC, decltype(all)&, true>(target_row(P, b, row, BF16), lo, hi, all, &r, &nan);
        if (threadIdx.x == 0) {
            s_part[t] = greedy_partial(r, nan);
            // the late word: taken when it comes, so it does not stay set
            const uint64_t t1 = wall_clock64();
            while (atomicExch(w + t, 0ull) == 0ull) {
                if (wall_clock64() - t1 > kFixedWaitTicks) break;
                __builtin_amdgcn_s_sleep(16);
            }
        }
        __syncthreads();
    }
    return true;
}

// Statistics workgroup of a one-kernel greedy path: chunk k % nc of target
// row k / nc of request b (rows used(s) only), published as greedy_word with
// an atomic exchange it does not wait for.
template <bool BF16, bool VEC, class U>
__device__ __forceinline__ void fused_greedy_stats(const VerifyParams& P, int b, int k, U&& used) {
    const int s = k / P.nc, ci = k % P.nc;
    const void* rp = target_row(P, b, s, BF16);
    const int lo = ci * P.chunk, hi = min(P.V, lo + P.chunk);
    ArgMax r;
    bool nan;
    if (!chunk_argmax<BF16, VEC>(rp, lo, hi, [&]() { return used(s); }, &r, &nan)) return;
    if (threadIdx.x == 0)
        atomicExch(reinterpret_cast<unsigned long long*>(P.ready) + static_cast<size_t>(b) * P.rows * P.nc + k,
                   greedy_word(r, nan));
}

}  // namespace specdec
