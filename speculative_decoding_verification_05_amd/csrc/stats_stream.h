// Streaming helpers of the statistics pass, shared by the statistics kernel
// (stats.hip) and the one-kernel sampling verify (verify.hip): one chunk of
// one logits row read once with branch-free 16-byte loads, the online
// softmax pair (max, sum of 2^((z - max) c)) of the softmax of z/T
// (AI-infra KB M013 s.04; "Speculative decoding tutorial" s.7.1).
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

__device__ __forceinline__ MaxSum block_combine(MaxSum v, float c) {
    __shared__ float s_m[kWaves], s_s[kWaves];
    v = wave_combine(v, c);
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    if (l == 0) { s_m[w] = v.m; s_s[w] = v.s; }
    __syncthreads();
    MaxSum r{s_m[0], s_s[0]};
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r = combine(r, MaxSum{s_m[k], s_s[k]}, c);
    return r;
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
template <bool BF16, bool VEC, class K>
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
        if (mn == neg_inf()) return;
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
    if (!stream_row<BF16, VEC, kUnroll>(rp, lo, hi, consume, keep)) return false;
    *out = block_combine(MaxSum{m, sum}, c);
    return true;
}

}  // namespace specdec
