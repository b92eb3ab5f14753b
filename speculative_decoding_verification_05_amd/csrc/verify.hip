// specdec_verify: the verify half of a speculative-decoding round on gfx950.
//
// What is computed (page titles and sections as cited in specdec.h):
//   - p_i, q_i are the softmax of z/T of target row i and draft row i
//     (AI-infra KB M013 s.04: the actual sampling distributions);
//   - draft i is accepted iff u_i < min(1, p_i(d_i) / q_i(d_i)), scanning
//     left to right and stopping at the first rejection ("Speculative
//     decoding tutorial" s.7.1, s.7.3, s.2);
//   - on a rejection at m the next token is drawn from
//     normalize(max(p_m - q_m, 0)), otherwise from p_gamma (same tutorial
//     s.7.2 and s.5.3; KB M013 s.05);
//   - greedy mode keeps draft i iff it equals argmax of target row i and emits
//     the argmax at the first mismatch (tutorial s.3-4; KB M013 s.03);
//   - without draft rows (a deterministic proposer such as n-gram lookup),
//     q_i is the point mass on d_i: the test becomes u_i < p_i(d_i) and the
//     residual is p_m without d_m (KB M013 s.08 and s.04).
//
// Kernels (all HBM-bandwidth bound, no matrix cores: nothing is a contraction):
//   k_stats          (stats.hip) the one full pass over every used row, one
//                    partial per (chunk, row).
//   k_decide_sample  workgroup (chunk, request).  Every workgroup of a request
//                    combines the request's partials, runs the acceptance tests
//                    on one wave and takes m from a ballot (identical results in
//                    all of them); each then computes its chunk's sampling mass
//                    (max(p_m - q_m, 0), or p_gamma on a full accept).  The
//                    request's last workgroup to finish finds the chunk where
//                    the running mass passes u*R, re-scans it with a block
//                    prefix sum, and writes every output of the request.
//   k_decide_greedy  one workgroup per request: row argmaxes from the
//                    partials, the argmax-equality prefix and every output.
//   k_greedy_fused   greedy in one launch: the statistics workgroups publish
//                    each chunk's (max, lowest index) as one 64-bit word, and
//                    one decision workgroup per request, launched after all
//                    of them, collects its words and decides as above.
//   k_verify_fused   sampling without truncation in one launch: the
//                    statistics workgroups of every request come first in
//                    launch order, then the decision workgroups, each of
//                    which waits (bounded) until its request's partials are
//                    published.  Same arithmetic as the two kernels above,
//                    same results; it saves the kernel boundary and lets the
//                    decision workgroups start while the last rows stream.
// Cross-workgroup hand-offs use device-scope atomics.  In the two-kernel
// paths nothing waits on another workgroup; in the one-kernel paths only
// decision workgroups wait, and only on workgroups that precede them in
// launch order (statistics workgroups, which never wait, and in sampling the
// request's earlier decision workgroups, which wait only on statistics).
#include "stats_stream.h"

#include <hip/hip_ext.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace specdec {
namespace {

// ------------------------------------------------------------------ sampling pass

// The mass the draw at position m samples from: max(p - q, 0) on a
// rejection, p itself when q is absent (bonus, or the empty-residual
// fallback).  p = 2^((z - max) c) / sum, q likewise.  CUT: p and q are
// truncated to their kept sets, given by cut records (token v of logit z is
// kept iff z > tau, or z == tau and v <= iota), sum being the kept mass.
struct MassRows {
    const void* p;
    const void* q;
    float mp, isp, mq, isq, c;
    int point;  // point-mass draft: this token carries no residual mass (-1: none)
    float tp, tq;  // CUT: boundary logits of p and q
    int ip, iq;    // CUT: last kept index at the boundary logit
};

template <bool CUT>
__device__ __forceinline__ float mass_at(const MassRows& a, float zp, float zq, int v) {
    float pv = __builtin_amdgcn_exp2f((zp - a.mp) * a.c) * a.isp;
    if constexpr (CUT) pv = (zp > a.tp || (zp == a.tp && v <= a.ip)) ? pv : 0.0f;
    if (!a.q) return pv;
    float qv = __builtin_amdgcn_exp2f((zq - a.mq) * a.c) * a.isq;
    if constexpr (CUT) qv = (zq > a.tq || (zq == a.tq && v <= a.iq)) ? qv : 0.0f;
    return fmaxf(pv - qv, 0.0f);
}

// The three kinds of sampling mass, told apart once per call (a uniform
// branch) so that the per-element loops carry neither the test for a draft
// row nor the point-mass token's: a residual max(p - q, 0) with draft rows,
// p itself (bonus, or the empty-residual fallback), p without one token
// (point-mass drafts).  Same operations per element as mass_at, so the same
// bits; three fewer vector operations per element of about fifteen.  The
// decision over cut records (CUT) keeps one generic loop (kAny, mass_at's
// tests per element): its membership tests leave it the tightest on
// registers, and three copies of its walk cost it more than they saved.
enum class MassKind { kResidual, kTarget, kTargetButOne, kAny };

template <MassKind K, bool CUT>
__device__ __forceinline__ float mass_of(const MassRows& a, float zp, float zq, int v) {
    if constexpr (K == MassKind::kAny) {
        const float r = mass_at<CUT>(a, zp, zq, v);
        return v == a.point ? 0.0f : r;
    }
    float pv = __builtin_amdgcn_exp2f((zp - a.mp) * a.c) * a.isp;
    if constexpr (CUT) pv = (zp > a.tp || (zp == a.tp && v <= a.ip)) ? pv : 0.0f;
    if constexpr (K == MassKind::kResidual) {
        float qv = __builtin_amdgcn_exp2f((zq - a.mq) * a.c) * a.isq;
        if constexpr (CUT) qv = (zq > a.tq || (zq == a.tq && v <= a.iq)) ? qv : 0.0f;
        return fmaxf(pv - qv, 0.0f);
    } else if constexpr (K == MassKind::kTargetButOne) {
        return v == a.point ? 0.0f : pv;
    } else {
        return pv;
    }
}

// Calls f with the kind of mass a describes (kAny for the cut decision).
template <bool CUT, class F>
__device__ __forceinline__ auto with_mass_kind(const MassRows& a, F&& f) {
    if constexpr (CUT) return f(std::integral_constant<MassKind, MassKind::kAny>{});
    if (a.q) return f(std::integral_constant<MassKind, MassKind::kResidual>{});
    if (a.point >= 0) return f(std::integral_constant<MassKind, MassKind::kTargetButOne>{});
    return f(std::integral_constant<MassKind, MassKind::kTarget>{});
}

// One chunk of the sampling pass is one tile: lane l holds the 16-byte
// vectors u*kThreads + l, u < kUnroll2, of each row.  Loads are clamped into
// the row (a vector is wholly inside [lo, hi) or wholly past it) and the
// values of out-of-range vectors are discarded after use, so no load sits
// behind a branch.  CACHED: ordinary loads (the lines may stay in the
// caches), else streaming ones.
template <bool BF16, bool VEC>
struct ChunkRegs {
    uint4 p[kUnroll2], q[kUnroll2];
};

template <bool BF16, bool VEC, bool CACHED>
__device__ __forceinline__ void load_chunk(ChunkRegs<BF16, VEC>& r, const MassRows& a, int lo, int hi) {
    constexpr int N = Vec<BF16>::N;
#pragma unroll
    for (int u = 0; u < kUnroll2; ++u) {
        const int e = min(lo + (u * kThreads + static_cast<int>(threadIdx.x)) * N, hi - N);
        if constexpr (CACHED) {
            r.p[u] = load16<BF16>(a.p, e);
            if (a.q) r.q[u] = load16<BF16>(a.q, e);
        } else {
            r.p[u] = load16_stream<BF16>(a.p, e);
            if (a.q) r.q[u] = load16_stream<BF16>(a.q, e);
        }
    }
}

// A chunk of the sampling pass is kUnroll2 = 2 halves in token order: half u
// is the kThreads vectors u*kThreads .. u*kThreads + kThreads - 1, lane l
// holding vector u*kThreads + l of each.  The pass keeps the two halves'
// masses apart, so that the final search reads and weighs only the half
// where the running mass crosses u*R (half the vector work of searching the
// whole chunk, on the decision's critical path).
static_assert(kUnroll2 == 2, "a sampling chunk is two halves, one vector per lane each");

// Lane's share of each half's mass (VEC layout), for mass kind K.
template <MassKind K, bool BF16, bool VEC, bool CUT = false>
__device__ __forceinline__ float2 lane_mass(const ChunkRegs<BF16, VEC>& r, const MassRows& a, int lo, int hi) {
    constexpr int N = Vec<BF16>::N;
    float h[kUnroll2];
#pragma unroll
    for (int u = 0; u < kUnroll2; ++u) {
        const Vec<BF16> vp = widen<BF16>(r.p[u]);
        Vec<BF16> vq;
        if constexpr (K == MassKind::kResidual) vq = widen<BF16>(r.q[u]);
        if constexpr (K == MassKind::kAny) {
            if (a.q) vq = widen<BF16>(r.q[u]);
        }
        const int e = lo + (u * kThreads + threadIdx.x) * N;
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < N; ++k)
            s += mass_of<K, CUT>(a, vp.x[k], K != MassKind::kTarget && K != MassKind::kTargetButOne && a.q ? vq.x[k] : 0.0f, e + k);
        h[u] = (e < hi) ? s : 0.0f;
    }
    return make_float2(h[0], h[1]);
}

// Lane's share of the chunk's mass with element loads (rows not 16-byte
// aligned): a slow path kept simple.
template <bool BF16, bool CUT = false>
__device__ float2 lane_mass_elements(const MassRows& a, int lo, int hi) {
    constexpr int N = Vec<BF16>::N;
    float h[kUnroll2] = {0.0f, 0.0f};
    for (int u = 0; u < kUnroll2; ++u) {
        const int e = lo + (u * kThreads + threadIdx.x) * N;
        for (int k = 0; k < N; ++k) {
            if (e + k >= hi) break;
            const float zp = load_logit<BF16>(a.p, e + k);
            const float zq = a.q ? load_logit<BF16>(a.q, e + k) : 0.0f;
            if (e + k != a.point) h[u] += mass_at<CUT>(a, zp, zq, e + k);
        }
    }
    return make_float2(h[0], h[1]);
}

// Masses of chunks [k0, k1), handed to emit(k, h0, h1) by thread 0, h0 and
// h1 the masses of the chunk's two halves (the chunk's mass is their sum,
// chunk_total).  Loads go in groups of GROUP chunks, into two register sets
// in turn (no copies between them), so the next group's loads are in flight
// while the current group is reduced.  Nothing inside the walk waits on other
// waves or on memory writes: each half's wave sums go to LDS (scr: 2 kWaves
// floats per chunk), and after one barrier thread 0 adds them in wave order
// and emits the whole batch at once (batches of 1024 / (2 kWaves) chunks).
// Returns the OR of emit's results (a dependency for arrive_last when emit
// publishes).
template <MassKind K, bool BF16, bool VEC, int GROUP, bool CACHED, bool CUT, class Emit>
__device__ __forceinline__ uint32_t mass_chunks_of(const MassRows& a, int k0, int k1, int chunk2, int V, float* scr,
                                   Emit&& emit) {
    uint32_t dep = 0;
    if (k0 >= k1) return dep;
    if constexpr (VEC) {
        const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
        constexpr int kBatch = 1024 / (kUnroll2 * kWaves);
        for (int b0 = k0; b0 < k1; b0 += kBatch) {
            const int b1 = min(k1, b0 + kBatch);
            auto load_group = [&](ChunkRegs<BF16, VEC>(&r)[GROUP], int kb) {
#pragma unroll
                for (int j = 0; j < GROUP; ++j) {
                    const int k = min(kb + j, b1 - 1);  // past b1: the last chunk again, unused
                    load_chunk<BF16, VEC, CACHED>(r[j], a, k * chunk2, min(V, (k + 1) * chunk2));
                }
            };
            auto reduce_group = [&](ChunkRegs<BF16, VEC>(&r)[GROUP], int kb) {
#pragma unroll
                for (int j = 0; j < GROUP; ++j) {
                    if (kb + j >= b1) break;
                    const int lo = (kb + j) * chunk2, hi = min(V, lo + chunk2);
                    const float2 h = lane_mass<K, BF16, VEC, CUT>(r[j], a, lo, hi);
                    const float s0 = wave_sum(h.x), s1 = wave_sum(h.y);
                    if (l == 0) {
                        scr[((kb + j - b0) * kUnroll2 + 0) * kWaves + w] = s0;
                        scr[((kb + j - b0) * kUnroll2 + 1) * kWaves + w] = s1;
                    }
                }
            };
            ChunkRegs<BF16, VEC> ra[GROUP], rb[GROUP];
            load_group(ra, b0);
            if constexpr (!CUT) {
                // no load under a branch between a group's loads and their
                // reduction (the compiler would wait there for every load in
                // flight, the next group's included): the last one or two
                // groups after the loop, ra holding [kb, kb + GROUP)
                int kb = b0;
                for (; kb + 2 * GROUP < b1; kb += 2 * GROUP) {
                    load_group(rb, kb + GROUP);
                    reduce_group(ra, kb);
                    load_group(ra, kb + 2 * GROUP);
                    reduce_group(rb, kb + GROUP);
                }
                if (kb + GROUP < b1) {
                    load_group(rb, kb + GROUP);
                    reduce_group(ra, kb);
                    reduce_group(rb, kb + GROUP);
                } else {
                    reduce_group(ra, kb);
                }
            } else {
                // one copy of the (generic, membership-testing) reduction:
                // the cut decision's registers do not hold a second
                for (int kb = b0; kb < b1; kb += 2 * GROUP) {
                    if (kb + GROUP < b1) load_group(rb, kb + GROUP);
                    reduce_group(ra, kb);
                    if (kb + GROUP >= b1) break;
                    if (kb + 2 * GROUP < b1) load_group(ra, kb + 2 * GROUP);
                    reduce_group(rb, kb + GROUP);
                }
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                for (int k = b0; k < b1; ++k) {
                    const float* s = scr + (k - b0) * kUnroll2 * kWaves;
                    float h0 = s[0], h1 = s[kWaves];
#pragma unroll
                    for (int q = 1; q < kWaves; ++q) {
                        h0 += s[q];
                        h1 += s[kWaves + q];
                    }
                    dep |= emit(k, h0, h1);
                }
            }
            __syncthreads();  // scr is reused by the next batch and by the caller
        }
    } else {
        for (int k = k0; k < k1; ++k) {
            const int lo = k * chunk2, hi = min(V, lo + chunk2);
            const float2 h = lane_mass_elements<BF16, CUT>(a, lo, hi);
            const float h0 = block_sum(h.x), h1 = block_sum(h.y);
            if (threadIdx.x == 0) dep |= emit(k, h0, h1);
        }
    }
    return dep;
}

// mass_chunks_of for the kind of mass a describes, chosen once for the whole
// walk, with no branch on the kind between one group's loads and their
// reduction.  Each copy of the walk is inlined: a walk left as a call takes
// its register sets by reference, which puts them in scratch memory (the cut
// decision with two-chunk groups went from 22.3 to 33.1 us that way).
template <bool BF16, bool VEC, int GROUP, bool CACHED, bool CUT = false, class Emit>
__device__ uint32_t mass_chunks(const MassRows& a, int k0, int k1, int chunk2, int V, float* scr,
                                Emit&& emit) {
    return with_mass_kind<CUT>(a, [&](auto kind) {
        return mass_chunks_of<decltype(kind)::value, BF16, VEC, GROUP, CACHED, CUT>(a, k0, k1, chunk2, V, scr,
                                                                                     emit);
    });
}

// A chunk's mass from its halves' (every path adds them the same way).
__device__ __forceinline__ float chunk_total(float h0, float h1) { return h0 + h1; }

// Masses of one chunk's halves (the empty-residual fallback path).
template <bool BF16, bool VEC, bool CUT = false>
__device__ float2 chunk_mass(const MassRows& a, int lo, int hi) {
    float2 h;
    if constexpr (VEC) {
        ChunkRegs<BF16, VEC> r;
        load_chunk<BF16, VEC, false>(r, a, lo, hi);
        h = with_mass_kind<CUT>(a, [&](auto kind) {
            return lane_mass<decltype(kind)::value, BF16, VEC, CUT>(r, a, lo, hi);
        });
    } else {
        h = lane_mass_elements<BF16, CUT>(a, lo, hi);
    }
    const float h0 = block_sum(h.x);
    const float h1 = block_sum(h.y);
    return make_float2(h0, h1);
}

// First v of one half [lo, hi) of a chunk (at most kThreads*N elements, hi
// >= N) with base + prefix(v) > target, scanning the mass in ascending token
// order.  Lane l holds the N consecutive elements starting at lo + l*N (one
// vector), so one block-wide exclusive scan of the lane totals gives each
// lane its offset.  Returns 0x7fffffff if none; *last_pos receives the half's
// largest v with mass > 0.
template <bool BF16, bool VEC, bool CUT = false>
__device__ int search_half(const MassRows& a, int lo, int hi, float base, float target,
                           int* last_pos) {
    constexpr int N = Vec<BF16>::N;
    constexpr int PER = N;  // elements per lane
    __shared__ float s_wtot[kWaves];
    __shared__ int s_found[kWaves], s_last[kWaves];
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    const int e0 = lo + threadIdx.x * PER;
    Vec<BF16> vp, vq;
    if constexpr (VEC) {
        // clamped into the row: a vector lies wholly inside [lo, hi) or past it
        const int ec = min(e0, hi - N);
        vp = widen<BF16>(load16<BF16>(a.p, ec));
        if (a.q) vq = widen<BF16>(load16<BF16>(a.q, ec));
    } else {
        vp = load_vec<BF16, VEC>(a.p, e0, hi, neg_inf());
        if (a.q) vq = load_vec<BF16, VEC>(a.q, e0, hi, neg_inf());
    }
    float r[PER];
    float run = 0.0f;
    int lastp = -1;
    with_mass_kind<CUT>(a, [&](auto kind) {
        constexpr MassKind K = decltype(kind)::value;
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int v = e0 + k;
            const float x =
                v < hi ? mass_of<K, CUT>(a, vp.x[k], K != MassKind::kTarget && K != MassKind::kTargetButOne && a.q ? vq.x[k] : 0.0f, v)
                       : 0.0f;
            if (x > 0.0f) lastp = v;
            r[k] = x;
            run += x;
        }
        return 0;
    });
    // exclusive scan of the lane totals: inclusive within the wave, shifted,
    // plus the totals of the waves before
    const float incl = wave_prefix_sum(run);
    const float ex = wave_shift_right(incl);
    if (l == kWave - 1) s_wtot[w] = incl;
    __syncthreads();
    float woff = 0.0f;
    for (int k = 0; k < w; ++k) woff += s_wtot[k];
    float acc = base + (woff + ex);
    int first = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        acc += r[k];
        if (first == 0x7fffffff && acc > target) first = e0 + k;
    }
    // lanes hold ascending token ranges: the lowest crossing lane has the
    // first crossing, the highest lane with mass the last token with mass
    const uint64_t cross = __ballot(first != 0x7fffffff);
    const uint64_t pos = __ballot(lastp >= 0);
    const int f = cross ? lane_value(first, __builtin_ctzll(cross)) : 0x7fffffff;
    const int lp = pos ? lane_value(lastp, 63 - __builtin_clzll(pos)) : -1;
    if (l == 0) {
        s_found[w] = f;
        s_last[w] = lp;
    }
    __syncthreads();
    int found = 0x7fffffff, last = -1;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
        found = min(found, s_found[k]);
        last = max(last, s_last[k]);
    }
    *last_pos = last;
    return found;
}

// Stage the request's chunk partials in LDS with one batch of independent
// loads (rows x chunks <= kMaxPart).
__device__ __forceinline__ void stage_partials(const VerifyParams& P, int b, float4* s_part) {
    const int n = P.rows * P.nc;
    const float4* src = P.part + static_cast<size_t>(b) * n;
    for (int t = threadIdx.x; t < n; t += kThreads) s_part[t] = src[t];
}

// Waits for request b's statistics in the one-kernel path.  The (max, sum)
// word of every used (row, chunk) is nonzero once published (a published
// pair never has all-zero bits: a chunk's sum is >= 1 unless its max is
// -inf, whose bits are nonzero), and zero at rest.  Lane 0 first polls the
// word of the request's last used (row, chunk) in launch order, the one
// usually published last; then every word is read (and, if still zero,
// polled) by a lane of its own.  Polls sleep in between, and atomic reads
// see the device-scope exchanges that published the words.  A word still
// missing after P.wait_ticks of the 100 MHz constant clock is computed here
// from its row, with the statistics workgroup's arithmetic (chunk_maxsum on
// the same chunk), so the result does not change; returns true (to every
// lane) if a wait gave up.
template <bool BF16, bool VEC>
__device__ bool wait_partials(const VerifyParams& P, int b, int g, float4* s_part) {
    const int n = P.rows * P.nc;
    unsigned long long* rdy = reinterpret_cast<unsigned long long*>(P.ready) + static_cast<size_t>(b) * n;
    const uint64_t t0 = wall_clock64();
    bool late = false;
    if (threadIdx.x == 0) {
        const int s_last = P.point ? g : (g > 0 ? P.G + g : 0);
        unsigned long long* last = rdy + s_last * P.nc + P.nc - 1;
        while (atomicOr(last, 0ull) == 0ull) {
            if (wall_clock64() - t0 > P.wait_ticks) break;
            __builtin_amdgcn_s_sleep(16);
        }
    }
    for (int t = threadIdx.x; t < n; t += kThreads) {
        const int s = t / P.nc;
        const bool used = (s <= P.G) ? (s <= g) : (s - (P.G + 1) < g);
        unsigned long long v = 0;
        bool miss = false;
        if (used) {
            while ((v = atomicOr(rdy + t, 0ull)) == 0ull) {
                if (wall_clock64() - t0 > P.wait_ticks) { miss = true; break; }
                __builtin_amdgcn_s_sleep(16);
            }
        }
        late |= miss;
        // (w = 1 marks a partial that did not come)
        s_part[t] = make_float4(__uint_as_float(static_cast<uint32_t>(v)),
                                __uint_as_float(static_cast<uint32_t>(v >> 32)), 0.0f, miss ? 1.0f : 0.0f);
    }
    if (!__syncthreads_or(late)) return false;
    for (int t = 0; t < n; ++t) {
        if (s_part[t].w == 0.0f) continue;
        const int s = t / P.nc, ci = t % P.nc;
        const void* rp = s <= P.G ? target_row(P, b, s, BF16) : draft_row(P, b, s - (P.G + 1), BF16);
        const int lo = ci * P.chunk, hi = min(P.V, lo + P.chunk);
        MaxSum r;
        if constexpr (VEC) {
            r = chunk_maxsum_lean<BF16>(rp, lo, hi, P.c);
        } else {
            auto all = []() { return true; };
            chunk_maxsum<BF16, VEC, decltype(all)&, true>(rp, lo, hi, P.c, all, &r);
        }
        __syncthreads();  // every lane has read s_part[t].w
        if (threadIdx.x == 0) s_part[t] = make_float4(r.m, r.s, 0.0f, 0.0f);
        __syncthreads();
    }
    return true;
}

// Back to zero for the next call: every used word of request b (run by the
// request's last decision workgroup, after every workgroup has read them).
// Without a late partial anywhere in the request every word was published
// before it was read, and each is cleared by an exchange nobody waits for.
// After a wait gave up (careful), a word is taken only once it has been
// published, within the fixed 20 ms bound, since it may still land now;
// returns true (to every lane) if one never came (it may land later and stay
// set: the workspace must then be cleared).
__device__ __forceinline__ bool clear_partials(const VerifyParams& P, int b, int g, bool careful) {
    const int n = P.rows * P.nc;
    unsigned long long* rdy = reinterpret_cast<unsigned long long*>(P.ready) + static_cast<size_t>(b) * n;
    if (!careful) {
        for (int t = threadIdx.x; t < n; t += kThreads) {
            const int s = t / P.nc;
            const bool used = (s <= P.G) ? (s <= g) : (s - (P.G + 1) < g);
            if (used) atomicExch(rdy + t, 0ull);
        }
        return false;
    }
    bool lost = false;
    for (int t = threadIdx.x; t < n; t += kThreads) {
        const int s = t / P.nc;
        const bool used = (s <= P.G) ? (s <= g) : (s - (P.G + 1) < g);
        if (!used) continue;
        const uint64_t t0 = wall_clock64();
        while (atomicExch(rdy + t, 0ull) == 0ull) {
            if (wall_clock64() - t0 > kFixedWaitTicks) { lost = true; break; }
            __builtin_amdgcn_s_sleep(16);
        }
    }
    return __syncthreads_or(lost);
}

// One-kernel path: the chunk masses of request b's decision workgroups
// other than the last, words [0, n) of cm.  Each publisher writes its word
// once, the chunk's two half masses packed by pack_halves, by an atomic
// exchange it does not wait for.  The last decision
// workgroup (launched after all of them) reads them here, a lane per word:
// each read is an exchange with zero, so a word is cleared for the next call
// as it is taken.  Polls sleep in between, bounded like the statistics wait;
// a word that did not come leaves kMassMissing in s_csum (the caller
// computes it and takes the late word).  Returns true (to every lane) if a
// wait gave up.
constexpr uint32_t kMassMissing = 0x7fc0deadu;  // a NaN pattern

// A published chunk-mass word: bit 63 set (never all zero), bit 62 if the
// publisher's own statistics wait gave up, then the two halves' masses as
// 31-bit floats without their sign bit (masses are >= 0; a NaN stays a NaN).
__device__ __forceinline__ unsigned long long pack_halves(float h0, float h1, bool late) {
    return (1ull << 63) | (late ? (1ull << 62) : 0ull) |
           (static_cast<unsigned long long>(__float_as_uint(h0) & 0x7fffffffu) << 31) |
           static_cast<unsigned long long>(__float_as_uint(h1) & 0x7fffffffu);
}

__device__ __forceinline__ float2 unpack_halves(unsigned long long v) {
    return make_float2(__uint_as_float(static_cast<uint32_t>(v >> 31) & 0x7fffffffu),
                       __uint_as_float(static_cast<uint32_t>(v) & 0x7fffffffu));
}

__device__ bool collect_masses(const VerifyParams& P, unsigned long long* cm, int n, float* s_csum,
                               float2* s_half) {
    const uint64_t t0 = wall_clock64();
    bool late = false;
    for (int k = threadIdx.x; k < n; k += kThreads) {
        unsigned long long v;
        while ((v = atomicExch(cm + k, 0ull)) == 0ull) {
            if (wall_clock64() - t0 > P.wait_ticks) { late = true; break; }
            __builtin_amdgcn_s_sleep(16);
        }
        late |= ((v >> 62) & 1ull) != 0;
        const float2 h = unpack_halves(v);
        s_half[k] = h;
        s_csum[k] = v == 0ull ? __uint_as_float(kMassMissing) : chunk_total(h.x, h.y);
    }
    return __syncthreads_or(late);
}

// Decision workgroup wg of request b.  FUSED: the statistics come from the
// same kernel's statistics workgroups (wait_partials), and the drafted
// tokens' logits are read from the rows directly; otherwise from the
// partials the statistics kernel stored.  CUT: p and q are truncated, each
// row's (max, kept mass) and kept set coming from its cut record
// (k_trunc_cut); everything else as without truncation.
template <bool BF16, bool VEC, int GROUP, bool FUSED, bool CACHED, bool CUT = false>
__device__ __forceinline__ void decide_sample(const VerifyParams& P, const int wg, const int b) {
    __shared__ float4 s_part[kMaxPart];
    __shared__ float2 s_stat[127];
    __shared__ float2 s_cut[CUT ? 127 : 1];  // (boundary logit, last kept index at it as bits)
    __shared__ float s_csum[1024];
    __shared__ float2 s_half[1024];  // each chunk's half masses
    __shared__ int s_m, s_dm;
    __shared__ uint32_t s_fl;
    __shared__ float s_R, s_um;
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    const int i = l;
    const float c = P.c;

    // (0) independent loads first: partials, the drafted tokens, gamma_b;
    // the uniforms of position i (lane i of wave 0) while they are in flight
    if constexpr (!FUSED) stage_partials(P, b, s_part);
    int d = -1;
    if (w == 0 && i < P.G) d = P.tokens[static_cast<size_t>(b) * P.G + i];
    // gamma_b read once: clamped into [0, G], flagged if it was outside
    const int graw = P.gamma ? P.gamma[b] : P.G;
    const int g = min(max(graw, 0), P.G);
    float u_acc = 0.0f, u_draw = 0.0f;
    if (w == 0) {
        const uint4 r = philox4x32_10(make_uint4(static_cast<uint32_t>(i), static_cast<uint32_t>(b),
                                                 P.round, 0u), P.key0, P.key1);
        u_acc = uniform24(r.x);
        u_draw = uniform24(r.y);
    }
    // logits of the drafted token in target row i and draft row i
    float zt = 0.0f, zq = 0.0f;
    bool late = false;
    if constexpr (FUSED) {
        if (w == 0 && i < g && d >= 0 && d < P.V) {
            zt = load_logit<BF16>(target_row(P, b, i, BF16), d);
            if (!P.point) zq = load_logit<BF16>(draft_row(P, b, i, BF16), d);
        }
        late = wait_partials<BF16, VEC>(P, b, g, s_part);
    } else {
        __syncthreads();
        if (w == 0 && i < g && d >= 0 && d < P.V) {
            const int cd = d / P.chunk;
            zt = s_part[i * P.nc + cd].z;
            if (!P.point) zq = s_part[(P.G + 1 + i) * P.nc + cd].z;
        }
    }

    // (1) (max, sum) of every used row from its chunk partials: a lane per
    // row over a few partials, else a wave per row (CUT: (max, kept mass)
    // and the kept set from the row's cut record)
    if constexpr (CUT) {
        for (int s = threadIdx.x; s < P.rows; s += kThreads) {
            const bool used = (s <= P.G) ? (s <= g) : (s - (P.G + 1) < g);
            if (!used) continue;
            const uint4 r = P.cut[static_cast<size_t>(b) * P.rows + s];
            s_stat[s] = make_float2(__uint_as_float(r.x), __uint_as_float(r.y));
            s_cut[s] = make_float2(__uint_as_float(r.z), __uint_as_float(r.w));
        }
    } else if (P.nc <= kSerialParts) {
        for (int s = threadIdx.x; s < P.rows; s += kThreads) {
            const bool used = (s <= P.G) ? (s <= g) : (s - (P.G + 1) < g);
            if (!used) continue;
            // the maximum first, then each partial's sum rescaled to it and
            // added in chunk order (no chain of dependent exponentials)
            float m = neg_inf();
            for (int k = 0; k < P.nc; ++k) m = fmaxf(m, s_part[s * P.nc + k].x);
            float sum = 0.0f;
            for (int k = 0; k < P.nc; ++k) {
                const float4 q = s_part[s * P.nc + k];
                sum += q.x == neg_inf() ? 0.0f : q.y * exp2f((q.x - m) * c);
            }
            s_stat[s] = make_float2(m, sum);
        }
    } else {
        for (int s = w; s < P.rows; s += kWaves) {
            const bool used = (s <= P.G) ? (s <= g) : (s - (P.G + 1) < g);
            if (!used) continue;
            // as above, a lane per partial
            float ml = neg_inf();
            for (int k = l; k < P.nc; k += kWave) ml = fmaxf(ml, s_part[s * P.nc + k].x);
            const float m = wave_max(ml);
            float sl = 0.0f;
            for (int k = l; k < P.nc; k += kWave) {
                const float4 q = s_part[s * P.nc + k];
                sl += q.x == neg_inf() ? 0.0f : q.y * exp2f((q.x - m) * c);
            }
            const float sum = wave_sum(sl);
            if (l == 0) s_stat[s] = make_float2(m, sum);
        }
    }
    __syncthreads();

    // (2) acceptance tests, lane i = position i of wave 0; m from a ballot
    float pd = 0.0f, qd = 0.0f;
    if (w == 0) {
        uint32_t fl = (i == 0 && (graw < 0 || graw > P.G)) ? SPECDEC_FLAG_BAD_GAMMA : 0u;
        bool acc = false;
        if (i <= g) {
            const float2 t = s_stat[i];
            if (!(t.x < pos_inf()) || !(t.y == t.y)) fl |= SPECDEC_FLAG_NONFINITE;
        }
        if (i < g) {
            const float2 t = s_stat[i];
            float2 q = make_float2(0.0f, 1.0f);
            if (!P.point) {
                q = s_stat[P.G + 1 + i];
                if (!(q.x < pos_inf()) || !(q.y == q.y)) fl |= SPECDEC_FLAG_NONFINITE;
            }
            float a = 0.0f;
            if (d >= 0 && d < P.V) {
                pd = exp2f((zt - t.x) * c) / t.y;
                if (P.point) {
                    qd = 1.0f;  // point-mass draft: q_i(d_i) = 1
                } else {
                    qd = exp2f((zq - q.x) * c) / q.y;
                }
                if constexpr (CUT) {
                    // a token outside a kept set has probability 0 there
                    const float2 kt = s_cut[i], kq = s_cut[P.G + 1 + i];
                    if (!(zt > kt.x || (zt == kt.x && d <= __float_as_int(kt.y)))) pd = 0.0f;
                    if (!P.point && !(zq > kq.x || (zq == kq.x && d <= __float_as_int(kq.y)))) qd = 0.0f;
                }
                if (qd > 0.0f) a = fminf(1.0f, pd / qd);
                else a = pd > 0.0f ? 1.0f : 0.0f;
            } else {
                fl |= SPECDEC_FLAG_TOKEN_RANGE;
            }
            acc = u_acc < a;
        } else {
            d = -1;
        }
        const uint64_t mask = __ballot(acc);
        const int m = min(g, static_cast<int>(__builtin_ctzll(~mask)));
        fl = wave_or(fl);
        const int dm = lane_value(d, min(m, kWave - 1));  // the rejected draft (m < g)
        const float um = lane_value(u_draw, min(m, kWave - 1));  // the draw's uniform
        if (l == 0) { s_m = m; s_fl = fl; s_dm = dm; s_um = um; }
    }
    __syncthreads();
    const int m = s_m;

    // (3) this workgroup's chunks of the sampling mass at position m
    const bool resid = m < g;
    MassRows a;
    const float2 tp = s_stat[m];
    a.p = target_row(P, b, m, BF16);
    a.mp = tp.x;
    a.isp = 1.0f / tp.y;
    a.c = c;
    a.q = nullptr;
    a.mq = 0.0f;
    a.isq = 0.0f;
    a.point = -1;
    a.tp = a.tq = neg_inf();
    a.ip = a.iq = 0x7fffffff;
    if constexpr (CUT) {
        a.tp = s_cut[m].x;
        a.ip = __float_as_int(s_cut[m].y);
    }
    if (resid && P.point) {
        // max(p - delta_d, 0): p itself without the rejected token
        a.point = s_dm;
    } else if (resid) {
        const float2 tq = s_stat[P.G + 1 + m];
        a.q = draft_row(P, b, m, BF16);
        a.mq = tq.x;
        a.isq = 1.0f / tq.y;
        if constexpr (CUT) {
            a.tq = s_cut[P.G + 1 + m].x;
            a.iq = __float_as_int(s_cut[P.G + 1 + m].y);
        }
    }
    const int k0 = wg * P.cpw, k1 = min(P.nc2, k0 + P.cpw);
    float* scr = reinterpret_cast<float*>(s_part);  // the partials are combined: free
    if constexpr (FUSED) {
        // the request's last decision workgroup (chunks [k0, nc2)) keeps its
        // masses in LDS and collects the others' published words
        unsigned long long* cm = reinterpret_cast<unsigned long long*>(P.cmass) + static_cast<size_t>(b) * P.nc2;
        mass_chunks<BF16, VEC, GROUP, CACHED>(a, k0, k1, P.chunk2, P.V, scr,
                                              [&](int k, float h0, float h1) -> uint32_t {
                                                  s_half[k] = make_float2(h0, h1);
                                                  s_csum[k] = chunk_total(h0, h1);
                                                  return 0u;
                                              });
        // (mass_chunks ends with a barrier: s_csum[k0, k1) is visible)
        if (wg != P.wpr - 1) {
            for (int k = k0 + threadIdx.x; k < k1; k += kThreads)
                atomicExch(cm + k, pack_halves(s_half[k].x, s_half[k].y, late));
            return;
        }
        if (collect_masses(P, cm, k0, s_csum, s_half)) {
            late = true;
            // a publisher that did not come in time: its chunks' masses
            // computed here (mass_chunks gives each chunk the same value
            // whatever the range; a real mass that happens to carry the
            // marker's bits is only computed again), then its late words taken
            for (int k = 0; k < k0; ++k) {
                if (__float_as_uint(s_csum[k]) != kMassMissing) continue;
                __syncthreads();  // every lane has read s_csum[k]
                mass_chunks<BF16, VEC, GROUP, CACHED>(a, k, k + 1, P.chunk2, P.V, scr,
                                                      [&](int kk, float h0, float h1) -> uint32_t {
                                                          s_half[kk] = make_float2(h0, h1);
                                                          s_csum[kk] = chunk_total(h0, h1);
                                                          return 0u;
                                                      });
                if (threadIdx.x == 0) {
                    const uint64_t t1 = wall_clock64();
                    while (atomicExch(cm + k, 0ull) == 0ull) {
                        if (wall_clock64() - t1 > kFixedWaitTicks) break;
                        __builtin_amdgcn_s_sleep(16);
                    }
                }
                __syncthreads();
            }
        }
        // every decision workgroup of the request has read the statistics
        // words before publishing its masses (a late one has been awaited)
        if (late) late = clear_partials(P, b, g, true) || late;
        else clear_partials(P, b, g, false);
    } else {
        uint32_t* csum = P.csum + static_cast<size_t>(b) * P.nc2 * 2;  // (h0, h1) per chunk
        const uint32_t dep = mass_chunks<BF16, VEC, GROUP, CACHED, CUT>(
            a, k0, k1, P.chunk2, P.V, scr, [&](int k, float h0, float h1) {
                return publish(csum + 2 * k, __float_as_uint(h0)) | publish(csum + 2 * k + 1, __float_as_uint(h1));
            });
        if (!arrive_last(P.cnt + b, static_cast<uint32_t>(P.wpr), dep)) return;
        for (int k = threadIdx.x; k < P.nc2; k += kThreads) {
            const float2 h = make_float2(__uint_as_float(fetch(csum + 2 * k)), __uint_as_float(fetch(csum + 2 * k + 1)));
            s_half[k] = h;
            s_csum[k] = chunk_total(h.x, h.y);
        }
        __syncthreads();
    }

    // (4) last workgroup of the request: R, the chunk where the running mass
    // passes u*R, the token inside it, then every output of the request.
    // Wave 0 walks the chunk sums in chunk order: lane l takes a run of
    // consecutive chunks, and a wave prefix sum of the runs' totals gives R
    // and each run its offset.  scan() leaves R in s_R, and in s_chunk /
    // s_before the chunk where the running mass first passes u*R and the
    // mass before it (or, if rounding leaves none, the last chunk with mass
    // and +inf).
    __shared__ int s_chunk;
    __shared__ float s_before;
    const int per = (P.nc2 + kWave - 1) / kWave;
    const int r0 = l * per, r1 = min(P.nc2, r0 + per);
    auto scan = [&]() {
        if (w == 0) {
            float run = 0.0f;
            for (int k = r0; k < r1; ++k) run += s_csum[k];
            const float incl = wave_prefix_sum(run);
            const float R = lane63(incl);
            const float target = s_um * R;
            float before = wave_shift_right(incl);
            int found = -1, lastk = -1;
            float fb = 0.0f;
            for (int k = r0; k < r1; ++k) {
                const float next = before + s_csum[k];
                if (found < 0 && next > target) { found = k; fb = before; }
                if (s_csum[k] > 0.0f) lastk = k;
                before = next;
            }
            const uint64_t hit = __ballot(found >= 0);
            const uint64_t pos = __ballot(lastk >= 0);
            int cstar;
            float bef;
            if (hit) {
                const int src = __builtin_ctzll(hit);
                cstar = lane_value(found, src);
                bef = lane_value(fb, src);
            } else {
                // rounding left u*R at or above the total: the last chunk with mass
                cstar = pos ? lane_value(lastk, 63 - __builtin_clzll(pos)) : 0;
                bef = pos_inf();  // no crossing: take its last token with mass
            }
            if (l == 0) { s_R = R; s_chunk = cstar; s_before = bef; }
        }
        __syncthreads();
    };
    uint32_t fl2 = 0;
    float R_report = 0.0f;
    scan();
    if (resid) {
        R_report = s_R;
        if (!(s_R > 0.0f)) {
            // empty residual: draw from p_m instead (never divide by zero)
            fl2 |= SPECDEC_FLAG_RESIDUAL_FALLBACK;
            a.q = nullptr;
            a.point = -1;
            for (int k = 0; k < P.nc2; ++k) {
                const float2 h = chunk_mass<BF16, VEC, CUT>(a, k * P.chunk2, min(P.V, (k + 1) * P.chunk2));
                if (threadIdx.x == 0) {
                    s_half[k] = h;
                    s_csum[k] = chunk_total(h.x, h.y);
                }
            }
            __syncthreads();
            scan();
        }
    }
    const float target = s_um * s_R;
    int lastp;
    // The chosen chunk's half: the first if the mass before the chunk plus
    // the first half's passes u*R, else the second, after the first's mass.
    // Without a crossing (s_before = +inf: rounding left u*R at or above the
    // total), the last token with mass is taken, in the chunk's last half
    // with mass.  A half of the last chunk may be empty (past V): never chosen.
    constexpr int kHalf = kThreads * Vec<BF16>::N;
    const int l2 = s_chunk * P.chunk2, h2 = min(P.V, l2 + P.chunk2), lm = min(h2, l2 + kHalf);
    const float2 hc = s_half[s_chunk];
    const bool none = !(s_before < pos_inf());
    const bool second = lm < h2 && (none ? hc.y > 0.0f : !(s_before + hc.x > target));
    const float base = second ? s_before + hc.x : s_before;
    int token = search_half<BF16, VEC, CUT>(a, second ? lm : l2, second ? h2 : lm, base, target, &lastp);
    // The chunk sums and the in-half prefixes associate the additions
    // differently; if that rounding leaves no element above u*R in the chosen
    // half, the crossing is its last token with mass.
    if (none || token == 0x7fffffff) token = lastp;

    if (w == 0) {
        fl2 |= write_round(P, b, m, i < m ? d : token);
        if (i < P.G) {
            if (P.p_draft) P.p_draft[static_cast<size_t>(b) * P.G + i] = pd;
            if (P.q_draft) P.q_draft[static_cast<size_t>(b) * P.G + i] = qd;
        }
        if (i == 0) {
            if (P.residual_mass) P.residual_mass[b] = R_report;
            if (P.flags) P.flags[b] = s_fl | fl2 | (late ? SPECDEC_FLAG_WAIT_TIMEOUT : 0u);
        }
    }
}

template <bool BF16, bool VEC, int GROUP>
__global__ __launch_bounds__(kThreads) void k_decide_sample(VerifyParams P) {
    decide_sample<BF16, VEC, GROUP, false, false>(P, blockIdx.x, blockIdx.y);
}

// The sampling decision over truncated rows given by cut records.
template <bool BF16, bool VEC, int GROUP>
__global__ __launch_bounds__(kThreads) void k_decide_cut(VerifyParams P) {
    decide_sample<BF16, VEC, GROUP, false, false, true>(P, blockIdx.x, blockIdx.y);
}

// ------------------------------------------------------------------ one-kernel sampling verify

// Workgroup roles of the one-kernel path, in launch order.  Request j
// contributes its S = rows x nc statistics workgroups; the W = wpr decision
// workgroups of request j are placed right after the statistics workgroups
// of request j + lag (after the last request's when j + lag >= B).  So every
// decision workgroup comes later in launch order than each statistics
// workgroup it waits for, and those never wait: with workgroups dispatched
// in launch order, every wait ends (and a bounded wait guards the rest).
constexpr int kXcds = 8;  // XCDs of one gfx950 device (8 x 32 compute units)

struct Role {
    bool stats;
    int b;
    int k;  // statistics: row * nc + chunk; decision: workgroup of the request
};

__device__ __forceinline__ Role fused_role(const VerifyParams& P, int x) {
    const int S = P.rows * P.nc, W = P.wpr, lag = P.lag;
    if (x < lag * S) return Role{true, x / S, x % S};
    x -= lag * S;
    if (P.resid_cached && lag == P.B && (P.B % kXcds) == 0 && ((P.B * S) % kXcds) == 0) {
        // Decision workgroups, each request's on one XCD: workgroups go to
        // the XCDs round-robin by launch index, so request b's take indices
        // congruent to b mod kXcds, and the crossing chunk the request's
        // last workgroup reads again was loaded (with cached loads) into
        // that XCD's L2 by the workgroup that summed it.  The request's last
        // workgroup still has the largest index of the request's.  (Measured
        // on two boxes: fp32 B=8 x V=32000 14.3-14.6 -> 13.2 us, p90 17.5-18.3
        // -> 13.7 us; B=64 x V=128256 bf16 38.2-38.6 us either way.)
        const int xcd = x % kXcds, slot = x / kXcds;
        return Role{false, (slot / W) * kXcds + xcd, slot % W};
    }
    const int mid = (P.B - lag) * (S + W);
    if (x < mid) {
        const int j = lag + x / (S + W), r = x % (S + W);
        if (r < S) return Role{true, j, r};
        return Role{false, j - lag, r - S};
    }
    x -= mid;
    return Role{false, P.B - lag + x / W, x % W};
}

// Statistics workgroup of the one-kernel path: the chunk's (max, sum) pair,
// published as one 64-bit word with a device-scope atomic exchange whose
// result is not awaited (an atomic with return, or an arrival counter
// behind it, waits a memory round trip that the full HBM stream makes long).
template <bool BF16, bool VEC>
__device__ __forceinline__ void fused_stats(const VerifyParams& P, int b, int k) {
    const int s = k / P.nc, ci = k % P.nc;
    const bool is_target = s <= P.G;
    const int i = is_target ? s : s - (P.G + 1);
    const void* rp = is_target ? target_row(P, b, i, BF16) : draft_row(P, b, i, BF16);
    const int lo = ci * P.chunk;
    const int hi = min(P.V, lo + P.chunk);
    auto keep = [&]() {
        if (!P.gamma) return true;
        const int g = request_gamma(P, b);
        return is_target ? i <= g : i < g;
    };
    MaxSum r;
    if (!chunk_maxsum<BF16, VEC>(rp, lo, hi, P.c, keep, &r)) return;
    if (threadIdx.x == 0) {
        const unsigned long long v =
            (static_cast<unsigned long long>(__float_as_uint(r.s)) << 32) | __float_as_uint(r.m);
        atomicExch(reinterpret_cast<unsigned long long*>(P.ready) +
                       static_cast<size_t>(b) * P.rows * P.nc + k, v);
    }
}

// CACHED: ordinary loads for the residual / bonus rows (see verify_impl).
template <bool BF16, bool VEC, int GROUP, bool CACHED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6))) void k_verify_fused(VerifyParams P) {
    const Role r = fused_role(P, blockIdx.x);
    if (r.stats) fused_stats<BF16, VEC>(P, r.b, r.k);
    else decide_sample<BF16, VEC, GROUP, true, CACHED>(P, r.k, r.b);
}

// ------------------------------------------------------------------ greedy decision

// Greedy decision of request b.  FUSED: the partials are the words the same
// kernel's statistics workgroups publish (collect_greedy); otherwise those
// the statistics kernel stored.
template <bool FUSED, bool BF16 = true, bool VEC = true>
__device__ __forceinline__ void decide_greedy(const VerifyParams& P, const int b) {
    __shared__ float4 s_part[kMaxPart];
    __shared__ int s_arg[64];
    __shared__ uint32_t s_nan[64];
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    if constexpr (!FUSED) stage_partials(P, b, s_part);
    const int i = l;
    int d = -1;
    if (w == 0 && i < P.G) d = P.tokens[static_cast<size_t>(b) * P.G + i];
    const int graw = P.gamma ? P.gamma[b] : P.G;  // read once, clamped, flagged below
    const int g = min(max(graw, 0), P.G);
    bool late = false;
    if constexpr (FUSED) late = collect_greedy<BF16, VEC>(P, b, [&](int s) { return s <= g; }, s_part);
    __syncthreads();
    // a lane per row over a few partials, else a wave per row
    auto part_argmax = [&](int s, int k0, int step, ArgMax& best, uint32_t& nan) {
        for (int k = k0; k < P.nc; k += step) {
            const float4 q = s_part[s * P.nc + k];
            const uint32_t word = __float_as_uint(q.y);  // index, bit 31: a NaN was seen
            const int idx = static_cast<int>(word & 0x7fffffffu);
            if (idx != 0x7fffffff) best = better(best, ArgMax{q.x, idx});
            nan |= word >> 31;
        }
    };
    if (P.nc <= kSerialParts) {
        for (int s = threadIdx.x; s <= g; s += kThreads) {
            ArgMax best{neg_inf(), 0x7fffffff};
            uint32_t nan = 0;
            part_argmax(s, 0, 1, best, nan);
            s_arg[s] = best.i;
            s_nan[s] = nan;
        }
    } else {
        for (int s = w; s <= g; s += kWaves) {
            ArgMax best{neg_inf(), 0x7fffffff};
            uint32_t nan = 0;
            part_argmax(s, l, kWave, best, nan);
            best = wave_argmax(best);
            nan = wave_or(nan);
            if (l == 0) { s_arg[s] = best.i; s_nan[s] = nan; }
        }
    }
    __syncthreads();
    if (w != 0) return;
    uint32_t fl = (i == 0 && (graw < 0 || graw > P.G)) ? SPECDEC_FLAG_BAD_GAMMA : 0u;
    bool acc = false;
    if (i <= g && s_nan[i]) fl |= SPECDEC_FLAG_NONFINITE;
    if (i < g) {
        if (d < 0 || d >= P.V) fl |= SPECDEC_FLAG_TOKEN_RANGE;
        acc = (d == s_arg[i]);
    } else {
        d = -1;
    }
    const uint64_t mask = __ballot(acc);
    const int m = min(g, static_cast<int>(__builtin_ctzll(~mask)));
    fl = wave_or(fl);
    fl |= write_round(P, b, m, i < m ? d : s_arg[m]);
    if (i == 0 && P.flags) P.flags[b] = fl | (late ? SPECDEC_FLAG_WAIT_TIMEOUT : 0u);
}

__global__ __launch_bounds__(kThreads) void k_decide_greedy(VerifyParams P) {
    decide_greedy<false>(P, blockIdx.x);
}

// One-kernel greedy verify: the B x S statistics workgroups (S = rows x nc,
// request by request) first in launch order, then one decision workgroup per
// request, which waits only on statistics workgroups launched before it.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void k_greedy_fused(VerifyParams P) {
    const int S = P.rows * P.nc;
    const int x = blockIdx.x;
    if (x < P.B * S) {
        const int b = x / S;
        fused_greedy_stats<BF16, VEC>(P, b, x % S, [&](int s) { return s <= request_gamma(P, b); });
    } else {
        decide_greedy<true, BF16, VEC>(P, x - P.B * S);
    }
}

// ------------------------------------------------------------------ host side

// Truncation mode: sampling with an effective top-k or with top-p.
bool truncation_mode(const specdec_verify_desc_t* d) {
    return d->mode == SPECDEC_SAMPLE &&
           ((d->top_k > 0 && d->top_k < d->vocab) || d->top_p < 1.0f);
}

// Truncation whose kept sets may be too long to list (top-p alone over more
// than kTruncCap tokens, or a top-k past kNucCap): cut records instead of
// kept-token records.  The debug build can force this path for any
// truncation (SPECDEC_TRUNC_CUT=1), for the tests that compare the two.
bool truncation_cut(const specdec_verify_desc_t* d) {
    if (!truncation_mode(d)) return false;
    const bool use_k = d->top_k > 0 && d->top_k < d->vocab;
    if (use_k ? d->top_k > kNucCap : d->vocab > kTruncCap) return true;
    const char* s = debug_knob("SPECDEC_TRUNC_CUT");
    return s && s[0] == '1';
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// a debug-build tuning switch (see debug_knob), else the default
int env_int(const char* name, int dflt) {
    const char* s = debug_knob(name);
    if (!s) return dflt;
    const int v = atoi(s);
    return v > 0 ? v : dflt;
}

// Decision workgroups of request j trail the statistics of request j + lag
// (B: after all of them); the debug build's SPECDEC_FUSED_LAG overrides (0..B).
int fused_lag(int B) {
    const char* s = debug_knob("SPECDEC_FUSED_LAG");
    const int v = s ? atoi(s) : B;
    return std::min(std::max(v, 0), B);
}

bool valid_desc(const specdec_verify_desc_t* d) {
    if (!d) return false;
    if (d->batch < 0 || d->batch > 65535 || d->gamma_max < 0 || d->gamma_max > 63 || d->vocab < 1)
        return false;
    if (d->dtype != SPECDEC_F32 && d->dtype != SPECDEC_BF16) return false;
    // at most 1024 sampling chunks of 256 lanes x 2 x 16 bytes per row
    if (d->vocab > 1024 * kThreads * kUnroll2 * (d->dtype == SPECDEC_BF16 ? 8 : 4)) return false;
    if (d->mode != SPECDEC_SAMPLE && d->mode != SPECDEC_GREEDY) return false;
    if (d->eos_plus1 < 0 || d->eos_plus1 > d->vocab) return false;
    if (d->mode == SPECDEC_SAMPLE) {
        const float T = d->temperature;
        if (!(T > 0.0f) || !(T < 3.0e38f)) return false;
        if (d->top_k < 0) return false;
        if (!(d->top_p > 0.0f) || !(d->top_p <= 1.0f)) return false;
    }
    return true;
}

}  // namespace

// Chunking.  Statistics pass, sampling: about one round of workgroups
// resident at once (8 per CU x 256 CUs), so that every workgroup streams from
// the start and none waits for a slot; greedy: two tiles per chunk; whole
// tiles per chunk either way.  Sampling pass: one tile of
// 256 lanes x 2 vectors per chunk (at most 1024 per row), each workgroup
// taking a run of consecutive chunks of one request.
Layout make_layout(const specdec_verify_desc_t* d, bool point) {
    Layout L{};
    const bool bf16 = d->dtype == SPECDEC_BF16;
    const int n = bf16 ? 8 : 4;
    const int tile = kThreads * n * kUnroll;
    const int vt = (d->vocab + tile - 1) / tile;
    L.rows = (d->mode == SPECDEC_SAMPLE && !point) ? 2 * d->gamma_max + 1 : d->gamma_max + 1;
    const double rows_total = static_cast<double>(d->batch > 0 ? d->batch : 1) * L.rows;
    int nc_want = static_cast<int>(2048.0 / rows_total);
    nc_want = nc_want < 1 ? 1 : nc_want;
    int tiles = (vt + nc_want - 1) / nc_want;
    // greedy rows (a compare per element, no exponential): chunks of two
    // tiles, many rounds of small workgroups (measured fastest: 622 MB in
    // 89 us against 101 us for one round of whole-row workgroups)
    if (d->mode == SPECDEC_GREEDY) tiles = 2;
    tiles = env_int("SPECDEC_STATS_TILES", tiles < 1 ? 1 : tiles);
    // the decision kernels stage rows x chunks partials in LDS
    while (static_cast<long>(L.rows) * ((vt + tiles - 1) / tiles) > kMaxPart) ++tiles;
    L.chunk = tile * tiles;
    L.nc = (d->vocab + L.chunk - 1) / L.chunk;
    L.chunk2 = kThreads * n * kUnroll2;
    L.nc2 = (d->vocab + L.chunk2 - 1) / L.chunk2;
    // sampling pass, all workgroups resident from the start: about 512 (two
    // per CU) when each then holds at most kMassGroupWide chunks, its whole
    // share loaded at once; else about 1024 (four per CU) of the leaner
    // double-buffered kind
    const int bb = d->batch > 0 ? d->batch : 1;
    const int w512 = max(1, static_cast<int>(512.0 / bb + 0.5));
    const bool short_share = L.nc2 <= kMassGroupWide * w512;
    const int wpr0 = short_share ? w512 : max(1, static_cast<int>(1024.0 / bb + 0.5));
    const int wpr = env_int("SPECDEC_SAMPLE_WPR", wpr0 > L.nc2 ? L.nc2 : wpr0);
    L.cpw = (L.nc2 + wpr - 1) / wpr;
    L.wpr = (L.nc2 + L.cpw - 1) / L.cpw;
    // a share of up to kMassGroupWide chunks is loaded as one group of
    // exactly its size; longer shares go in double-buffered pairs
    L.group = L.cpw <= kMassGroupWide ? L.cpw : kMassGroupChunks;
    // one-kernel path: twice as many decision workgroups, one chunk per
    // group (measured fastest on B=64 x V=128256 and B=512 x V=262144)
    const int fwpr = env_int("SPECDEC_SAMPLE_WPR", std::min(L.nc2, 2 * wpr0));
    L.fcpw = (L.nc2 + fwpr - 1) / fwpr;
    L.fwpr = (L.nc2 + L.fcpw - 1) / L.fcpw;
    const size_t B = static_cast<size_t>(d->batch);
    size_t off = 0;
    // zero at rest: arrival counters (two-kernel sampling path), statistics
    // words and chunk-mass words (one-kernel paths)
    L.off_cnt = off; off = align256(off + B * 4);
    L.off_ready = off; off = align256(off + B * L.rows * L.nc * sizeof(uint64_t));
    L.off_cmass = off; off = align256(off + B * L.nc2 * sizeof(uint64_t));
    L.off_part = off; off = align256(off + B * L.rows * L.nc * sizeof(float4));
    L.off_csum = off; off = align256(off + B * L.nc2 * 2 * sizeof(uint32_t));
    L.trunc = truncation_mode(d);
    // point-mass drafts under truncation: the cut path (its decision serves
    // point masses; the listed path's does not)
    L.cut = truncation_cut(d) || (point && L.trunc);
    // the cut decision's membership tests take registers: groups of at most
    // two chunks (larger ones spill).  Where shares of two chunks still keep
    // the decision's workgroups within about one resident round (2048), take
    // twice the workgroups, each loading its whole share at once.
    if (L.cut && L.cpw > kMassGroupChunks) {
        const int wpr2 = (L.nc2 + kMassGroupChunks - 1) / kMassGroupChunks;
        if (static_cast<long>(bb) * wpr2 <= 2048) {
            L.cpw = kMassGroupChunks;
            L.wpr = (L.nc2 + L.cpw - 1) / L.cpw;
            L.group = L.cpw;
        }
    }
    if (L.cut && L.group > kMassGroupChunks) L.group = kMassGroupChunks;
    L.off_nuc = off;  // kept-token records, or cut records
    if (L.cut) off = align256(off + B * L.rows * sizeof(uint4));
    else if (L.trunc) off = align256(off + B * L.rows * (1 + kNucCap) * sizeof(uint2));
    L.total = off;
    return L;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

__global__ void k_zero_words(uint32_t* p, size_t n) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

// ------------------------------------------------------------------ allocation-free variant
// The workspace of specdec_verify_noalloc: a file-scope device array, one
// copy per GPU the library runs on, held until the process ends.  Host code
// never passes the array's name to a kernel (in host code it is only a
// stand-in for the symbol): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kNoAllocBytes = size_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];
constexpr int kNoAllocDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocDevices] = {};

// The current device's copy of `scratch` (set up on its first use).
specdec_status_t noalloc_workspace(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocDevices) return SPECDEC_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SPECDEC_ERR_DEVICE;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SPECDEC_OK;
}

// Launch the passes of one call.  ev (may be null) holds start/stop events of
// the statistics pass and of the sampling pass; they bracket the kernels
// themselves (hipExtLaunchKernel), not the host-side enqueue.
template <bool BF16, bool VEC>
specdec_status_t launch_all(const specdec_verify_desc_t* d, const VerifyParams& P, const Layout& L,
                            bool fused, hipStream_t stream, hipEvent_t* ev) {
    const dim3 block(kThreads);
    hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
    hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
    auto launch = [&](auto kernel, dim3 grid, hipEvent_t start, hipEvent_t stop) {
        if (ev)
            hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, P);
        else
            hipLaunchKernelGGL(kernel, grid, block, 0, stream, P);
    };
    const bool greedy = d->mode == SPECDEC_GREEDY;
    if (fused && greedy) {
        const dim3 grid(static_cast<unsigned>(d->batch) * (L.rows * L.nc + 1));
        launch(k_greedy_fused<BF16, VEC>, grid, e0, e1);
        // the decision runs inside that kernel: its events mark the end
        if (e2 && hipEventRecord(e2, stream) != hipSuccess) return SPECDEC_ERR_DEVICE;
        if (e3 && hipEventRecord(e3, stream) != hipSuccess) return SPECDEC_ERR_DEVICE;
        return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
    }
    if (fused) {
        // one kernel: statistics and decision workgroups interleaved
        // (one chunk per group keeps the register count near the statistics
        // pass's, so that the streaming workgroups keep their occupancy)
        const dim3 grid(static_cast<unsigned>(d->batch) * (L.rows * L.nc + L.fwpr));
        if (P.resid_cached) launch(k_verify_fused<BF16, VEC, 1, true>, grid, e0, e1);
        else launch(k_verify_fused<BF16, VEC, 1, false>, grid, e0, e1);
        // the decision runs inside that kernel: its events mark the end
        if (e2 && hipEventRecord(e2, stream) != hipSuccess) return SPECDEC_ERR_DEVICE;
        if (e3 && hipEventRecord(e3, stream) != hipSuccess) return SPECDEC_ERR_DEVICE;
        return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
    }
    if (launch_stats(P, BF16, VEC, greedy, dim3(L.nc, L.rows, d->batch), stream, e0, e1) != SPECDEC_OK)
        return SPECDEC_ERR_DEVICE;
    if (greedy) {
        launch(k_decide_greedy, dim3(d->batch), e2, e3);
    } else {
        const dim3 grid(L.wpr, d->batch);
        switch (L.group) {
            case 1: launch(k_decide_sample<BF16, VEC, 1>, grid, e2, e3); break;
            case 3: launch(k_decide_sample<BF16, VEC, 3>, grid, e2, e3); break;
            case 4: launch(k_decide_sample<BF16, VEC, 4>, grid, e2, e3); break;
            default: launch(k_decide_sample<BF16, VEC, 2>, grid, e2, e3); break;
        }
    }
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
}

// Truncation by cut records: the statistics pass, the cut records, then the
// sampling decision over the truncated rows.  ev (may be null): start/stop
// of the cut kernel (the pass that dominates) and of the decision.
template <bool BF16, bool VEC>
specdec_status_t launch_cut(const specdec_verify_desc_t* d, const VerifyParams& P, const Layout& L,
                            hipStream_t stream, hipEvent_t* ev) {
    hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
    hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
    if (launch_stats(P, BF16, VEC, false, dim3(L.nc, L.rows, d->batch), stream, nullptr, nullptr) != SPECDEC_OK)
        return SPECDEC_ERR_DEVICE;
    if (launch_trunc_cut(P, BF16, VEC, stream, e0, e1) != SPECDEC_OK) return SPECDEC_ERR_DEVICE;
    const dim3 grid(L.wpr, d->batch), block(kThreads);
    auto launch = [&](auto kernel) {
        if (ev)
            hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, e2, e3, 0, P);
        else
            hipLaunchKernelGGL(kernel, grid, block, 0, stream, P);
    };
    if (L.group == 1) launch(k_decide_cut<BF16, VEC, 1>);
    else launch(k_decide_cut<BF16, VEC, 2>);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
}

specdec_status_t verify_impl(const specdec_verify_desc_t* d, const void* target_logits,
                             const void* draft_logits, const int32_t* draft_tokens,
                             const int32_t* gamma, const int32_t* max_tokens,
                             int32_t* accept_count, int32_t* num_tokens, int32_t* out_tokens,
                             float* p_draft, float* q_draft, float* residual_mass, uint32_t* flags,
                             void* workspace, size_t workspace_bytes, hipStream_t stream,
                             hipEvent_t* ev, bool clear_counters = false) {
    if (!valid_desc(d)) return SPECDEC_ERR_INVALID_ARGUMENT;
    const bool sample = d->mode == SPECDEC_SAMPLE;
    if (!target_logits || !accept_count || !out_tokens || !workspace)
        return SPECDEC_ERR_INVALID_ARGUMENT;
    if (d->gamma_max > 0 && !draft_tokens) return SPECDEC_ERR_INVALID_ARGUMENT;
    // sampling without draft rows: point-mass drafts of a deterministic proposer
    // (with gamma_max = 0 there is no draft row either way)
    const bool point = sample && !draft_logits && d->gamma_max > 0;
    const Layout L = make_layout(d, point);
    if (workspace_bytes < L.total) return SPECDEC_ERR_WORKSPACE_TOO_SMALL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (d->batch == 0) return SPECDEC_OK;
    if (clear_counters) {
        // the sections that must be zero at first use (arrival counters and
        // hand-off words) lie before the partials: one fill kernel
        const size_t n = L.off_part / 4;
        const unsigned grid = static_cast<unsigned>(std::min<size_t>((n + kThreads - 1) / kThreads, 1024));
        hipLaunchKernelGGL(k_zero_words, dim3(grid), dim3(kThreads), 0, stream,
                           static_cast<uint32_t*>(workspace), n);
        if (hipGetLastError() != hipSuccess) return SPECDEC_ERR_DEVICE;
    }

    VerifyParams P{};
    P.target = target_logits;
    P.draft = draft_logits;
    P.tokens = draft_tokens;
    P.gamma = gamma;
    P.max_tokens = max_tokens;
    P.accept_count = accept_count;
    P.num_tokens = num_tokens;
    P.out_tokens = out_tokens;
    P.p_draft = p_draft;
    P.q_draft = q_draft;
    P.residual_mass = residual_mass;
    P.flags = flags;
    char* ws = static_cast<char*>(workspace);
    P.cnt = reinterpret_cast<uint32_t*>(ws + L.off_cnt);
    P.ready = reinterpret_cast<uint64_t*>(ws + L.off_ready);
    P.cmass = reinterpret_cast<uint64_t*>(ws + L.off_cmass);
    P.part = reinterpret_cast<float4*>(ws + L.off_part);
    P.csum = reinterpret_cast<uint32_t*>(ws + L.off_csum);
    P.nuc = reinterpret_cast<uint2*>(ws + L.off_nuc);
    P.cut = reinterpret_cast<uint4*>(ws + L.off_nuc);
    P.top_k = d->top_k;
    P.top_p = d->top_p;
    P.B = d->batch;
    P.G = d->gamma_max;
    P.V = d->vocab;
    P.rows = L.rows;
    P.nc = L.nc;
    P.chunk = L.chunk;
    P.nc2 = L.nc2;
    P.chunk2 = L.chunk2;
    // sampling without truncation and greedy verification run as one kernel
    // unless SPECDEC_FUSED=0
    const bool fused = !L.trunc && fused_enabled();
    P.wpr = fused && sample ? L.fwpr : L.wpr;
    P.cpw = fused && sample ? L.fcpw : L.cpw;
    P.lag = fused_lag(d->batch);
    P.wait_ticks = fused_wait_ticks();
    P.c = sample ? static_cast<float>(1.4426950408889634 / static_cast<double>(d->temperature)) : 1.0f;
    P.key0 = static_cast<uint32_t>(d->seed & 0xffffffffu);
    P.key1 = static_cast<uint32_t>(d->seed >> 32);
    P.round = d->round;
    P.eos = d->eos_plus1 - 1;  // -1: none
    P.point = point;

    const bool bf16 = d->dtype == SPECDEC_BF16;
    const size_t es = bf16 ? 2 : 4;
    // Residual / bonus loads of the one-kernel sampling pass: ordinary loads
    // while the batch's row pairs (B x 2 x V) fit in kResidCachedBytes, so the last
    // workgroup's reload of the crossing chunk can hit the caches (headline
    // shape: 40.9 -> 40.1 us per call); streaming loads above that, where
    // lines kept from a re-read of hundreds of MB only delay the write-back
    // of what the following kernels write (B = 512 x V = 262144 round:
    // 618 -> 662 us per round with ordinary loads).
    P.resid_cached = static_cast<size_t>(d->batch) * 2 * static_cast<size_t>(d->vocab) * es <=
                     kResidCachedBytes;
    const bool vec = aligned16(target_logits) && (!sample || aligned16(draft_logits)) &&
                     (static_cast<size_t>(d->vocab) * es) % 16 == 0;
    if (L.cut) return bf16 ? (vec ? launch_cut<true, true>(d, P, L, stream, ev) : launch_cut<true, false>(d, P, L, stream, ev))
                           : (vec ? launch_cut<false, true>(d, P, L, stream, ev) : launch_cut<false, false>(d, P, L, stream, ev));
    if (L.trunc) return launch_truncated(P, bf16, vec, stream, ev);
    if (bf16)
        return vec ? launch_all<true, true>(d, P, L, fused, stream, ev)
                   : launch_all<true, false>(d, P, L, fused, stream, ev);
    return vec ? launch_all<false, true>(d, P, L, fused, stream, ev)
               : launch_all<false, false>(d, P, L, fused, stream, ev);
}

}  // namespace
}  // namespace specdec

using namespace specdec;

extern "C" size_t specdec_verify_workspace_bytes(const specdec_verify_desc_t* desc) {
    if (!valid_desc(desc)) return 0;
    // enough for draft rows and for point-mass drafts alike
    return std::max(make_layout(desc, false).total, make_layout(desc, true).total);
}

extern "C" specdec_status_t specdec_verify(const specdec_verify_desc_t* d,
                                           const void* target_logits, const void* draft_logits,
                                           const int32_t* draft_tokens, const int32_t* gamma,
                                           const int32_t* max_tokens, int32_t* accept_count,
                                           int32_t* num_tokens, int32_t* out_tokens,
                                           float* p_draft, float* q_draft, float* residual_mass,
                                           uint32_t* flags, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
    return verify_impl(d, target_logits, draft_logits, draft_tokens, gamma, max_tokens,
                       accept_count, num_tokens, out_tokens, p_draft, q_draft, residual_mass,
                       flags, workspace, workspace_bytes, stream, nullptr);
}

extern "C" specdec_status_t specdec_verify_profiled(
    const specdec_verify_desc_t* d, const void* target_logits, const void* draft_logits,
    const int32_t* draft_tokens, const int32_t* gamma, const int32_t* max_tokens,
    int32_t* accept_count, int32_t* num_tokens, int32_t* out_tokens, float* p_draft,
    float* q_draft, float* residual_mass, uint32_t* flags, void* workspace,
    size_t workspace_bytes, hipStream_t stream, hipEvent_t* stage_events) {
    return verify_impl(d, target_logits, draft_logits, draft_tokens, gamma, max_tokens,
                       accept_count, num_tokens, out_tokens, p_draft, q_draft, residual_mass,
                       flags, workspace, workspace_bytes, stream, stage_events);
}

extern "C" specdec_status_t specdec_verify_noalloc(
    const specdec_verify_desc_t* d, const void* target_logits, const void* draft_logits,
    const int32_t* draft_tokens, const int32_t* gamma, const int32_t* max_tokens,
    int32_t* accept_count, int32_t* num_tokens, int32_t* out_tokens, float* p_draft,
    float* q_draft, float* residual_mass, uint32_t* flags, hipStream_t stream) {
    if (!valid_desc(d)) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (specdec_verify_workspace_bytes(d) > kNoAllocBytes) return SPECDEC_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    const specdec_status_t st = noalloc_workspace(&ws);
    if (st != SPECDEC_OK) return st;
    // the array keeps the previous call's contents (maybe another layout):
    // its zero-at-first-use sections are cleared on the stream first
    return verify_impl(d, target_logits, draft_logits, draft_tokens, gamma, max_tokens,
                       accept_count, num_tokens, out_tokens, p_draft, q_draft, residual_mass,
                       flags, ws, kNoAllocBytes, stream, nullptr, true);
}
