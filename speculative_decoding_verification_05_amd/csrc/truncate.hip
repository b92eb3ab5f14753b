// Truncated sampling distributions (top-k, then top-p) for specdec_verify.
//
// p and q must be the distributions the two models actually sample from,
// after temperature and truncation, and the acceptance test and the residual
// use those filtered probabilities (AI-infra KB M013 s.04; the nxmr.cn note
// on lossless acceleration: processing such as top-p must show in p and q).
// Definition used (the pages leave the details open):
//   top-k: keep every token whose raw logit is >= the k-th largest raw logit
//          (ties at the boundary kept);
//   top-p: order the kept tokens by probability, i.e. raw logit, descending
//          and token index ascending; keep the shortest prefix whose
//          cumulative probability under softmax(z/T) over the top-k set
//          reaches top_p;
//   then p (or q) is softmax(z/T) restricted to, and renormalised over, what
//   is kept.  Target and draft rows are filtered independently.
//
// k_trunc_select  one 256-lane workgroup per used row, one streaming read of
//                 the row.  Each lane keeps the four largest of its
//                 per-vector maxima (the maximum of one 16-byte vector), each
//                 packed with its vector's number into one word: distinct
//                 elements of the row, so the k-th largest of these 1024
//                 values bounds the row's k-th largest logit from below, and
//                 every element at or above that bound lies in one of its
//                 lane's four tracked vectors (or the lane's fourth maximum
//                 reaches the bound while the lane has more vectors, and its
//                 whole share is read again).  Those vectors (one cache line
//                 each) are read again and their elements at or above the
//                 bound go to per-wave LDS regions: a few dozen of 128K
//                 tokens for the tested shapes.  One wave then ranks them by
//                 (logit desc, index asc), keeps the exact top-k set (ties kept) and the
//                 top-p prefix, and records the kept tokens sorted by index
//                 with their weights 2^((z - max) c) and the kept total
//                 (longer lists go through LDS bitonic sorts; lists past the
//                 LDS capacity through an exact bitwise search over re-reads).
// k_decide_trunc  one workgroup per request: p(d_i), q(d_i) from the records,
//                 the acceptance tests, m, then the inverse CDF of the
//                 residual (or bonus) over the short kept list in ascending
//                 token order, and every output of the request.
#include "verify_internal.h"

#include <hip/hip_ext.h>

#include <type_traits>


namespace specdec {
namespace {

constexpr int kSelCap = 2048;                 // LDS candidate slots per row
constexpr int kWaveCap = kSelCap / kWaves;   // each wave's region of them
static_assert(kTruncCap <= kSelCap, "a top-p-only row fits the candidate buffer whole");
constexpr uint32_t kRowOverflow = 1u << 16;   // record header: kept set clipped
constexpr uint32_t kRowNonfinite = 1u << 17;  // record header: NaN or +inf in the row

// Monotone map of a float to an unsigned key (larger float, larger key).
__device__ __forceinline__ uint32_t ordered_key(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// (z, i) precedes (z2, i2): larger logit first, then lower index.
__device__ __forceinline__ bool precedes(float z, int i, float z2, int i2) {
    return z > z2 || (z == z2 && i < i2);
}

__device__ __forceinline__ int block_count(int v) {
    __shared__ int s_w[kWaves];
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    v = wave_isum(v);
    __syncthreads();
    if (l == 0) s_w[w] = v;
    __syncthreads();
    int r = 0;
    for (int k = 0; k < kWaves; ++k) r += s_w[k];
    return r;
}

// Bitonic sort of n (a power of two) entries (z, i) in LDS into `precedes` order.
__device__ void bitonic_sort(float* z, int* id, int n) {
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int p = threadIdx.x; p < n / 2; p += kThreads) {
                const int a = ((p & ~(j - 1)) << 1) | (p & (j - 1)), c = a + j;  // j: a power of two
                const bool up = (a & k) == 0;
                const bool swap = up ? precedes(z[c], id[c], z[a], id[a])
                                     : precedes(z[a], id[a], z[c], id[c]);
                if (swap) {
                    const float tz = z[a]; z[a] = z[c]; z[c] = tz;
                    const int ti = id[a]; id[a] = id[c]; id[c] = ti;
                }
            }
            __syncthreads();
        }
    }
}

// Bitonic sort of n entries (i, e) in LDS by ascending i.
__device__ void bitonic_sort_index(int* id, float* e, int n) {
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int p = threadIdx.x; p < n / 2; p += kThreads) {
                const int a = ((p & ~(j - 1)) << 1) | (p & (j - 1)), c = a + j;  // j: a power of two
                const bool up = (a & k) == 0;
                const bool swap = up ? (id[c] < id[a]) : (id[a] < id[c]);
                if (swap) {
                    const int ti = id[a]; id[a] = id[c]; id[c] = ti;
                    const float te = e[a]; e[a] = e[c]; e[c] = te;
                }
            }
            __syncthreads();
        }
    }
}

__device__ __forceinline__ int pow2_at_least(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

__device__ __forceinline__ uint2* row_record(const VerifyParams& P, int b, int s) {
    return P.nuc + (static_cast<size_t>(b) * P.rows + s) * (1 + kNucCap);
}

// Appends the lanes' hits (x >= bound) of one element position to the LDS
// buffer: one LDS atomic per wave, slots in lane order.
__device__ __forceinline__ void append_hits(bool hit, float x, int e, float* bz, int* bi,
                                            int* count) {
    const uint64_t mask = __ballot(hit);
    if (!mask) return;
    const int l = threadIdx.x % kWave;
    int base = 0;
    if (l == __builtin_ctzll(mask)) base = atomicAdd(count, __popcll(mask));
    base = lane_value(base, __builtin_ctzll(mask));
    if (hit) {
        const int slot = base + __popcll(mask & ((1ull << l) - 1ull));
        if (slot < kSelCap) { bz[slot] = x; bi[slot] = e; }
    }
}

// Element q of a 16-byte vector of bf16 or fp32 logits, widened to float.
template <bool BF16>
__device__ __forceinline__ float elem(const uint4& r, int q) {
    if constexpr (BF16) {
        const uint32_t w = q < 2 ? r.x : q < 4 ? r.y : q < 6 ? r.z : r.w;
        return (q & 1) ? bf16_hi(w) : bf16_lo(w);
    } else {
        return __uint_as_float(q == 0 ? r.x : q == 1 ? r.y : q == 2 ? r.z : r.w);
    }
}

// The 16-byte vector holding the values of v (which came from such a vector,
// or are -inf).
template <bool BF16>
__device__ __forceinline__ uint4 narrow(const Vec<BF16>& v) {
    if constexpr (BF16) {
        auto pair = [&](int k) {
            return (__float_as_uint(v.x[k]) >> 16) | (__float_as_uint(v.x[k + 1]) & 0xffff0000u);
        };
        return make_uint4(pair(0), pair(2), pair(4), pair(6));
    } else {
        return make_uint4(__float_as_uint(v.x[0]), __float_as_uint(v.x[1]),
                          __float_as_uint(v.x[2]), __float_as_uint(v.x[3]));
    }
}

// The 16-byte vector of elements [e, e+N) of a row clipped to [.., V),
// -inf past V (load_vec's clamping, without widening).
template <bool BF16, bool VEC>
__device__ __forceinline__ uint4 load_raw(const void* rp, int e, int V) {
    if constexpr (VEC) {
        constexpr int N = Vec<BF16>::N;
        const uint4 w = *reinterpret_cast<const uint4*>(
            static_cast<const char*>(rp) + static_cast<size_t>(min(e, V - N)) * (BF16 ? 2 : 4));
        const uint32_t f = BF16 ? 0xff80ff80u : 0xff800000u;
        return e < V ? w : make_uint4(f, f, f, f);
    } else {
        return narrow<BF16>(load_vec<BF16, false>(rp, e, V, neg_inf()));
    }
}

// mag with the magnitude bits of a raw 16-byte vector folded in: per 16-bit
// half with a packed maximum (bf16), per word (fp32).  A half (word) above
// 0x7f80 (0x7f800000) afterwards means a NaN was seen.
template <bool BF16>
__device__ __forceinline__ uint32_t nan_mag(uint32_t mag, const uint4& r) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    if constexpr (BF16) {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        u16x2 a = __builtin_bit_cast(u16x2, mag);
#pragma unroll
        for (int j = 0; j < 4; ++j) a = __builtin_elementwise_max(a, __builtin_bit_cast(u16x2, w[j] & 0x7fff7fffu));
        return __builtin_bit_cast(uint32_t, a);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) mag = max(mag, w[j] & 0x7fffffffu);
        return mag;
    }
}

// One pass over a whole row in tiles of 256 lanes x kUnroll 16-byte vectors;
// f(r, t0) sees a lane's kUnroll raw vectors of the tile at t0 (vector u
// holds tokens t0 + (u * 256 + lane) * N ...), -inf past V.  VEC: every
// tile, the clipped last one included, goes through one pipeline (the next
// tile's loads in flight while the current one is visited) with addresses
// clamped into the row, so each byte of the row is fetched once; the last
// tile's vectors past V (wholly past it: V is a multiple of N) become -inf
// before its visit.  PEEL: every tile but the last is whole, so the loop
// issues the next tile's loads unconditionally and the last tile is visited
// after it (a load under a branch makes the compiler wait for every load in
// flight, the next tile's included, before each visit); the visit's code is
// then there twice, which costs registers.  Without PEEL one loop covers
// every tile, the next tile's loads under a branch.
template <bool BF16, bool VEC, bool PEEL, int NT = kThreads, class F>
__device__ __forceinline__ void stream_tiles(const void* rp, int V, F&& f) {
    constexpr int N = Vec<BF16>::N;
    constexpr int TILE = NT * N * kUnroll;
    const int t = threadIdx.x;
    if constexpr (VEC) {
        const int ntiles = (V + TILE - 1) / TILE;
        auto load_tile = [&](uint4 (&r)[kUnroll], int t0) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                r[u] = load16_stream<BF16>(rp, min(t0 + (u * NT + t) * N, V - N));
        };
        const uint32_t ninf = BF16 ? 0xff80ff80u : 0xff800000u;
        uint4 cur[kUnroll];
        load_tile(cur, 0);
        if constexpr (PEEL) {
            int t0 = 0;
            for (int k = 0; k + 1 < ntiles; ++k, t0 += TILE) {
                uint4 nxt[kUnroll];
                load_tile(nxt, t0 + TILE);
                f(cur, t0);
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) cur[u] = nxt[u];
            }
            if (t0 + TILE > V) {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    if (t0 + (u * NT + t) * N >= V) cur[u] = make_uint4(ninf, ninf, ninf, ninf);
            }
            f(cur, t0);
        } else {
            for (int k = 0; k < ntiles; ++k) {
                const int t0 = k * TILE;
                uint4 nxt[kUnroll];
                if (k + 1 < ntiles) load_tile(nxt, t0 + TILE);
                if (t0 + TILE > V) {
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u)
                        if (t0 + (u * NT + t) * N >= V) cur[u] = make_uint4(ninf, ninf, ninf, ninf);
                }
                f(cur, t0);
                if (k + 1 < ntiles) {
#pragma unroll
                    for (int u = 0; u < kUnroll; ++u) cur[u] = nxt[u];
                }
            }
        }
    } else {
        for (int t0 = 0; t0 < V; t0 += TILE) {
            uint4 r[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                r[u] = narrow<BF16>(load_vec<BF16, false>(rp, t0 + (u * NT + t) * N, V, neg_inf()));
            f(r, t0);
        }
    }
}

// Candidates s_z/s_i[0..C), C <= 64, to the kept-token record, by one wave:
// each candidate's rank by (logit desc, index asc) and by index, counted
// against every other candidate read by broadcast from LDS (no sorting
// network), a prefix of the weights in rank order the same way, and the kept
// tokens placed by index rank.  s_z/s_i[64..192) serve as scratch.
__device__ void select_in_wave(const VerifyParams& P, int b, int s, int C, bool use_k,
                               float* s_z, int* s_i, uint32_t rowflags) {
    const int l = threadIdx.x % kWave;
    const bool in = l < C;
    const float z = in ? s_z[l] : neg_inf();
    const int id = in ? s_i[l] : 0x7fffffff;
    // sentinels past C, which precede nothing: whole float4 reads, no checks
    if (l < 4) {
        s_z[C + l] = neg_inf();
        s_i[C + l] = 0x7fffffff;
    }
    int rank = 0, lower = 0;
#pragma unroll 4
    for (int j0 = 0; j0 < C; j0 += 4) {
        const float4 zj = *reinterpret_cast<const float4*>(s_z + j0);
        const int4 ij = *reinterpret_cast<const int4*>(s_i + j0);
        const float zz[4] = {zj.x, zj.y, zj.z, zj.w};
        const int ii[4] = {ij.x, ij.y, ij.z, ij.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            rank += static_cast<int>((zz[k] > z) | ((zz[k] == z) & (ii[k] < id)));
            lower += static_cast<int>(ii[k] < id);
        }
    }
    auto lane_of = [&](bool pred) { return __builtin_ctzll(__ballot(pred)); };
    int K = C;
    if (use_k && P.top_k <= C) {
        const float tau = lane_value(z, lane_of(in && rank == P.top_k - 1));
        K = __popcll(__ballot(in && z >= tau));
    }
    const float M = lane_value(z, lane_of(in && rank == 0));
    const float e = in && rank < K ? exp2f((z - M) * P.c) : 0.0f;
    // inclusive prefix of the weights in rank order, summed in candidate
    // order (monotone in rank: every term is non-negative)
    float* s_e = s_z + 2 * kWave;
    int* s_r = s_i + 2 * kWave;
    s_e[l] = e;
    s_r[l] = in ? rank : 0x7fffffff;
    float pre = 0.0f;
#pragma unroll 4
    for (int j0 = 0; j0 < C; j0 += 4) {
        const float4 ej = *reinterpret_cast<const float4*>(s_e + j0);
        const int4 rj = *reinterpret_cast<const int4*>(s_r + j0);
        pre += rj.x <= rank ? ej.x : 0.0f;
        pre += rj.y <= rank ? ej.y : 0.0f;
        pre += rj.z <= rank ? ej.z : 0.0f;
        pre += rj.w <= rank ? ej.w : 0.0f;
    }
    int Nk = K;
    if (P.top_p < 1.0f) {
        const float goal = P.top_p * lane_value(pre, lane_of(in && rank == K - 1));
        Nk = min(K, static_cast<int>(__popcll(__ballot(in && rank < K && pre < goal))) + 1);
    }
    const float Sn = lane_value(pre, lane_of(in && rank == Nk - 1));
    // the kept tokens by ascending index: every candidate at its index rank,
    // then the kept ones compacted in that order
    const bool kept = in && rank < Nk;
    if (in) {
        s_i[kWave + lower] = kept ? id : -1;
        s_z[kWave + lower] = e;
    }
    const int id2 = in ? s_i[kWave + l] : -1;
    const float e2 = in ? s_z[kWave + l] : 0.0f;
    const uint64_t km = __ballot(id2 >= 0);
    uint2* rec = row_record(P, b, s);
    if (id2 >= 0)
        rec[1 + __popcll(km & ((1ull << l) - 1ull))] = make_uint2(static_cast<uint32_t>(id2), __float_as_uint(e2));
    if (l == 0) rec[0] = make_uint2(static_cast<uint32_t>(Nk) | rowflags, __float_as_uint(Sn));
}

// Inverse of ordered_key, clamped to -inf below the key of -inf (never a NaN).
__device__ __forceinline__ float key_value(uint32_t key) {
    if (key < 0x007fffffu) return neg_inf();
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void k_trunc_select(VerifyParams P) {
    __shared__ __align__(16) float s_z[kSelCap];
    __shared__ __align__(16) int s_i[kSelCap];
    __shared__ float s_wt[kWaves];
    __shared__ int s_count, s_cut;
    __shared__ int s_cw[kWaves];
    __shared__ uint32_t s_hist[kThreads];
    __shared__ int s_sel[3];
    constexpr int N = Vec<BF16>::N;
    constexpr int TILE = kThreads * N * kUnroll;
    const int s = blockIdx.x, b = blockIdx.y;
    const bool is_target = s <= P.G;
    const int i = is_target ? s : s - (P.G + 1);
    const int g = request_gamma(P, b);
    if (is_target ? (i > g) : (i >= g)) return;  // padding row
    const void* rp = is_target ? target_row(P, b, i, BF16) : draft_row(P, b, i, BF16);
    const int V = P.V;
    const int t = threadIdx.x, w = t / kWave, l = t % kWave;
    const uint64_t below = (1ull << l) - 1ull;
    const bool use_k = P.top_k > 0 && P.top_k < V;

    // (1) the one read.  Per lane, the four largest of its per-vector maxima,
    // each packed with its vector's unit number (tile * kUnroll + u) into one
    // word: the top 16 bits of the maximum's order-preserving key (-0 taken
    // as +0), then the unit.  Cutting a key's low bits only lowers the value
    // it stands for (a widened bf16 loses nothing when positive).  The units
    // hold distinct elements of the row.  0: no unit.
    uint32_t k1 = 0u, k2 = 0u, k3 = 0u, k4 = 0u;
    // NaNs: the lane's largest magnitude bits per 16-bit half (bf16) or per
    // word (fp32); a NaN's exceed +inf's.  The tail's -inf does not.
    uint32_t mag = 0;
    auto visit = [&](const uint4 (&r)[kUnroll], int t0) {
        const uint32_t unit0 = static_cast<uint32_t>(t0 / TILE) * kUnroll;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float m = neg_inf();  // the tail is filled with -inf; NaNs are skipped
#pragma unroll
            for (int q = 0; q < N; ++q) m = fmaxf(m, elem<BF16>(r[u], q));
            mag = nan_mag<BF16>(mag, r[u]);
            const uint32_t key = (ordered_key(m + 0.0f) & 0xffff0000u) | (unit0 + u);
            k4 = max(k4, min(key, k3));
            k3 = max(k3, min(key, k2));
            k2 = max(k2, min(key, k1));
            k1 = max(k1, key);
        }
    };
    stream_tiles<BF16, VEC, true>(rp, V, visit);
    const bool lane_nan = BF16 ? ((mag & 0xffffu) > 0x7f80u || (mag >> 16) > 0x7f80u) : mag > 0x7f800000u;
    // wave-uniform: a NaN or a +inf (key 0xff80....) was seen
    const uint64_t bad = __ballot(lane_nan || (k1 >> 16) >= 0xff80u);

    // (2) the bound: the k-th largest of the 4 x 256 tracked keys, a lower
    // bound on the row's k-th largest logit.  Radix select over the keys'
    // top 16 bits, 8 a round from the top: an LDS histogram of the digit
    // among the keys that share the digits chosen so far, then one wave
    // scans the bins from the top for the one where the running count
    // reaches k.
    uint32_t bkey = 0u;  // no bound: every unit reaches
    if (t == 0) s_count = 0;
    if (use_k) {
        const uint32_t kk[4] = {k1 & 0xffff0000u, k2 & 0xffff0000u, k3 & 0xffff0000u, k4 & 0xffff0000u};
        uint32_t prefix = 0;
        int need = P.top_k;
        bool found = true;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int shift = 24 - 8 * r;
            s_hist[t] = 0u;  // kThreads == 256 bins
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool same = r == 0 || (kk[j] >> (shift + 8)) == (prefix >> (shift + 8));
                if (same) atomicAdd(&s_hist[(kk[j] >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (w == 0) {
                // lane l holds bins 255-4l .. 252-4l (descending)
                int cnt[4];
                int tot = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    cnt[q] = static_cast<int>(s_hist[255 - 4 * l - q]);
                    tot += cnt[q];
                }
                const int incl = wave_scan(tot, 0, [](int x, int y) { return x + y; });
                const int excl = incl - tot;
                const uint64_t hit = __ballot(incl >= need);
                if (hit) {
                    const int src = __builtin_ctzll(hit);
                    int digit = 0, rest = 0;
                    if (l == src) {
                        int run = excl;
                        for (int q = 0; q < 4; ++q) {
                            if (run + cnt[q] >= need) { digit = 255 - 4 * l - q; rest = need - run; break; }
                            run += cnt[q];
                        }
                    }
                    if (l == src) { s_sel[0] = digit; s_sel[1] = rest; s_sel[2] = 1; }
                } else if (l == 0) {
                    s_sel[2] = 0;  // fewer than k keys share the prefix: no finite bound
                }
            }
            __syncthreads();
            if (!s_sel[2]) { found = false; break; }
            prefix |= static_cast<uint32_t>(s_sel[0]) << shift;
            need = s_sel[1];
        }
        bkey = found ? prefix : 0u;
    }
    const float bound = key_value(bkey);  // -inf when there is no bound
    __syncthreads();

    // (3) every element at or above the bound lies in a vector whose maximum
    // reaches it, so in one of the lane's four tracked vectors unless the
    // fourth reaches it too and the lane has other vectors (more than one
    // tile): then its whole share is read again by its wave.  Otherwise the
    // reaching tracked vectors are read again (one batch of loads) and their
    // elements >= bound appended to the wave's own LDS region (a
    // wave-uniform count, no atomics).
    float* zw = s_z + w * kWaveCap;
    int* iw = s_i + w * kWaveCap;
    int c = 0;
    auto append = [&](bool h, float x, int e) {
        const uint64_t mask = __ballot(h);
        if (!mask) return;
        const int slot = c + __popcll(mask & below);
        if (h && slot < kWaveCap) {
            zw[slot] = x;
            iw[slot] = e;
        }
        c += __popcll(mask);
    };
    const int ntiles = (V + TILE - 1) / TILE;
    auto reach = [&](uint32_t k) { return k != 0u && k >= bkey; };
    const bool all = ntiles > 1 && reach(k4);
    const uint32_t kt[4] = {k1, k2, k3, k4};
    int ue[4];  // first element of each vector to read again, or -1
    int nt = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int unit = static_cast<int>(kt[j] & 0xffffu);
        ue[j] = reach(kt[j]) && !all ? (unit / kUnroll) * TILE + ((unit % kUnroll) * kThreads + t) * N : -1;
        if (__ballot(ue[j] >= 0)) nt = j + 1;
    }
    if (nt > 0) {
        uint4 rv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j >= nt) break;
            // only lanes with a vector to read load (the others' loads are
            // masked off; their address stays inside the row all the same)
            rv[j] = ue[j] >= 0 ? load_raw<BF16, VEC>(rp, max(ue[j], 0), V) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j >= nt) break;
#pragma unroll
            for (int q = 0; q < N; ++q) {
                const int e = ue[j] + q;
                const float x = elem<BF16>(rv[j], q);
                append(ue[j] >= 0 && e < V && x >= bound, x, e);
            }
        }
    }
    {
        // whole-share re-reads, one lane at a time: lane l reads tiles l, l + 64, ...
        uint64_t heavy = __ballot(all);
        while (heavy) {
            const int L = __builtin_ctzll(heavy);
            heavy &= heavy - 1ull;
            const int lane = t - l + L;  // the heavy lane's thread index
            for (int tile0 = 0; tile0 < ntiles; tile0 += kWave) {
                const int tile = tile0 + l;
                const int base = min(tile, ntiles - 1) * TILE;
                uint4 v[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    v[u] = tile < ntiles ? load_raw<BF16, VEC>(rp, base + (u * kThreads + lane) * N, V)
                                         : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                    for (int q = 0; q < N; ++q) {
                        const int e = base + (u * kThreads + lane) * N + q;
                        const float x = elem<BF16>(v[u], q);
                        append(tile < ntiles && e < V && x >= bound, x, e);
                    }
            }
        }
    }
    if (l == 0) s_cw[w] = c;
    uint32_t rowflags = 0;
    if (__syncthreads_or(bad != 0)) rowflags = kRowNonfinite;
    int C = 0;
    bool spill = false;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
        const int cq = s_cw[q];
        C += cq;
        spill |= cq > kWaveCap;
    }
    if (spill) C = kSelCap + 1;
    // wave 0 moves the wave regions' entries together into s_z/s_i[0..C)
    // (every destination at or before its source, each chunk read before
    // any of it is written)
    auto gather = [&]() {
        int dst = 0;
        for (int q = 0; q < kWaves; ++q) {
            const int cq = s_cw[q];
            for (int j0 = 0; j0 < cq; j0 += kWave) {
                const int p = j0 + l;
                const bool in = p < cq;
                const float zv = in ? s_z[q * kWaveCap + p] : 0.0f;
                const int iv = in ? s_i[q * kWaveCap + p] : 0;
                if (in) {
                    s_z[dst + l] = zv;
                    s_i[dst + l] = iv;
                }
                dst += min(kWave, cq - j0);
            }
        }
    };
    bool packed = false;

    if (C > kSelCap) {
        // Overflow (heavy ties, or very flat rows with a large k): the exact
        // k-th largest value by a bitwise search on ordered keys (largest key
        // t with count(key >= t) >= k), each step one read of the row, then
        // the buffer is refilled with the elements at or above it.  Without
        // an effective top-k every element is a candidate (key 0 keeps all
        // but NaNs; such rows have V <= kTruncCap <= kSelCap).
        uint32_t key = 0;
        for (int bit = 31; use_k && bit >= 0; --bit) {
            const uint32_t trial = key | (1u << bit);
            int cnt = 0;
            for (int e0 = t * N; e0 < V; e0 += kThreads * N) {
                const Vec<BF16> v = load_vec<BF16, VEC>(rp, e0, V, neg_inf());
#pragma unroll
                for (int k = 0; k < N; ++k)
                    cnt += (e0 + k < V) && (v.x[k] == v.x[k]) && ordered_key(v.x[k]) >= trial;
            }
            if (block_count(cnt) >= (use_k ? P.top_k : 1)) key = trial;
        }
        if (t == 0) s_count = 0;
        __syncthreads();
        for (int e0 = 0; e0 < V; e0 += kThreads * N) {
            const int e = e0 + t * N;
            const Vec<BF16> v = load_vec<BF16, VEC>(rp, e, V, neg_inf());
#pragma unroll
            for (int k = 0; k < N; ++k) {
                const float x = v.x[k];
                append_hits(e + k < V && (x == x) && ordered_key(x) >= key, x, e + k, s_z, s_i, &s_count);
            }
        }
        __syncthreads();
        C = s_count;
        if (C > kSelCap) { rowflags |= kRowOverflow; C = kSelCap; }
        packed = true;
    }
    if (C <= kWave) {
        // The usual case: one wave finishes the row (no barriers).
        if (t >= kWave) return;
        if (!packed) gather();
        select_in_wave(P, b, s, C, use_k, s_z, s_i, rowflags);
        return;
    }
    if (!packed) {
        if (t < kWave) gather();
        __syncthreads();
    }
    const int n = pow2_at_least(C < 2 ? 2 : C);
    for (int p = C + t; p < n; p += kThreads) { s_z[p] = neg_inf(); s_i[p] = 0x7fffffff; }
    __syncthreads();

    // (3) sorted by (logit desc, index asc); the exact top-k set is a prefix
    bitonic_sort(s_z, s_i, n);
    int K = C;
    if (use_k && P.top_k <= C) {
        const float tau = s_z[P.top_k - 1];
        int c = 0;
        for (int p = t; p < C; p += kThreads) c += s_z[p] >= tau;
        K = block_count(c);
    }
    const float M = s_z[0];
    const float cc = P.c;

    // (4) top-p: the shortest prefix whose weight reaches top_p of the top-k weight
    int Nk = K;
    float part = 0.0f;
    for (int p = t; p < K; p += kThreads) part += exp2f((s_z[p] - M) * cc);
    float Sn = block_sum(part);
    if (P.top_p < 1.0f) {
        const float goal = P.top_p * Sn;
        const int w = t / kWave, l = t % kWave;
        if (t == 0) s_cut = K - 1;
        __syncthreads();
        float carry = 0.0f;
        for (int base = 0; base < K; base += kThreads) {
            const int p = base + t;
            float x = p < K ? exp2f((s_z[p] - M) * cc) : 0.0f;
            x = wave_prefix_sum(x);
            __syncthreads();
            if (l == kWave - 1) s_wt[w] = x;
            __syncthreads();
            float off = carry, tot = carry;
            for (int k = 0; k < kWaves; ++k) {
                if (k < w) off += s_wt[k];
                tot += s_wt[k];
            }
            const uint64_t mask = __ballot(p < K && off + x >= goal);
            if (l == 0 && mask) atomicMin(&s_cut, base + w * kWave + __builtin_ctzll(mask));
            carry = tot;
            __syncthreads();
            if (s_cut < K - 1) break;
        }
        Nk = s_cut + 1;
        part = 0.0f;
        for (int p = t; p < Nk; p += kThreads) part += exp2f((s_z[p] - M) * cc);
        Sn = block_sum(part);
    }
    if (Nk > kNucCap) { Nk = kNucCap; rowflags |= kRowOverflow; }

    // (5) the kept tokens by ascending index, with their weights
    __syncthreads();
    float* s_e = s_z;  // weights replace logits in place
    for (int p = t; p < Nk; p += kThreads) s_e[p] = exp2f((s_z[p] - M) * cc);
    const int n2 = pow2_at_least(Nk < 2 ? 2 : Nk);
    for (int p = Nk + t; p < n2; p += kThreads) { s_i[p] = 0x7fffffff; s_e[p] = 0.0f; }
    __syncthreads();
    bitonic_sort_index(s_i, s_e, n2);
    uint2* rec = row_record(P, b, s);
    for (int p = t; p < Nk; p += kThreads)
        rec[1 + p] = make_uint2(static_cast<uint32_t>(s_i[p]), __float_as_uint(s_e[p]));
    if (t == 0) rec[0] = make_uint2(static_cast<uint32_t>(Nk) | rowflags, __float_as_uint(Sn));
}

// ------------------------------------------------------------------ decision

// Weight of token d in a record (0 if not kept), searched by a whole wave.
__device__ __forceinline__ float record_weight(const uint2* rec, int n, int d) {
    const int l = threadIdx.x % kWave;
    float e = 0.0f;
    for (int base = 0; base < n; base += kWave) {
        const int p = base + l;
        const uint2 ent = p < n ? rec[1 + p] : make_uint2(0xffffffffu, 0u);
        const bool hit = static_cast<int>(ent.x) == d;
        const uint64_t mask = __ballot(hit);
        if (mask) {
            e = lane_value(__uint_as_float(ent.y), __builtin_ctzll(mask));
            break;
        }
    }
    return e;
}

__global__ __launch_bounds__(kThreads) void k_decide_trunc(VerifyParams P) {
    __shared__ uint32_t s_n[127];
    __shared__ float s_S[127];
    __shared__ float s_p[64], s_q[64];
    __shared__ int s_d[64], s_acc[64];
    __shared__ int s_pi[kNucCap];
    __shared__ float s_pe[kNucCap];
    __shared__ int s_qi[kNucCap];
    __shared__ float s_qe[kNucCap];
    __shared__ float s_wt[kWaves];
    __shared__ int s_found, s_last, s_m;
    __shared__ uint32_t s_fl;
    const int b = blockIdx.x;
    const int t = threadIdx.x, w = t / kWave, l = t % kWave;
    const int g = request_gamma(P, b);

    // record headers of the used rows
    if (t == 0) s_fl = gamma_flag(P, b);
    __syncthreads();
    for (int s = t; s < P.rows; s += kThreads) {
        const bool used = (s <= P.G) ? (s <= g) : (s - (P.G + 1) < g);
        if (!used) continue;
        const uint2 h = row_record(P, b, s)[0];
        s_n[s] = h.x & 0xffffu;
        s_S[s] = __uint_as_float(h.y);
        uint32_t f = 0;
        if (h.x & kRowNonfinite) f |= SPECDEC_FLAG_NONFINITE;
        if (h.x & kRowOverflow) f |= SPECDEC_FLAG_TRUNC_OVERFLOW;
        if (f) atomicOr(&s_fl, f);
    }
    __syncthreads();

    // acceptance tests, one wave per position
    for (int i = w; i < g; i += kWaves) {
        const int d = P.tokens[static_cast<size_t>(b) * P.G + i];
        float pd = 0.0f, qd = 0.0f;
        bool in_range = d >= 0 && d < P.V;
        if (in_range) {
            const int st = i, sq = P.G + 1 + i;
            pd = record_weight(row_record(P, b, st), static_cast<int>(s_n[st]), d) / s_S[st];
            qd = record_weight(row_record(P, b, sq), static_cast<int>(s_n[sq]), d) / s_S[sq];
        }
        if (l == 0) {
            float a = 0.0f;
            if (in_range) {
                if (qd > 0.0f) a = fminf(1.0f, pd / qd);
                else a = pd > 0.0f ? 1.0f : 0.0f;
            } else {
                atomicOr(&s_fl, SPECDEC_FLAG_TOKEN_RANGE);
            }
            const uint4 r = philox4x32_10(make_uint4(static_cast<uint32_t>(i), static_cast<uint32_t>(b),
                                                     P.round, 0u), P.key0, P.key1);
            s_p[i] = pd;
            s_q[i] = qd;
            s_d[i] = d;
            s_acc[i] = uniform24(r.x) < a;
        }
    }
    __syncthreads();
    if (t == 0) {
        int m = 0;
        while (m < g && s_acc[m]) ++m;
        s_m = m;
    }
    __syncthreads();
    const int m = s_m;
    const bool resid = m < g;

    // the sampling list: kept tokens of target row m (ascending index), and
    // of draft row m for the residual
    const int np = static_cast<int>(s_n[m]);
    const float Sp = s_S[m];
    const uint2* rp = row_record(P, b, m);
    for (int p = t; p < np; p += kThreads) {
        const uint2 ent = rp[1 + p];
        s_pi[p] = static_cast<int>(ent.x);
        s_pe[p] = __uint_as_float(ent.y);
    }
    int nq = 0;
    float Sq = 1.0f;
    if (resid) {
        nq = static_cast<int>(s_n[P.G + 1 + m]);
        Sq = s_S[P.G + 1 + m];
        const uint2* rq = row_record(P, b, P.G + 1 + m);
        for (int p = t; p < nq; p += kThreads) {
            const uint2 ent = rq[1 + p];
            s_qi[p] = static_cast<int>(ent.x);
            s_qe[p] = __uint_as_float(ent.y);
        }
    }
    __syncthreads();
    // mass of list entry p: max(p - q, 0) (q found by binary search), or p
    auto mass = [&](int p, bool with_q) -> float {
        const float pv = s_pe[p] / Sp;
        if (!with_q) return pv;
        const int v = s_pi[p];
        int lo = 0, hi = nq;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_qi[mid] < v) lo = mid + 1; else hi = mid;
        }
        const float qv = (lo < nq && s_qi[lo] == v) ? s_qe[lo] / Sq : 0.0f;
        return fmaxf(pv - qv, 0.0f);
    };
    bool with_q = resid;
    float part = 0.0f;
    for (int p = t; p < np; p += kThreads) part += mass(p, with_q);
    float R = block_sum(part);
    const float R_report = resid ? R : 0.0f;
    uint32_t fl2 = 0;
    if (resid && !(R > 0.0f)) {
        // empty residual: draw from p_m instead (never divide by zero)
        fl2 |= SPECDEC_FLAG_RESIDUAL_FALLBACK;
        with_q = false;
        part = 0.0f;
        for (int p = t; p < np; p += kThreads) part += mass(p, false);
        R = block_sum(part);
    }
    const uint4 rnd = philox4x32_10(make_uint4(static_cast<uint32_t>(m), static_cast<uint32_t>(b),
                                               P.round, 0u), P.key0, P.key1);
    const float target = uniform24(rnd.y) * R;

    // inverse CDF over the list in ascending token order
    if (t == 0) { s_found = 0x7fffffff; s_last = -1; }
    __syncthreads();
    float carry = 0.0f;
    for (int base = 0; base < np; base += kThreads) {
        const int p = base + t;
        const float r = p < np ? mass(p, with_q) : 0.0f;
        float x = r;
        x = wave_prefix_sum(x);
        __syncthreads();
        if (l == kWave - 1) s_wt[w] = x;
        __syncthreads();
        float off = carry, tot = carry;
        for (int k = 0; k < kWaves; ++k) {
            if (k < w) off += s_wt[k];
            tot += s_wt[k];
        }
        const uint64_t cross = __ballot(p < np && off + x > target);
        const uint64_t pos = __ballot(p < np && r > 0.0f);
        if (l == 0 && cross) atomicMin(&s_found, base + w * kWave + __builtin_ctzll(cross));
        if (l == 0 && pos) atomicMax(&s_last, base + w * kWave + 63 - __builtin_clzll(pos));
        carry = tot;
        __syncthreads();
        if (s_found != 0x7fffffff) break;
    }
    __syncthreads();
    const int pick = s_found != 0x7fffffff ? s_found : s_last;
    const int token = pick >= 0 ? s_pi[pick] : -1;

    if (w == 0) {
        const int i = l;
        fl2 |= write_round(P, b, m, i < m ? s_d[i] : token);
        if (i < P.G) {
            if (P.p_draft) P.p_draft[static_cast<size_t>(b) * P.G + i] = i < g ? s_p[i] : 0.0f;
            if (P.q_draft) P.q_draft[static_cast<size_t>(b) * P.G + i] = i < g ? s_q[i] : 0.0f;
        }
        if (i == 0) {
            if (P.residual_mass) P.residual_mass[b] = R_report;
            if (P.flags) P.flags[b] = s_fl | fl2;
        }
    }
}

// ------------------------------------------------------------------ cut records
// Top-p without an effective top-k, or a top-k past kNucCap: the kept set can
// hold most of the row, so it is not listed.  The kept tokens are the first
// Nk in (logit desc, index asc) order, i.e. the set
//   { v : z_v > tau } + { v : z_v == tau and v <= iota }
// for the logit tau and index iota of the Nk-th (iota = INT_MAX when every
// token at tau is kept).  k_trunc_cut finds (tau, iota) and the kept mass of
// each used row; the sampling decision (decide_sample in its cut mode) tests
// membership element by element as it reads the rows.
//
// The search is a radix select over order-preserving keys of the logits
// (-0 taken as +0, so that equal logits have equal keys; a bf16 logit's key
// is its 16-bit pattern's, in the top half): a 12-bit digit histogram over
// the whole row, then histograms of the next digit over the chosen bin only,
// down to exact values (bf16: 12 + 4 bits; fp32: 12 + 12 + 8).  top-k counts
// elements; top-p weighs them by 2^((z - max) c) held as integers of 2^-40,
// so every sum is exact and the same whatever order the lanes add in, and a
// value's weight in the last digit is its count times its one element weight.
// An element whose weight is below 2^-40 of the row's largest counts as 0: a
// relative error below V * 2^-40 of the kept mass.  The last digit's pass
// also counts each value per segment of the row, so the tie index iota is
// found by reading one segment again.
constexpr int kCutBins = 4096;  // 12-bit digits
constexpr int kCutSegs = 8192;  // last digit: values x segments of tie counters
constexpr float kFix = 1099511627776.0f;  // 2^40

template <bool BF16>
__device__ __forceinline__ uint32_t cut_key(float x) {
    const uint32_t k = ordered_key(x + 0.0f);  // -0 + 0 = +0
    return BF16 ? (k & 0xffff0000u) : k;
}

// The logit whose key is k (k from cut_key).
template <bool BF16>
__device__ __forceinline__ float cut_value(uint32_t k) {
    if constexpr (BF16) {
        const uint32_t h = k >> 16;
        const uint32_t u = (h & 0x8000u) ? (h & 0x7fffu) : (~h & 0xffffu);
        return __uint_as_float(u << 16);
    } else {
        return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
    }
}

__device__ __forceinline__ unsigned long long fixed_weight(float x, float M, float c) {
    return static_cast<unsigned long long>(__builtin_amdgcn_exp2f((x - M) * c) * kFix);
}

// Digit d of the keys: bits [shift, shift + width).
template <bool BF16>
__device__ __forceinline__ int digit_shift(int d) { return d == 0 ? 20 : BF16 ? 16 : (d == 1 ? 8 : 0); }
template <bool BF16>
__device__ __forceinline__ int digit_width(int d) { return d == 0 ? 12 : BF16 ? 4 : (d == 1 ? 12 : 8); }

struct Cross {
    int bin;                   // -1: base plus the bins' total stays below the goal
    unsigned long long above;  // base plus the weight of the bins past it
    unsigned long long total;  // base plus the weight of all the bins
};

// Bins [0, n) read from the top (n a power of two <= kCutBins, weights w(j)),
// after `base` (the weight already above them): the highest bin j with
// base + above(j) < goal <= base + above(j) + w(j), above(j) being the
// weight of the bins past j.  Every test compares an exact integer sum with
// the goal the same way, so successive searches agree at their edges.
// Thread t < kThreads sums a run of consecutive bins from the top into
// s_run[t] (kThreads entries of LDS; larger workgroups leave their other
// lanes out), wave 0 scans the runs four to a lane, and the crossing lane
// walks its runs and then bins.
template <class W>
__device__ Cross find_cross(int n, double goal, unsigned long long base, unsigned long long* s_run, W&& w) {
    __shared__ Cross s_res;
    const int t = threadIdx.x, l = t % kWave;
    const int per = n >= kThreads ? n / kThreads : 1;
    const int nthr = n / per;
    unsigned long long run = 0;
    if (t < nthr)
        for (int k = 0; k < per; ++k) run += w(n - 1 - (t * per + k));
    if (t < kThreads) s_run[t] = run;
    __syncthreads();
    if (t < kWave) {
        const unsigned long long q = s_run[4 * l] + s_run[4 * l + 1] + s_run[4 * l + 2] + s_run[4 * l + 3];
        unsigned long long incl = q;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const unsigned long long o = __shfl_up(incl, d);
            if (l >= d) incl += o;
        }
        const unsigned long long total = base + __shfl(incl, kWave - 1);
        const uint64_t hit = __ballot(static_cast<double>(base + incl) >= goal);
        if (!hit) {
            if (l == 0) s_res = Cross{-1, total, total};
        } else if (l == static_cast<int>(__builtin_ctzll(hit))) {
            unsigned long long above = base + incl - q;
            int j = -1;
            for (int r = 4 * l; r < 4 * l + 4 && j < 0; ++r) {
                if (static_cast<double>(above + s_run[r]) < goal) {
                    above += s_run[r];
                    continue;
                }
                for (int k = 0; k < per; ++k) {
                    const int bin = n - 1 - (r * per + k);
                    const unsigned long long x = w(bin);
                    if (static_cast<double>(above + x) >= goal) {
                        j = bin;
                        break;
                    }
                    above += x;
                }
            }
            s_res = Cross{j, above, total};
        }
    }
    __syncthreads();
    const Cross r = s_res;
    __syncthreads();  // s_run and s_res serve the next call
    return r;
}

// Exclusive prefix sum over the workgroup's lanes (NW waves) in thread
// order; *total receives the sum (same on every lane).
template <int NW = kWaves>
__device__ __forceinline__ int block_excl_scan(int v, int* total) {
    __shared__ int s_w[NW];
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    const int incl = wave_scan(v, 0, [](int x, int y) { return x + y; });
    __syncthreads();
    if (l == kWave - 1) s_w[w] = incl;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        if (k < w) off += s_w[k];
        tot += s_w[k];
    }
    *total = tot;
    return off + incl - v;
}

// 512 lanes per row: one workgroup per row leaves about two rows per CU on
// the tested batches, and with 256 lanes the passes were bound by latency
// (too few loads in flight and waves to hide the arithmetic): 130 us against
// 113 us at 512 lanes and 146 us at 1024 (B=64 x V=128256, top-p 0.9).
constexpr int kCutThreads = 512;

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kCutThreads) void k_trunc_cut(VerifyParams P) {
    constexpr int NT = kCutThreads;
    // one buffer for each pass's histogram: top-k counts (uint32), top-p
    // weights (uint64), or the last digit's tie counters (uint32)
    __shared__ unsigned long long s_buf[kCutBins];
    __shared__ uint32_t s_vcnt[256];  // the last top-p digit: count per value
    __shared__ unsigned long long s_run[kThreads];
    __shared__ float s_ms[2];
    __shared__ int s_tie;
    constexpr int N = Vec<BF16>::N;
    constexpr int TILE = NT * N * kUnroll;
    constexpr int NDIG = BF16 ? 2 : 3;
    const int s = blockIdx.x, b = blockIdx.y;
    const bool is_target = s <= P.G;
    const int i = is_target ? s : s - (P.G + 1);
    const int g = request_gamma(P, b);
    if (is_target ? (i > g) : (i >= g)) return;  // padding row
    const void* rp = is_target ? target_row(P, b, i, BF16) : draft_row(P, b, i, BF16);
    const int V = P.V, t = threadIdx.x;
    const float c = P.c;
    uint4* rec = P.cut + static_cast<size_t>(b) * P.rows + s;

    // (0) the row's (max, sum) from its statistics partials
    if (t < kWave) {
        MaxSum acc{neg_inf(), 0.0f};
        const float4* part = P.part + (static_cast<size_t>(b) * P.rows + s) * P.nc;
        for (int k = t; k < P.nc; k += kWave) {
            const float4 q = part[k];
            acc = combine(acc, MaxSum{q.x, q.y}, c);
        }
        acc = wave_combine(acc, c);
        if (t == 0) { s_ms[0] = acc.m; s_ms[1] = acc.s; }
    }
    __syncthreads();
    const float M = s_ms[0];
    if (!(M < pos_inf()) || !(M > neg_inf()) || !(s_ms[1] == s_ms[1])) {
        // a NaN or +inf in the row, or nothing but -inf: the decision flags it
        if (t == 0)
            *rec = make_uint4(__float_as_uint(pos_inf()), __float_as_uint(1.0f), __float_as_uint(neg_inf()),
                              0x7fffffffu);
        return;
    }
    const bool use_k = P.top_k > 0 && P.top_k < V;
    const bool use_p = P.top_p < 1.0f;

    // one read of the row: f(x, key, t0) for every element e < V of the tile
    // at t0 (each_w: also for the -inf filling past V, which weighs nothing,
    // for the passes that only add weights)
    auto each_impl = [&](auto&& f, auto check) {
        stream_tiles<BF16, VEC, false, NT>(rp, V, [&](const uint4 (&r)[kUnroll], int t0) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
#pragma unroll
                for (int q = 0; q < N; ++q) {
                    const float x = elem<BF16>(r[u], q);
                    if (!decltype(check)::value || t0 + (u * NT + t) * N + q < V)
                        f(x, cut_key<BF16>(x), t0);
                }
        });
        __syncthreads();
    };
    auto each = [&](auto&& f) { each_impl(f, std::true_type{}); };
    auto each_w = [&](auto&& f) { each_impl(f, std::false_type{}); };
    uint32_t* const s_cnt = reinterpret_cast<uint32_t*>(s_buf);
    unsigned long long* const s_wt = s_buf;
    auto clear = [&](int n) {  // n 64-bit entries (2n counts)
        for (int j = t; j < n; j += NT) s_buf[j] = 0ull;
        __syncthreads();
    };
    auto fixed_mask = [&](int d) -> uint32_t {  // the key bits above digit d
        const int top = digit_shift<BF16>(d) + digit_width<BF16>(d);
        return top >= 32 ? 0u : ~((1u << top) - 1u);
    };

    // (1) top-k: the key of the k-th largest logit, by counts; kept keys are >= lo
    uint32_t lo = 0;
    if (use_k) {
        uint32_t prefix = 0;
        unsigned long long above = 0;  // elements with keys past the prefix's range
        for (int d = 0; d < NDIG; ++d) {
            const int sh = digit_shift<BF16>(d), nb = 1 << digit_width<BF16>(d);
            const uint32_t fm = fixed_mask(d);
            clear(nb);
            each([&](float, uint32_t key, int) {
                if ((key & fm) == prefix) atomicAdd(&s_cnt[(key >> sh) & (nb - 1)], 1u);
            });
            const Cross cr = find_cross(nb, static_cast<double>(P.top_k), above, s_run,
                                        [&](int j) { return static_cast<unsigned long long>(s_cnt[j]); });
            // (top_k < V elements: the count always reaches it)
            prefix |= static_cast<uint32_t>(max(cr.bin, 0)) << sh;
            above = cr.above;
        }
        lo = prefix;
    }

    // (2) the weight of keys >= lo by the top digit (without top-p, their
    // total is the kept mass)
    auto coarse = [&](int j) { return s_wt[j]; };
    uint32_t kappa = lo;       // kept: keys > kappa, and key == kappa up to index iota
    bool all_from_lo = true;   // ... or every key >= lo (top-k alone, or no crossing)
    int iota = 0x7fffffff;
    unsigned long long kept = 0;
    clear(kCutBins);
    each_w([&](float x, uint32_t key, int) {
        if (key >= lo) {
            const unsigned long long f = fixed_weight(x, M, c);
            if (f) atomicAdd(&s_wt[key >> 20], f);
        }
    });
    const double goal_frac = static_cast<double>(P.top_p);
    // (a goal past any total: the bins' total alone)
    const unsigned long long total = find_cross(kCutBins, 1e300, 0ull, s_run, coarse).total;
    Cross cr{-1, 0, 0};
    if (use_p) cr = find_cross(kCutBins, goal_frac * static_cast<double>(total), 0ull, s_run, coarse);
    if (!use_p) {
        kept = total;
    } else {
        // (3) top-p: the value at which the running weight, from the top,
        // first reaches top_p of the total, digit by digit
        const double goal = goal_frac * static_cast<double>(total);
        bool found = cr.bin >= 0;
        uint32_t prefix = static_cast<uint32_t>(max(cr.bin, 0)) << 20;
        unsigned long long above = cr.above;
        for (int d = 1; found && d < NDIG - 1; ++d) {  // fp32's middle digit
            const int sh = digit_shift<BF16>(d), nb = 1 << digit_width<BF16>(d);
            const uint32_t fm = fixed_mask(d);
            clear(nb);
            each_w([&](float x, uint32_t key, int) {
                if (key >= lo && (key & fm) == prefix) {
                    const unsigned long long f = fixed_weight(x, M, c);
                    if (f) atomicAdd(&s_wt[(key >> sh) & (nb - 1)], f);
                }
            });
            cr = find_cross(nb, goal, above, s_run, coarse);
            found = cr.bin >= 0;
            prefix |= static_cast<uint32_t>(max(cr.bin, 0)) << sh;
            above = cr.above;
        }
        // last digit: counts per value (a value's weight is count x its
        // element weight) and per value and segment of the row
        const int d = NDIG - 1;
        const int sh = digit_shift<BF16>(d), nb = 1 << digit_width<BF16>(d);
        const uint32_t fm = fixed_mask(d);
        const int ntiles = (V + TILE - 1) / TILE;
        const int nseg = kCutSegs / nb;
        const int tps = (ntiles + nseg - 1) / nseg;  // tiles per segment
        uint32_t* const seg = s_cnt;  // kCutSegs counters
        if (found) {
            for (int j = t; j < nb; j += NT) s_vcnt[j] = 0u;
            clear(kCutSegs / 2);
            // (the -inf filling past V never shares the crossing value's
            // prefix: it weighs nothing, and the crossing value weighs more)
            each_w([&](float, uint32_t key, int t0) {
                if (key >= lo && (key & fm) == prefix) {
                    const int v = static_cast<int>((key >> sh) & static_cast<uint32_t>(nb - 1));
                    atomicAdd(&s_vcnt[v], 1u);
                    atomicAdd(&seg[v * nseg + (t0 / TILE) / tps], 1u);
                }
            });
            auto value_weight = [&](int j) {
                const uint32_t k = prefix | (static_cast<uint32_t>(j) << sh);
                return static_cast<unsigned long long>(s_vcnt[j]) * fixed_weight(cut_value<BF16>(k), M, c);
            };
            cr = find_cross(nb, goal, above, s_run, value_weight);
            found = cr.bin >= 0;
        }
        if (!found) {
            // (not reached: the goal lies past the total) every key >= lo
            kept = total;
        } else {
            const int v = cr.bin;
            kappa = prefix | (static_cast<uint32_t>(v) << sh);
            all_from_lo = false;
            above = cr.above;
            const unsigned long long fk = fixed_weight(cut_value<BF16>(kappa), M, c);
            auto reach = [&](unsigned long long x) { return static_cast<double>(x) >= goal; };
            const int64_t cnt = static_cast<int64_t>(s_vcnt[v]);
            // the fewest tokens at kappa that reach the goal, in [1, cnt]
            int64_t n = fk ? static_cast<int64_t>(ceil((goal - static_cast<double>(above)) / static_cast<double>(fk))) : cnt;
            n = n < 1 ? 1 : (n > cnt ? cnt : n);
            while (n > 1 && reach(above + static_cast<unsigned long long>(n - 1) * fk)) --n;
            while (n < cnt && !reach(above + static_cast<unsigned long long>(n) * fk)) ++n;
            kept = above + static_cast<unsigned long long>(n) * fk;
            if (n < cnt) {
                // iota: the n-th token at kappa in index order.  The segment
                // holding it from the per-segment counts (ascending order read
                // as bins from the top), then that segment read again.
                const Cross sc = find_cross(nseg, static_cast<double>(n), 0ull, s_run,
                                            [&](int j) { return static_cast<unsigned long long>(seg[v * nseg + nseg - 1 - j]); });
                const int sg = nseg - 1 - max(sc.bin, 0);
                int r = static_cast<int>(n - static_cast<int64_t>(sc.above));  // rank inside the segment, from 1
                if (t == 0) s_tie = 0x7fffffff;
                __syncthreads();
                for (int tile = sg * tps; tile < min(ntiles, (sg + 1) * tps) && r > 0; ++tile) {
                    for (int u = 0; u < kUnroll && r > 0; ++u) {
                        const int e = tile * TILE + (u * NT + t) * N;
                        const uint4 raw = load_raw<BF16, VEC>(rp, e, V);
                        int hits = 0;
#pragma unroll
                        for (int q = 0; q < N; ++q)
                            hits += (e + q < V && cut_key<BF16>(elem<BF16>(raw, q)) == kappa) ? 1 : 0;
                        int tot;
                        const int ex = block_excl_scan<NT / kWave>(hits, &tot);
                        if (ex < r && r <= ex + hits) {
                            int k = r - ex;
#pragma unroll
                            for (int q = 0; q < N; ++q) {
                                if (e + q < V && cut_key<BF16>(elem<BF16>(raw, q)) == kappa && --k == 0) s_tie = e + q;
                            }
                        }
                        r -= tot;
                    }
                }
                __syncthreads();
                iota = s_tie;
            }
        }
    }
    if (t == 0) {
        const float kept_f = static_cast<float>(static_cast<double>(kept) * (1.0 / 1099511627776.0));
        const float tau = (all_from_lo && !use_k) ? neg_inf() : cut_value<BF16>(kappa);
        *rec = make_uint4(__float_as_uint(M), __float_as_uint(kept_f), __float_as_uint(tau),
                          static_cast<uint32_t>(iota));
    }
}

}  // namespace

specdec_status_t launch_truncated(const VerifyParams& P, bool bf16, bool vec, hipStream_t stream,
                                  hipEvent_t* ev) {
    hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
    hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
    const dim3 grid(P.rows, P.B);
    auto launch = [&](auto kernel, dim3 g, dim3 block, hipEvent_t a, hipEvent_t b) {
        if (ev)
            hipExtLaunchKernelGGL(kernel, g, block, 0, stream, a, b, 0, P);
        else
            hipLaunchKernelGGL(kernel, g, block, 0, stream, P);
    };
    const dim3 tb(kThreads);
    if (bf16) {
        if (vec) launch(k_trunc_select<true, true>, grid, tb, e0, e1);
        else launch(k_trunc_select<true, false>, grid, tb, e0, e1);
    } else {
        if (vec) launch(k_trunc_select<false, true>, grid, tb, e0, e1);
        else launch(k_trunc_select<false, false>, grid, tb, e0, e1);
    }
    if (hipGetLastError() != hipSuccess) return SPECDEC_ERR_DEVICE;
    launch(k_decide_trunc, dim3(P.B), dim3(kThreads), e2, e3);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
}


specdec_status_t launch_trunc_cut(const VerifyParams& P, bool bf16, bool vec, hipStream_t stream,
                                  hipEvent_t start, hipEvent_t stop) {
    const dim3 grid(P.rows, P.B);
    auto launch = [&](auto kernel) {
        if (start || stop)
            hipExtLaunchKernelGGL(kernel, grid, dim3(kCutThreads), 0, stream, start, stop, 0, P);
        else
            hipLaunchKernelGGL(kernel, grid, dim3(kCutThreads), 0, stream, P);
    };
    if (bf16) vec ? launch(k_trunc_cut<true, true>) : launch(k_trunc_cut<true, false>);
    else vec ? launch(k_trunc_cut<false, true>) : launch(k_trunc_cut<false, false>);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
}

}  // namespace specdec
