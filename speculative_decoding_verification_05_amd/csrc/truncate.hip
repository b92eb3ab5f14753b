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
// k_trunc_select  one 256-lane workgroup per used row.  One full streaming
//                 read keeps, per lane, the maximum of each of 8 slots of
//                 consecutive tiles; the k-th largest of the 256 lane maxima
//                 is a lower bound on the row's k-th largest logit (they are
//                 distinct elements of the row).  Only the lane-slots whose
//                 maximum reaches the bound are read again (a few percent of
//                 the row, from cache), their elements at or above the bound
//                 are appended to an LDS buffer with wave ballots (a few dozen
//                 of 128K for the tested shapes), and the buffer is
//                 bitonic-sorted by (logit desc, index asc) and
//                 cut to the exact top-k set (ties kept) and then to the top-p
//                 prefix.  The kept tokens are recorded sorted by token index
//                 with their weights 2^((z - max) c) and the kept total.  If
//                 the buffer overflows (very flat rows, heavy ties) the k-th
//                 value is found exactly by a bitwise search over re-reads of
//                 the row instead.
// k_decide_trunc  one workgroup per request: p(d_i), q(d_i) from the records,
//                 the acceptance tests, m, then the inverse CDF of the
//                 residual (or bonus) over the short kept list in ascending
//                 token order, and every output of the request.
#include "verify_internal.h"

#include <hip/hip_ext.h>

namespace specdec {
namespace {

constexpr int kSelCap = 2048;                 // LDS candidate slots per row
constexpr int kSlots = 8;                     // per-lane tile-slot maxima of the first read
constexpr int kMaxTps = 2;                    // tiles re-read per batch
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
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
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
    base = __shfl(base, __builtin_ctzll(mask), kWave);
    if (hit) {
        const int slot = base + __popcll(mask & ((1ull << l) - 1ull));
        if (slot < kSelCap) { bz[slot] = x; bi[slot] = e; }
    }
}

// One pass over a whole row in tiles of 256 lanes x kUnroll 16-byte vectors
// (the next tile's loads in flight while the current one is visited), then
// a clipped tail; f(v, t0) sees a lane's kUnroll vectors of the tile at t0
// (vector u holds tokens t0 + (u * 256 + lane) * N ...).
template <bool BF16, bool VEC, class F>
__device__ __forceinline__ void stream_tiles(const void* rp, int V, F&& f) {
    constexpr int N = Vec<BF16>::N;
    constexpr int TILE = kThreads * N * kUnroll;
    const int t = threadIdx.x;
    const int full_end = VEC ? (V / TILE) * TILE : 0;
    int t0 = 0;
    if (t0 < full_end) {
        uint4 cur[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) cur[u] = load16_stream<BF16>(rp, t0 + (u * kThreads + t) * N);
        for (; t0 < full_end; t0 += TILE) {
            const int tn = min(t0 + TILE, full_end - TILE);  // re-loads the last tile once: no branch
            uint4 nxt[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) nxt[u] = load16_stream<BF16>(rp, tn + (u * kThreads + t) * N);
            Vec<BF16> v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) v[u] = widen<BF16>(cur[u]);
            f(v, t0);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) cur[u] = nxt[u];
        }
    }
    for (; t0 < V; t0 += TILE) {
        Vec<BF16> v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = load_vec<BF16, VEC>(rp, t0 + (u * kThreads + t) * N, V, neg_inf());
        f(v, t0);
    }
}

// Largest number of set bits of `hits` in the workgroup (the re-read rounds).
__device__ __forceinline__ int __reduce_max_hits(uint32_t hits) {
    __shared__ int s_r;
    if (threadIdx.x == 0) s_r = 0;
    __syncthreads();
    int c = __popc(hits);
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) c = max(c, __shfl_xor(c, o, kWave));
    if (threadIdx.x % kWave == 0) atomicMax(&s_r, c);
    __syncthreads();
    return s_r;
}

// Sorting network step of a wave-wide bitonic sort held one entry per lane:
// exchange with lane l ^ j, keeping the entry that belongs at this lane.
template <class Before>
__device__ __forceinline__ void wave_bitonic_step(float& z, int& id, int k, int j, Before before) {
    const int l = threadIdx.x % kWave;
    const float zp = __shfl_xor(z, j, kWave);
    const int ip = __shfl_xor(id, j, kWave);
    const bool up = (l & k) == 0;
    const bool low = (l & j) == 0;
    // the lower lane of an ascending (up) pair keeps the entry that comes first
    const bool partner_first = before(zp, ip, z, id);
    const bool take = (low == up) ? partner_first : before(z, id, zp, ip);
    if (take) { z = zp; id = ip; }
}

// Candidates s_z/s_i[0..C), C <= 64, to the kept-token record, by one wave.
__device__ void select_in_wave(const VerifyParams& P, int b, int s, int C, bool use_k,
                               const float* s_z, const int* s_i, uint32_t rowflags) {
    const int l = threadIdx.x % kWave;
    float z = l < C ? s_z[l] : neg_inf();
    int id = l < C ? s_i[l] : 0x7fffffff;
    auto by_logit = [](float za, int ia, float zb, int ib) { return precedes(za, ia, zb, ib); };
    for (int k = 2; k <= kWave; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) wave_bitonic_step(z, id, k, j, by_logit);
    // lane l now holds the l-th entry by (logit desc, index asc)
    int K = C;
    if (use_k && P.top_k <= C) {
        const float tau = __shfl(z, P.top_k - 1, kWave);
        K = __popcll(__ballot(l < C && z >= tau));
    }
    const float M = __shfl(z, 0, kWave);
    const float e = l < K ? exp2f((z - M) * P.c) : 0.0f;
    float pre = e;  // inclusive prefix in that order
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const float y = __shfl_up(pre, o, kWave);
        if (l >= o) pre += y;
    }
    int Nk = K;
    if (P.top_p < 1.0f) {
        const float goal = P.top_p * __shfl(pre, K - 1, kWave);
        const uint64_t hit = __ballot(l < K && pre >= goal);
        Nk = hit ? __builtin_ctzll(hit) + 1 : K;
    }
    const float Sn = __shfl(pre, Nk - 1, kWave);
    // the kept tokens by ascending index
    float ek = l < Nk ? e : 0.0f;
    int ik = l < Nk ? id : 0x7fffffff;
    auto by_index = [](float, int ia, float, int ib) { return ia < ib; };
    for (int k = 2; k <= kWave; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) wave_bitonic_step(ek, ik, k, j, by_index);
    uint2* rec = row_record(P, b, s);
    if (l < Nk) rec[1 + l] = make_uint2(static_cast<uint32_t>(ik), __float_as_uint(ek));
    if (l == 0) rec[0] = make_uint2(static_cast<uint32_t>(Nk) | rowflags, __float_as_uint(Sn));
}

// ------------------------------------------------------------------ selection

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void k_trunc_select(VerifyParams P) {
    __shared__ float s_z[kSelCap];
    __shared__ int s_i[kSelCap];
    __shared__ float s_tm[kSlots * kThreads];
    __shared__ float s_wt[kWaves];
    __shared__ int s_count, s_cut;
    constexpr int N = Vec<BF16>::N;
    const int s = blockIdx.x, b = blockIdx.y;
    const bool is_target = s <= P.G;
    const int i = is_target ? s : s - (P.G + 1);
    const int g = request_gamma(P, b);
    if (is_target ? (i > g) : (i >= g)) return;  // padding row
    const void* rp = is_target ? target_row(P, b, i, BF16) : draft_row(P, b, i, BF16);
    const int V = P.V;
    const int t = threadIdx.x;
    const bool use_k = P.top_k > 0 && P.top_k < V;
    uint64_t bad = 0;  // wave-uniform: a NaN or +inf was seen

    // (1) the one full read: per lane, the maximum of each slot of
    // consecutive tiles (kSlots slots per row, in LDS) and non-finite values;
    // then the bound, the k-th largest lane maximum (k distinct elements of
    // the row, so a lower bound on its k-th largest logit)
    constexpr int TILE = kThreads * N * kUnroll;
    const int ntiles = (V + TILE - 1) / TILE;
    const int tps = (ntiles + kSlots - 1) / kSlots;  // tiles per slot
    float run = neg_inf(), lm = neg_inf();
    int cur_slot = 0;
    auto tile_max = [&](const Vec<BF16> (&v)[kUnroll], int t0) {
        const int slot = (t0 / TILE) / tps;
        if (slot != cur_slot) {  // uniform: tiles are visited in order
            s_tm[cur_slot * kThreads + t] = run;
            run = neg_inf();
            cur_slot = slot;
        }
        float m = neg_inf();
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int e0 = t0 + (u * kThreads + t) * N;
#pragma unroll
            for (int k = 0; k < N; ++k) {
                const float x = v[u].x[k];
                const bool valid = e0 + k < V;
                m = valid ? fmaxf(m, x) : m;
                bad |= __ballot(valid && __builtin_isnan(x));
            }
        }
        run = fmaxf(run, m);
        lm = fmaxf(lm, m);
    };
    stream_tiles<BF16, VEC>(rp, V, tile_max);
    s_tm[cur_slot * kThreads + t] = run;
    for (int sl = cur_slot + 1; sl < kSlots; ++sl) s_tm[sl * kThreads + t] = neg_inf();
    bad |= __ballot(lm == pos_inf());
    float bound = neg_inf();
    if (t == 0) s_count = 0;
    if (use_k && V > kSelCap && P.top_k <= kThreads) {
        // the k-th largest lane maximum: every wave runs the same bitwise
        // search over the 256 staged values (ballot counts, no barriers)
        s_z[t] = lm;
        __syncthreads();
        const int l = t % kWave;
        uint32_t kq[kWaves];
#pragma unroll
        for (int q = 0; q < kWaves; ++q) kq[q] = ordered_key(s_z[q * kWave + l]);
        uint32_t key = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t trial = key | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int q = 0; q < kWaves; ++q) cnt += __popcll(__ballot(kq[q] >= trial));
            if (cnt >= P.top_k) key = trial;
        }
        bound = __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
    }
    __syncthreads();

    // (2) re-read only the lane-slots whose maximum reaches the bound (a few
    // percent of them), one batch of loads per round, and append every
    // element >= bound
    uint32_t hits = 0;
    for (int sl = 0; sl < kSlots; ++sl)
        if (s_tm[sl * kThreads + t] >= bound) hits |= 1u << sl;
    const int rounds = __reduce_max_hits(hits);
    for (int r = 0; r < rounds; ++r) {
        const int sl = hits ? __builtin_ctz(hits) : -1;
        hits &= hits - 1u;
        // the slot's tiles in batches of kMaxTps, each batch's loads issued together
        for (int tb = 0; tb < tps; tb += kMaxTps) {
            Vec<BF16> v[kMaxTps][kUnroll];
#pragma unroll
            for (int tt = 0; tt < kMaxTps; ++tt) {
                const int tile = sl * tps + tb + tt;
                const int t0 = (sl >= 0 && tb + tt < tps && tile < ntiles ? tile : 0) * TILE;
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    v[tt][u] = load_vec<BF16, VEC>(rp, t0 + (u * kThreads + t) * N, V, neg_inf());
            }
#pragma unroll
            for (int tt = 0; tt < kMaxTps; ++tt) {
                const int tile = sl * tps + tb + tt;
                const bool live = sl >= 0 && tb + tt < tps && tile < ntiles;
                const int t0 = (live ? tile : 0) * TILE;
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int e0 = t0 + (u * kThreads + t) * N;
#pragma unroll
                    for (int k = 0; k < N; ++k) {
                        const float x = v[tt][u].x[k];
                        append_hits(live && e0 + k < V && x >= bound, x, e0 + k, s_z, s_i, &s_count);
                    }
                }
            }
        }
    }
    __syncthreads();
    int C = s_count;
    uint32_t rowflags = bad ? kRowNonfinite : 0u;
    const bool any_bad = __syncthreads_or(bad != 0);
    if (any_bad) rowflags = kRowNonfinite;

    if (C > kSelCap) {
        // Overflow: the exact k-th largest value by a bitwise search on
        // ordered keys (largest key t with count(key >= t) >= k), each step
        // one read of the row, then the buffer is refilled with the elements
        // at or above it.
        uint32_t key = 0;
        for (int bit = 31; bit >= 0; --bit) {
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
    }
    if (C <= kWave) {
        // The usual case: one wave finishes the row in registers (shuffle
        // bitonic sorts, ballots and a wave prefix scan; no barriers).
        if (t >= kWave) return;
        select_in_wave(P, b, s, C, use_k, s_z, s_i, rowflags);
        return;
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
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const float y = __shfl_up(x, o, kWave);
                if (l >= o) x += y;
            }
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
            e = __shfl(__uint_as_float(ent.y), __builtin_ctzll(mask), kWave);
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
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const float y = __shfl_up(x, o, kWave);
            if (l >= o) x += y;
        }
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
        int32_t* out = P.out_tokens + static_cast<size_t>(b) * (P.G + 1);
        if (i <= P.G) out[i] = i < m ? s_d[i] : (i == m ? token : -1);
        if (i < P.G) {
            if (P.p_draft) P.p_draft[static_cast<size_t>(b) * P.G + i] = i < g ? s_p[i] : 0.0f;
            if (P.q_draft) P.q_draft[static_cast<size_t>(b) * P.G + i] = i < g ? s_q[i] : 0.0f;
        }
        if (i == 0) {
            P.accept_count[b] = m;
            if (P.residual_mass) P.residual_mass[b] = R_report;
            if (P.flags) P.flags[b] = s_fl | fl2;
        }
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

}  // namespace specdec
