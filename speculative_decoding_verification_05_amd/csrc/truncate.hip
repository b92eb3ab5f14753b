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
// k_truncate      one 1024-lane workgroup per used row keeps the whole row
//                 in registers (16 x 16-byte vectors per lane).  The k-th
//                 largest of the 1024 lane maxima bounds the k-th largest
//                 logit from below (they are k distinct elements), so only
//                 the few elements above that bound are compacted into LDS,
//                 bitonic-sorted by (logit desc, index asc), cut to the exact
//                 top-k set and then to the top-p prefix.  The kept tokens
//                 are recorded sorted by token index with their weights
//                 2^((z - max) c) and the kept total.  A row with too many
//                 candidates falls back to an exact bitwise search for the
//                 k-th value over the registers.
// k_decide_trunc  one workgroup per request: p(d_i), q(d_i) from the records,
//                 the acceptance tests, m, then the inverse CDF of the
//                 residual (or bonus) over the short kept list in ascending
//                 token order, and every output of the request.
#include "verify_internal.h"

#include <hip/hip_ext.h>

namespace specdec {
namespace {

constexpr int kTWaves = kTruncThreads / kWave;
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

// ---- block-wide helpers for 1024 lanes
__device__ __forceinline__ int block_excl_scan_1024(int v, int* total) {
    __shared__ int s_w[kTWaves];
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    int x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (l >= o) x += y;
    }
    __syncthreads();
    if (l == kWave - 1) s_w[w] = x;
    __syncthreads();
    int off = 0, tot = 0;
    for (int k = 0; k < kTWaves; ++k) {
        if (k < w) off += s_w[k];
        tot += s_w[k];
    }
    *total = tot;
    return off + x - v;
}

__device__ __forceinline__ float block_sum_1024(float v) {
    __shared__ float s_w[kTWaves];
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    v = wave_sum(v);
    __syncthreads();
    if (l == 0) s_w[w] = v;
    __syncthreads();
    float r = 0.0f;
    for (int k = 0; k < kTWaves; ++k) r += s_w[k];
    return r;
}

__device__ __forceinline__ int block_count_1024(int v) {
    __shared__ int s_w[kTWaves];
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    __syncthreads();
    if (l == 0) s_w[w] = v;
    __syncthreads();
    int r = 0;
    for (int k = 0; k < kTWaves; ++k) r += s_w[k];
    return r;
}

// Bitonic sort of n (a power of two, <= 2 x 1024) entries (z, i) in LDS
// into `precedes` order.
__device__ void bitonic_sort(float* z, int* id, int n) {
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int p = threadIdx.x; p < n / 2; p += kTruncThreads) {
                const int a = 2 * j * (p / j) + (p % j), c = a + j;
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
            for (int p = threadIdx.x; p < n / 2; p += kTruncThreads) {
                const int a = 2 * j * (p / j) + (p % j), c = a + j;
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

// ------------------------------------------------------------------ selection

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kTruncThreads) void k_truncate(VerifyParams P) {
    __shared__ float s_z[kTruncCap];
    __shared__ int s_i[kTruncCap];
    __shared__ float s_lm[kTruncThreads];
    __shared__ float s_wt[kTWaves];
    __shared__ int s_cut;
    constexpr int N = Vec<BF16>::N;
    const int s = blockIdx.x, b = blockIdx.y;
    const bool is_target = s <= P.G;
    const int i = is_target ? s : s - (P.G + 1);
    const int g = request_gamma(P, b);
    if (is_target ? (i > g) : (i >= g)) return;  // padding row
    const void* rp = is_target ? target_row(P, b, i, BF16) : draft_row(P, b, i, BF16);
    const int V = P.V;
    const int nvec = (V + N - 1) / N;
    const int t = threadIdx.x;

    // (1) the row into registers: lane t holds vectors t + u * 1024
    uint4 raw[kTruncVecs];
#pragma unroll
    for (int u = 0; u < kTruncVecs; ++u) {
        const int j = min(t + u * kTruncThreads, nvec - 1);
        if constexpr (VEC) {
            raw[u] = load16<BF16>(rp, j * N);
        } else {
            Vec<BF16> v = load_vec<BF16, false>(rp, j * N, V, neg_inf());
            uint32_t w[4];
            if constexpr (BF16) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w[q] = (__float_as_uint(v.x[2 * q]) >> 16) | (__float_as_uint(v.x[2 * q + 1]) & 0xffff0000u);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) w[q] = __float_as_uint(v.x[q]);
            }
            raw[u] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
    // element (u, k) is token (t + u * 1024) * N + k, valid below V
    auto for_each = [&](auto&& f) {
#pragma unroll
        for (int u = 0; u < kTruncVecs; ++u) {
            const Vec<BF16> v = widen<BF16>(raw[u]);
            const int e0 = (t + u * kTruncThreads) * N;
#pragma unroll
            for (int k = 0; k < N; ++k)
                if (e0 + k < V) f(v.x[k], e0 + k);
        }
    };

    // (2) lane maxima, row maximum, non-finite values
    float lm = neg_inf();
    bool bad = false;
    for_each([&](float x, int) {
        lm = fmaxf(lm, x);
        bad |= (x != x) || (x == pos_inf());
    });
    const bool any_bad = __syncthreads_or(bad);

    // (3) a lower bound on the k-th largest logit: the k-th largest lane max
    const bool use_k = P.top_k > 0 && P.top_k < V;
    float lo = neg_inf();
    if (use_k && V > kTruncCap) {
        s_lm[t] = lm;
        __syncthreads();
        for (int k = 2; k <= kTruncThreads; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                const int x = t ^ j;
                if (x > t) {
                    const float a = s_lm[t], c = s_lm[x];
                    const bool desc = (t & k) == 0;
                    if (desc ? (a < c) : (a > c)) { s_lm[t] = c; s_lm[x] = a; }
                }
                __syncthreads();
            }
        }
        lo = s_lm[P.top_k - 1];
    }

    // (4) candidates: every element >= lo (all of a row that fits in LDS)
    int mine = 0;
    for_each([&](float x, int) { mine += (x >= lo); });
    int C;
    int pos = block_excl_scan_1024(mine, &C);
    uint32_t rowflags = any_bad ? kRowNonfinite : 0u;
    if (C > kTruncCap) {
        // Too many elements above the bound (heavy ties or a flat row): find
        // the exact k-th largest value by a bitwise search on ordered keys,
        // keeping the largest key t with count(key >= t) >= k.
        uint32_t key = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t trial = key | (1u << bit);
            int cnt = 0;
            for_each([&](float x, int) { cnt += (x == x) && ordered_key(x) >= trial; });
            if (block_count_1024(cnt) >= P.top_k) key = trial;
        }
        mine = 0;
        for_each([&](float x, int) { mine += (x == x) && ordered_key(x) >= key; });
        pos = block_excl_scan_1024(mine, &C);
        if (C > kTruncCap) rowflags |= kRowOverflow;  // more ties than slots: clipped
        for_each([&](float x, int e) {
            if ((x == x) && ordered_key(x) >= key) {
                if (pos < kTruncCap) { s_z[pos] = x; s_i[pos] = e; }
                ++pos;
            }
        });
    } else {
        for_each([&](float x, int e) {
            if (x >= lo) { s_z[pos] = x; s_i[pos] = e; ++pos; }
        });
    }
    C = min(C, kTruncCap);
    const int n = pow2_at_least(C < 2 ? 2 : C);
    for (int p = C + t; p < n; p += kTruncThreads) { s_z[p] = neg_inf(); s_i[p] = 0x7fffffff; }
    __syncthreads();

    // (5) sorted by (logit desc, index asc); the exact top-k set is a prefix
    bitonic_sort(s_z, s_i, n);
    int K = C;
    if (use_k) {
        const float tau = s_z[P.top_k - 1];
        int c = 0;
        for (int p = t; p < C; p += kTruncThreads) c += s_z[p] >= tau;
        K = block_count_1024(c);
    }
    const float M = s_z[0];
    const float cc = P.c;

    // (6) top-p: the shortest prefix whose mass reaches top_p of the top-k mass
    int Nk = K;
    float Sn;
    {
        float part = 0.0f;
        for (int p = t; p < K; p += kTruncThreads) part += exp2f((s_z[p] - M) * cc);
        const float Sk = block_sum_1024(part);
        Sn = Sk;
        if (P.top_p < 1.0f) {
            const float goal = P.top_p * Sk;
            if (t == 0) s_cut = K - 1;
            __syncthreads();
            float carry = 0.0f;
            for (int base = 0; base < K; base += kTruncThreads) {
                const int p = base + t;
                const float e = p < K ? exp2f((s_z[p] - M) * cc) : 0.0f;
                // inclusive prefix of e in sorted order (fp32)
                float x = e;
                const int w = t / kWave, l = t % kWave;
#pragma unroll
                for (int o = 1; o < kWave; o <<= 1) {
                    const float y = __shfl_up(x, o, kWave);
                    if (l >= o) x += y;
                }
                __syncthreads();
                if (l == kWave - 1) s_wt[w] = x;
                __syncthreads();
                float off = carry;
                float tot = carry;
                for (int k = 0; k < kTWaves; ++k) {
                    if (k < w) off += s_wt[k];
                    tot += s_wt[k];
                }
                const bool hit = p < K && off + x >= goal;
                const uint64_t mask = __ballot(hit);
                if (l == 0 && mask) atomicMin(&s_cut, base + w * kWave + __builtin_ctzll(mask));
                carry = tot;
                __syncthreads();
                if (s_cut < K - 1 || base + kTruncThreads >= K) break;
            }
            Nk = s_cut + 1;
            float part2 = 0.0f;
            for (int p = t; p < Nk; p += kTruncThreads) part2 += exp2f((s_z[p] - M) * cc);
            Sn = block_sum_1024(part2);
        }
    }
    if (Nk > kNucCap) { Nk = kNucCap; rowflags |= kRowOverflow; }

    // (7) the kept tokens by ascending index, with their weights
    __syncthreads();
    float* s_e = s_z;  // reuse: weights replace logits
    for (int p = t; p < Nk; p += kTruncThreads) s_e[p] = exp2f((s_z[p] - M) * cc);
    const int n2 = pow2_at_least(Nk < 2 ? 2 : Nk);
    for (int p = Nk + t; p < n2; p += kTruncThreads) { s_i[p] = 0x7fffffff; s_e[p] = 0.0f; }
    __syncthreads();
    bitonic_sort_index(s_i, s_e, n2);
    uint2* rec = row_record(P, b, s);
    for (int p = t; p < Nk; p += kTruncThreads)
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
    const dim3 tb(kTruncThreads);
    if (bf16) {
        if (vec) launch(k_truncate<true, true>, grid, tb, e0, e1);
        else launch(k_truncate<true, false>, grid, tb, e0, e1);
    } else {
        if (vec) launch(k_truncate<false, true>, grid, tb, e0, e1);
        else launch(k_truncate<false, false>, grid, tb, e0, e1);
    }
    if (hipGetLastError() != hipSuccess) return SPECDEC_ERR_DEVICE;
    launch(k_decide_trunc, dim3(P.B), dim3(kThreads), e2, e3);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
}

}  // namespace specdec
