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
//     the argmax at the first mismatch (tutorial s.3-4; KB M013 s.03).
//
// Kernels (all HBM-bandwidth bound, no matrix cores: nothing is a contraction):
//   k_stats_sample  one pass over every used logits row, split in chunks of
//                   32 KB.  Each workgroup streams its chunk with 16-byte loads,
//                   four in flight per lane, and reduces it to an online
//                   (max, sum 2^((z-max)c)) pair; the chunk that holds the
//                   drafted token also records that logit.  The last workgroup
//                   of a request to finish (arrival counter) combines the
//                   request's pairs, runs the acceptance tests on one wave and
//                   finds m with a ballot: m = count of trailing ones.
//   k_stats_greedy  the same pass computing (max, lowest index) per chunk;
//                   its last workgroup per request compares drafts with the
//                   row argmaxes and writes every output.
//   k_sample        the draw at position m.  Workgroup (chunk, request)
//                   computes the chunk's residual (or p_gamma) mass with a
//                   block prefix scan; the request's last workgroup finds the
//                   chunk where the running mass passes u*R, re-scans it and
//                   takes the first token whose prefix exceeds u*R.
// Cross-workgroup hand-off uses device-scope release/acquire fences around a
// per-request atomic counter; nothing ever waits on another workgroup, so
// every workgroup finishes regardless of scheduling order.
#include "specdec.h"
#include "specdec_device.h"

#include <stdint.h>
#include <stdlib.h>

namespace specdec {
namespace {

constexpr int kUnroll = 4;   // 16-byte loads in flight per lane in the stats pass

struct VerifyParams {
    const void* target;
    const void* draft;
    const int32_t* tokens;
    const int32_t* gamma;
    int32_t* accept_count;
    int32_t* out_tokens;
    float* p_draft;
    float* q_draft;
    float* residual_mass;
    uint32_t* flags;
    // workspace
    uint32_t* cnt1;     // [B] arrivals in the stats pass
    uint32_t* cnt2;     // [B] arrivals in the sampling pass
    float4* part;       // [B][R][nc] per-chunk partials, R = 2G+1 (sample) or G+1 (greedy)
    float2* rowstat;    // [B][2G+1] (max, sum) of every used row
    float* csum;        // [B][nc2] chunk masses of the sampling pass
    int B, G, V;
    int rows;           // R
    int nc, chunk;      // stats pass: chunks per row, elements per chunk
    int nc2, chunk2;    // sampling pass
    float c;            // log2(e) / T
    uint32_t key0, key1, round;
};

// gamma_b clamped into [0, G] (an out-of-range value is flagged by the
// decision step), so no row past the padded layout is ever addressed.
__device__ __forceinline__ int request_gamma(const VerifyParams& P, int b) {
    const int g = P.gamma ? P.gamma[b] : P.G;
    return min(max(g, 0), P.G);
}

__device__ __forceinline__ uint32_t gamma_flag(const VerifyParams& P, int b) {
    const int g = P.gamma ? P.gamma[b] : P.G;
    return (g < 0 || g > P.G) ? SPECDEC_FLAG_BAD_GAMMA : 0u;
}

__device__ __forceinline__ const void* row_ptr(const void* base, size_t row, int V, bool bf16) {
    return static_cast<const char*>(base) + row * static_cast<size_t>(V) * (bf16 ? 2 : 4);
}

// Arrival at a per-request counter after this workgroup's results are stored.
// Returns true (to every lane) in the last workgroup to arrive; that
// workgroup then reads what the others wrote.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t total) {
    __shared__ int s_last;
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();  // release this workgroup's partials device-wide
        const uint32_t old = atomicAdd(counter, 1u);
        s_last = (old == total - 1);
        if (s_last) *counter = 0;  // leave the workspace ready for the next call
    }
    __syncthreads();
    if (s_last) __threadfence();  // acquire the other workgroups' partials
    return s_last;
}

// ------------------------------------------------------------------ sampling

// Block reduction of the per-lane online pairs.
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

// The per-request decision of sampling mode, run by the whole workgroup that
// arrived last: (max, sum) of every used row, then the acceptance tests.
__device__ void decide_sample(const VerifyParams& P, int b, int g) {
    __shared__ float2 s_stat[127];
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    const float c = P.c;
    // rows 0..g are target rows, G+1 .. G+g draft rows
    for (int s = w; s < P.rows; s += kWaves) {
        const bool used = (s <= P.G) ? (s <= g) : (s - (P.G + 1) < g);
        if (!used) continue;
        const float4* pr = P.part + (static_cast<size_t>(b) * P.rows + s) * P.nc;
        MaxSum acc{neg_inf(), 0.0f};
        for (int k = l; k < P.nc; k += kWave) {
            const float4 q = pr[k];
            acc = combine(acc, MaxSum{q.x, q.y}, c);
        }
        acc = wave_combine(acc, c);
        if (l == 0) {
            s_stat[s] = make_float2(acc.m, acc.s);
            P.rowstat[static_cast<size_t>(b) * P.rows + s] = make_float2(acc.m, acc.s);
        }
    }
    __syncthreads();
    if (w != 0) return;
    // lane i: position i
    const int i = l;
    uint32_t fl = 0;
    bool acc = false;
    float pd = 0.0f, qd = 0.0f;
    int d = -1;
    if (i == 0) fl |= gamma_flag(P, b);
    if (i <= g) {
        const float2 t = s_stat[i];
        if (!(t.x < pos_inf()) || !(t.y == t.y)) fl |= SPECDEC_FLAG_NONFINITE;
    }
    if (i < g) {
        d = P.tokens[static_cast<size_t>(b) * P.G + i];
        const float2 t = s_stat[i];
        const float2 q = s_stat[P.G + 1 + i];
        if (!(q.x < pos_inf()) || !(q.y == q.y)) fl |= SPECDEC_FLAG_NONFINITE;
        float a = 0.0f;
        if (d >= 0 && d < P.V) {
            const int cd = d / P.chunk;
            const float zt = P.part[(static_cast<size_t>(b) * P.rows + i) * P.nc + cd].z;
            const float zq = P.part[(static_cast<size_t>(b) * P.rows + P.G + 1 + i) * P.nc + cd].z;
            pd = exp2f((zt - t.x) * c) / t.y;
            qd = exp2f((zq - q.x) * c) / q.y;
            if (qd > 0.0f) a = fminf(1.0f, pd / qd);
            else a = pd > 0.0f ? 1.0f : 0.0f;
        } else {
            fl |= SPECDEC_FLAG_TOKEN_RANGE;
        }
        const uint4 r = philox4x32_10(make_uint4(static_cast<uint32_t>(i), static_cast<uint32_t>(b),
                                                 P.round, 0u), P.key0, P.key1);
        acc = uniform24(r.x) < a;
    }
    const uint64_t mask = __ballot(acc);
    // m = number of leading accepted positions (ones from bit 0), capped at g
    const int m = min(g, static_cast<int>(__builtin_ctzll(~mask)));
    fl = wave_or(fl);
    int32_t* out = P.out_tokens + static_cast<size_t>(b) * (P.G + 1);
    if (i <= P.G && i != m) out[i] = i < m ? d : -1;
    if (i < P.G) {
        if (P.p_draft) P.p_draft[static_cast<size_t>(b) * P.G + i] = pd;
        if (P.q_draft) P.q_draft[static_cast<size_t>(b) * P.G + i] = qd;
    }
    if (i == 0) {
        P.accept_count[b] = m;
        if (P.flags) P.flags[b] = fl;
    }
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void k_stats_sample(VerifyParams P) {
    const int ci = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
    const int g = request_gamma(P, b);
    const bool is_target = s <= P.G;
    const int i = is_target ? s : s - (P.G + 1);
    if (is_target ? (i > g) : (i >= g)) return;  // padding row: never read
    const size_t row = is_target ? static_cast<size_t>(b) * (P.G + 1) + i
                                 : static_cast<size_t>(b) * P.G + i;
    const void* rp = row_ptr(is_target ? P.target : P.draft, row, P.V, BF16);
    const int lo = ci * P.chunk;
    const int hi = min(P.V, lo + P.chunk);
    const float c = P.c;
    constexpr int N = Vec<BF16>::N;
    constexpr int TILE = kThreads * N * kUnroll;

    // Tiles wholly inside the chunk stream with branch-free 16-byte loads (all
    // kUnroll of a lane in flight together); only the last tile of a row's
    // last chunk takes the clipped path.
    float m = neg_inf(), sum = 0.0f;
    auto consume = [&](const Vec<BF16> (&v)[kUnroll]) {
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
    const int full_end = VEC ? lo + ((hi - lo) / TILE) * TILE : lo;
    for (int t0 = lo; t0 < full_end; t0 += TILE) {
        uint4 raw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) raw[u] = load16<BF16>(rp, t0 + (u * kThreads + threadIdx.x) * N);
        Vec<BF16> v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = widen<BF16>(raw[u]);
        consume(v);
    }
    for (int t0 = full_end; t0 < hi; t0 += TILE) {
        Vec<BF16> v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = load_vec<BF16, VEC>(rp, t0 + (u * kThreads + threadIdx.x) * N, hi, neg_inf());
        consume(v);
    }
    const MaxSum r = block_combine(MaxSum{m, sum}, c);

    // the logit of the token this row judges (target) or proposed (draft)
    if (threadIdx.x == 0) {
        float zd = 0.0f;
        if (i < g) {
            const int d = P.tokens[static_cast<size_t>(b) * P.G + i];
            if (d >= lo && d < hi) zd = load_logit<BF16>(rp, d);
        }
        P.part[(static_cast<size_t>(b) * P.rows + s) * P.nc + ci] = make_float4(r.m, r.s, zd, 0.0f);
    }
    const uint32_t total = static_cast<uint32_t>((2 * g + 1) * P.nc);
    if (!arrive_last(P.cnt1 + b, total)) return;
    decide_sample(P, b, g);
}

// ------------------------------------------------------------------ greedy

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

__device__ void decide_greedy(const VerifyParams& P, int b, int g) {
    __shared__ int s_arg[64];
    __shared__ uint32_t s_nan[64];
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    for (int s = w; s <= g; s += kWaves) {
        const float4* pr = P.part + (static_cast<size_t>(b) * P.rows + s) * P.nc;
        ArgMax best{neg_inf(), 0x7fffffff};
        uint32_t nan = 0;
        for (int k = l; k < P.nc; k += kWave) {
            const float4 q = pr[k];
            const int idx = __float_as_int(q.y);
            if (idx != 0x7fffffff) best = better(best, ArgMax{q.x, idx});
            nan |= __float_as_uint(q.z);
        }
        best = wave_argmax(best);
        nan = wave_or(nan);
        if (l == 0) { s_arg[s] = best.i; s_nan[s] = nan; }
    }
    __syncthreads();
    if (w != 0) return;
    const int i = l;
    uint32_t fl = 0;
    bool acc = false;
    int d = -1;
    if (i == 0) fl |= gamma_flag(P, b);
    if (i <= g && s_nan[i]) fl |= SPECDEC_FLAG_NONFINITE;
    if (i < g) {
        d = P.tokens[static_cast<size_t>(b) * P.G + i];
        if (d < 0 || d >= P.V) fl |= SPECDEC_FLAG_TOKEN_RANGE;
        acc = (d == s_arg[i]);
    }
    const uint64_t mask = __ballot(acc);
    const int m = min(g, static_cast<int>(__builtin_ctzll(~mask)));
    fl = wave_or(fl);
    int32_t* out = P.out_tokens + static_cast<size_t>(b) * (P.G + 1);
    if (i <= P.G) out[i] = i < m ? d : (i == m ? s_arg[m] : -1);
    if (i == 0) {
        P.accept_count[b] = m;
        if (P.flags) P.flags[b] = fl;
    }
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void k_stats_greedy(VerifyParams P) {
    const int ci = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
    const int g = request_gamma(P, b);
    if (i > g) return;
    const void* rp = row_ptr(P.target, static_cast<size_t>(b) * (P.G + 1) + i, P.V, BF16);
    const int lo = ci * P.chunk;
    const int hi = min(P.V, lo + P.chunk);
    constexpr int N = Vec<BF16>::N;
    constexpr int TILE = kThreads * N * kUnroll;
    // Each lane visits its elements in ascending index order, so a strict ">"
    // keeps the lowest index among equal maxima.
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
    const int full_end = VEC ? lo + ((hi - lo) / TILE) * TILE : lo;
    for (int t0 = lo; t0 < full_end; t0 += TILE) {
        uint4 raw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) raw[u] = load16<BF16>(rp, t0 + (u * kThreads + threadIdx.x) * N);
        Vec<BF16> v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = widen<BF16>(raw[u]);
        consume(v, t0);
    }
    for (int t0 = full_end; t0 < hi; t0 += TILE) {
        Vec<BF16> v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = load_vec<BF16, VEC>(rp, t0 + (u * kThreads + threadIdx.x) * N, hi, neg_inf());
        consume(v, t0);
    }
    const ArgMax r = block_argmax(best);
    const bool any_nan = __syncthreads_or(nan);
    if (threadIdx.x == 0)
        P.part[(static_cast<size_t>(b) * P.rows + i) * P.nc + ci] =
            make_float4(r.v, __int_as_float(r.i), __uint_as_float(any_nan ? 1u : 0u), 0.0f);
    const uint32_t total = static_cast<uint32_t>((g + 1) * P.nc);
    if (!arrive_last(P.cnt1 + b, total)) return;
    decide_greedy(P, b, g);
}

// ------------------------------------------------------------------ sampling pass

struct ScanRow {
    const void* p;   // target row m (or gamma)
    const void* q;   // draft row m, or nullptr when the mass is p itself
    float mp, sp, mq, sq, c;
};

template <bool BF16>
__device__ __forceinline__ float mass_at(const ScanRow& a, float zp, float zq) {
    const float pv = exp2f((zp - a.mp) * a.c) / a.sp;
    if (!a.q) return pv;
    const float qv = exp2f((zq - a.mq) * a.c) / a.sq;
    return fmaxf(pv - qv, 0.0f);
}

// Chunk [lo, hi) of the sampling mass r (max(p - q, 0), or p), scanned in
// ascending token order in tiles of 256 lanes x 16 bytes.  Returns the
// chunk's total, defined as the inclusive prefix at its last element.
// With base + prefix(v) > target for some v in the chunk, *tok receives the
// first such v.  *last_pos receives the largest v with r(v) > 0.
// Kept out of line so that the chunk total of the mass pass and the prefix
// values of the search pass come from the very same instructions.
template <bool BF16, bool VEC>
__device__ __noinline__ float scan_chunk(const ScanRow a, int lo, int hi, float base, float target,
                                         int* tok, int* last_pos) {
    constexpr int N = Vec<BF16>::N;
    constexpr int TILE = kThreads * N;
    __shared__ float s_wtot[kWaves];
    __shared__ float s_tile_end;
    __shared__ int s_found, s_last;
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    __syncthreads();  // a previous call's results have been read by every lane
    if (threadIdx.x == 0) { s_found = 0x7fffffff; s_last = -1; }
    float tile_base = 0.0f;
    for (int t0 = lo; t0 < hi; t0 += TILE) {
        const int e = t0 + threadIdx.x * N;
        const Vec<BF16> vp = load_vec<BF16, VEC>(a.p, e, hi, neg_inf());
        Vec<BF16> vq;
        if (a.q) vq = load_vec<BF16, VEC>(a.q, e, hi, neg_inf());
        float r[N], inc[N];
        int lastp = -1;
#pragma unroll
        for (int k = 0; k < N; ++k) {
            r[k] = (e + k < hi) ? mass_at<BF16>(a, vp.x[k], a.q ? vq.x[k] : 0.0f) : 0.0f;
            if (r[k] > 0.0f) lastp = e + k;
        }
        inc[0] = r[0];
#pragma unroll
        for (int k = 1; k < N; ++k) inc[k] = inc[k - 1] + r[k];
        // exclusive scan of lane totals: inclusive within the wave, shifted
        float x = inc[N - 1];
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const float y = __shfl_up(x, o, kWave);
            if (l >= o) x += y;
        }
        float ex = __shfl_up(x, 1, kWave);
        if (l == 0) ex = 0.0f;
        __syncthreads();
        if (l == kWave - 1) s_wtot[w] = x;
        __syncthreads();
        float woff = 0.0f;
        for (int k = 0; k < w; ++k) woff += s_wtot[k];
        const float lane_base = tile_base + (woff + ex);
        int first = 0x7fffffff;
#pragma unroll
        for (int k = N - 1; k >= 0; --k) {
            const float pre = lane_base + inc[k];
            if (base + pre > target) first = e + k;
        }
        if (first != 0x7fffffff) atomicMin(&s_found, first);
        if (lastp >= 0) atomicMax(&s_last, lastp);
        if (threadIdx.x == kThreads - 1) s_tile_end = lane_base + inc[N - 1];
        __syncthreads();
        tile_base = s_tile_end;
        if (s_found != 0x7fffffff) break;
    }
    __syncthreads();
    *tok = s_found;
    *last_pos = s_last;
    return tile_base;
}

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void k_sample(VerifyParams P) {
    __shared__ float s_csum[1024];
    __shared__ float s_R;
    const int ci = blockIdx.x, b = blockIdx.y;
    const int g = request_gamma(P, b);
    const int m = min(max(P.accept_count[b], 0), g);  // written by the stats pass
    const bool resid = m < g;
    const float2 st = P.rowstat[static_cast<size_t>(b) * P.rows + m];
    ScanRow a;
    a.p = row_ptr(P.target, static_cast<size_t>(b) * (P.G + 1) + m, P.V, BF16);
    a.mp = st.x;
    a.sp = st.y;
    a.c = P.c;
    a.q = nullptr;
    a.mq = 0.0f;
    a.sq = 1.0f;
    if (resid) {
        const float2 sq = P.rowstat[static_cast<size_t>(b) * P.rows + P.G + 1 + m];
        a.q = row_ptr(P.draft, static_cast<size_t>(b) * P.G + m, P.V, BF16);
        a.mq = sq.x;
        a.sq = sq.y;
    }
    int tok, lastp;
    const int lo = ci * P.chunk2, hi = min(P.V, lo + P.chunk2);
    const float cs = scan_chunk<BF16, VEC>(a, lo, hi, 0.0f, pos_inf(), &tok, &lastp);
    if (threadIdx.x == 0) P.csum[static_cast<size_t>(b) * P.nc2 + ci] = cs;
    if (!arrive_last(P.cnt2 + b, static_cast<uint32_t>(P.nc2))) return;

    // Last workgroup of request b: R, the chunk where the mass passes u*R,
    // then the token inside it.
    for (int k = threadIdx.x; k < P.nc2; k += kThreads)
        s_csum[k] = P.csum[static_cast<size_t>(b) * P.nc2 + k];
    __syncthreads();
    uint32_t fl = 0;
    float R_report = 0.0f;
    if (threadIdx.x == 0) {
        float R = 0.0f;
        for (int k = 0; k < P.nc2; ++k) R += s_csum[k];
        s_R = R;
    }
    __syncthreads();
    if (resid) {
        R_report = s_R;
        if (!(s_R > 0.0f)) {
            // empty residual: draw from p_m instead (never divide by zero)
            fl |= SPECDEC_FLAG_RESIDUAL_FALLBACK;
            a.q = nullptr;
            for (int k = 0; k < P.nc2; ++k) {
                const int l2 = k * P.chunk2, h2 = min(P.V, l2 + P.chunk2);
                int t2, lp2;
                const float v = scan_chunk<BF16, VEC>(a, l2, h2, 0.0f, pos_inf(), &t2, &lp2);
                if (threadIdx.x == 0) s_csum[k] = v;
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                float R = 0.0f;
                for (int k = 0; k < P.nc2; ++k) R += s_csum[k];
                s_R = R;
            }
            __syncthreads();
        }
    }
    const uint4 rnd = philox4x32_10(make_uint4(static_cast<uint32_t>(m), static_cast<uint32_t>(b),
                                               P.round, 0u), P.key0, P.key1);
    const float target = uniform24(rnd.y) * s_R;
    __shared__ int s_chunk;
    __shared__ float s_before;
    if (threadIdx.x == 0) {
        float C = 0.0f;
        int cstar = -1;
        float before = 0.0f;
        for (int k = 0; k < P.nc2; ++k) {
            const float next = C + s_csum[k];
            if (next > target) { cstar = k; before = C; break; }
            C = next;
        }
        s_chunk = cstar;
        s_before = before;
    }
    __syncthreads();
    int token = -1;
    if (s_chunk >= 0) {
        const int l2 = s_chunk * P.chunk2, h2 = min(P.V, l2 + P.chunk2);
        int t2, lp2;
        scan_chunk<BF16, VEC>(a, l2, h2, s_before, target, &t2, &lp2);
        // The chunk total ends a partial last tile with a differently
        // associated sum than its last element's prefix; if that rounding
        // leaves no element above u*R, the crossing is the chunk's last token
        // with mass.
        token = t2 != 0x7fffffff ? t2 : lp2;
    } else {
        // rounding left u*R at or above the total: the last token with mass
        int k = P.nc2 - 1;
        while (k > 0 && !(s_csum[k] > 0.0f)) --k;
        const int l2 = k * P.chunk2, h2 = min(P.V, l2 + P.chunk2);
        int t2, lp2;
        scan_chunk<BF16, VEC>(a, l2, h2, 0.0f, pos_inf(), &t2, &lp2);
        token = lp2;
    }
    if (threadIdx.x == 0) {
        P.out_tokens[static_cast<size_t>(b) * (P.G + 1) + m] = token;
        if (P.residual_mass) P.residual_mass[b] = R_report;
        if (P.flags && fl) P.flags[b] |= fl;
    }
}

// ------------------------------------------------------------------ host side

struct Layout {
    int rows, nc, chunk, nc2, chunk2;
    size_t off_cnt1, off_cnt2, off_part, off_rowstat, off_csum, total;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int env_int(const char* name, int dflt) {
    const char* s = getenv(name);
    if (!s || !*s) return dflt;
    const int v = atoi(s);
    return v > 0 ? v : dflt;
}

bool valid_desc(const specdec_verify_desc_t* d) {
    if (!d) return false;
    if (d->batch < 0 || d->batch > 65535 || d->gamma_max < 0 || d->gamma_max > 63 || d->vocab < 1) return false;
    if (d->dtype != SPECDEC_F32 && d->dtype != SPECDEC_BF16) return false;
    if (d->mode != SPECDEC_SAMPLE && d->mode != SPECDEC_GREEDY) return false;
    if (d->reserved != 0) return false;
    if (d->mode == SPECDEC_SAMPLE) {
        const float T = d->temperature;
        if (!(T > 0.0f) || !(T < 3.0e38f)) return false;
        if (d->top_k < 0) return false;
        if (!(d->top_p > 0.0f) || !(d->top_p <= 1.0f)) return false;
    }
    return true;
}

Layout make_layout(const specdec_verify_desc_t* d) {
    Layout L{};
    const bool bf16 = d->dtype == SPECDEC_BF16;
    const int n = bf16 ? 8 : 4;
    const int tile = kThreads * n * kUnroll;
    const int tiles = env_int("SPECDEC_STATS_TILES", 2);
    L.rows = d->mode == SPECDEC_SAMPLE ? 2 * d->gamma_max + 1 : d->gamma_max + 1;
    L.chunk = tile * tiles;
    L.nc = (d->vocab + L.chunk - 1) / L.chunk;
    // sampling pass: chunks of 2 tiles of 256 x 16 B, at most 1024 of them
    const int tile2 = kThreads * n;
    L.chunk2 = tile2 * env_int("SPECDEC_SAMPLE_TILES", 2);
    while ((d->vocab + L.chunk2 - 1) / L.chunk2 > 1024) L.chunk2 *= 2;
    L.nc2 = (d->vocab + L.chunk2 - 1) / L.chunk2;
    const size_t B = static_cast<size_t>(d->batch);
    size_t off = 0;
    L.off_cnt1 = off; off = align256(off + B * 4);
    L.off_cnt2 = off; off = align256(off + B * 4);
    L.off_part = off; off = align256(off + B * L.rows * L.nc * sizeof(float4));
    L.off_rowstat = off; off = align256(off + B * L.rows * sizeof(float2));
    L.off_csum = off; off = align256(off + B * L.nc2 * sizeof(float));
    L.total = off;
    return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <bool BF16, bool VEC>
specdec_status_t launch_all(const specdec_verify_desc_t* d, const VerifyParams& P, const Layout& L,
                            hipStream_t stream) {
    const dim3 block(kThreads);
    if (d->mode == SPECDEC_GREEDY) {
        const dim3 grid(L.nc, d->gamma_max + 1, d->batch);
        hipLaunchKernelGGL((k_stats_greedy<BF16, VEC>), grid, block, 0, stream, P);
    } else {
        const dim3 grid(L.nc, 2 * d->gamma_max + 1, d->batch);
        hipLaunchKernelGGL((k_stats_sample<BF16, VEC>), grid, block, 0, stream, P);
        if (hipGetLastError() != hipSuccess) return SPECDEC_ERR_DEVICE;
        const dim3 grid2(L.nc2, d->batch);
        hipLaunchKernelGGL((k_sample<BF16, VEC>), grid2, block, 0, stream, P);
    }
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
}

}  // namespace
}  // namespace specdec

using namespace specdec;

extern "C" size_t specdec_verify_workspace_bytes(const specdec_verify_desc_t* desc) {
    if (!valid_desc(desc)) return 0;
    return make_layout(desc).total;
}

extern "C" specdec_status_t specdec_verify(const specdec_verify_desc_t* d,
                                           const void* target_logits, const void* draft_logits,
                                           const int32_t* draft_tokens, const int32_t* gamma,
                                           int32_t* accept_count, int32_t* out_tokens,
                                           float* p_draft, float* q_draft, float* residual_mass,
                                           uint32_t* flags, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
    if (!valid_desc(d)) return SPECDEC_ERR_INVALID_ARGUMENT;
    const bool sample = d->mode == SPECDEC_SAMPLE;
    if (!target_logits || !accept_count || !out_tokens || !workspace)
        return SPECDEC_ERR_INVALID_ARGUMENT;
    if (d->gamma_max > 0 && !draft_tokens) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (sample && d->gamma_max > 0 && !draft_logits) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (sample && (d->top_k != 0 || d->top_p < 1.0f)) return SPECDEC_ERR_UNSUPPORTED;
    const Layout L = make_layout(d);
    if (workspace_bytes < L.total) return SPECDEC_ERR_WORKSPACE_TOO_SMALL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (d->batch == 0) return SPECDEC_OK;

    VerifyParams P{};
    P.target = target_logits;
    P.draft = draft_logits;
    P.tokens = draft_tokens;
    P.gamma = gamma;
    P.accept_count = accept_count;
    P.out_tokens = out_tokens;
    P.p_draft = p_draft;
    P.q_draft = q_draft;
    P.residual_mass = residual_mass;
    P.flags = flags;
    char* ws = static_cast<char*>(workspace);
    P.cnt1 = reinterpret_cast<uint32_t*>(ws + L.off_cnt1);
    P.cnt2 = reinterpret_cast<uint32_t*>(ws + L.off_cnt2);
    P.part = reinterpret_cast<float4*>(ws + L.off_part);
    P.rowstat = reinterpret_cast<float2*>(ws + L.off_rowstat);
    P.csum = reinterpret_cast<float*>(ws + L.off_csum);
    P.B = d->batch;
    P.G = d->gamma_max;
    P.V = d->vocab;
    P.rows = L.rows;
    P.nc = L.nc;
    P.chunk = L.chunk;
    P.nc2 = L.nc2;
    P.chunk2 = L.chunk2;
    P.c = sample ? static_cast<float>(1.4426950408889634 / static_cast<double>(d->temperature)) : 1.0f;
    P.key0 = static_cast<uint32_t>(d->seed & 0xffffffffu);
    P.key1 = static_cast<uint32_t>(d->seed >> 32);
    P.round = d->round;

    const bool bf16 = d->dtype == SPECDEC_BF16;
    const size_t es = bf16 ? 2 : 4;
    const bool vec = aligned16(target_logits) && (!sample || aligned16(draft_logits)) &&
                     (static_cast<size_t>(d->vocab) * es) % 16 == 0;
    if (bf16) return vec ? launch_all<true, true>(d, P, L, stream) : launch_all<true, false>(d, P, L, stream);
    return vec ? launch_all<false, true>(d, P, L, stream) : launch_all<false, false>(d, P, L, stream);
}
