// specdec_propose_ngram: prompt-lookup (n-gram) drafting on gfx950.
//
// What is computed (AI-infra KB M013 s.08: candidates from repeated patterns
// in the text; "The math behind the speedup": pattern-based drafting searches
// the existing context for a matching sequence at near-zero cost;
// "Speculative decoding tutorial" s.13.1 and s.14: prompt lookup / n-gram
// candidates from the prompt or the history):
//   for n = n_max down to n_min, the most recent earlier occurrence of the
//   history's last n tokens (ending before the last position); the first n
//   with one wins, and the up to gamma tokens after it are the proposal.
//
// Equivalent single pass: for every end position e <= L-2 let l(e) be the
// length of the common suffix of h[..e] and h[..L-1], capped at n_max.  The
// winner maximises (l(e), e) over the e with l(e) >= n_min.  One workgroup
// per request streams its history through LDS in segments (with the n_max-1
// tokens before each segment as a halo); every lane scores the positions it
// owns against the pattern held in LDS, keeps the best packed key
// (l << 24 | e), and a block maximum picks the winner.  One read of the
// history: bound by HBM bandwidth and, for short histories, by latency.
#include "specdec.h"
#include "specdec_device.h"

#include <stdint.h>

namespace specdec {
namespace {

constexpr int kSeg = 8192;          // history positions per LDS segment
constexpr int kMaxN = 32;           // largest n_max
constexpr int kLoadsPerLane = kSeg / kThreads;

__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
    return lane63(wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; }));
}

struct NgramParams {
    const int32_t* history;   // [B][max_len]
    const int32_t* hist_len;  // [B]
    int32_t* tokens;          // [B][G]
    int32_t* count;           // [B]
    int32_t* match;           // [B] or null
    int B, max_len, n_min, n_max, G;
};

__global__ __launch_bounds__(kThreads) void k_propose_ngram(NgramParams P) {
    __shared__ int32_t s_h[kMaxN - 1 + kSeg];
    __shared__ int32_t s_pat[kMaxN];
    __shared__ uint32_t s_w[kWaves];
    const int b = blockIdx.x;
    const int l = threadIdx.x;
    const int32_t* h = P.history + static_cast<size_t>(b) * P.max_len;
    const int L = min(max(P.hist_len[b], 0), P.max_len);
    const int halo = P.n_max - 1;
    // the pattern: pat[k] = h[L-1-k]
    if (l < P.n_max && l < L) s_pat[l] = h[L - 1 - l];
    uint32_t best = 0;  // (l << 24) | e; 0: none
    const int e_end = L - 1;  // candidate end positions e < L-1
    for (int p0 = 0; p0 < e_end; p0 += kSeg) {
        const int p1 = min(p0 + kSeg, e_end);
        const int lo = max(p0 - halo, 0);  // first position held in LDS
        // every load of the segment in flight at once
        int32_t v[kLoadsPerLane];
#pragma unroll
        for (int i = 0; i < kLoadsPerLane; ++i) {
            const int p = p0 + l + i * kThreads;
            v[i] = p < p1 ? h[p] : 0;
        }
        int32_t hv = 0;
        if (l < p0 - lo) hv = h[lo + l];  // halo (lo + l < p0)
        __syncthreads();  // the previous segment's readers are done
        if (l < p0 - lo) s_h[l] = hv;
#pragma unroll
        for (int i = 0; i < kLoadsPerLane; ++i) {
            const int p = p0 + l + i * kThreads;
            if (p < p1) s_h[p - lo] = v[i];
        }
        __syncthreads();
        // score the positions this lane owns (ascending, so the last best wins)
        for (int i = 0; i < kLoadsPerLane; ++i) {
            const int e = p0 + l + i * kThreads;
            if (e >= p1) break;
            int k = 0;
            while (k < P.n_max && e - k >= 0 && s_h[e - k - lo] == s_pat[k]) ++k;
            if (k >= P.n_min) {
                const uint32_t key = (static_cast<uint32_t>(k) << 24) | static_cast<uint32_t>(e);
                best = key > best ? key : best;
            }
        }
    }
    // block maximum of the keys
    best = wave_umax(best);
    if (l % kWave == 0) s_w[l / kWave] = best;
    __syncthreads();
    uint32_t key = s_w[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) key = s_w[w] > key ? s_w[w] : key;
    const int n = static_cast<int>(key >> 24);
    const int first = static_cast<int>(key & 0xffffffu) + 1;  // the token after the occurrence
    const int cnt = key ? min(P.G, L - first) : 0;
    if (l < P.G) P.tokens[static_cast<size_t>(b) * P.G + l] = l < cnt ? h[first + l] : -1;
    if (l == 0) {
        P.count[b] = cnt;
        if (P.match) P.match[b] = n;
    }
}

bool valid_ngram(const specdec_ngram_desc_t* d) {
    if (!d) return false;
    if (d->batch < 0 || d->batch > 65535 || d->max_len < 1 || d->max_len >= (1 << 24)) return false;
    if (d->n_min < 1 || d->n_max < d->n_min || d->n_max > kMaxN) return false;
    if (d->gamma_max < 0 || d->gamma_max > 63 || d->reserved != 0) return false;
    return true;
}

}  // namespace
}  // namespace specdec

using namespace specdec;

extern "C" specdec_status_t specdec_propose_ngram(const specdec_ngram_desc_t* d,
                                                  const int32_t* history, const int32_t* hist_len,
                                                  int32_t* draft_tokens, int32_t* num_drafts,
                                                  int32_t* match_len, hipStream_t stream) {
    if (!valid_ngram(d)) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (!history || !hist_len || !num_drafts || (d->gamma_max > 0 && !draft_tokens))
        return SPECDEC_ERR_INVALID_ARGUMENT;
    if (d->batch == 0) return SPECDEC_OK;
    NgramParams P{};
    P.history = history;
    P.hist_len = hist_len;
    P.tokens = draft_tokens;
    P.count = num_drafts;
    P.match = match_len;
    P.B = d->batch;
    P.max_len = d->max_len;
    P.n_min = d->n_min;
    P.n_max = d->n_max;
    P.G = d->gamma_max;
    hipLaunchKernelGGL(k_propose_ngram, dim3(d->batch), dim3(kThreads), 0, stream, P);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
}
