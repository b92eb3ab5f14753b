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
// winner maximises (l(e), e) over the e with l(e) >= n_min.  A lane keeps
// the best packed key (l << 24 | e) of its positions and a block maximum
// that of the workgroup.  Rows of at most 8192 tokens take one 1024-lane
// workgroup per request, the whole history in LDS (k_propose_ngram_whole);
// longer rows are split into segments of end positions, one workgroup each,
// combined by a device-scope atomic maximum, and the last segment to arrive
// writes the proposal (k_propose_ngram).  One read of the history: bound by
// HBM bandwidth and, for short histories, by latency.
#include "verify_internal.h"

#include <stdint.h>

namespace specdec {
namespace {

constexpr int kSeg = 2048;                  // end positions scored per workgroup
constexpr int kPerLane = kSeg / kThreads;   // ... per lane, kThreads apart
constexpr int kMaxN = 32;                   // largest n_max

__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
    return lane63(wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; }));
}

struct NgramParams {
    const int32_t* history;   // [B][max_len]
    const int32_t* hist_len;  // [B]
    int32_t* tokens;          // [B][G]
    int32_t* count;           // [B]
    int32_t* match;           // [B] or null
    uint32_t* key;            // [B] workspace: running best key
    uint32_t* cnt;            // [B] workspace: arrivals
    int B, max_len, n_min, n_max, G;
};

// Workgroup (segment sg, request b) scores end positions [sg*kSeg, ...).
// Lane l loads the tokens of its positions e = base + l + i*kThreads; the
// first comparison (h[e] against the history's last token) uses them
// directly, and only the positions that pass it look further back, in LDS:
// the segment with the n_max-1 tokens before it, and the pattern (the
// history's last n_max tokens, last first).
__global__ __launch_bounds__(kThreads) void k_propose_ngram(NgramParams P) {
    __shared__ int32_t s_h[kMaxN - 1 + kSeg];
    __shared__ int32_t s_pat[kMaxN];
    __shared__ uint32_t s_w[kWaves];
    const int sg = blockIdx.x, b = blockIdx.y;
    const int l = threadIdx.x;
    const int32_t* h = P.history + static_cast<size_t>(b) * P.max_len;
    const int base = sg * kSeg;
    // the segment's loads go out with the length's (the row holds max_len
    // tokens, so they are in bounds whatever the length); the entries past
    // the history are discarded below
    int32_t v[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int e = base + l + i * kThreads;
        v[i] = e < P.max_len ? h[e] : 0;
    }
    const int L = min(max(P.hist_len[b], 0), P.max_len);
    const int e_end = L - 1;                                  // end positions e < L-1
    const int nseg = e_end > 0 ? (e_end + kSeg - 1) / kSeg : 1;
    if (sg >= nseg) return;                                   // past this request's history
    const int lo = max(base - (P.n_max - 1), 0);              // first position held in LDS
    // then the halo before the segment and the pattern
    const int32_t halo = (l < base - lo) ? h[lo + l] : 0;
    const int32_t pat = (l < P.n_max && l < L) ? h[L - 1 - l] : 0;
    if (l < base - lo) s_h[l] = halo;
    if (l < P.n_max) s_pat[l] = pat;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int e = base + l + i * kThreads;
        if (e < e_end) s_h[e - lo] = v[i];
    }
    __syncthreads();
    const int32_t last = s_pat[0];
    uint32_t best = 0;  // (l << 24) | e; 0: none
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int e = base + l + i * kThreads;
        if (e < e_end && v[i] == last) {
            int k = 1;
            while (k < P.n_max && e - k >= 0 && s_h[e - k - lo] == s_pat[k]) ++k;
            if (k >= P.n_min) {
                const uint32_t key = (static_cast<uint32_t>(k) << 24) | static_cast<uint32_t>(e);
                best = key > best ? key : best;
            }
        }
    }
    best = wave_umax(best);
    if (l % kWave == 0) s_w[l / kWave] = best;
    __syncthreads();
    uint32_t key = s_w[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) key = s_w[w] > key ? s_w[w] : key;
    // combine the segments: the largest key wins; the last segment to arrive
    // writes the outputs
    uint32_t dep = 0;
    if (l == 0) dep = atomicMax(P.key + b, key);
    if (!arrive_last(P.cnt + b, static_cast<uint32_t>(nseg), dep)) return;
    __shared__ uint32_t s_key;
    if (l == 0) s_key = atomicExch(P.key + b, 0u);  // the final key, reset for the next call
    __syncthreads();
    key = s_key;
    const int n = static_cast<int>(key >> 24);
    const int first = static_cast<int>(key & 0xffffffu) + 1;  // the token after the occurrence
    const int cnt = key ? min(P.G, L - first) : 0;
    if (l < P.G) P.tokens[static_cast<size_t>(b) * P.G + l] = l < cnt ? h[first + l] : -1;
    if (l == 0) {
        P.count[b] = cnt;
        if (P.match) P.match[b] = n;
    }
}

// Rows of at most kWhole tokens: one workgroup per request.  After the
// length, every token of the history is loaded at once (8 per lane) and kept
// in LDS; positions are scored as in k_propose_ngram and the proposal is read
// back from LDS: two memory round trips and no combine across workgroups.
constexpr int kWhole = 8192;
constexpr int kWholeThreads = 1024;  // 16 waves: 8 positions per lane, as in a segment
constexpr int kWholePerLane = kWhole / kWholeThreads;
constexpr int kWholeWaves = kWholeThreads / kWave;

__global__ __launch_bounds__(kWholeThreads) void k_propose_ngram_whole(NgramParams P) {
    __shared__ int32_t s_h[kWhole];
    __shared__ uint32_t s_w[kWholeWaves];
    const int b = blockIdx.x;
    const int l = threadIdx.x;
    const int32_t* h = P.history + static_cast<size_t>(b) * P.max_len;
    const int L = min(max(P.hist_len[b], 0), P.max_len);
    int32_t v[kWholePerLane];
#pragma unroll
    for (int i = 0; i < kWholePerLane; ++i) {
        const int e = l + i * kWholeThreads;
        v[i] = e < L ? h[e] : 0;
    }
#pragma unroll
    for (int i = 0; i < kWholePerLane; ++i) {
        const int e = l + i * kWholeThreads;
        if (e < L) s_h[e] = v[i];
    }
    __syncthreads();
    const int e_end = L - 1;  // end positions e < L-1
    const int32_t last = L > 0 ? s_h[L - 1] : 0;
    uint32_t best = 0;  // (l << 24) | e; 0: none
#pragma unroll
    for (int i = 0; i < kWholePerLane; ++i) {
        const int e = l + i * kWholeThreads;
        if (e < e_end && v[i] == last) {
            int k = 1;
            while (k < P.n_max && e - k >= 0 && s_h[e - k] == s_h[L - 1 - k]) ++k;
            if (k >= P.n_min) {
                const uint32_t key = (static_cast<uint32_t>(k) << 24) | static_cast<uint32_t>(e);
                best = key > best ? key : best;
            }
        }
    }
    best = wave_umax(best);
    if (l % kWave == 0) s_w[l / kWave] = best;
    __syncthreads();
    uint32_t key = s_w[0];
#pragma unroll
    for (int w = 1; w < kWholeWaves; ++w) key = s_w[w] > key ? s_w[w] : key;
    const int n = static_cast<int>(key >> 24);
    const int first = static_cast<int>(key & 0xffffffu) + 1;  // the token after the occurrence
    const int cnt = key ? min(P.G, L - first) : 0;
    if (l < P.G) P.tokens[static_cast<size_t>(b) * P.G + l] = l < cnt ? s_h[first + l] : -1;
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

size_t ngram_workspace(const specdec_ngram_desc_t* d) {
    return (static_cast<size_t>(d->batch) * 8 + 255) & ~static_cast<size_t>(255);
}

}  // namespace
}  // namespace specdec

using namespace specdec;

extern "C" size_t specdec_propose_ngram_workspace_bytes(const specdec_ngram_desc_t* d) {
    return valid_ngram(d) ? ngram_workspace(d) : 0;
}

extern "C" specdec_status_t specdec_propose_ngram(const specdec_ngram_desc_t* d,
                                                  const int32_t* history, const int32_t* hist_len,
                                                  int32_t* draft_tokens, int32_t* num_drafts,
                                                  int32_t* match_len, void* workspace,
                                                  size_t workspace_bytes, hipStream_t stream) {
    if (!valid_ngram(d)) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (!history || !hist_len || !num_drafts || (d->gamma_max > 0 && !draft_tokens) || !workspace)
        return SPECDEC_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < ngram_workspace(d)) return SPECDEC_ERR_WORKSPACE_TOO_SMALL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 3u) != 0) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (d->batch == 0) return SPECDEC_OK;
    NgramParams P{};
    P.history = history;
    P.hist_len = hist_len;
    P.tokens = draft_tokens;
    P.count = num_drafts;
    P.match = match_len;
    P.key = static_cast<uint32_t*>(workspace);
    P.cnt = P.key + d->batch;
    P.B = d->batch;
    P.max_len = d->max_len;
    P.n_min = d->n_min;
    P.n_max = d->n_max;
    P.G = d->gamma_max;
    if (d->max_len <= kWhole) {
        hipLaunchKernelGGL(k_propose_ngram_whole, dim3(d->batch), dim3(kWholeThreads), 0, stream, P);
    } else {
        const int nseg = (d->max_len + kSeg - 1) / kSeg;
        hipLaunchKernelGGL(k_propose_ngram, dim3(nseg, d->batch), dim3(kThreads), 0, stream, P);
    }
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
}
