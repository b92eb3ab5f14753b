// Internal interface shared by the verify kernels (verify.hip) and the
// truncation kernels (truncate.hip): the per-call parameter block and small
// device helpers.  Not part of the public ABI.
#pragma once

#include "specdec.h"
#include "specdec_device.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

namespace specdec {

constexpr int kUnroll = 4;        // 16-byte vectors per lane per tile, statistics pass
constexpr int kUnroll2 = 2;       // per row per tile, sampling pass
constexpr int kMaxPart = 512;     // partials per request the decision kernels stage in LDS
constexpr int kTruncCap = 2048;   // vocabulary limit of top-p without an effective top-k
constexpr int kMassGroupWide = 4;    // sampling-pass chunks loaded at once (short shares)
constexpr int kMassGroupChunks = 2;  // ... and per double-buffered group (long shares)
constexpr int kSerialParts = 16;  // at most this many partials per row: one lane combines them
constexpr int kNucCap = 1024;     // kept tokens recorded per row (and the top-k limit)
constexpr size_t kResidCachedBytes = size_t{64} << 20;  // see verify_impl: residual loads cached up to this



struct VerifyParams {
    const void* target;
    const void* draft;
    const int32_t* tokens;
    const int32_t* gamma;
    const int32_t* nodes;       // tree mode: [B] node counts (rows used), or null
    const int32_t* parents;     // tree mode: [B][G+1] parent of each node
    int32_t* path;              // tree mode: [B][G+1] kept path (output)
    const int32_t* max_tokens;  // [B] token budget of the round, or null
    int32_t* accept_count;
    int32_t* num_tokens;        // [B] or null
    int32_t* out_tokens;
    float* p_draft;
    float* q_draft;
    float* residual_mass;
    uint32_t* flags;
    // workspace
    float4* part;       // [B][R][nc] chunk partials, R = 2G+1 (sample) or G+1 (greedy)
    uint32_t* cnt;      // [B] arrivals in the sampling pass
    uint32_t* csum;     // [B][nc2] chunk masses of the sampling pass (float bits)
    uint64_t* ready;    // [B][R][nc] one-kernel path: published (max, sum) words, 0 at rest
    uint64_t* cmass;    // [B][nc2] one-kernel path: published chunk masses, 0 at rest
    int lag;            // one-kernel path: decision workgroups trail by this many requests
    uint64_t wait_ticks;  // one-kernel path: bound of a decision workgroup's wait
    int B, G, V;
    int rows;           // R
    int nc, chunk;      // statistics pass: chunks per row, elements per chunk
    int nc2, chunk2;    // sampling pass: chunks per row, elements per chunk (one tile)
    int wpr, cpw;       // sampling pass: workgroups per request, chunks per workgroup
    float c;            // log2(e) / T
    uint32_t key0, key1, round;
    int eos;            // end-of-sequence token, -1: none
    bool point;         // sampling with point-mass drafts: no draft rows, q_i = delta(d_i)
    bool resid_cached;  // one-kernel sampling pass: ordinary (cached) loads for the residual / bonus rows
    // truncation (top-k / top-p) mode
    int top_k;          // 0 or >= V: no top-k
    float top_p;        // 1: no top-p
    uint2* nuc;         // [B][R][1 + kNucCap] kept-token records
    uint4* cut;         // [B][R] cut records: (max, kept mass, boundary logit, last kept index at it)
};

// gamma_b clamped into [0, G] (an out-of-range value is flagged by the
// decision step), so no row past the padded layout is ever addressed.
__device__ __forceinline__ int request_gamma(const VerifyParams& P, int b) {
    const int g = P.gamma ? P.gamma[b] : P.G;
    return min(max(g, 0), P.G);
}

// Tree mode: nodes of request b clamped into [1, G+1] (G+1 = padded nodes).
__device__ __forceinline__ int tree_nodes(const VerifyParams& P, int b) {
    const int n = P.nodes ? P.nodes[b] : P.G + 1;
    return min(max(n, 1), P.G + 1);
}

__device__ __forceinline__ uint32_t gamma_flag(const VerifyParams& P, int b) {
    const int g = P.gamma ? P.gamma[b] : P.G;
    return (g < 0 || g > P.G) ? SPECDEC_FLAG_BAD_GAMMA : 0u;
}

__device__ __forceinline__ const void* row_ptr(const void* base, size_t row, int V, bool bf16) {
    return static_cast<const char*>(base) + row * static_cast<size_t>(V) * (bf16 ? 2 : 4);
}

__device__ __forceinline__ const void* target_row(const VerifyParams& P, int b, int i, bool bf16) {
    return row_ptr(P.target, static_cast<size_t>(b) * (P.G + 1) + i, P.V, bf16);
}

__device__ __forceinline__ const void* draft_row(const VerifyParams& P, int b, int i, bool bf16) {
    return row_ptr(P.draft, static_cast<size_t>(b) * P.G + i, P.V, bf16);
}

// Cross-workgroup hand-off.  A device-scope fence costs an L2 write-back and
// invalidate, and those serialise per XCD (measured: ~0.4 us each, which made
// a fence per workgroup dominate a pass).  Instead, the words another
// workgroup must read are published with device-scope atomic exchanges and
// read back with atomic read-modify-writes; both are performed at the
// device's coherence point, so no cache maintenance is needed.  The arrival
// increment uses an address that depends on the exchanges' returned values
// (through an empty asm statement the optimiser cannot see through), so it is
// issued only once the published words have landed.
__device__ __forceinline__ uint32_t publish(uint32_t* p, uint32_t v) { return atomicExch(p, v); }
__device__ __forceinline__ uint32_t fetch(uint32_t* p) { return atomicOr(p, 0u); }

// Arrival at a per-request counter; lane 0 passes the OR of its publish()
// results as `dep`.  Returns true (to every lane) in the last workgroup to
// arrive, which may then fetch() what the others published.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t total, uint32_t dep) {
    __shared__ int s_last;
    if (threadIdx.x == 0) {
        uint32_t zero = 0u;
        asm volatile("" : "+v"(zero) : "v"(dep));
        const uint32_t old = atomicAdd(counter + zero, 1u);
        s_last = (old == total - 1);
        if (s_last) atomicExch(counter, 0u);  // ready for the next call
    }
    __syncthreads();
    return s_last;
}

// Round end, on one wave (lane i = position i, i <= G).  The list the round
// would commit is c_0..c_m: the accepted drafts d_0..d_{m-1}, then the drawn
// token x; lane i passes c_i (ignored past m).  The list is cut after its
// first end-of-sequence token and after the request's token budget (AI-infra
// KB M013 s.03; "Speculative decoding tutorial" s.11 and s.5.2).  Writes
// out_tokens (-1 past the cut), accept_count (drafts left: min(m, n)) and
// num_tokens (n); returns the EOS / LENGTH flag bits (same in every lane).
__device__ __forceinline__ uint32_t write_round(const VerifyParams& P, int b, int m, int c) {
    const int i = threadIdx.x % kWave;
    int n = m + 1;
    uint32_t fl = 0;
    int e = 64;
    if (P.eos >= 0) {
        const uint64_t hit = __ballot(i <= m && c == P.eos);
        if (hit) e = __builtin_ctzll(hit);
        n = min(n, e + 1);
    }
    if (P.max_tokens) {
        const int cap = max(P.max_tokens[b], 0);
        if (cap <= n) {
            n = cap;
            fl |= SPECDEC_FLAG_LENGTH;
        }
    }
    if (e < n) fl |= SPECDEC_FLAG_EOS;
    int32_t* out = P.out_tokens + static_cast<size_t>(b) * (P.G + 1);
    if (i <= P.G) out[i] = i < n ? c : -1;
    if (i == 0) {
        P.accept_count[b] = min(m, n);
        if (P.num_tokens) P.num_tokens[b] = n;
    }
    return fl;
}

// Sum over the kThreads lanes of a workgroup (same value returned to all).
__device__ __forceinline__ float block_sum(float v) {
    __shared__ float s_v[kWaves];
    v = wave_sum(v);
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    __syncthreads();
    if (l == 0) s_v[w] = v;
    __syncthreads();
    float r = s_v[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) r += s_v[k];
    return r;
}

// Tuning and test switches.  The product library reads no environment: it
// always takes the measured defaults below.  The debug build of the same
// sources (libspecdec_debug.so, compiled with SPECDEC_DEBUG_KNOBS) reads
// SPECDEC_FUSED, SPECDEC_FUSED_WAIT_TICKS, SPECDEC_FUSED_LAG,
// SPECDEC_STATS_TILES, SPECDEC_SAMPLE_WPR and SPECDEC_TRUNC_CUT, for the tests that compare
// paths or force a timeout, and for tuning sweeps.
constexpr uint64_t kFixedWaitTicks = 2000000ull;  // 20 ms of the 100 MHz constant clock

inline const char* debug_knob(const char* name) {
#ifdef SPECDEC_DEBUG_KNOBS
    const char* s = getenv(name);
    return (s && *s) ? s : nullptr;
#else
    (void)name;
    return nullptr;
#endif
}

// One-kernel paths (statistics and decision workgroups in one launch) for
// sampling without truncation, greedy chains and greedy trees; the debug
// build's SPECDEC_FUSED=0 selects the two-kernel paths.
inline bool fused_enabled() {
    const char* s = debug_knob("SPECDEC_FUSED");
    return !(s && s[0] == '0');
}

// First bound of a one-kernel decision workgroup's waits (20 ms; the debug
// build's SPECDEC_FUSED_WAIT_TICKS lowers it to force the recompute path).
// A wait that gives up computes the missing partial itself; the late word is
// then drained under the fixed 20 ms bound so the workspace stays clean.
inline uint64_t fused_wait_ticks() {
    const char* s = debug_knob("SPECDEC_FUSED_WAIT_TICKS");
    return s ? strtoull(s, nullptr, 10) : kFixedWaitTicks;
}

// Workspace layout and chunking of one verify call (shared by the chain and
// tree entry points).
struct Layout {
    int rows, nc, chunk, nc2, chunk2, wpr, cpw;
    int group;          // sampling-pass chunks loaded together (1..kMassGroupWide)
    int fwpr, fcpw;     // one-kernel path: decision workgroups per request, chunks each
    bool trunc;
    bool cut;           // truncation by cut records (kept sets not listed)
    size_t off_cnt, off_ready, off_cmass, off_part, off_csum, off_nuc, total;
};
// point: sampling with point-mass drafts (no draft rows)
Layout make_layout(const specdec_verify_desc_t* d, bool point = false);

// The statistics pass (one partial per chunk of every used row); start/stop
// events (either may be null) bracket the kernel.
specdec_status_t launch_stats(const VerifyParams& P, bool bf16, bool vec, bool greedy, dim3 grid,
                              hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// Truncation mode (top-k and/or top-p): one pass that selects and records
// every used row's kept tokens, then the per-request decision over them.
specdec_status_t launch_truncated(const VerifyParams& P, bool bf16, bool vec, hipStream_t stream,
                                  hipEvent_t* ev);

// Truncation whose kept set is not listed (top-p without an effective top-k,
// or top-k past kNucCap): the cut record of every used row, from the row and
// its statistics partials (run the statistics pass first).  start/stop
// events (both null, or both set) bracket the kernel.
specdec_status_t launch_trunc_cut(const VerifyParams& P, bool bf16, bool vec, hipStream_t stream,
                                  hipEvent_t start, hipEvent_t stop);

}  // namespace specdec
