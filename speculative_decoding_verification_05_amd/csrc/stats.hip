// k_stats: the one full pass over every used logits row of specdec_verify.
//
// Each workgroup streams one chunk of one row with branch-free 16-byte loads
// (four per lane per tile, the next tile in flight while the current one is
// reduced) and stores one partial: the online-softmax pair (max, sum of
// 2^((z - max) c)) plus the logit at the drafted token in sampling mode
// (the softmax of z/T: AI-infra KB M013 s.04; "Speculative decoding
// tutorial" s.7.1), or (max, lowest index) in greedy mode (tutorial s.3-4).
// No atomics and no cross-workgroup traffic: the kernel boundary publishes
// the partials to the decision pass.  HBM-bandwidth bound, no matrix cores.
#include "stats_stream.h"

#include <hip/hip_ext.h>

namespace specdec {
namespace {

// ------------------------------------------------------------------ statistics pass

// Workgroup (chunk ci, row slot s, request b).  Slots 0..G are target rows,
// G+1..2G draft rows (sampling only).  Rows past gamma_b are abandoned after
// their first loads are issued, so the gamma_b load never stalls the stream.
template <bool BF16, bool VEC, bool GREEDY>
__global__ __launch_bounds__(kThreads) void k_stats(VerifyParams P) {
    const int ci = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
    const bool is_target = s <= P.G;
    const int i = is_target ? s : s - (P.G + 1);
    const void* rp = is_target ? target_row(P, b, i, BF16) : draft_row(P, b, i, BF16);
    const int lo = ci * P.chunk;
    const int hi = min(P.V, lo + P.chunk);
    auto keep = [&]() {
        if (P.nodes) return i < tree_nodes(P, b);
        if (!P.gamma) return true;
        const int g = request_gamma(P, b);
        return is_target ? i <= g : i < g;
    };
    float4* slot = P.part + (static_cast<size_t>(b) * P.rows + s) * P.nc + ci;
    if constexpr (GREEDY) {
        ArgMax r;
        bool nan;
        if (!chunk_argmax<BF16, VEC>(rp, lo, hi, keep, &r, &nan)) return;
        if (threadIdx.x == 0) *slot = greedy_partial(r, nan);
    } else {
        // the token this row judges (target) or proposed (draft); its logit
        // rides along with the partial of the chunk that holds it
        const int d = i < P.G ? P.tokens[static_cast<size_t>(b) * P.G + i] : -1;
        MaxSum r;
        if (!chunk_maxsum<BF16, VEC>(rp, lo, hi, P.c, keep, &r)) return;
        if (threadIdx.x == 0) {
            const float zd = (d >= lo && d < hi) ? load_logit<BF16>(rp, d) : 0.0f;
            *slot = make_float4(r.m, r.s, zd, 0.0f);
        }
    }
}

}  // namespace

specdec_status_t launch_stats(const VerifyParams& P, bool bf16, bool vec, bool greedy, dim3 grid,
                              hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    auto launch = [&](auto kernel) {
        if (start || stop)
            hipExtLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, start, stop, 0, P);
        else
            hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, P);
    };
    if (bf16) {
        if (vec) greedy ? launch(k_stats<true, true, true>) : launch(k_stats<true, true, false>);
        else greedy ? launch(k_stats<true, false, true>) : launch(k_stats<true, false, false>);
    } else {
        if (vec) greedy ? launch(k_stats<false, true, true>) : launch(k_stats<false, true, false>);
        else greedy ? launch(k_stats<false, false, true>) : launch(k_stats<false, false, false>);
    }
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
}

}  // namespace specdec
