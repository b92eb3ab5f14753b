// specdec_verify_tree: greedy verification of a draft tree on gfx950.
//
// What is computed ("The apprentice's draft" s.5.3: the target checks every
// node of a draft tree in one forward and the longest accepted root-to-leaf
// path is kept; the greedy rule of "Speculative decoding tutorial" s.3-4 and
// AI-infra KB M013 s.03 on every edge):
//   - g_j = argmax of target row j (raw logits, lowest index on ties): the
//     target's next token after the path root..j;
//   - node j >= 1 is kept iff its parent is kept and token_j == g_parent(j);
//   - the committed path ends at the deepest kept node (lowest node index
//     among equally deep ones) and is followed by g of that node.
//
// Kernels (HBM-bandwidth bound, no matrix cores):
//   k_tree_fused     (default) one launch: the statistics workgroups of every
//                    request (greedy mode over the N rows of each tree, one
//                    (max, lowest index) word per (chunk, row), published
//                    with an atomic exchange), then one decision workgroup
//                    per request, which collects its request's words (all
//                    launched before it) and decides as k_decide_tree.
//   k_stats          (stats.hip) + k_decide_tree, the two-kernel path
//                    (SPECDEC_FUSED=0): one streaming read with one partial
//                    per (chunk, row), then one workgroup per request.
// The decision: row argmaxes from the partials, then one wave with a lane
// per node: edge matches, pointer jumping (log2 N rounds of lane shuffles)
// for "every ancestor kept" and the depth, a ballot for the deepest kept
// node, the path, and every output (round end shared with specdec_verify).
#include "stats_stream.h"

#include <hip/hip_ext.h>
#include <stdint.h>

namespace specdec {
namespace {

// Tree decision of request b.  FUSED: the partials are the words the same
// kernel's statistics workgroups publish (collect_greedy); otherwise those
// the statistics kernel stored.
template <bool FUSED, bool BF16 = true, bool VEC = true>
__device__ __forceinline__ void decide_tree(const VerifyParams& P, const int b) {
    __shared__ float4 s_part[kMaxPart];
    __shared__ int s_arg[64];
    __shared__ uint32_t s_nan[64];
    __shared__ int s_par[64];
    __shared__ int s_path[64];
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    const int N = P.G + 1;
    const int n = tree_nodes(P, b);
    // independent loads first: partials, the node's token and parent
    if constexpr (!FUSED) {
        const float4* src = P.part + static_cast<size_t>(b) * P.rows * P.nc;
        for (int t = threadIdx.x; t < n * P.nc; t += kThreads) s_part[t] = src[t];
    }
    int tok = -1, par = 0;
    if (w == 0 && l < n && l > 0) {
        tok = P.tokens[static_cast<size_t>(b) * N + l];
        par = P.parents[static_cast<size_t>(b) * N + l];
    }
    bool late = false;
    if constexpr (FUSED) late = collect_greedy<BF16, VEC>(P, b, [&](int s) { return s < n; }, s_part);
    __syncthreads();
    // argmax of every used row: a lane per row over a few partials, else a wave
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
        for (int s = threadIdx.x; s < n; s += kThreads) {
            ArgMax best{neg_inf(), 0x7fffffff};
            uint32_t nan = 0;
            part_argmax(s, 0, 1, best, nan);
            s_arg[s] = best.i;
            s_nan[s] = nan;
        }
    } else {
        for (int s = w; s < n; s += kWaves) {
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

    // one lane per node
    uint32_t fl = 0;
    const bool live = l < n;
    bool parent_ok = true;
    if (live && l > 0) {
        parent_ok = par >= 0 && par < l;
        if (!parent_ok) fl |= SPECDEC_FLAG_BAD_TREE;
        else if (tok < 0 || tok >= P.V) fl |= SPECDEC_FLAG_TOKEN_RANGE;
    }
    if (live && s_nan[l]) fl |= SPECDEC_FLAG_NONFINITE;
    const int up = (live && l > 0 && parent_ok) ? par : 0;  // pointer to the parent (root: itself)
    s_par[l] = up;
    int ok = (l == 0) ? 1 : (live && parent_ok && tok == s_arg[up]) ? 1 : 0;
    // pointer jumping: after r rounds, `a` is the ancestor 2^r levels up (or
    // the root), ok is the AND of the edge matches on the way and d the
    // distance; the root has d = 0 and points to itself, so 6 rounds give
    // every node of a 64-node tree its depth and its whole-path verdict.
    int a = up, d = (l == 0 || !live) ? 0 : 1;
#pragma unroll
    for (int r = 0; r < 6; ++r) {
        const int ok_a = __shfl(ok, a);
        const int d_a = __shfl(d, a);
        const int a_a = __shfl(a, a);
        ok &= ok_a;
        d += d_a;
        a = a_a;
    }
    // deepest kept node, lowest index among equals
    const int key = (live && ok) ? d : -1;
    int dmax = key;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dmax = max(dmax, __shfl_xor(dmax, off));
    const uint64_t at = __ballot(key == dmax);
    const int best = __builtin_ctzll(at);
    const int m = dmax;  // >= 0: the root always qualifies
    if (l == 0) {
        int x = best;
        for (int k = m; k >= 0; --k) {
            s_path[k] = x;
            x = s_par[x];
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const int node_k = l <= m ? s_path[l] : -1;               // node at depth l
    const int next = l + 1 <= m ? s_path[l + 1] : -1;         // node at depth l+1
    const int tok_next = __shfl(tok, next < 0 ? 0 : next);    // its token
    const int c = l < m ? tok_next : s_arg[best];
    fl = wave_or(fl);
    fl |= write_round(P, b, m, c);
    if (l < N) P.path[static_cast<size_t>(b) * N + l] = node_k;
    if (l == 0 && P.flags) P.flags[b] = fl | (late ? SPECDEC_FLAG_WAIT_TIMEOUT : 0u);
}

__global__ __launch_bounds__(kThreads) void k_decide_tree(VerifyParams P) {
    decide_tree<false>(P, blockIdx.x);
}

// One-kernel tree verify: the B x S statistics workgroups (S = N rows x nc,
// request by request) first in launch order, then one decision workgroup per
// request, which waits only on statistics workgroups launched before it.
// 8 waves per SIMD (63 VGPRs, no spills): 68.7 against 69.4 us per tree
// step at the compiler's 7 (the same cap on k_greedy_fused cost 0.7 us)
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void k_tree_fused(VerifyParams P) {
    const int S = P.rows * P.nc;
    const int x = blockIdx.x;
    if (x < P.B * S) {
        const int b = x / S;
        fused_greedy_stats<BF16, VEC>(P, b, x % S, [&](int s) { return s < tree_nodes(P, b); });
    } else {
        decide_tree<true, BF16, VEC>(P, x - P.B * S);
    }
}

bool valid_tree(const specdec_tree_desc_t* d) {
    if (!d) return false;
    if (d->batch < 0 || d->batch > 65535 || d->num_nodes < 1 || d->num_nodes > 64 || d->vocab < 1)
        return false;
    if (d->dtype != SPECDEC_F32 && d->dtype != SPECDEC_BF16) return false;
    if (d->vocab > 1024 * kThreads * kUnroll2 * (d->dtype == SPECDEC_BF16 ? 8 : 4)) return false;
    if (d->eos_plus1 < 0 || d->eos_plus1 > d->vocab || d->reserved != 0) return false;
    return true;
}

// The chain verifier's layout in greedy mode with N = G+1 rows per request.
specdec_verify_desc_t as_chain_desc(const specdec_tree_desc_t* d) {
    specdec_verify_desc_t v{};
    v.batch = d->batch;
    v.gamma_max = d->num_nodes - 1;
    v.vocab = d->vocab;
    v.dtype = d->dtype;
    v.mode = SPECDEC_GREEDY;
    v.temperature = 1.0f;
    v.top_p = 1.0f;
    v.eos_plus1 = d->eos_plus1;
    return v;
}

}  // namespace
}  // namespace specdec

using namespace specdec;

extern "C" size_t specdec_verify_tree_workspace_bytes(const specdec_tree_desc_t* d) {
    if (!valid_tree(d)) return 0;
    const specdec_verify_desc_t v = as_chain_desc(d);
    return make_layout(&v).total;
}

namespace specdec {
namespace {

specdec_status_t tree_impl(const specdec_tree_desc_t* d, const void* target_logits,
                           const int32_t* node_tokens, const int32_t* parents,
                           const int32_t* num_nodes, const int32_t* max_tokens,
                           int32_t* accept_count, int32_t* num_tokens, int32_t* out_tokens,
                           int32_t* path, uint32_t* flags, void* workspace,
                           size_t workspace_bytes, hipStream_t stream, hipEvent_t* ev) {
    if (!valid_tree(d)) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (!target_logits || !node_tokens || !parents || !accept_count || !out_tokens || !path ||
        !workspace)
        return SPECDEC_ERR_INVALID_ARGUMENT;
    const specdec_verify_desc_t v = as_chain_desc(d);
    const Layout L = make_layout(&v);
    if (workspace_bytes < L.total) return SPECDEC_ERR_WORKSPACE_TOO_SMALL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (d->batch == 0) return SPECDEC_OK;
    VerifyParams P{};
    P.target = target_logits;
    P.tokens = node_tokens;
    P.nodes = num_nodes;
    P.parents = parents;
    P.path = path;
    P.max_tokens = max_tokens;
    P.accept_count = accept_count;
    P.num_tokens = num_tokens;
    P.out_tokens = out_tokens;
    P.flags = flags;
    char* ws = static_cast<char*>(workspace);
    P.part = reinterpret_cast<float4*>(ws + L.off_part);
    P.ready = reinterpret_cast<uint64_t*>(ws + L.off_ready);
    P.wait_ticks = fused_wait_ticks();
    P.B = d->batch;
    P.G = d->num_nodes - 1;
    P.V = d->vocab;
    P.rows = L.rows;
    P.nc = L.nc;
    P.chunk = L.chunk;
    P.c = 1.0f;
    P.eos = d->eos_plus1 - 1;  // -1: none
    const bool bf16 = d->dtype == SPECDEC_BF16;
    const size_t es = bf16 ? 2 : 4;
    const bool vec = (reinterpret_cast<uintptr_t>(target_logits) & 15u) == 0 &&
                     (static_cast<size_t>(d->vocab) * es) % 16 == 0;
    if (fused_enabled()) {
        // one kernel; ev[0]/ev[1] bracket it, ev[2]/ev[3] mark its end
        const dim3 grid(static_cast<unsigned>(d->batch) * (L.rows * L.nc + 1));
        auto launch = [&](auto kernel) {
            if (ev)
                hipExtLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, ev[0], ev[1], 0, P);
            else
                hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, P);
        };
        if (bf16) vec ? launch(k_tree_fused<true, true>) : launch(k_tree_fused<true, false>);
        else vec ? launch(k_tree_fused<false, true>) : launch(k_tree_fused<false, false>);
        // (any entry may be NULL)
        if (ev && ev[2] && hipEventRecord(ev[2], stream) != hipSuccess) return SPECDEC_ERR_DEVICE;
        if (ev && ev[3] && hipEventRecord(ev[3], stream) != hipSuccess) return SPECDEC_ERR_DEVICE;
        return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
    }
    if (launch_stats(P, bf16, vec, true, dim3(L.nc, L.rows, d->batch), stream,
                     ev ? ev[0] : nullptr, ev ? ev[1] : nullptr) != SPECDEC_OK)
        return SPECDEC_ERR_DEVICE;
    if (ev)
        hipExtLaunchKernelGGL(k_decide_tree, dim3(d->batch), dim3(kThreads), 0, stream, ev[2],
                              ev[3], 0, P);
    else
        hipLaunchKernelGGL(k_decide_tree, dim3(d->batch), dim3(kThreads), 0, stream, P);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
}

}  // namespace
}  // namespace specdec

extern "C" specdec_status_t specdec_verify_tree(const specdec_tree_desc_t* d,
                                                const void* target_logits,
                                                const int32_t* node_tokens,
                                                const int32_t* parents, const int32_t* num_nodes,
                                                const int32_t* max_tokens, int32_t* accept_count,
                                                int32_t* num_tokens, int32_t* out_tokens,
                                                int32_t* path, uint32_t* flags, void* workspace,
                                                size_t workspace_bytes, hipStream_t stream) {
    return tree_impl(d, target_logits, node_tokens, parents, num_nodes, max_tokens, accept_count,
                     num_tokens, out_tokens, path, flags, workspace, workspace_bytes, stream,
                     nullptr);
}

extern "C" specdec_status_t specdec_verify_tree_profiled(
    const specdec_tree_desc_t* d, const void* target_logits, const int32_t* node_tokens,
    const int32_t* parents, const int32_t* num_nodes, const int32_t* max_tokens,
    int32_t* accept_count, int32_t* num_tokens, int32_t* out_tokens, int32_t* path,
    uint32_t* flags, void* workspace, size_t workspace_bytes, hipStream_t stream,
    hipEvent_t* stage_events) {
    return tree_impl(d, target_logits, node_tokens, parents, num_nodes, max_tokens, accept_count,
                     num_tokens, out_tokens, path, flags, workspace, workspace_bytes, stream,
                     stage_events);
}
