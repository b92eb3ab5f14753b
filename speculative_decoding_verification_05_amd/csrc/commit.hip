// specdec_commit_kv: the commit half of a speculative-decoding round.
//
// After verification keeps m drafts, the K/V of the pending token and of the
// m accepted drafts become cache history and the rejected entries must not
// stay readable; the cache length becomes t + m + 1 (AI-infra KB M013 s.06;
// "Speculative decoding tutorial" s.5.2: trim to t+m, the replacement then
// makes t+m+1; "The apprentice's draft" s.5.4: of the gamma+1 entries the
// verify pass produced, the accepted ones are written into the cache, on a
// paged (block-table) cache).
//
// specdec_rollback_kv runs the same kernel on the draft model's cache with
// no scratch: the draft wrote its own entries for positions t..t+gamma-1
// while proposing, so the kept ones stay where they are, positions
// t+m+1..t+gamma-1 are zero-filled and the length becomes t+min(m+1, gamma)
// (KB M013 s.06: both caches return to the committed context; tutorial
// s.5.1-5.3: equal lengths, trim to the accepted prefix, and on a full accept
// the draft still has to consume its last draft and the bonus).
//
// One workgroup per (slot j, request b) moves that slot's L x 2 runs of
// H x D bf16 with 16-byte vector loads and stores: the scratch side is one
// contiguous span, the pool side one contiguous run per (layer, K|V) inside a
// physical block.  Pure copy/zero-fill traffic, bound by HBM bandwidth.
// The last workgroup of a request (arrival counter) writes the new length, so
// no workgroup can read a length that was already advanced.
#include "specdec.h"
#include "specdec_device.h"

#include <stdint.h>

namespace specdec {
namespace {

constexpr int kCopyUnroll = 8;  // 16-byte vectors per lane in flight while copying a slot

struct CommitParams {
    const uint16_t* scratch;   // [B][S][L][2][H][D]; null: draft-cache rollback
    const int32_t* slot_map;   // [B][G+1] scratch slot per window position, or null (identity)
    uint16_t* pool;            // [L][2][NB][BS][H][D]
    const int32_t* table;      // [B][maxb]
    const int32_t* accept;
    const int32_t* gamma;
    int32_t* seq_lens;
    uint32_t* flags;
    uint32_t* cnt;             // [B]
    int B, G, L, H, D, BS, maxb, S;
    int64_t NB;
    int hd;                    // H * D elements per run
};

// Window position j of request b (one workgroup).
template <bool VEC>
__device__ __forceinline__ void commit_slot(const CommitParams& P, const int j, const int b) {
    // independent loads first (the slot map entry is in bounds for every j)
    const int g = P.gamma ? P.gamma[b] : P.G;
    const int m = P.accept[b];
    const int t = P.seq_lens[b];
    const int mapped = P.slot_map ? P.slot_map[static_cast<size_t>(b) * (P.G + 1) + j] : j;
    const bool rollback = P.scratch == nullptr;
    const bool valid = g >= 0 && g <= P.G && m >= 0 && m <= g && t >= 0;
    if (!valid || j > g) {
        // past the window, or a request left untouched (flagged once)
        const bool bad = (g < 0 || g > P.G) || (!valid && j == 0);
        if (bad && threadIdx.x == 0 && P.flags) atomicOr(P.flags + b, SPECDEC_FLAG_BAD_BLOCK);
        return;
    }
    const bool work = rollback ? (j > m && j < g) : true;
    const int64_t pos = static_cast<int64_t>(t) + j;
    const int64_t lb = pos / P.BS;
    const int off = static_cast<int>(pos % P.BS);
    const int32_t phys = (work && lb < P.maxb) ? P.table[static_cast<size_t>(b) * P.maxb + lb] : -1;
    const bool keep = work && !rollback && j <= m;
    const size_t runs = static_cast<size_t>(P.L) * 2;
    const int slot = keep ? mapped : 0;
    const bool slot_ok = slot >= 0 && slot < P.S;
    const uint16_t* src = P.scratch ? P.scratch + (static_cast<size_t>(b) * P.S + (slot_ok ? slot : 0)) * runs * P.hd
                                    : nullptr;
    // VEC: kCopyUnroll 16-byte vectors per lane per group, all loads of a
    // group issued before its stores.  The first group's source loads go out
    // together with the block-table load above (they depend only on the
    // slot), so the copy does not wait for the physical block first.
    const int nv = P.hd / 8;  // 16-byte vectors per run
    const int total = static_cast<int>(runs) * nv;
    const bool load_src = keep && slot_ok;
    uint4 v[kCopyUnroll];
    auto load_group = [&](int e0) {
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int e = e0 + u * kThreads;
            v[u] = make_uint4(0u, 0u, 0u, 0u);
            if (load_src && e < total) {
                const int run = e / nv, w = e - run * nv;
                const u32x4_t x = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4_t*>(src + static_cast<size_t>(run) * P.hd + w * 8));
                v[u] = make_uint4(x.x, x.y, x.z, x.w);
            }
        }
    };
    if (VEC) load_group(threadIdx.x);
    // The new length is written by the last of the window's g+1 workgroups to
    // arrive.  Every wave of each of them has read t before the barrier, so
    // none can see an advanced length: no fence is needed, only the
    // device-scope counter.  The arrival is issued before the copy so that
    // its round trip overlaps the copy's.
    __syncthreads();
    uint32_t arrived = 0;
    if (threadIdx.x == 0) arrived = atomicAdd(P.cnt + b, 1u);
    bool bad = false;
    if (work) {
        if (phys < 0 || phys >= P.NB) {
            bad = true;
        } else {
            if (!slot_ok) {
                bad = true;
            } else if (VEC) {
                for (int e0 = threadIdx.x; e0 < total; e0 += kThreads * kCopyUnroll) {
                    if (e0 != static_cast<int>(threadIdx.x)) load_group(e0);
#pragma unroll
                    for (int u = 0; u < kCopyUnroll; ++u) {
                        const int e = e0 + u * kThreads;
                        if (e < total) {
                            const int run = e / nv, w = e - run * nv;  // run = layer * 2 + (K|V)
                            uint16_t* dst = P.pool + ((static_cast<size_t>(run) * P.NB + phys) * P.BS + off) * P.hd + w * 8;
                            *reinterpret_cast<uint4*>(dst) = v[u];
                        }
                    }
                }
            } else {
                const size_t n_el = runs * P.hd;
                for (size_t e = threadIdx.x; e < n_el; e += kThreads) {
                    const size_t run = e / P.hd, w = e % P.hd;
                    uint16_t* dst = P.pool + ((run * P.NB + phys) * P.BS + off) * P.hd + w;
                    *dst = keep ? src[run * P.hd + w] : static_cast<uint16_t>(0);
                }
            }
        }
    }
    if (threadIdx.x == 0) {
        if (bad && P.flags) atomicOr(P.flags + b, SPECDEC_FLAG_BAD_BLOCK);
        if (arrived == static_cast<uint32_t>(g)) {
            atomicExch(P.cnt + b, 0u);  // ready for the next call
            P.seq_lens[b] = t + (rollback ? min(m + 1, g) : m + 1);
        }
    }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_commit(CommitParams P) {
    commit_slot<VEC>(P, blockIdx.x, blockIdx.y);
}

// A target commit (z = 0) and a draft rollback (z = 1) of one round in one
// launch: both depend only on the accept counts, so their workgroups run
// side by side.  Each branch reads its own kernel argument directly.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_commit_pair(CommitParams A, CommitParams R) {
    if (blockIdx.z == 0) commit_slot<VEC>(A, blockIdx.x, blockIdx.y);
    else commit_slot<VEC>(R, blockIdx.x, blockIdx.y);
}

__global__ void k_fill_zero(uint32_t* p, size_t n) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

bool valid_kv(const specdec_kv_desc_t* d) {
    if (!d) return false;
    if (d->batch < 0 || d->batch > 65535 || d->gamma_max < 0 || d->gamma_max > 63) return false;
    if (d->num_layers < 1 || d->num_kv_heads < 1 || d->head_dim < 1 || d->block_size < 1)
        return false;
    if (d->max_blocks_per_req < 1 || d->num_blocks < 1 || d->scratch_slots < 0) return false;
    if (static_cast<int64_t>(d->num_kv_heads) * d->head_dim > (1 << 24)) return false;
    // element offsets inside one slot stay in 32-bit range
    if (static_cast<int64_t>(d->num_layers) * 2 * d->num_kv_heads * d->head_dim >= (int64_t{1} << 31))
        return false;
    return true;
}

specdec_status_t launch_commit(const specdec_kv_desc_t* d, const void* scratch_kv,
                               const int32_t* slot_map, void* kv_pool,
                               const int32_t* block_table, const int32_t* accept_count,
                               const int32_t* gamma, int32_t* seq_lens, uint32_t* flags,
                               void* workspace, hipStream_t stream);

}  // namespace
}  // namespace specdec

using namespace specdec;

extern "C" size_t specdec_commit_kv_workspace_bytes(const specdec_kv_desc_t* d) {
    if (!valid_kv(d)) return 0;
    return (static_cast<size_t>(d->batch) * 4 + 255) & ~static_cast<size_t>(255);
}

namespace specdec {
namespace {

// Host-side checks of a commit's arguments (accept_count checked by the callers).
specdec_status_t check_commit(const specdec_kv_desc_t* d, const void* scratch_kv, void* kv_pool,
                              const int32_t* block_table, const int32_t* slot_map,
                              int32_t* seq_lens, void* workspace, size_t workspace_bytes) {
    if (!valid_kv(d)) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (!scratch_kv || !kv_pool || !block_table || !seq_lens || !workspace)
        return SPECDEC_ERR_INVALID_ARGUMENT;
    // without a slot map, window position j reads slot j: S must cover G+1
    if (!slot_map && d->scratch_slots != 0 && d->scratch_slots < d->gamma_max + 1)
        return SPECDEC_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < specdec_commit_kv_workspace_bytes(d)) return SPECDEC_ERR_WORKSPACE_TOO_SMALL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 3u) != 0) return SPECDEC_ERR_INVALID_ARGUMENT;
    return SPECDEC_OK;
}

// ... and of a rollback's.
specdec_status_t check_rollback(const specdec_kv_desc_t* d, void* kv_pool, const int32_t* block_table,
                                int32_t* seq_lens, void* workspace, size_t workspace_bytes) {
    if (!valid_kv(d)) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (!kv_pool || !block_table || !seq_lens || !workspace) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (d->scratch_slots != 0) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < specdec_commit_kv_workspace_bytes(d)) return SPECDEC_ERR_WORKSPACE_TOO_SMALL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 3u) != 0) return SPECDEC_ERR_INVALID_ARGUMENT;
    return SPECDEC_OK;
}

}  // namespace
}  // namespace specdec

extern "C" specdec_status_t specdec_commit_kv(const specdec_kv_desc_t* d, const void* scratch_kv,
                                              void* kv_pool, const int32_t* block_table,
                                              const int32_t* accept_count, const int32_t* gamma,
                                              const int32_t* slot_map, int32_t* seq_lens,
                                              uint32_t* flags, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream) {
    const specdec_status_t st = check_commit(d, scratch_kv, kv_pool, block_table, slot_map, seq_lens,
                                             workspace, workspace_bytes);
    if (st != SPECDEC_OK) return st;
    if (!accept_count) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (d->batch == 0) return SPECDEC_OK;
    return launch_commit(d, scratch_kv, slot_map, kv_pool, block_table, accept_count, gamma,
                         seq_lens, flags, workspace, stream);
}

namespace specdec {
namespace {

// Kernel parameters of one commit (scratch_kv null: a rollback); *vec:
// whether 16-byte vectors fit the rows and both buffers' alignment.
CommitParams commit_params(const specdec_kv_desc_t* d, const void* scratch_kv,
                           const int32_t* slot_map, void* kv_pool, const int32_t* block_table,
                           const int32_t* accept_count, const int32_t* gamma, int32_t* seq_lens,
                           uint32_t* flags, void* workspace, bool* vec) {
    CommitParams P{};
    P.scratch = static_cast<const uint16_t*>(scratch_kv);
    P.slot_map = slot_map;
    P.S = d->scratch_slots > 0 ? d->scratch_slots : d->gamma_max + 1;
    P.pool = static_cast<uint16_t*>(kv_pool);
    P.table = block_table;
    P.accept = accept_count;
    P.gamma = gamma;
    P.seq_lens = seq_lens;
    P.flags = flags;
    P.cnt = static_cast<uint32_t*>(workspace);
    P.B = d->batch;
    P.G = d->gamma_max;
    P.L = d->num_layers;
    P.H = d->num_kv_heads;
    P.D = d->head_dim;
    P.BS = d->block_size;
    P.maxb = d->max_blocks_per_req;
    P.NB = d->num_blocks;
    P.hd = d->num_kv_heads * d->head_dim;
    *vec = (P.hd % 8 == 0) && (reinterpret_cast<uintptr_t>(scratch_kv) & 15u) == 0 &&
           (reinterpret_cast<uintptr_t>(kv_pool) & 15u) == 0;
    return P;
}

specdec_status_t launch_commit(const specdec_kv_desc_t* d, const void* scratch_kv,
                               const int32_t* slot_map, void* kv_pool,
                               const int32_t* block_table, const int32_t* accept_count,
                               const int32_t* gamma, int32_t* seq_lens, uint32_t* flags,
                               void* workspace, hipStream_t stream) {
    bool vec;
    const CommitParams P = commit_params(d, scratch_kv, slot_map, kv_pool, block_table, accept_count,
                                         gamma, seq_lens, flags, workspace, &vec);
    const dim3 grid(d->gamma_max + 1, d->batch);
    if (vec)
        hipLaunchKernelGGL(k_commit<true>, grid, dim3(kThreads), 0, stream, P);
    else
        hipLaunchKernelGGL(k_commit<false>, grid, dim3(kThreads), 0, stream, P);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
}

}  // namespace
}  // namespace specdec

extern "C" specdec_status_t specdec_rollback_kv(const specdec_kv_desc_t* d, void* kv_pool,
                                                const int32_t* block_table,
                                                const int32_t* accept_count, const int32_t* gamma,
                                                int32_t* seq_lens, uint32_t* flags,
                                                void* workspace, size_t workspace_bytes,
                                                hipStream_t stream) {
    const specdec_status_t st = check_rollback(d, kv_pool, block_table, seq_lens, workspace,
                                               workspace_bytes);
    if (st != SPECDEC_OK) return st;
    if (!accept_count) return SPECDEC_ERR_INVALID_ARGUMENT;
    if (d->batch == 0) return SPECDEC_OK;
    return launch_commit(d, nullptr, nullptr, kv_pool, block_table, accept_count, gamma, seq_lens,
                         flags, workspace, stream);
}

extern "C" specdec_status_t specdec_commit_and_rollback_kv(
    const specdec_kv_desc_t* d, const void* scratch_kv, void* kv_pool, const int32_t* block_table,
    const int32_t* slot_map, int32_t* seq_lens, uint32_t* flags, void* workspace,
    size_t workspace_bytes, const specdec_kv_desc_t* dd, void* draft_pool,
    const int32_t* draft_block_table, int32_t* draft_seq_lens, uint32_t* draft_flags,
    void* draft_workspace, size_t draft_workspace_bytes, const int32_t* accept_count,
    const int32_t* gamma, hipStream_t stream) {
    specdec_status_t st = check_commit(d, scratch_kv, kv_pool, block_table, slot_map, seq_lens,
                                       workspace, workspace_bytes);
    if (st != SPECDEC_OK) return st;
    st = check_rollback(dd, draft_pool, draft_block_table, draft_seq_lens, draft_workspace,
                        draft_workspace_bytes);
    if (st != SPECDEC_OK) return st;
    if (!accept_count || d->batch != dd->batch || d->gamma_max != dd->gamma_max)
        return SPECDEC_ERR_INVALID_ARGUMENT;
    // the two halves run side by side, each with its own arrival counters
    // and lengths: a shared or overlapping workspace (or length array) would
    // let their arrivals race on one counter
    auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
        const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
        return na > 0 && nb > 0 && x < y + nb && y < x + na;
    };
    if (overlap(workspace, specdec_commit_kv_workspace_bytes(d), draft_workspace,
                specdec_commit_kv_workspace_bytes(dd)) ||
        overlap(seq_lens, static_cast<size_t>(d->batch) * 4, draft_seq_lens, static_cast<size_t>(dd->batch) * 4))
        return SPECDEC_ERR_INVALID_ARGUMENT;
    if (d->batch == 0) return SPECDEC_OK;
    bool va, vr;
    const CommitParams A = commit_params(d, scratch_kv, slot_map, kv_pool, block_table, accept_count,
                                         gamma, seq_lens, flags, workspace, &va);
    const CommitParams R = commit_params(dd, nullptr, nullptr, draft_pool, draft_block_table,
                                         accept_count, gamma, draft_seq_lens, draft_flags,
                                         draft_workspace, &vr);
    if (!(va && vr)) {
        // rows that do not take 16-byte vectors: the two launches one after the other
        st = launch_commit(d, scratch_kv, slot_map, kv_pool, block_table, accept_count, gamma,
                           seq_lens, flags, workspace, stream);
        if (st != SPECDEC_OK) return st;
        return launch_commit(dd, nullptr, nullptr, draft_pool, draft_block_table, accept_count,
                             gamma, draft_seq_lens, draft_flags, draft_workspace, stream);
    }
    hipLaunchKernelGGL(k_commit_pair<true>, dim3(d->gamma_max + 1, d->batch, 2), dim3(kThreads), 0,
                       stream, A, R);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
}

extern "C" specdec_status_t specdec_workspace_clear(void* workspace, size_t bytes, hipStream_t stream) {
    if (!workspace || (bytes & 3u) != 0 || (reinterpret_cast<uintptr_t>(workspace) & 3u) != 0)
        return SPECDEC_ERR_INVALID_ARGUMENT;
    if (bytes == 0) return SPECDEC_OK;
    const size_t n = bytes / 4;
    const size_t blocks = (n + kThreads - 1) / kThreads;
    const unsigned grid = static_cast<unsigned>(blocks < 4096 ? blocks : 4096);
    hipLaunchKernelGGL(k_fill_zero, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<uint32_t*>(workspace), n);
    return hipGetLastError() == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_DEVICE;
}

extern "C" const char* specdec_status_string(specdec_status_t s) {
    switch (s) {
        case SPECDEC_OK: return "SPECDEC_OK";
        case SPECDEC_ERR_INVALID_ARGUMENT: return "SPECDEC_ERR_INVALID_ARGUMENT: bad descriptor or pointer";
        case SPECDEC_ERR_WORKSPACE_TOO_SMALL: return "SPECDEC_ERR_WORKSPACE_TOO_SMALL";
        case SPECDEC_ERR_UNSUPPORTED: return "SPECDEC_ERR_UNSUPPORTED: request not implemented";
        case SPECDEC_ERR_DEVICE: return "SPECDEC_ERR_DEVICE: HIP launch failed";
    }
    return "unknown specdec status";
}

extern "C" int32_t specdec_abi_version(void) { return SPECDEC_ABI_VERSION; }
