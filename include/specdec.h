/* specdec.h -- verify-and-commit step of speculative decoding on one AMD
 * Instinct MI355X (gfx950).  C ABI of libspecdec.so.
 *
 * One speculative round proposes gamma draft tokens, runs the target once over
 * the pending token plus the drafts, then (this library) decides how many
 * drafts to keep, draws the next token, and commits the surviving K/V entries:
 *
 *   specdec_verify     temperature (+ optional top-k / top-p) on target and
 *                      draft rows, the min(1, p/q) acceptance test (or argmax
 *                      equality in greedy mode), the longest contiguous
 *                      accepted prefix, then the correction token from
 *                      normalize(max(p - q, 0)) or the bonus token from the
 *                      last target row.
 *   specdec_commit_kv  copies the K/V of the kept slots into a paged cache,
 *                      invalidates the rejected slots and sets the new length.
 *   specdec_rollback_kv  brings the draft model's paged cache back to the
 *                      committed sequence.
 *   specdec_commit_and_rollback_kv  both of the above for one round, in one
 *                      launch.
 *
 * Passages defining these operations (page title, section):
 *   - "Speculative decoding tutorial: from distribution preservation and
 *     KV-cache rollback to break-even": s.2 (four stages, contiguous prefix),
 *     s.3-4 (greedy verification, logits alignment table), s.5.2-5.3
 *     (rollback to t+m then t+m+1; bonus token), s.7.1-7.3 (acceptance
 *     probability, residual distribution, left-to-right over positions),
 *     s.13.2 (keep decisions on the GPU; no per-token host sync).
 *   - AI-infra knowledge base page M013: s.03 (greedy walk-through), s.04
 *     (p and q are the distributions after temperature and truncation), s.05
 *     (three-option example), s.06 (commit or roll back the caches).
 *   - "The apprentice's draft" (engineering half): s.2 Steps 2-4; s.5.4 (the
 *     gamma+1 K/V entries of the verify pass, accepted ones written back).
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers to caller-owned memory; the
 *     descriptor structs are HOST pointers read during the call only.  The
 *     library allocates nothing and holds no state between calls.
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call
 *     returns without synchronising; outputs are valid once the stream has
 *     reached that point.  Nothing is copied back to the host.
 *   - A non-OK status means that NOTHING was enqueued (argument errors are
 *     found on the host before any launch), except SPECDEC_ERR_DEVICE, which
 *     reports a launch failure from the HIP runtime.  Launches are checked
 *     with hipGetLastError, which also returns (and clears) an error that an
 *     earlier HIP call on the calling thread left pending: check and clear
 *     your own calls' errors before calling in.
 *   - Data anomalies (a draft token outside [0,V), a non-finite logit, an
 *     empty residual, an unusable block-table entry) never change the status;
 *     they are reported per request in the optional `flags` output.
 *   - Calls that share a workspace must be ordered (same stream, or
 *     synchronised streams): concurrent calls on one workspace race.
 */
#ifndef SPECDEC_H
#define SPECDEC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPECDEC_ABI_VERSION 3

typedef enum specdec_status {
    SPECDEC_OK = 0,
    SPECDEC_ERR_INVALID_ARGUMENT = 1,   /* bad descriptor, NULL or misaligned pointer */
    SPECDEC_ERR_WORKSPACE_TOO_SMALL = 2,
    SPECDEC_ERR_UNSUPPORTED = 3,        /* valid request the library does not implement
                                           (no entry point of this version returns it) */
    SPECDEC_ERR_DEVICE = 4              /* the HIP runtime refused a launch */
} specdec_status_t;

typedef enum specdec_dtype { SPECDEC_F32 = 0, SPECDEC_BF16 = 1 } specdec_dtype_t;
typedef enum specdec_mode { SPECDEC_SAMPLE = 0, SPECDEC_GREEDY = 1 } specdec_mode_t;

/* Per-request flag bits (the `flags` outputs). */
#define SPECDEC_FLAG_RESIDUAL_FALLBACK 0x2u  /* rejected, but sum max(p-q,0) <= 0: sampled p */
#define SPECDEC_FLAG_NONFINITE         0x4u  /* NaN or +inf in a used logits row */
#define SPECDEC_FLAG_TOKEN_RANGE       0x8u  /* a draft token outside [0,V): rejected */
#define SPECDEC_FLAG_BAD_BLOCK         0x10u /* commit: window not committable, slot(s) skipped */
#define SPECDEC_FLAG_BAD_GAMMA         0x20u /* verify: gamma_b outside [0,G], clamped into it */
#define SPECDEC_FLAG_TRUNC_OVERFLOW    0x40u /* verify: a kept set exceeded 1024 tokens (ties): clipped */
#define SPECDEC_FLAG_EOS               0x80u /* verify: the committed list ends with the EOS token */
#define SPECDEC_FLAG_LENGTH            0x100u /* verify: the token budget ended the committed list */
#define SPECDEC_FLAG_BAD_TREE          0x200u /* tree: a parent index outside [0, node): node rejected */
#define SPECDEC_FLAG_WAIT_TIMEOUT      0x400u /* verify, verify_tree: in a one-kernel path
                                                 (sampling without truncation, greedy, tree)
                                                 a decision workgroup gave up waiting (20 ms)
                                                 for a partial of the request and computed it
                                                 itself from the logits: the outputs are
                                                 still valid.  The late partial is then awaited
                                                 another 20 ms and taken; only if it never
                                                 came may a workspace word stay set, and the
                                                 workspace must be cleared before its next use */

/* ------------------------------------------------------------------ verify */

typedef struct specdec_verify_desc {
    int32_t batch;        /* B in [0, 65535] requests */
    int32_t gamma_max;    /* G in [0, 63]: padded draft length */
    int32_t vocab;        /* V >= 1; at most 4194304 (bf16) / 2097152 (fp32) */
    int32_t dtype;        /* specdec_dtype_t of both logits tensors */
    int32_t mode;         /* specdec_mode_t */
    int32_t top_k;        /* SAMPLE only: 0 = off, else keep logits >= k-th largest */
    float temperature;    /* SAMPLE only: > 0 and finite */
    float top_p;          /* SAMPLE only: (0, 1]; 1 = off */
    uint64_t seed;        /* Philox4x32-10 key (low word, high word) */
    uint32_t round;       /* Philox counter word 2 (make it differ per round) */
    int32_t eos_plus1;    /* 0: no end-of-sequence handling (so a zero-filled
                             descriptor has none); else the EOS token id + 1,
                             in [1, V] */
} specdec_verify_desc_t;

/* Bytes of device workspace specdec_verify needs for `desc` (0 on a bad
 * descriptor).  The workspace holds per-chunk partial statistics, per-request
 * arrival counters and hand-off words.  Its counter words must be zero before the
 * first call that uses it (allocate it zero-filled, or run
 * specdec_workspace_clear once); every completed call leaves them zero again,
 * so one workspace serves any number of ordered calls with one descriptor.
 * Clear it again before using it with another descriptor (the counters of one
 * layout may lie where another left partials).  Rounded to 256 B. */
size_t specdec_verify_workspace_bytes(const specdec_verify_desc_t* desc);

/* Verify one round for B requests.
 *
 * Round end (AI-infra KB M013 s.03: an end-of-sequence token or the output
 * length limit can end a round early; "Speculative decoding tutorial" s.11:
 * decoding continues while fewer than max_new_tokens were produced and stops
 * right after emitting EOS; s.5.2: nothing after an EOS in the candidate
 * block may reach the cache).  The list a round commits is d_0..d_{m-1} and
 * then the correction or bonus token; it is cut after its first EOS token
 * (desc->eos_plus1 > 0) and after max_tokens[b] tokens.  accept_count then
 * counts the drafts left in the list, so specdec_commit_kv and
 * specdec_rollback_kv keep exactly the committed tokens' K/V.
 *
 * Inputs (device, row-major, 16-byte aligned for full speed):
 *   target_logits [B][G+1][V] dtype: row i of request b is the target's
 *       distribution that judges draft token i (row 0 is produced by the
 *       pending token, i.e. the last committed token whose K/V is not yet in
 *       the cache); row gamma_b yields the bonus token.
 *   draft_logits  [B][G][V] dtype: row i is the draft distribution that
 *       proposed draft token i.  Not read in GREEDY mode (may be NULL).  NULL
 *       in SAMPLE mode means a deterministic proposer (specdec_propose_ngram):
 *       q_i is the point mass on d_i, so draft i is accepted with probability
 *       p_i(d_i) and a rejection draws from p_i with d_i removed (AI-infra KB
 *       M013 s.08 asks for the candidates' probability representation; the
 *       rule of s.04 then applies unchanged).  With truncation, p_i is the
 *       truncated target distribution (s.04) and q_i stays the point mass.
 *       With G = 0 there are no draft rows and NULL is simply the absent
 *       array.
 *   draft_tokens  [B][G] int32: the proposed tokens d_0..d_{gamma_b - 1}.
 *   gamma         [B] int32 in [0, G], or NULL (every request uses G).  Rows
 *       and tokens past gamma_b are never read.  A value outside [0, G] is
 *       clamped into it and flagged (SPECDEC_FLAG_BAD_GAMMA).
 *   max_tokens    [B] int32, or NULL (no limit): the most tokens request b
 *       may commit this round (its remaining output length); values below 0
 *       count as 0.
 * Outputs (device):
 *   accept_count  [B] int32: m_b, the number of leading drafts kept (after
 *       the round-end cut; without EOS or budget, the accepted prefix).
 *   num_tokens    [B] int32, or NULL: n_b, tokens committed this round
 *       (m_b + 1 unless the cut removed the drawn token).  When it is m_b + 1
 *       and neither EOS nor LENGTH is flagged, out_tokens[b][m_b] is the next
 *       round's pending token; otherwise the request has finished.
 *   out_tokens    [B][G+1] int32: d_0..d_{m-1}, then the correction (m <
 *       gamma_b) or bonus (m = gamma_b) token at index m, then -1; with a
 *       round-end cut, -1 from index n_b on.
 *   p_draft, q_draft [B][G] float, or NULL: p_i(d_i), q_i(d_i) after
 *       temperature and truncation (0 past gamma_b).  Not written in GREEDY.
 *   residual_mass [B] float, or NULL: sum_v max(p_m - q_m, 0) at the rejected
 *       position, 0 when every draft was accepted.  Not written in GREEDY.
 *   flags         [B] uint32, or NULL: SPECDEC_FLAG_* bits.
 * Randomness: two uniforms per (request b, position i) from Philox4x32-10
 *   with key = seed and counter = (i, b, round, 0); word 0 drives the accept
 *   test (accept iff u < min(1, p/q)), word 1 the inverse-CDF draw at the
 *   position where the round ends (token = min{v : cumsum(r)(v) > u R});
 *   u = (word >> 8) * 2^-24.
 * Greedy: draft i is kept iff it equals the argmax of target row i (raw
 *   logits, lowest index on ties); the token at m is the argmax of row m.
 * Errors: INVALID_ARGUMENT for a bad descriptor or a NULL required pointer;
 *   WORKSPACE_TOO_SMALL if workspace_bytes < specdec_verify_workspace_bytes.
 *   In each case nothing is enqueued.
 * Kernels: sampling without truncation and greedy verification run as one
 *   kernel (statistics and decision workgroups in one launch; the library's
 *   debug build, libspecdec_debug.so, can select a two-kernel path with the
 *   same results through SPECDEC_FUSED=0 in the environment; this library
 *   reads no environment);
 *   truncation with top_k <= 1024, or top-p alone on V <= 2048, runs a
 *   selection kernel that lists each row's kept tokens, then a decision
 *   kernel over the lists; other truncation (top-p alone on larger
 *   vocabularies, top_k > 1024, any truncation with point-mass drafts)
 *   runs the statistics pass, a kernel that
 *   finds each row's cut (the boundary logit and, among the tokens tied at
 *   it, the last kept index) by a radix select over the logits' order
 *   keys, and the sampling decision testing each token against the cut.
 * Truncation: top-k keeps every token whose raw logit is >= the k-th largest
 *   raw logit (ties kept); top-p then keeps the shortest prefix, in order of
 *   raw logit descending and token index ascending, whose cumulative
 *   probability under softmax(z/T) over the top-k set reaches top_p.  p and q
 *   are softmax(z/T) renormalised over their own kept sets, and both the
 *   acceptance test and the residual use them. */
specdec_status_t specdec_verify(const specdec_verify_desc_t* desc,
                                const void* target_logits, const void* draft_logits,
                                const int32_t* draft_tokens, const int32_t* gamma,
                                const int32_t* max_tokens,
                                int32_t* accept_count, int32_t* num_tokens, int32_t* out_tokens,
                                float* p_draft, float* q_draft, float* residual_mass,
                                uint32_t* flags,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* specdec_verify with per-pass timing for profilers and benchmarks.
 * stage_events: NULL, or a host array of 4 hipEvent_t created by the caller
 * (any entry may be NULL): [0]/[1] are recorded at the start/end of the
 * statistics pass kernel (the one full read of the logits), [2]/[3] at the
 * start/end of the decision kernel (acceptance tests and, when sampling, the
 * correction/bonus draw).  The events bracket the kernels' execution
 * (hipExtLaunchKernel), not the enqueue.  Sampling without truncation and
 * greedy verification run both passes in one kernel: [0]/[1] bracket that
 * kernel and [2]/[3] are recorded right after it.  With truncation, [0]/[1]
 * bracket the pass that dominates instead: the selection kernel that lists
 * the kept tokens, or the kernel that finds the cut records (the statistics
 * kernel launched before it is then not bracketed); [2]/[3] bracket the
 * decision kernel as above.
 * Everything else, including every error, is as for specdec_verify. */
specdec_status_t specdec_verify_profiled(const specdec_verify_desc_t* desc,
                                         const void* target_logits, const void* draft_logits,
                                         const int32_t* draft_tokens, const int32_t* gamma,
                                         const int32_t* max_tokens,
                                         int32_t* accept_count, int32_t* num_tokens,
                                         int32_t* out_tokens,
                                         float* p_draft, float* q_draft, float* residual_mass,
                                         uint32_t* flags,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream, hipEvent_t* stage_events);

/* specdec_verify for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as specdec_verify, without the
 * workspace: the library uses its own, a 16 MiB device array per GPU (held
 * until the process ends), located with hipGetSymbolAddress on the first call
 * on each device, with that device current.  The call allocates nothing.
 *   - WORKSPACE_TOO_SMALL when specdec_verify_workspace_bytes(desc) exceeds
 *     16 MiB (nothing is enqueued).
 *   - Each call first clears, on `stream`, the parts of the array that must be
 *     zero (a fill kernel, no hipMemset), so consecutive calls may use any
 *     descriptors.
 *   - All calls on one GPU share the array: calls that overlap on one GPU
 *     (different streams without ordering, several host threads) race.
 *   - `stream` must belong to the current device. */
specdec_status_t specdec_verify_noalloc(const specdec_verify_desc_t* desc,
                                        const void* target_logits, const void* draft_logits,
                                        const int32_t* draft_tokens, const int32_t* gamma,
                                        const int32_t* max_tokens,
                                        int32_t* accept_count, int32_t* num_tokens,
                                        int32_t* out_tokens,
                                        float* p_draft, float* q_draft, float* residual_mass,
                                        uint32_t* flags, hipStream_t stream);

/* ------------------------------------------------------------- commit K/V */

typedef struct specdec_kv_desc {
    int32_t batch;              /* B in [0, 65535] */
    int32_t gamma_max;          /* G in [0, 63] */
    int32_t num_layers;         /* L >= 1 */
    int32_t num_kv_heads;       /* H >= 1 */
    int32_t head_dim;           /* D >= 1 */
    int32_t block_size;         /* tokens per physical block, >= 1 */
    int32_t max_blocks_per_req; /* columns of the block table */
    int32_t scratch_slots;      /* S: K/V slots per request in the scratch; 0 = G+1
                                   (specdec_commit_kv only; must be 0 for rollback) */
    int64_t num_blocks;         /* physical blocks in the pool */
} specdec_kv_desc_t;
/* Descriptor limits checked on the host (INVALID_ARGUMENT otherwise):
 * max_blocks_per_req >= 1, num_blocks >= 1, scratch_slots >= 0, H*D <= 2^24
 * and L*2*H*D < 2^31 (element offsets inside one slot stay 32-bit). */

/* Bytes of device workspace specdec_commit_kv needs (per-request arrival
 * counters; same zero-at-first-use rule as the verify workspace). */
size_t specdec_commit_kv_workspace_bytes(const specdec_kv_desc_t* desc);

/* Commit the verified slots of one round into a paged K/V cache.
 *   scratch_kv  [B][S][L][2][H][D] bf16: the K (index 0) and V (index 1)
 *       the verify forward produced, S = desc->scratch_slots (0: G+1).
 *       Without a slot map, slot j of request b belongs to position
 *       seq_lens[b] + j (slot 0 = the pending token).
 *   slot_map    [B][G+1] int32 or NULL: position seq_lens[b] + j takes slot
 *       slot_map[b][j] (only j <= m_b is read).  For a tree round this is
 *       specdec_verify_tree's `path` ("The apprentice's draft" s.5.3: only the
 *       accepted path becomes history); a slot outside [0, S) skips that
 *       position and flags SPECDEC_FLAG_BAD_BLOCK.
 *   kv_pool     [L][2][num_blocks][block_size][H][D] bf16, updated in place.
 *   block_table [B][max_blocks_per_req] int32: physical block of each logical
 *       block; entries covering positions t_b .. t_b + gamma_b must be valid.
 *   accept_count [B] int32 (m_b, e.g. specdec_verify's output), gamma [B]
 *       int32 or NULL (= G), both device-resident.
 *   seq_lens    [B] int32, in place: in t_b (valid cache entries before the
 *       round), out t_b + m_b + 1.  Within the kernel the new length is
 *       written by the request's last workgroup to start its slot, possibly
 *       before the other workgroups' copies land; everything ordered after
 *       the call (a later kernel or copy on the stream, or after a
 *       synchronisation) sees both the new length and every placed slot.
 *   flags       [B] uint32 or NULL: SPECDEC_FLAG_BAD_BLOCK is OR-ed in when a
 *       block-table entry needed by the window is outside [0, num_blocks) or
 *       past the table (that slot is skipped), or when gamma_b, m_b or t_b is
 *       out of range (nothing of that request is touched, its length kept).
 * For j = 0..m_b the slot is copied to position t_b + j; for j = m_b+1 ..
 * gamma_b the position is zero-filled (bf16 +0.0) so no rejected entry stays
 * readable; positions outside [t_b, t_b + gamma_b] are not touched.
 * Errors: INVALID_ARGUMENT for a bad descriptor or NULL pointer;
 * WORKSPACE_TOO_SMALL; nothing is enqueued in either case. */
specdec_status_t specdec_commit_kv(const specdec_kv_desc_t* desc,
                                   const void* scratch_kv, void* kv_pool,
                                   const int32_t* block_table, const int32_t* accept_count,
                                   const int32_t* gamma, const int32_t* slot_map,
                                   int32_t* seq_lens, uint32_t* flags,
                                   void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* ------------------------------------------------------------ tree verify */

typedef struct specdec_tree_desc {
    int32_t batch;        /* B in [0, 65535] requests */
    int32_t num_nodes;    /* N in [1, 64]: padded nodes per tree, node 0 = root */
    int32_t vocab;        /* V >= 1, as for specdec_verify */
    int32_t dtype;        /* specdec_dtype_t of the target logits */
    int32_t eos_plus1;    /* 0: none; else the EOS id + 1, in [1, V] */
    int32_t reserved;     /* must be 0 */
} specdec_tree_desc_t;

/* Bytes of device workspace specdec_verify_tree needs (0 on a bad descriptor). */
size_t specdec_verify_tree_workspace_bytes(const specdec_tree_desc_t* desc);

/* Greedy verification of a draft tree ("The apprentice's draft", s.5.3: the
 * target checks all nodes of a draft tree in one forward and the longest
 * accepted path is kept; "Speculative decoding tutorial" s.13.3 and s.14:
 * tree speculation verifies several candidate branches at once).  The greedy
 * rule of specdec_verify holds on every edge: node j (j >= 1) is kept iff its
 * parent was kept and its token equals the argmax of the parent's target row
 * (raw logits, lowest index on ties).  The committed path ends at the deepest
 * kept node (lowest node index among equally deep ones); the next token is
 * the argmax of that node's row (a correction if it has children, else the
 * bonus).  The committed list is cut at EOS / max_tokens as in specdec_verify.
 * Sampling over trees is not provided (the pages give no rule for it).
 * Inputs (device):
 *   target_logits [B][N][V] dtype: row j is the target's distribution after
 *       the path root..j (the verify forward over the tree with a tree mask);
 *       node 0 is the pending token.
 *   node_tokens   [B][N] int32: token of node j (entry 0 ignored).
 *   parents       [B][N] int32: parent of node j, in [0, j) (entry 0
 *       ignored); nodes come in topological order.  A bad parent rejects the
 *       node (and so its subtree) and flags SPECDEC_FLAG_BAD_TREE.
 *   num_nodes     [B] int32 in [1, N], or NULL (= N); rows and entries past
 *       it are never read (clamped into [1, N]).
 *   max_tokens    [B] int32 or NULL: token budget, as for specdec_verify.
 * Outputs (device):
 *   accept_count  [B] int32: depth of the committed path (drafts kept, after
 *       the round-end cut).
 *   num_tokens    [B] int32 or NULL: tokens committed this round.
 *   out_tokens    [B][N] int32: the path's tokens, then the next token, -1
 *       after (cut as for specdec_verify).
 *   path          [B][N] int32: node at each depth of the kept path (path[0]
 *       = 0), -1 after; feed it to specdec_commit_kv as the slot map with
 *       scratch_slots = N.
 *   flags         [B] uint32 or NULL: BAD_TREE, TOKEN_RANGE, NONFINITE,
 *       EOS, LENGTH, WAIT_TIMEOUT.
 * Runs as one kernel (statistics and decision workgroups in one launch);
 * (The debug build selects a two-kernel path with SPECDEC_FUSED=0.)
 * Errors: INVALID_ARGUMENT (bad descriptor, NULL required pointer,
 *   misaligned workspace), WORKSPACE_TOO_SMALL; nothing is enqueued. */
specdec_status_t specdec_verify_tree(const specdec_tree_desc_t* desc, const void* target_logits,
                                     const int32_t* node_tokens, const int32_t* parents,
                                     const int32_t* num_nodes, const int32_t* max_tokens,
                                     int32_t* accept_count, int32_t* num_tokens,
                                     int32_t* out_tokens, int32_t* path, uint32_t* flags,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* specdec_verify_tree with per-kernel timing: stage_events as for
 * specdec_verify_profiled ([0]/[1] around the statistics pass, [2]/[3]
 * around the tree decision kernel).  Everything else as specdec_verify_tree. */
specdec_status_t specdec_verify_tree_profiled(const specdec_tree_desc_t* desc,
                                              const void* target_logits,
                                              const int32_t* node_tokens, const int32_t* parents,
                                              const int32_t* num_nodes, const int32_t* max_tokens,
                                              int32_t* accept_count, int32_t* num_tokens,
                                              int32_t* out_tokens, int32_t* path, uint32_t* flags,
                                              void* workspace, size_t workspace_bytes,
                                              hipStream_t stream, hipEvent_t* stage_events);

/* ------------------------------------------------------------ n-gram drafts */

typedef struct specdec_ngram_desc {
    int32_t batch;        /* B in [0, 65535] requests */
    int32_t max_len;      /* row stride of the history, in [1, 2^24) */
    int32_t n_min;        /* shortest n-gram matched, >= 1 */
    int32_t n_max;        /* longest n-gram matched, in [n_min, 32] */
    int32_t gamma_max;    /* G in [0, 63]: most tokens proposed */
    int32_t reserved;     /* must be 0 */
} specdec_ngram_desc_t;

/* Prompt-lookup / n-gram drafting (AI-infra KB M013 s.08: candidates from
 * repeated patterns in the text; "The math behind the speedup": pattern-based
 * drafting searches the existing context for a matching sequence at near-zero
 * cost; "Speculative decoding tutorial" s.13.1 and s.14: prompt lookup and
 * n-gram candidates come from the prompt or the history).  For n = n_max down
 * to n_min, the last n tokens of a request's history are looked up at their
 * most recent earlier occurrence (one that ends before the last position);
 * the first n with an occurrence wins and the tokens following it, at most G
 * and never past the end of the history, are proposed.
 *   history      [B][max_len] int32 (device): committed tokens, the pending
 *       token last; only the first hist_len[b] entries of a row are read.
 *   hist_len     [B] int32 (device), clamped into [0, max_len].
 *   draft_tokens [B][G] int32 out: the proposal, -1 after it.
 *   num_drafts   [B] int32 out: its length (0: no occurrence); pass it to
 *       specdec_verify as `gamma`.
 *   match_len    [B] int32 out or NULL: the n that matched (0 if none).
 * The proposer is deterministic, so its q is a point mass: verify its
 * proposals with specdec_verify in GREEDY mode, or in SAMPLE mode with
 * draft_logits = NULL.
 * Errors: INVALID_ARGUMENT for a bad descriptor, a NULL required pointer or a
 * misaligned workspace; WORKSPACE_TOO_SMALL.  Nothing is enqueued then. */
specdec_status_t specdec_propose_ngram(const specdec_ngram_desc_t* desc, const int32_t* history,
                                       const int32_t* hist_len, int32_t* draft_tokens,
                                       int32_t* num_drafts, int32_t* match_len,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* Bytes of device workspace specdec_propose_ngram needs (0 on a bad
 * descriptor): per-request best-match keys and arrival counters, which must
 * be zero before first use (allocate zero-filled or specdec_workspace_clear);
 * every completed call leaves them zero. */
size_t specdec_propose_ngram_workspace_bytes(const specdec_ngram_desc_t* desc);

/* Bring the draft model's paged cache back to the committed sequence after
 * specdec_verify (AI-infra KB M013 s.06: the target cache and the draft cache
 * must both return to the correct context; "Speculative decoding tutorial"
 * s.5.1: both lengths equal the committed length after a round, s.5.2: both
 * are trimmed to the accepted prefix, s.5.3: on a full accept the draft
 * still has to consume the last draft and the bonus token).
 *   kv_pool     the draft's [L][2][num_blocks][block_size][H][D] bf16 pool
 *       (desc describes the draft model), updated in place.
 *   block_table [B][max_blocks_per_req] int32, accept_count [B] (m_b),
 *       gamma [B] or NULL (= G): as for specdec_commit_kv.
 *   seq_lens    [B] int32, in place: in t_b, the draft cache length before
 *       the round (equal to the target's); out t_b + min(m_b + 1, gamma_b).
 *   flags       [B] uint32 or NULL: SPECDEC_FLAG_BAD_BLOCK as for commit.
 * While proposing, the draft wrote its own K/V in place for the pending token
 * and d_0 .. d_{gamma_b - 2}, i.e. positions t_b .. t_b + gamma_b - 1.  The
 * entries of the pending token and of the kept drafts stay; positions
 * t_b + m_b + 1 .. t_b + gamma_b - 1 are zero-filled (bf16 +0.0); nothing
 * else is touched.  After the call the draft cache holds the committed
 * sequence except, when m_b = gamma_b, d_{gamma_b - 1}, which the draft has
 * not consumed yet; the new pending token is consumed by the next round.
 * Workspace: specdec_commit_kv_workspace_bytes(desc) bytes, same rules.
 * Errors: as for specdec_commit_kv. */
specdec_status_t specdec_rollback_kv(const specdec_kv_desc_t* desc, void* kv_pool,
                                     const int32_t* block_table, const int32_t* accept_count,
                                     const int32_t* gamma, int32_t* seq_lens, uint32_t* flags,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* specdec_commit_kv on the target's cache and specdec_rollback_kv on the
 * draft's, for the same round, in one launch (AI-infra KB M013 s.06: both
 * caches return to the committed context after verification; both updates
 * depend only on accept_count, so their workgroups run side by side).
 * Arguments and results are exactly those of the two calls: the first group
 * (desc ... workspace_bytes) as for specdec_commit_kv, the second (draft_desc
 * ... draft_workspace_bytes) as for specdec_rollback_kv, with accept_count and
 * gamma shared; the two descriptors must agree on batch and gamma_max.  Rows
 * that do not take 16-byte vectors are served by two launches in order.
 * Errors: as for the two calls, plus INVALID_ARGUMENT when batch or gamma_max
 * differ, when the two workspaces overlap (the halves run side by side,
 * each with its own arrival counters: one workspace for both would let their
 * arrivals race; the two separate calls may share one), or when seq_lens and
 * draft_seq_lens overlap; nothing is enqueued in any error case. */
specdec_status_t specdec_commit_and_rollback_kv(
    const specdec_kv_desc_t* desc, const void* scratch_kv, void* kv_pool,
    const int32_t* block_table, const int32_t* slot_map, int32_t* seq_lens, uint32_t* flags,
    void* workspace, size_t workspace_bytes,
    const specdec_kv_desc_t* draft_desc, void* draft_pool, const int32_t* draft_block_table,
    int32_t* draft_seq_lens, uint32_t* draft_flags, void* draft_workspace,
    size_t draft_workspace_bytes,
    const int32_t* accept_count, const int32_t* gamma, hipStream_t stream);

/* ------------------------------------------------------------------ misc */

/* Zero `bytes` of device memory at `workspace` with a fill kernel on
 * `stream` (no hipMemset, so it may sit inside a captured graph).  bytes must
 * be a multiple of 4 and workspace 4-byte aligned. */
specdec_status_t specdec_workspace_clear(void* workspace, size_t bytes, hipStream_t stream);

/* Static description of a status code. */
const char* specdec_status_string(specdec_status_t status);

/* SPECDEC_ABI_VERSION of the loaded library. */
int32_t specdec_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPECDEC_H */
