/* CPU oracle of the speculative-decoding verify-and-commit step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code: it exists so that tests, the smoke check and the CPU
 * baseline of the benchmark can compare the HIP path against a plain,
 * single-threaded, double-precision restatement of what the step computes.
 * It shares no code with the HIP path.
 *
 * Layouts match the device layouts so the same host buffers feed both sides:
 *   target  [B][G+1][V]  float32 or bfloat16 bit patterns (uint16)
 *   draft   [B][G][V]    same type (unused in greedy mode; NULL in sampling
 *                        mode: point-mass drafts, q_i = 1 at d_i)
 *   tokens  [B][G] int32, gamma [B] int32 (NULL: every request uses G)
 */
#ifndef SPECDEC_ORACLE_H
#define SPECDEC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t batch;        /* B */
    int32_t gamma_max;    /* G */
    int32_t vocab;        /* V */
    int32_t is_bf16;      /* 1: logits are bfloat16 bit patterns, 0: float32 */
    int32_t greedy;       /* 1: argmax-equality verification */
    int32_t top_k;        /* 0: off */
    double temperature;   /* > 0, sampling only */
    double top_p;         /* 1.0: off */
    uint64_t seed;        /* Philox key */
    uint32_t round;       /* Philox counter word 2 */
    int32_t eos_token;    /* -1: none; else the end-of-sequence token id */
} oracle_verify_args;

/* Flag bits (per request), same meaning as on the device side. */
#define ORACLE_FLAG_RESIDUAL_FALLBACK 0x2u  /* rejected but sum of [p-q]+ <= 0 */
#define ORACLE_FLAG_NONFINITE         0x4u  /* NaN or +inf in a used row */
#define ORACLE_FLAG_TOKEN_RANGE       0x8u  /* a draft token outside [0,V) */
#define ORACLE_FLAG_EOS               0x80u /* the committed list ends with an EOS token */
#define ORACLE_FLAG_LENGTH            0x100u /* the token budget ended the committed list */

/* Verify selected requests.  req_ids[n] picks the requests (NULL: 0..B-1 and
 * n must equal B); every output is indexed by the position in that list:
 *   accept_count [n]: drafts kept (after the EOS / budget cut),
 *   num_tokens [n] (may be NULL): tokens committed this round,
 *   out_tokens [n][G+1] (-1 padded), p_draft/q_draft [n][G]
 *   (0 past gamma_i; untouched in greedy mode), residual_mass [n], flags [n],
 *   near_pos [n]: smallest position whose output-determining decision lies
 *   within 1e-6 of its threshold (accept test, inverse-CDF edge or top-p cut),
 *   -1 if none.
 * u_accept / u_sample [n][G+1] (may be NULL) replace the Philox uniforms.
 * max_tokens [B] (indexed by request, may be NULL): the most tokens request b
 *   may commit this round (values below 0 count as 0).
 * Returns 0, or a negative value on a malformed argument. */
int oracle_verify(const oracle_verify_args* a, const void* target, const void* draft,
                  const int32_t* draft_tokens, const int32_t* gamma,
                  const int32_t* max_tokens,
                  const int32_t* req_ids, int32_t n,
                  const double* u_accept, const double* u_sample,
                  int32_t* accept_count, int32_t* num_tokens, int32_t* out_tokens,
                  double* p_draft, double* q_draft, double* residual_mass,
                  uint32_t* flags, int32_t* near_pos);

/* Dense sampling distribution of one logits row after temperature, top-k and
 * top-p.  near_cut (may be NULL) is set to 1 if the top-p cumulative lies
 * within 1e-6 of top_p at the cut.  Returns the number of kept tokens. */
int oracle_row_distribution(const void* row, int32_t is_bf16, int32_t vocab,
                            double temperature, int32_t top_k, double top_p,
                            double* prob, int32_t* near_cut);

/* Philox4x32-10 block: out = philox(ctr, key). */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* Greedy verification of a draft tree.
 *   target  [B][N][V]: row j is the target's distribution after the path from
 *           the root (node 0, the pending token) to node j
 *   tokens  [B][N] int32 (node 0's entry ignored), parents [B][N] int32
 *           (parents[b][0] ignored; 0 <= parent < j otherwise)
 *   num_nodes [B] in [1, N] or NULL (N)
 * Outputs per request: accept_count (depth of the committed path after the
 * EOS / budget cut), num_tokens (may be NULL), out_tokens [B][N] (the path's
 * tokens, then the target's choice after its last node; -1 padded),
 * path [B][N] (node of each depth along the accepted path, root first, -1
 * padded; not cut), flags [B] (ORACLE_FLAG_BAD_TREE for a malformed parent,
 * ORACLE_FLAG_TOKEN_RANGE for a token outside [0,V); such nodes reject).
 * Returns 0, or a negative value on a malformed argument. */
#define ORACLE_FLAG_BAD_TREE 0x200u
int oracle_verify_tree(int32_t batch, int32_t num_nodes_max, int32_t vocab, int32_t is_bf16,
                       const void* target, const int32_t* tokens, const int32_t* parents,
                       const int32_t* num_nodes, int32_t eos_token, const int32_t* max_tokens,
                       int32_t* accept_count, int32_t* num_tokens, int32_t* out_tokens,
                       int32_t* path, uint32_t* flags);

/* Commit the verified K/V slots of every request into the paged pool.
 *   scratch  [B][S][L][2][H][D] bf16 bits, S = scratch_slots (0: G+1)
 *   slot_map [B][G+1] or NULL: position t_i + j takes scratch slot
 *            slot_map[i][j] (NULL: slot j, the chain case)
 *   pool     [L][2][num_blocks][block][H][D] bf16 bits
 *   block_table [B][max_blocks], accept_count [B], gamma [B] (NULL: G)
 *   seq_lens [B] in: t_i, out: t_i + m_i + 1
 * Positions t_i .. t_i + m_i receive their slots, t_i + m_i + 1 .. t_i + gamma_i
 * are zero-filled.
 * Returns 0, or a negative value if a needed block-table entry is invalid. */
int oracle_commit_kv(int32_t batch, int32_t gamma_max, int32_t layers, int32_t kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t max_blocks,
                     int64_t num_blocks, int32_t scratch_slots, const uint16_t* scratch,
                     const int32_t* slot_map, uint16_t* pool,
                     const int32_t* block_table, const int32_t* accept_count,
                     const int32_t* gamma, int32_t* seq_lens);

/* Roll back the draft model's paged cache after verification.  While
 * proposing, the draft wrote positions t_i .. t_i + gamma_i - 1 in place (the
 * pending token, then d_0 .. d_{gamma_i - 2}).  Positions t_i + m_i + 1 ..
 * t_i + gamma_i - 1 are zero-filled and seq_lens becomes
 * t_i + min(m_i + 1, gamma_i).
 *   pool [L][2][num_blocks][block][H][D] bf16 bits; the rest as for commit.
 * Returns 0, or a negative value if a needed block-table entry is invalid. */
int oracle_rollback_kv(int32_t batch, int32_t gamma_max, int32_t layers, int32_t kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t max_blocks,
                       int64_t num_blocks, uint16_t* pool, const int32_t* block_table,
                       const int32_t* accept_count, const int32_t* gamma, int32_t* seq_lens);

/* Prompt-lookup / n-gram proposal.
 *   history [B][max_len] int32, hist_len [B] in [0, max_len]
 *   draft_tokens [B][gamma_max] (-1 padded), num_drafts [B] (0: no match),
 *   match_len [B] (the n that matched, 0 if none; may be NULL)
 * For n = n_max down to n_min, the last n tokens are looked up at their most
 * recent earlier occurrence; the tokens after it (at most gamma_max, not past
 * the end) are proposed.  Returns 0, or a negative value on bad arguments. */
int oracle_propose_ngram(int32_t batch, int32_t max_len, const int32_t* history,
                         const int32_t* hist_len, int32_t n_min, int32_t n_max, int32_t gamma_max,
                         int32_t* draft_tokens, int32_t* num_drafts, int32_t* match_len);

#ifdef __cplusplus
}
#endif
#endif
