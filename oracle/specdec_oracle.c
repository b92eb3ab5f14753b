/* CPU oracle of the speculative-decoding verify-and-commit step.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU
 * baseline leg of the benchmark; never by the product path.  Plain,
 * single-threaded, double precision, loops in ascending vocabulary order,
 * shares no code with the HIP kernels.
 *
 * Sources (the pages this restates; section names are the pages' own):
 *  [KB]   AI-infra knowledge base, detail page M013 "speculative decoding":
 *         s.03 greedy walk-through, s.04 exact sampling rule, s.05 the
 *         three-option worked example and its derivation, s.06 KV commit.
 *  [TUT]  "Speculative decoding tutorial: from distribution preservation and
 *         KV-cache rollback to break-even": s.3 greedy verification, s.4
 *         logits alignment, s.5.2/5.3 rollback and bonus, s.7.1-7.3 sampling.
 *  [APP]  "The apprentice's draft" (engineering half): s.2 Steps 2-4.
 *  [NOTE] nxmr.cn note on "lossless acceleration": the exact-fraction check,
 *         the R = 0 warning, filters must show in p and q.
 *  Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 *         easy as 1, 2, 3", SC'11.
 *
 * Readings where the pages leave a step open (all listed in the design notes):
 *  - row alignment: target row i judges draft token i; row gamma_i gives the
 *    bonus token ([TUT] s.4 table, with row 0 the pending-token row);
 *  - accept iff u < min(1, p/q) with u in [0,1) ([APP] Step 3);
 *  - q(d) = 0 accepts iff p(d) > 0; a token outside [0,V) is rejected;
 *  - residual mass <= 0 on a reject falls back to sampling p (flagged);
 *  - sampling is the inverse CDF in ascending token order with a strict ">":
 *    token = min{v : sum_{w<=v} r(w) > u * R};
 *  - uniforms: Philox4x32-10, key = seed, counter = (position, request,
 *    round, 0); word 0 -> accept test, word 1 -> sampling; u = (w >> 8) 2^-24;
 *  - greedy ties go to the lowest token index, on raw logits;
 *  - the committed list (accepted drafts, then the drawn token) is cut after
 *    its first end-of-sequence token and after the request's token budget;
 *    the accept count reported is the number of drafts left in it;
 *  - top-k keeps every token whose raw logit is >= the k-th largest raw
 *    logit; top-p then orders the kept tokens by probability (equivalently
 *    raw logit) descending, index ascending, keeps the shortest prefix whose
 *    cumulative probability is >= top_p, and both p and q are renormalized
 *    softmaxes over their own kept sets.
 */
#include "specdec_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define NEAR_EPS 1e-6

/* ---------------------------------------------------------------- Philox */

/* Philox4x32-10 (SC'11): ten rounds of two 32x32->64 multiplies with the
 * published multipliers, the key bumped by the published Weyl constants
 * between rounds. */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t prod0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        uint64_t prod1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        uint32_t n0 = (uint32_t)(prod1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)prod1;
        uint32_t n2 = (uint32_t)(prod0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)prod0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The two uniforms of (position, request): 24 high bits of words 0 and 1. */
static void philox_uniforms(uint64_t seed, uint32_t round, int32_t position, int32_t request,
                            double* u_accept, double* u_sample)
{
    uint32_t ctr[4] = {(uint32_t)position, (uint32_t)request, round, 0u};
    uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
    uint32_t w[4];
    oracle_philox4x32_10(ctr, key, w);
    *u_accept = (double)(w[0] >> 8) * (1.0 / 16777216.0);
    *u_sample = (double)(w[1] >> 8) * (1.0 / 16777216.0);
}

/* ---------------------------------------------------------------- logits */

static double logit_at(const void* row, int32_t is_bf16, int64_t v)
{
    if (is_bf16) {
        uint32_t bits = (uint32_t)((const uint16_t*)row)[v] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float*)row)[v];
}

static int row_nonfinite(const void* row, int32_t is_bf16, int32_t V)
{
    for (int64_t v = 0; v < V; ++v) {
        double z = logit_at(row, is_bf16, v);
        if (isnan(z) || (isinf(z) && z > 0)) return 1;
    }
    return 0;
}

/* qsort helpers ---------------------------------------------------------- */
static int cmp_double_desc(const void* a, const void* b)
{
    double x = *(const double*)a, y = *(const double*)b;
    return (x < y) - (x > y);
}

typedef struct { double z; int32_t v; } zidx;
static int cmp_z_desc_idx_asc(const void* a, const void* b)
{
    const zidx* x = (const zidx*)a;
    const zidx* y = (const zidx*)b;
    if (x->z > y->z) return -1;
    if (x->z < y->z) return 1;
    return (x->v > y->v) - (x->v < y->v);
}

/* The sampling distribution of one row ([KB] s.04: p and q are the actual
 * sampling distributions after temperature and truncation; [NOTE]: filters
 * must show in the probabilities).  Softmax of z/T over the kept set. */
int oracle_row_distribution(const void* row, int32_t is_bf16, int32_t V, double T,
                            int32_t top_k, double top_p, double* prob, int32_t* near_cut)
{
    if (near_cut) *near_cut = 0;
    char* keep = (char*)malloc((size_t)V);
    for (int64_t v = 0; v < V; ++v) keep[v] = 1;

    /* top-k on raw logits: threshold = k-th largest value, ties kept. */
    if (top_k > 0 && top_k < V) {
        double* sorted = (double*)malloc(sizeof(double) * (size_t)V);
        for (int64_t v = 0; v < V; ++v) sorted[v] = logit_at(row, is_bf16, v);
        qsort(sorted, (size_t)V, sizeof(double), cmp_double_desc);
        double tau = sorted[top_k - 1];
        free(sorted);
        for (int64_t v = 0; v < V; ++v) keep[v] = logit_at(row, is_bf16, v) >= tau;
    }

    /* softmax of z/T over the kept set */
    double M = -INFINITY;
    for (int64_t v = 0; v < V; ++v)
        if (keep[v]) {
            double x = logit_at(row, is_bf16, v) / T;
            if (x > M) M = x;
        }
    double S = 0.0;
    for (int64_t v = 0; v < V; ++v)
        if (keep[v]) S += exp(logit_at(row, is_bf16, v) / T - M);
    for (int64_t v = 0; v < V; ++v)
        prob[v] = keep[v] ? exp(logit_at(row, is_bf16, v) / T - M) / S : 0.0;

    /* top-p: shortest prefix (probability descending, index ascending) whose
     * cumulative probability reaches top_p; then renormalize over it. */
    if (top_p < 1.0) {
        int64_t n_kept = 0;
        for (int64_t v = 0; v < V; ++v) n_kept += keep[v];
        zidx* order = (zidx*)malloc(sizeof(zidx) * (size_t)n_kept);
        int64_t k = 0;
        for (int64_t v = 0; v < V; ++v)
            if (keep[v]) { order[k].z = logit_at(row, is_bf16, v); order[k].v = (int32_t)v; ++k; }
        qsort(order, (size_t)n_kept, sizeof(zidx), cmp_z_desc_idx_asc);
        double cum = 0.0, prev = 0.0;
        int64_t cut = n_kept - 1;
        for (int64_t j = 0; j < n_kept; ++j) {
            prev = cum;
            cum += prob[order[j].v];
            if (cum >= top_p) { cut = j; break; }
        }
        if (near_cut && (fabs(cum - top_p) < NEAR_EPS || fabs(prev - top_p) < NEAR_EPS))
            *near_cut = 1;
        for (int64_t j = cut + 1; j < n_kept; ++j) keep[order[j].v] = 0;
        free(order);
        double S2 = 0.0;
        for (int64_t v = 0; v < V; ++v)
            if (keep[v]) S2 += exp(logit_at(row, is_bf16, v) / T - M);
        for (int64_t v = 0; v < V; ++v)
            prob[v] = keep[v] ? exp(logit_at(row, is_bf16, v) / T - M) / S2 : 0.0;
    }
    int kept = 0;
    for (int64_t v = 0; v < V; ++v) kept += keep[v];
    free(keep);
    return kept;
}

/* Greedy choice of one row: largest raw logit, lowest index on ties
 * ([KB] s.03: a fixed tie rule; [TUT] s.3 g_T = argmax). */
static int32_t row_argmax(const void* row, int32_t is_bf16, int32_t V)
{
    int32_t best = 0;
    double best_z = logit_at(row, is_bf16, 0);
    for (int64_t v = 1; v < V; ++v) {
        double z = logit_at(row, is_bf16, v);
        if (z > best_z) { best_z = z; best = (int32_t)v; }
    }
    return best;
}

/* ---------------------------------------------------------------- verify */

static const void* row_ptr(const void* base, int32_t is_bf16, int64_t row, int32_t V)
{
    size_t es = is_bf16 ? 2 : 4;
    return (const char*)base + (size_t)row * (size_t)V * es;
}

static void note_near(int32_t* near, int32_t pos)
{
    if (*near < 0 || pos < *near) *near = pos;
}

/* Round end.  The list the step would commit is out[0..m]: the m accepted
 * drafts, then the correction or bonus token.  Decoding stops after an
 * end-of-sequence token and once the output-length limit is reached ([KB]
 * s.03: EOS and length limits can end a round early; [TUT] s.5.2: nothing
 * after an EOS in the candidate block may reach the cache; [TUT] s.11: the
 * loop runs while fewer than max_new_tokens were produced and stops after
 * emitting EOS).  So the list is cut after its first EOS and after `budget`
 * tokens (budget < 0: no limit).  Returns the number of tokens kept; *kept_m
 * receives the drafts among them, and the rest of out[] becomes -1. */
static int32_t round_end(int32_t m, int32_t G, int32_t* out, int32_t eos, int32_t budget,
                         uint32_t* fl, int32_t* kept_m)
{
    int32_t n = m + 1;
    int32_t e = -1;
    if (eos >= 0)
        for (int32_t j = 0; j <= m; ++j)
            if (out[j] == eos) { e = j; break; }
    if (e >= 0) n = e + 1;
    if (budget >= 0 && budget <= n) {
        n = budget;
        *fl |= ORACLE_FLAG_LENGTH;
    }
    if (e >= 0 && e < n) *fl |= ORACLE_FLAG_EOS;
    for (int32_t j = n; j <= G; ++j) out[j] = -1;
    *kept_m = m < n ? m : n;
    return n;
}

int oracle_verify(const oracle_verify_args* a, const void* target, const void* draft,
                  const int32_t* draft_tokens, const int32_t* gamma,
                  const int32_t* max_tokens,
                  const int32_t* req_ids, int32_t n,
                  const double* u_accept_in, const double* u_sample_in,
                  int32_t* accept_count, int32_t* num_tokens, int32_t* out_tokens,
                  double* p_draft, double* q_draft, double* residual_mass,
                  uint32_t* flags, int32_t* near_pos)
{
    const int32_t B = a->batch, G = a->gamma_max, V = a->vocab;
    if (B < 0 || G < 0 || G > 63 || V < 1 || !target || !draft_tokens || !accept_count
        || !out_tokens)
        return -1;
    if (!a->greedy && !(a->temperature > 0.0)) return -2;
    if (!req_ids && n != B) return -3;

    double* P = NULL; /* target distributions, rows 0..gamma_b, each V */
    double* Q = NULL; /* draft distributions, rows 0..gamma_b-1 */
    double* r = (double*)malloc(sizeof(double) * (size_t)V);
    if (!a->greedy) {
        P = (double*)malloc(sizeof(double) * (size_t)(G + 1) * (size_t)V);
        Q = (double*)malloc(sizeof(double) * (size_t)(G > 0 ? G : 1) * (size_t)V);
    }

    int rc = 0;
    for (int32_t k = 0; k < n; ++k) {
        const int32_t b = req_ids ? req_ids[k] : k;
        if (b < 0 || b >= B) { rc = -4; break; }
        const int32_t gb = gamma ? gamma[b] : G;
        if (gb < 0 || gb > G) { rc = -5; break; }
        const int32_t* d = draft_tokens + (size_t)b * G;
        int32_t* out = out_tokens + (size_t)k * (G + 1);
        uint32_t fl = 0;
        int32_t near = -1;
        int32_t committed_m = 0;
        for (int32_t j = 0; j <= G; ++j) out[j] = -1;
        for (int32_t i = 0; i < gb; ++i)
            if (d[i] < 0 || d[i] >= V) fl |= ORACLE_FLAG_TOKEN_RANGE;
        for (int32_t i = 0; i <= gb; ++i)
            if (row_nonfinite(row_ptr(target, a->is_bf16, (int64_t)b * (G + 1) + i, V), a->is_bf16, V))
                fl |= ORACLE_FLAG_NONFINITE;

        if (a->greedy) {
            /* [TUT] s.3-s.4 / [KB] s.03: longest prefix of drafts equal to the
             * target's argmax at their aligned rows; the first mismatch (or
             * the bonus row) contributes the target's own argmax. */
            int32_t m = 0;
            int32_t g = 0;
            for (int32_t i = 0; i <= gb; ++i) {
                g = row_argmax(row_ptr(target, a->is_bf16, (int64_t)b * (G + 1) + i, V), a->is_bf16, V);
                if (i == gb || d[i] != g) break;
                out[i] = d[i];
                ++m;
            }
            out[m] = g;
            if (residual_mass) residual_mass[k] = 0.0;
            committed_m = m;
        } else {
            for (int32_t i = 0; i < gb && draft; ++i)
                if (row_nonfinite(row_ptr(draft, a->is_bf16, (int64_t)b * G + i, V), a->is_bf16, V))
                    fl |= ORACLE_FLAG_NONFINITE;
            /* p_i, q_i: the actual sampling distributions ([KB] s.04). */
            for (int32_t i = 0; i <= gb; ++i) {
                int32_t nc = 0;
                oracle_row_distribution(row_ptr(target, a->is_bf16, (int64_t)b * (G + 1) + i, V),
                                        a->is_bf16, V, a->temperature, a->top_k, a->top_p,
                                        P + (size_t)i * V, &nc);
                if (nc) note_near(&near, i);
            }
            for (int32_t i = 0; i < gb; ++i) {
                if (!draft) {
                    /* No draft rows: the proposer is deterministic (n-gram
                     * lookup), so q_i is the point mass on d_i ([KB] s.08:
                     * such candidates need their probability representation
                     * stated; the exact rule of s.04 is then applied as is). */
                    for (int64_t v = 0; v < V; ++v) Q[(size_t)i * V + v] = 0.0;
                    if (d[i] >= 0 && d[i] < V) Q[(size_t)i * V + d[i]] = 1.0;
                    continue;
                }
                int32_t nc = 0;
                oracle_row_distribution(row_ptr(draft, a->is_bf16, (int64_t)b * G + i, V),
                                        a->is_bf16, V, a->temperature, a->top_k, a->top_p,
                                        Q + (size_t)i * V, &nc);
                if (nc) note_near(&near, i);
            }
            double ua[65], us[65];
            for (int32_t i = 0; i <= gb; ++i) {
                if (u_accept_in) {
                    ua[i] = u_accept_in[(size_t)k * (G + 1) + i];
                    us[i] = u_sample_in[(size_t)k * (G + 1) + i];
                } else {
                    philox_uniforms(a->seed, a->round, i, b, &ua[i], &us[i]);
                }
            }
            /* Per-position probabilities of the drafted tokens. */
            for (int32_t i = 0; i < G; ++i) {
                double pd = 0.0, qd = 0.0;
                if (i < gb && d[i] >= 0 && d[i] < V) {
                    pd = P[(size_t)i * V + d[i]];
                    qd = Q[(size_t)i * V + d[i]];
                }
                if (p_draft) p_draft[(size_t)k * G + i] = pd;
                if (q_draft) q_draft[(size_t)k * G + i] = qd;
            }
            /* Left-to-right acceptance ([TUT] s.7.1, s.7.3; [APP] Step 3):
             * accept d_i with probability min(1, p_i(d_i)/q_i(d_i)); stop at
             * the first rejection ([TUT] s.2: only a contiguous prefix). */
            int32_t m = 0;
            for (int32_t i = 0; i < gb; ++i) {
                double acc_p;
                if (d[i] < 0 || d[i] >= V) {
                    acc_p = 0.0;
                } else {
                    double pd = P[(size_t)i * V + d[i]];
                    double qd = Q[(size_t)i * V + d[i]];
                    if (qd > 0.0) acc_p = pd / qd < 1.0 ? pd / qd : 1.0;
                    else acc_p = pd > 0.0 ? 1.0 : 0.0;
                }
                if (fabs(ua[i] - acc_p) < NEAR_EPS) note_near(&near, i);
                if (!(ua[i] < acc_p)) break;
                out[i] = d[i];
                ++m;
            }
            /* Correction from normalize(max(p_m - q_m, 0)) on a rejection
             * ([KB] s.05, [TUT] s.7.2, [APP] Step 4), else the bonus token
             * from p_gamma ([TUT] s.5.3). */
            const double* pm = P + (size_t)m * V;
            double R = 0.0;
            if (m < gb) {
                const double* qm = Q + (size_t)m * V;
                for (int64_t v = 0; v < V; ++v) {
                    double diff = pm[v] - qm[v];
                    r[v] = diff > 0.0 ? diff : 0.0;
                    R += r[v];
                }
                if (residual_mass) residual_mass[k] = R;
                if (!(R > 0.0)) {
                    /* [KB] s.05 / [NOTE]: the reject branch is unreachable in
                     * exact arithmetic when R = 0; never divide by it. */
                    fl |= ORACLE_FLAG_RESIDUAL_FALLBACK;
                    R = 0.0;
                    for (int64_t v = 0; v < V; ++v) { r[v] = pm[v]; R += r[v]; }
                }
            } else {
                for (int64_t v = 0; v < V; ++v) { r[v] = pm[v]; R += r[v]; }
                if (residual_mass) residual_mass[k] = 0.0;
            }
            /* Inverse CDF, ascending token order. */
            const double target_mass = us[m] * R;
            double C = 0.0, C_prev = 0.0;
            int32_t tok = -1;
            for (int64_t v = 0; v < V; ++v) {
                C_prev = C;
                C += r[v];
                if (C > target_mass) { tok = (int32_t)v; break; }
            }
            if (tok < 0) {
                for (int64_t v = V - 1; v >= 0; --v)
                    if (r[v] > 0.0) { tok = (int32_t)v; break; }
                C_prev = C;
            }
            if (fabs(us[m] - C_prev / R) < NEAR_EPS || fabs(us[m] - C / R) < NEAR_EPS)
                note_near(&near, m);
            out[m] = tok;
            committed_m = m;
        }
        {
            const int32_t budget = max_tokens ? (max_tokens[b] < 0 ? 0 : max_tokens[b]) : -1;
            int32_t kept_m = 0;
            const int32_t nt = round_end(committed_m, G, out, a->eos_token, budget, &fl, &kept_m);
            accept_count[k] = kept_m;
            if (num_tokens) num_tokens[k] = nt;
        }
        if (flags) flags[k] = fl;
        if (near_pos) near_pos[k] = near;
    }
    free(r);
    free(P);
    free(Q);
    return rc;
}

/* ---------------------------------------------------------------- commit */

/* Keep the K/V of the pending token and the accepted drafts, invalidate the
 * rejected slots and set the new length ([KB] s.06; [TUT] s.5.2: trim to
 * t+m, then the replacement makes t+m+1; [APP] s.5.4: accepted entries are
 * written into the cache, the rest dropped).  Position t+j takes scratch slot
 * j (chain) or the slot of the path's node at depth j (tree: [APP] s.5.3,
 * only the accepted path becomes history); positions up to t+m are written,
 * t+m+1 .. t+gamma_i zero-filled. */
int oracle_commit_kv(int32_t B, int32_t G, int32_t L, int32_t H, int32_t D, int32_t bs,
                     int32_t max_blocks, int64_t num_blocks, int32_t scratch_slots,
                     const uint16_t* scratch, const int32_t* slot_map,
                     uint16_t* pool, const int32_t* block_table, const int32_t* accept_count,
                     const int32_t* gamma, int32_t* seq_lens)
{
    const size_t row = (size_t)H * (size_t)D;
    const int32_t S = scratch_slots > 0 ? scratch_slots : G + 1;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t gb = gamma ? gamma[b] : G;
        const int32_t m = accept_count[b];
        const int32_t t = seq_lens[b];
        if (gb < 0 || gb > G || m < 0 || m > gb || t < 0) return -1;
        for (int32_t j = 0; j <= gb; ++j) {
            const int64_t pos = (int64_t)t + j;
            if (pos / bs >= max_blocks) return -2;
            const int32_t blk = block_table[(size_t)b * max_blocks + pos / bs];
            if (blk < 0 || blk >= num_blocks) return -3;
            const int64_t off = pos % bs;
            for (int32_t l = 0; l < L; ++l)
                for (int32_t kv = 0; kv < 2; ++kv) {
                    uint16_t* dst = pool + ((((size_t)l * 2 + kv) * (size_t)num_blocks + (size_t)blk)
                                            * (size_t)bs + (size_t)off) * row;
                    if (j <= m) {
                        const int32_t slot = slot_map ? slot_map[(size_t)b * (G + 1) + j] : j;
                        if (slot < 0 || slot >= S) return -4;
                        const uint16_t* src = scratch
                            + ((((size_t)b * S + slot) * L + l) * 2 + kv) * row;
                        memcpy(dst, src, row * sizeof(uint16_t));
                    } else {
                        memset(dst, 0, row * sizeof(uint16_t));
                    }
                }
        }
    }
    for (int32_t b = 0; b < B; ++b) seq_lens[b] = seq_lens[b] + accept_count[b] + 1;
    return 0;
}

/* The draft's cache after verification ([KB] s.06: the target cache and the
 * draft cache must both return to the committed context; [TUT] s.5.1: their
 * lengths equal the committed length after every round; [TUT] s.5.2: trim to
 * t+m, then the replacement token is fed to both; [TUT] s.5.3: on a full
 * accept the draft still has to consume the last draft and the bonus).
 * Proposing wrote the pending token and d_0..d_{gamma-2} at positions
 * t..t+gamma-1, so the entries of the pending token and the m accepted drafts
 * (as far as they were written) stay, the later ones are zero-filled, and the
 * length becomes t + min(m + 1, gamma). */
int oracle_rollback_kv(int32_t B, int32_t G, int32_t L, int32_t H, int32_t D, int32_t bs,
                       int32_t max_blocks, int64_t num_blocks, uint16_t* pool,
                       const int32_t* block_table, const int32_t* accept_count,
                       const int32_t* gamma, int32_t* seq_lens)
{
    const size_t row = (size_t)H * (size_t)D;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t gb = gamma ? gamma[b] : G;
        const int32_t m = accept_count[b];
        const int32_t t = seq_lens[b];
        if (gb < 0 || gb > G || m < 0 || m > gb || t < 0) return -1;
        for (int32_t j = m + 1; j < gb; ++j) {
            const int64_t pos = (int64_t)t + j;
            if (pos / bs >= max_blocks) return -2;
            const int32_t blk = block_table[(size_t)b * max_blocks + pos / bs];
            if (blk < 0 || blk >= num_blocks) return -3;
            const int64_t off = pos % bs;
            for (int32_t l = 0; l < L; ++l)
                for (int32_t kv = 0; kv < 2; ++kv)
                    memset(pool + ((((size_t)l * 2 + kv) * (size_t)num_blocks + (size_t)blk)
                                   * (size_t)bs + (size_t)off) * row,
                           0, row * sizeof(uint16_t));
        }
    }
    for (int32_t b = 0; b < B; ++b) {
        const int32_t gb = gamma ? gamma[b] : G;
        const int32_t keep = accept_count[b] + 1 < gb ? accept_count[b] + 1 : gb;
        seq_lens[b] = seq_lens[b] + keep;
    }
    return 0;
}

/* ---------------------------------------------------------------- tree */

/* Greedy verification of a draft tree ([APP] s.5.3: the target checks every
 * node of the tree in one forward and the longest accepted root-to-leaf path
 * is kept; [TUT] s.13.3 and s.14: tree speculation verifies several
 * branches at once).  The greedy rule of [TUT] s.3-4 / [KB] s.03 applies
 * along every edge: the target's row after a node judges that node's
 * children, and a child is accepted when its token is the row's argmax
 * (lowest index on ties) and its parent was accepted.  The committed path
 * ends at the deepest accepted node (lowest node index among equally deep
 * ones); the token after it is the argmax of that node's row, which is the
 * correction when it has children and the bonus when it is a leaf.  The
 * committed list is then cut at EOS / budget exactly as for a chain. */
int oracle_verify_tree(int32_t B, int32_t N, int32_t V, int32_t is_bf16, const void* target,
                       const int32_t* tokens, const int32_t* parents, const int32_t* num_nodes,
                       int32_t eos_token, const int32_t* max_tokens, int32_t* accept_count,
                       int32_t* num_tokens, int32_t* out_tokens, int32_t* path, uint32_t* flags)
{
    if (B < 0 || N < 1 || N > 64 || V < 1 || !target || !tokens || !parents || !accept_count
        || !out_tokens || !path)
        return -1;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t n = num_nodes ? num_nodes[b] : N;
        if (n < 1 || n > N) return -2;
        const int32_t* tok = tokens + (size_t)b * N;
        const int32_t* par = parents + (size_t)b * N;
        uint32_t fl = 0;
        int32_t choice[64], depth[64], ok[64];
        for (int32_t j = 0; j < n; ++j)
            choice[j] = row_argmax(row_ptr(target, is_bf16, (int64_t)b * N + j, V), is_bf16, V);
        /* nodes in index order: a parent always precedes its children */
        ok[0] = 1;
        depth[0] = 0;
        for (int32_t j = 1; j < n; ++j) {
            ok[j] = 0;
            depth[j] = 0;
            if (par[j] < 0 || par[j] >= j) { fl |= ORACLE_FLAG_BAD_TREE; continue; }
            depth[j] = depth[par[j]] + 1;
            if (tok[j] < 0 || tok[j] >= V) { fl |= ORACLE_FLAG_TOKEN_RANGE; continue; }
            ok[j] = ok[par[j]] && tok[j] == choice[par[j]];
        }
        int32_t best = 0;
        for (int32_t j = 1; j < n; ++j)
            if (ok[j] && depth[j] > depth[best]) best = j;
        const int32_t m = depth[best];
        int32_t* pth = path + (size_t)b * N;
        int32_t* out = out_tokens + (size_t)b * N;
        for (int32_t j = 0; j < N; ++j) { pth[j] = -1; out[j] = -1; }
        for (int32_t x = best; ; x = par[x]) {
            pth[depth[x]] = x;
            if (x == 0) break;
        }
        for (int32_t k = 1; k <= m; ++k) out[k - 1] = tok[pth[k]];
        out[m] = choice[best];
        const int32_t budget = max_tokens ? (max_tokens[b] < 0 ? 0 : max_tokens[b]) : -1;
        int32_t kept_m = 0;
        const int32_t nt = round_end(m, N - 1, out, eos_token, budget, &fl, &kept_m);
        accept_count[b] = kept_m;
        if (num_tokens) num_tokens[b] = nt;
        if (flags) flags[b] = fl;
    }
    return 0;
}

/* ---------------------------------------------------------------- n-gram */

/* Prompt-lookup / n-gram proposal ([KB] s.08: candidates found from repeated
 * patterns in the text; [MATH]: pattern-based drafting searches the existing
 * context for a matching sequence at near-zero cost; [TUT] s.13.1 and s.14:
 * prompt lookup / n-gram candidates come from the prompt or the history).
 * For n = n_max down to n_min: the last n tokens of the history are searched
 * for their most recent earlier occurrence (one that ends before the last
 * position); the first n that has one wins, and the tokens that follow the
 * occurrence, at most gamma_max of them and never past the history's end,
 * are the proposal.  No occurrence: nothing is proposed. */
int oracle_propose_ngram(int32_t B, int32_t max_len, const int32_t* history,
                         const int32_t* hist_len, int32_t n_min, int32_t n_max, int32_t G,
                         int32_t* draft_tokens, int32_t* num_drafts, int32_t* match_len)
{
    if (B < 0 || max_len < 1 || n_min < 1 || n_max < n_min || G < 0 || !history || !hist_len
        || !draft_tokens || !num_drafts)
        return -1;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t L = hist_len[b];
        if (L < 0 || L > max_len) return -2;
        const int32_t* h = history + (size_t)b * max_len;
        int32_t* out = draft_tokens + (size_t)b * G;
        for (int32_t i = 0; i < G; ++i) out[i] = -1;
        num_drafts[b] = 0;
        if (match_len) match_len[b] = 0;
        for (int32_t n = n_max; n >= n_min; --n) {
            if (L < n + 1) continue;
            int32_t found = -1;
            for (int32_t s = L - n - 1; s >= 0 && found < 0; --s) {
                int32_t same = 1;
                for (int32_t k = 0; k < n; ++k)
                    if (h[s + k] != h[L - n + k]) { same = 0; break; }
                if (same) found = s;
            }
            if (found < 0) continue;
            const int32_t first = found + n;       /* the token after the occurrence */
            int32_t cnt = L - first < G ? L - first : G;
            for (int32_t i = 0; i < cnt; ++i) out[i] = h[first + i];
            num_drafts[b] = cnt;
            if (match_len) match_len[b] = n;
            break;
        }
    }
    return 0;
}
