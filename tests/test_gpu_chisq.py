"""Distribution preservation through the HIP kernels, by repeated sampling.

"Speculative decoding tutorial" s.12.3 and AI-infra KB M013 s.09 ask for the
sampling path to be checked by drawing many times on a small vocabulary and
comparing the empirical frequencies with the target distribution.  Here every
request of a batch carries the same target and draft rows, the drafts are
drawn on the host from q (or are fixed tokens, for point-mass drafts), and the
Philox round counter changes from call to call, so the batch and the rounds
give independent trials.  Among the trials that reach position i (every draft
before i kept), the committed token at i must follow p_i: a chi-square test
per position at p-value > 1e-3.  p_i is computed here in double from the
stored logits, independently of the oracle and of the kernels; with top-k or
top-p it is the truncated p~ (drafts drawn from the truncated q~), through the
kept-token lists and, forced in the debug build, through the cut records.
"""
import numpy as np
import pytest

from pins import P_MIN, chisq_fit
from gpu_helpers import env, gpu_verify, say
from speculative_decoding_verification_05_amd import synth

pytestmark = pytest.mark.gpu

B_CALL = 50_000   # requests per call (the descriptor allows up to 65535)

# (V, gamma, dtype, point-mass drafts, temperature, calls, top_k, top_p, cut path forced)
CASES = [
    (3, 1, "f32", False, 1.0, 4, 0, 1.0, False),
    (8, 4, "f32", False, 0.9, 4, 0, 1.0, False),
    (16, 4, "f32", False, 0.7, 5, 0, 1.0, False),
    (16, 1, "bf16", False, 1.0, 4, 0, 1.0, False),
    (8, 4, "f32", True, 0.9, 4, 0, 1.0, False),
    # truncated target and draft: kept-token lists, then cut records
    (16, 4, "f32", False, 0.8, 4, 6, 1.0, False),
    (16, 4, "f32", False, 0.8, 4, 0, 0.8, False),
    (16, 4, "bf16", False, 0.8, 4, 10, 0.85, True),
    (16, 2, "f32", True, 1.0, 4, 0, 0.7, False),
]


def truncated(z, T, top_k, top_p):
    """softmax(z/T) kept to top-k (ties at the k-th logit kept), then to the
    shortest prefix in (logit desc, index asc) order reaching top_p, and
    renormalised: computed here in double, apart from the oracle and the
    kernels (AI-infra KB M013 s.04; the nxmr.cn note: truncation shows in
    the probabilities)."""
    z = z.astype(np.float64)
    keep = np.ones(z.shape[0], bool)
    if 0 < top_k < z.shape[0]:
        keep = z >= np.sort(z)[::-1][top_k - 1]
    w = np.where(keep, np.exp(z / T - (z / T)[keep].max()), 0.0)
    w /= w.sum()
    if top_p < 1.0:
        order = np.lexsort((np.arange(z.shape[0]), -z))  # logit desc, index asc
        order = order[keep[order]]
        cum = np.cumsum(w[order])
        n = int(np.searchsorted(cum, top_p, side="left")) + 1
        cut = np.zeros_like(keep)
        cut[order[:min(n, order.size)]] = True
        w = np.where(cut, w, 0.0)
        w /= w.sum()
    return w


@pytest.mark.parametrize("V,G,dtype,point,T,calls,top_k,top_p,force_cut", CASES,
                         ids=[f"V{c[0]}-g{c[1]}-{c[2]}{'-point' if c[3] else ''}"
                              f"{f'-k{c[6]}' if c[6] else ''}{f'-p{c[7]}' if c[7] < 1 else ''}"
                              f"{'-cut' if c[8] else ''}" for c in CASES])
def test_committed_tokens_follow_the_target(V, G, dtype, point, T, calls, top_k, top_p, force_cut):
    rng = np.random.default_rng(1000 + 31 * V + G + (7 if point else 0))
    zt = (rng.standard_normal((G + 1, V)) * 1.2).astype(np.float32)
    zq = (zt[:G] + rng.standard_normal((G, V)) * 1.0).astype(np.float32)
    if dtype == "bf16":
        t_store, q_store = synth.f32_to_bf16_bits(zt), synth.f32_to_bf16_bits(zq)
        zt, zq = synth.bf16_bits_to_f32(t_store), synth.bf16_bits_to_f32(q_store)
    else:
        t_store, q_store = zt, zq
    p = np.stack([truncated(zt[i], T, top_k, top_p) for i in range(G + 1)])
    q = np.stack([truncated(zq[i], T, top_k, top_p) for i in range(G)])
    tgt = np.ascontiguousarray(np.broadcast_to(t_store, (B_CALL, G + 1, V)))
    drf = None if point else np.ascontiguousarray(np.broadcast_to(q_store, (B_CALL, G, V)))
    counts = np.zeros((G + 1, V), np.int64)
    for r in range(calls):
        if point:
            # a deterministic proposer: fixed tokens (here a random one per trial)
            d = rng.integers(0, V, (B_CALL, G)).astype(np.int32)
        else:
            d = np.stack([rng.choice(V, size=B_CALL, p=q[i]) for i in range(G)], axis=1).astype(np.int32)
        x = {"target": tgt, "draft": drf, "draft_tokens": d,
             "gamma": np.full(B_CALL, G, np.int32)}
        say(f"[chi-square] V={V} gamma={G} {dtype}{' point-mass' if point else ''} top_k={top_k} "
            f"top_p={top_p}{' (cut path)' if force_cut else ''}: round {r}")
        if force_cut:
            with env(SPECDEC_TRUNC_CUT=1):
                out = gpu_verify(x, bf16=dtype == "bf16", temperature=T, seed=77, round=r,
                                 top_k=top_k, top_p=top_p)
        else:
            out = gpu_verify(x, bf16=dtype == "bf16", temperature=T, seed=77, round=r,
                             top_k=top_k, top_p=top_p)
        m = out["accept_count"]
        for i in range(G + 1):
            reached = m >= i
            counts[i] += np.bincount(out["out_tokens"][reached, i], minlength=V)[:V]
        if point:
            # a rejection never commits the rejected token itself
            rej = m < G
            assert not np.any(out["out_tokens"][rej, m[rej]] == d[rej, m[rej]])
    bad = []
    for i in range(G + 1):
        if np.any(counts[i][p[i] == 0] != 0):
            bad.append(f"position {i}: tokens outside the kept set committed: {counts[i]}")
            continue
        pv = chisq_fit(counts[i], p[i])
        say(f"  position {i}: {counts[i].sum()} trials, p-value {pv:.3g}")
        if pv < P_MIN:
            bad.append(f"position {i}: p-value {pv:.2e}")
    assert not bad, "; ".join(bad)
    # the acceptance rate at position 0 is sum_v min(p, q) (point mass: p(d))
    n0 = calls * B_CALL
    acc0 = counts[1].sum() / n0
    want = float(np.minimum(p[0], q[0]).sum()) if not point else float(p[0].mean())
    assert abs(acc0 - want) < 5 * np.sqrt(want * (1 - want) / n0) + 1e-9, (acc0, want)
