"""GPU parity of truncation by cut records (top-p without an effective top-k
on large vocabularies, top-k past 1024, truncation with point-mass drafts)
against the CPU oracle.

p and q are softmax(z/T) restricted to their kept sets and renormalised
(AI-infra KB M013 s.04; the nxmr.cn note on lossless acceleration: top-p and
the like must show in the probabilities).  The kept set is a prefix of the
(logit desc, index asc) order, so the kernels keep it as a cut (boundary
logit, last kept index among the tokens tied at it) instead of a list; these
tests check that cut against the oracle's sorted prefix element by element,
including cuts that fall inside large groups of tied logits.  The same
comparison rules as the other parity tests apply (near-threshold decisions,
including a top-p cumulative within 1e-6 of top_p, excluded and counted).
"""
import numpy as np
import pytest

import speculative_decoding_verification_05_amd as sd
from speculative_decoding_verification_05_amd import synth
from gpu_helpers import compare, env, gpu_verify, oracle_verify, say

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    sd.lib()
    yield
    torch.cuda.empty_cache()


def check(wl, x=None, label=None, **kw):
    label = label or wl.name
    say(f"[cut] {label}: B={wl.batch} G={wl.gamma_max} V={wl.vocab} {wl.dtype} "
        f"top_k={kw.get('top_k', wl.top_k)} top_p={kw.get('top_p', wl.top_p)}")
    if x is None:
        x = synth.make_verify_inputs(wl)
    args = dict(temperature=wl.temperature, top_k=wl.top_k, top_p=wl.top_p, seed=wl.verify_seed)
    args.update(kw)
    got = gpu_verify(x, bf16=wl.dtype == "bf16", **args)
    ref = oracle_verify(x, **args)
    errs, near = compare(ref, got, x["gamma"], False, None, label)
    say(f"  near-threshold requests excluded from that decision on: {near}")
    assert not errs, "\n".join(errs[:20])
    return x, got, ref


def set_logits(x, key, vals):
    """Store float logits into x[key] in the workload's storage format,
    keeping its NaN padding rows."""
    arr = x[key]
    if arr.dtype == np.uint16:
        keep = arr == synth.BF16_QNAN
        arr[:] = synth.f32_to_bf16_bits(vals.astype(np.float32))
        arr[keep] = synth.BF16_QNAN
    else:
        keep = np.isnan(arr)
        arr[:] = vals.astype(np.float32)
        arr[keep] = np.nan


# ------------------------------------------------------------ full size

def test_top_p_alone_full_size_every_request():
    """B=64, gamma=4, V=128256 bf16, T=0.8, top-p 0.9 and no top-k: every
    request on the oracle."""
    check(W["b64_g4_v128256_topp09"])


def test_top_p_alone_262144_vocabulary():
    """The ragged recipe's 262144-token rows (T=1, ragged gamma), top-p 0.95."""
    wl = W["b512_ragged_v262144_kv"].scaled(40, top_k=0, top_p=0.95)
    check(wl)


def test_top_p_alone_fp32():
    """fp32 logits (three digits of the radix select): B=8, V=32000, top-p 0.9."""
    check(W["b8_g4_v32000_f32"], top_p=0.9)


@pytest.mark.parametrize("top_k,top_p", [(5000, 1.0), (2000, 0.95), (128255, 1.0), (1025, 0.5)])
def test_top_k_past_1024(top_k, top_p):
    """top-k above the listed-set limit, alone and followed by top-p, up to
    k = V - 1."""
    wl = W["b128_g4_v128256_topk50_topp09"].scaled(12, top_k=top_k, top_p=top_p)
    check(wl)


# ------------------------------------------------------------ forced cut path at small sizes

@pytest.mark.parametrize("vocab,top_k,top_p,dtype", [
    (40000, 50, 1.0, "bf16"), (40000, 1, 1.0, "bf16"), (40000, 1024, 0.95, "bf16"),
    (2000, 0, 0.8, "bf16"), (2000, 3000, 0.5, "bf16"), (10007, 50, 0.9, "bf16"),
    (5000, 0, 0.9, "f32"), (1500, 0, 0.99, "bf16"), (3001, 7, 0.3, "f32"), (64, 0, 0.6, "bf16")])
def test_forced_cut_path(vocab, top_k, top_p, dtype):
    """The debug build sends every truncation to the cut path: shapes the
    listed path also serves (unaligned rows, k = 1, the largest listed k,
    top-p alone on small vocabularies, fp32) against the oracle."""
    wl = W["b128_g4_v128256_topk50_topp09"].scaled(10, vocab, top_k=top_k, top_p=top_p, dtype=dtype)
    with env(SPECDEC_TRUNC_CUT=1):
        check(wl, label=f"forced cut V={vocab} k={top_k} p={top_p} {dtype}")


@pytest.mark.parametrize("top_k,top_p", [(0, 0.5), (0, 0.9), (5000, 1.0), (5000, 0.7), (0, 0.999)])
def test_cut_inside_large_tie_groups(top_k, top_p):
    """Integer logits in {0, 1, 2}: thousands of tokens share each value, so
    every cut falls inside a tie group and the index order decides (the
    listed path flags these rows as clipped; the cut path is exact)."""
    wl = W["b128_g4_v128256_topk50_topp09"].scaled(6, 60000, top_k=top_k, top_p=top_p)
    x = synth.make_verify_inputs(wl)
    rng = np.random.default_rng(8)
    for key in ("target", "draft"):
        set_logits(x, key, rng.integers(0, 3, x[key].shape).astype(np.float32))
    with env(SPECDEC_TRUNC_CUT=1):
        check(wl, x, label=f"ties k={top_k} p={top_p}")


def test_cut_tie_group_spanning_many_segments():
    """V=262144 with one tied value over a third of the row: the tie index is
    found from the per-segment counts and one segment read again."""
    wl = W["b512_ragged_v262144_kv"].scaled(4, top_k=0, top_p=0.5)
    x = synth.make_verify_inputs(wl)
    rng = np.random.default_rng(11)
    for key in ("target", "draft"):
        v = rng.choice(np.array([1.0, 0.5, -3.0], np.float32), size=x[key].shape, p=[0.3, 0.35, 0.35])
        set_logits(x, key, v)
    check(wl, x, label="tie group over many segments")


def test_cut_treats_negative_zero_as_zero():
    """Logits 0 stored as both +0 and -0 (bf16 0x0000 and 0x8000): equal
    logits, ordered by index alone."""
    wl = W["b128_g4_v128256_topk50_topp09"].scaled(6, 9000, top_k=0, top_p=0.6)
    x = synth.make_verify_inputs(wl)
    rng = np.random.default_rng(5)
    for key in ("target", "draft"):
        arr = x[key]
        pad = arr == synth.BF16_QNAN
        bits = np.where(rng.random(arr.shape) < 0.5, 0x0000, 0x8000).astype(np.uint16)
        top = rng.random(arr.shape) < 0.02
        bits[top] = synth.f32_to_bf16_bits(np.full(int(top.sum()), 0.75, np.float32))
        arr[:] = bits
        arr[pad] = synth.BF16_QNAN
    with env(SPECDEC_TRUNC_CUT=1):
        check(wl, x, label="signed zeros")


def test_cut_ragged_with_gamma_zero():
    """Ragged gamma with some gamma_b = 0 (a plain draw from the truncated
    bonus row) and padding rows never read."""
    wl = W["b512_ragged_v262144_kv"].scaled(24, 30000, top_k=0, top_p=0.85)
    x = synth.make_verify_inputs(wl)
    x["gamma"][::4] = 0
    check(wl, x, label="ragged, gamma 0")


def test_cut_nonfinite_rows_are_flagged():
    """A NaN in a used row flags the request (the row's cut is not searched)."""
    wl = W["b64_g4_v128256_topp09"].scaled(4, 20000)
    x = synth.make_verify_inputs(wl)
    x["target"][1, 0, 123] = synth.BF16_QNAN
    got = gpu_verify(x, bf16=True, temperature=wl.temperature, top_p=wl.top_p, seed=wl.verify_seed)
    assert got["flags"][1] & sd.FLAG_NONFINITE
    assert not np.any(got["flags"][[0, 2, 3]] & sd.FLAG_NONFINITE)


@pytest.mark.parametrize("vocab,top_k,top_p", [(128256, 50, 0.9), (128256, 0, 0.9), (32000, 2000, 1.0),
                                                (3000, 0, 0.5), (5000, 7, 1.0)])
def test_point_mass_drafts_with_truncation(vocab, top_k, top_p):
    """Point-mass drafts (no draft rows, as from an n-gram proposer) under
    truncation: p is the truncated target, q the point mass on the drafted
    token, so a draft is kept with probability p~(d) and a rejection draws
    from p~ without d (AI-infra KB M013 s.04 and s.08)."""
    wl = W["b128_g4_v128256_topk50_topp09"].scaled(16, vocab, top_k=top_k, top_p=top_p)
    x = synth.make_verify_inputs(wl)
    x["draft"] = None
    check(wl, x, label=f"point-mass drafts V={vocab} k={top_k} p={top_p}")


def test_cut_path_in_hip_graph_replays():
    """The cut path's three launches (statistics, cut records, decision; no
    fills) captured once and replayed three times, with eager calls on other
    inputs in between: every replay equals the eager call byte for byte, and
    the eager call the oracle."""
    import dataclasses
    import torch
    from gpu_helpers import to_dev
    wl = W["b64_g4_v128256_topp09"].scaled(16, 50000)
    x = synth.make_verify_inputs(wl)
    x2 = synth.make_verify_inputs(dataclasses.replace(wl, data_seed=wl.data_seed + 1))
    dev = "cuda"
    desc = sd.make_verify_desc(wl.batch, wl.gamma_max, wl.vocab, temperature=wl.temperature,
                               top_p=wl.top_p, seed=wl.verify_seed)
    ver = sd.Verifier(desc, dev)
    args = [to_dev(x[k], dev) for k in ("target", "draft", "draft_tokens", "gamma")]
    args2 = [to_dev(x2[k], dev) for k in ("target", "draft", "draft_tokens", "gamma")]
    names = ("accept_count", "num_tokens", "out_tokens", "p_draft", "q_draft", "residual_mass", "flags")

    def state():
        torch.cuda.synchronize()
        return {n: getattr(ver, n).cpu().numpy().copy() for n in names}

    say("[cut graph] eager call")
    ver(*args)
    want = state()
    ref = oracle_verify(x, temperature=wl.temperature, top_p=wl.top_p, seed=wl.verify_seed)
    errs, _ = compare(ref, want, x["gamma"], False, None, "cut graph")
    assert not errs, "\n".join(errs[:20])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        ver(*args)
    for k in range(3):
        ver(*args2)                      # eager work on other inputs between replays
        torch.cuda.synchronize()
        graph.replay()
        now = state()
        for n in names:
            assert np.array_equal(now[n], want[n]), (k, n)
        say(f"[cut graph] replay {k} matches the eager call")
