"""The one-kernel sampling verify against the two-kernel path on seeded
random shapes (batch, gamma_max, vocabulary, dtype, ragged gamma, point-mass
drafts, temperature): every output byte-equal, on two calls in a row with one
workspace; a third of the cases also against the CPU oracle."""
import dataclasses
import os

import numpy as np
import pytest

import speculative_decoding_verification_05_amd as sd
from speculative_decoding_verification_05_amd import synth
from gpu_helpers import compare, env, gpu_verify, oracle_verify, say

pytestmark = pytest.mark.gpu


def _cases(n=48, seed=20261202):
    rng = np.random.default_rng(seed)
    vocabs = [1, 8, 100, 1000, 4095, 4096, 4097, 10007, 32000, 65536, 128256, 200003]
    out = []
    while len(out) < n:
        B = int(rng.choice([1, 2, 3, 7, 16, 33, 100, 300]))
        G = int(rng.integers(0, 9))
        V = int(rng.choice(vocabs))
        if B * (2 * G + 1) * V > 40_000_000:
            continue
        out.append(dict(batch=B, gamma_max=G, vocab=V,
                        dtype=str(rng.choice(["bf16", "f32"])),
                        ragged=bool(rng.random() < 0.5) and G > 0,
                        point=bool(rng.random() < 0.25),
                        temperature=float(rng.choice([0.5, 0.8, 1.0, 1.7])),
                        data_seed=int(rng.integers(1, 1 << 30)),
                        verify_seed=int(rng.integers(0, 1 << 62)),
                        oracle=B * (2 * G + 1) * V <= 5_000_000 and len(out) % 3 == 0))
    return out


# SPECDEC_RANDOM_CASES / SPECDEC_RANDOM_SEED widen the sweep for a longer run
CASES = _cases(int(os.environ.get("SPECDEC_RANDOM_CASES", 48)),
               int(os.environ.get("SPECDEC_RANDOM_SEED", 20261202)))


@pytest.mark.parametrize("case", CASES, ids=[f"b{c['batch']}g{c['gamma_max']}v{c['vocab']}"
                                              f"{c['dtype']}{'r' if c['ragged'] else ''}"
                                              f"{'p' if c['point'] else ''}" for c in CASES])
def test_one_kernel_equals_two_kernel(case):
    wl = dataclasses.replace(synth.WORKLOADS[synth.HEADLINE], name="random", batch=case["batch"],
                             gamma_max=case["gamma_max"], vocab=case["vocab"],
                             dtype=case["dtype"], ragged=case["ragged"],
                             temperature=case["temperature"], data_seed=case["data_seed"],
                             verify_seed=case["verify_seed"])
    say(f"[one-kernel random] {case}")
    x = synth.make_verify_inputs(wl)
    if case["point"]:
        x["draft"] = None
    args = dict(bf16=wl.dtype == "bf16", temperature=wl.temperature, seed=wl.verify_seed)
    with env(SPECDEC_FUSED=0):
        ref = gpu_verify(x, **args)
    with env(SPECDEC_FUSED=None):
        outs = gpu_verify(x, reps=2, **args)
    for o in outs:
        for k in ref:
            assert np.array_equal(o[k], ref[k]), k
        assert not np.any(o["flags"] & sd.FLAG_WAIT_TIMEOUT)
    if case["oracle"]:
        oref = oracle_verify(x, temperature=wl.temperature, seed=wl.verify_seed)
        errs, near = compare(oref, ref, x["gamma"], False, None, "random")
        say(f"  oracle: near-threshold requests {near}")
        assert not errs, "\n".join(errs[:20])
