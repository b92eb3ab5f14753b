"""The seeded input generator: reproducible, per-request independent, with
the documented shapes and value recipes (no GPU)."""
import numpy as np
import pytest

from speculative_decoding_verification_05_amd import synth


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e-3, 65504.0], np.float32)
    h = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(h)
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa -> 1.0
    assert back[0] == 1.0 and back[1] == 1.0
    assert back[2] == np.float32(1.0 + 2 ** -7)
    assert back[3] == -2.5
    rel = np.abs(back - x) / np.abs(x)
    assert np.all(rel <= 2.0 ** -8)  # half a bf16 ulp (7 stored mantissa bits)


def test_subset_regeneration_is_bit_identical():
    wl = synth.WORKLOADS["b64_g4_v128256_bf16"].scaled(6, 3000)
    full = synth.make_verify_inputs(wl, threads=3)
    for b in (0, 4):
        one = synth.make_request_inputs(wl, b)
        assert np.array_equal(one["target"], full["target"][b])
        assert np.array_equal(one["draft"], full["draft"][b])
        assert np.array_equal(one["draft_tokens"], full["draft_tokens"][b])


def test_ragged_padding_and_gamma():
    wl = synth.WORKLOADS["b512_ragged_v262144_kv"].scaled(16, 512)
    x = synth.make_verify_inputs(wl)
    g = x["gamma"]
    assert g.min() >= 1 and g.max() <= 8
    for b in range(16):
        assert np.all(x["target"][b, g[b] + 1:] == synth.BF16_QNAN)
        assert np.all(x["draft"][b, g[b]:] == synth.BF16_QNAN)
        assert np.all(x["draft_tokens"][b, g[b]:] == -1)
        assert np.all((x["draft_tokens"][b, :g[b]] >= 0) & (x["draft_tokens"][b, :g[b]] < 512))


def test_top_swap_recipe_rate():
    wl = synth.WORKLOADS["b256_g7_v151936_greedy_kv"].scaled(64, 2000)
    x = synth.make_verify_inputs(wl)
    vals = synth.bf16_bits_to_f32(x["target"][:, :7])
    top = np.argmax(vals, axis=2)
    rate = (x["draft_tokens"] != top).mean()
    assert 0.17 < rate < 0.33


def test_kv_window_blocks_are_distinct_and_in_range():
    wl = synth.WORKLOADS["b256_g7_v151936_greedy_kv"].scaled(32, 100)
    kv = synth.make_kv_inputs(wl)
    used = kv.block_table[kv.block_table >= 0]
    assert used.size == np.unique(used).size == kv.num_blocks
    for b in range(32):
        t = kv.seq_lens[b]
        for j in range(8):
            assert kv.block_table[b, (t + j) // 16] >= 0
    assert np.all(kv.pool == synth.KV_POISON)


def test_tree_inputs_follow_the_recipe():
    wl = synth.WORKLOADS["tree_b64_n16_v151936_greedy_kv"].scaled(6, 3000)
    x = synth.make_tree_inputs(wl)
    par = np.array(synth.TREE16)
    assert x["target"].shape == (6, 16, 3000) and np.all(x["parents"] == par)
    assert synth.tree_depths(par).max() == 5
    z = synth.bf16_bits_to_f32(x["target"])
    kids = [[j for j in range(1, 16) if par[j] == p] for p in range(16)]
    for b in range(6):
        for p, ks in enumerate(kids):
            if not ks:
                continue
            order = np.lexsort((np.arange(3000), -z[b, p]))
            top = set(order[:len(ks) + 1].tolist())
            toks = [int(x["tokens"][b, j]) for j in ks]
            assert len(set(toks)) == len(toks)          # distinct siblings
            assert set(toks) <= top                      # the target's top-ranked tokens
    again = synth.make_tree_inputs(wl)
    assert np.array_equal(again["tokens"], x["tokens"])


def test_ngram_histories_repeat():
    wl = synth.WORKLOADS["ngram_b512_ctx1k8k_g8"].scaled(24)
    x = synth.make_ngram_inputs(wl)
    lo, hi = wl.ngram[2], wl.ngram[3]
    L = x["hist_len"]
    assert np.all((L >= lo) & (L <= hi))
    for b in range(24):
        h = x["history"][b]
        assert np.all(h[:L[b]] >= 0) and np.all(h[:L[b]] < wl.vocab) and np.all(h[L[b]:] == -1)
        # copied spans make 8-grams recur far more than chance would
        grams = {tuple(h[i:i + 8]) for i in range(L[b] - 8)}
        assert len(grams) < 0.9 * (L[b] - 8)


def test_draft_kv_holds_the_proposer_window():
    wl = synth.WORKLOADS["b512_ragged_v262144_kv"].scaled(10, 64)
    pool, table, seq, nb = synth.make_draft_kv_inputs(wl)
    dk = wl.draft_kv
    assert pool.shape == (dk.layers, 2, nb, dk.block_size, dk.kv_heads, dk.head_dim)
    written = 0
    for b in range(10):
        g = synth.request_gamma(wl, b)
        for j in range(g):
            pos = seq[b] + j
            blk = table[b, pos // dk.block_size]
            assert np.all(pool[:, :, blk, pos % dk.block_size] != synth.KV_POISON)
            written += 1
    per_pos = dk.layers * 2 * dk.kv_heads * dk.head_dim
    assert int((pool != synth.KV_POISON).sum()) == written * per_pos
