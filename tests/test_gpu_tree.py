"""GPU parity of specdec_verify_tree and the path commit against the oracle
(through the C ABI).  Greedy tree verification has no tolerance: accept
counts, committed tokens, paths, num_tokens and flags must be bit-exact, and
the committed K/V bytes identical."""
import numpy as np
import pytest

import oracle
import speculative_decoding_verification_05_amd as sd
from speculative_decoding_verification_05_amd import synth
from gpu_helpers import env, say, to_dev

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
TREE = "tree_b64_n16_v151936_greedy_kv"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    sd.lib()
    yield
    torch.cuda.empty_cache()


def gpu_tree(x, *, eos_token=-1, max_tokens=None, use_num_nodes=True, dev="cuda"):
    import torch
    t = x["target"]
    B, N, V = t.shape
    desc = sd.make_tree_desc(B, N, V, bf16=t.dtype == np.uint16, eos_token=eos_token)
    ws = torch.zeros(sd.specdec_verify_tree_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    i32 = torch.int32
    out = {"accept_count": torch.full((B,), -7, dtype=i32, device=dev),
           "num_tokens": torch.full((B,), -7, dtype=i32, device=dev),
           "out_tokens": torch.full((B, N), -7, dtype=i32, device=dev),
           "path": torch.full((B, N), -7, dtype=i32, device=dev),
           "flags": torch.full((B,), -1, dtype=i32, device=dev)}
    nn = to_dev(x["num_nodes"], dev) if use_num_nodes else None
    mt = None if max_tokens is None else to_dev(np.asarray(max_tokens, np.int32), dev)
    sd.specdec_verify_tree(desc, to_dev(t, dev), to_dev(x["tokens"], dev), to_dev(x["parents"], dev),
                           nn, mt, out["accept_count"], out["num_tokens"], out["out_tokens"],
                           out["path"], out["flags"], ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def check_tree(x, label, **kw):
    say(f"[tree] {label}: B={x['target'].shape[0]} N={x['target'].shape[1]} "
        f"V={x['target'].shape[2]}")
    got = gpu_tree(x, **kw)
    use_nn = kw.pop("use_num_nodes", True)
    ref = oracle.verify_tree(x["target"], x["tokens"], x["parents"],
                             x["num_nodes"] if use_nn else None, **kw)
    for k in ("accept_count", "num_tokens", "out_tokens", "path"):
        bad = np.argwhere(got[k] != ref[k])
        assert bad.size == 0, f"{label}: {k} differs at {bad[:5].tolist()}: " \
                              f"gpu {got[k][bad[0][0]]} oracle {ref[k][bad[0][0]]}"
    fl = got["flags"].astype(np.uint32)
    assert np.array_equal(fl, ref["flags"]), f"{label}: flags {fl} vs {ref['flags']}"
    return got, ref


def random_trees(B, N, V, rng, match=0.6, ties=True):
    z = (rng.integers(0, 4, (B, N, V)) if ties else rng.standard_normal((B, N, V)) * 3)
    z = z.astype(np.float32)
    am = np.argmax(z, axis=2)
    par = np.full((B, N), -1, np.int32)
    tok = rng.integers(0, V, (B, N)).astype(np.int32)
    for b in range(B):
        for j in range(1, N):
            par[b, j] = rng.integers(max(0, j - 6), j)
            if rng.random() < match:
                tok[b, j] = am[b, par[b, j]]
    return {"target": z, "tokens": tok, "parents": par,
            "num_nodes": rng.integers(1, N + 1, B).astype(np.int32)}


def test_one_kernel_tree_matches_two_kernel_path():
    """Tree verify in one launch writes the same bytes as the statistics
    kernel followed by the tree decision kernel (random trees with ties and
    ragged node counts, bf16 and fp32), on two calls in a row."""
    rng = np.random.default_rng(77)
    for B, N, V, bf16 in ((24, 16, 20000, True), (9, 64, 3000, False), (40, 5, 151936, True)):
        x = random_trees(B, N, V, rng)
        if bf16:
            x["target"] = synth.f32_to_bf16_bits(x["target"])
        label = f"B={B} N={N} V={V} {'bf16' if bf16 else 'fp32'}"
        with env(SPECDEC_FUSED=0):
            say(f"[one-kernel tree] {label}: two-kernel path (debug build)")
            ref = gpu_tree(x)
        say(f"[one-kernel tree] {label}: one kernel")
        outs = [gpu_tree(x) for _ in range(2)]
        for o in outs:
            for k in ref:
                assert np.array_equal(o[k], ref[k]), (label, k)


def test_drawn_tree_cases():
    """The tree of the drawing with the hand-derived outcomes of the oracle pin."""
    import pins
    rng = np.random.default_rng(91)
    rows = []
    for r in pins.golden_rows("tree_walkthrough.txt"):
        cols = [c.strip() for c in " ".join(r).split("|")]
        rows.append(([0] + [int(v) for v in cols[1].split()], [int(v) for v in cols[2].split()]))
    B, N, V = len(rows), 7, 100
    z = np.stack([pins._greedy_rows(ch, V, rng) for _, ch in rows])
    x = {"target": z, "tokens": np.array([t for t, _ in rows], np.int32),
         "parents": np.tile(np.array([-1, 0, 1, 2, 3, 2, 5], np.int32), (B, 1)),
         "num_nodes": np.full(B, N, np.int32)}
    check_tree(x, "drawn tree")


@pytest.mark.parametrize("B,N,V,ties", [(64, 12, 6, True), (40, 64, 50, True), (30, 1, 9, True),
                                        (24, 33, 20000, False), (16, 16, 8191, False)])
def test_random_trees(B, N, V, ties):
    """Random topologies (parents within 6 of the node), planted ties,
    ragged node counts, N = 1 and N = 64, unaligned rows (V = 8191)."""
    x = random_trees(B, N, V, np.random.default_rng(B * 1000 + N), ties=ties)
    check_tree(x, f"random N={N} V={V}")
    x["target"] = synth.f32_to_bf16_bits(x["target"])
    check_tree(x, f"random N={N} V={V} bf16")


def test_bad_parents_and_tokens_are_flagged():
    rng = np.random.default_rng(93)
    x = random_trees(12, 10, 30, rng)
    x["num_nodes"][:] = 10
    x["parents"][1, 4] = 4          # not below the node
    x["parents"][2, 7] = -3
    x["tokens"][3, 2] = 30          # outside [0, V)
    x["tokens"][4, 5] = -1
    got, _ = check_tree(x, "bad parents / tokens")
    assert got["flags"][1] & sd.FLAG_BAD_TREE and got["flags"][2] & sd.FLAG_BAD_TREE
    assert got["flags"][3] & sd.FLAG_TOKEN_RANGE and got["flags"][4] & sd.FLAG_TOKEN_RANGE


def test_eos_and_budget():
    rng = np.random.default_rng(95)
    x = random_trees(60, 20, 12, rng, match=0.8)
    mt = rng.integers(-1, 8, 60).astype(np.int32)
    for eos, budget in ((3, None), (-1, mt), (3, mt)):
        got, ref = check_tree(x, f"eos={eos} budget={budget is not None}", eos_token=eos,
                              max_tokens=budget)
    assert np.any(ref["flags"] & oracle.FLAG_EOS) and np.any(ref["flags"] & oracle.FLAG_LENGTH)


def test_no_num_nodes_means_all():
    x = random_trees(10, 9, 40, np.random.default_rng(97))
    x["num_nodes"][:] = 9
    check_tree(x, "num_nodes = NULL", use_num_nodes=False)


def test_tree_recipe_scaled():
    wl = W[TREE].scaled(16)
    check_tree(synth.make_tree_inputs(wl), "tree recipe B=16")


def test_tree_recipe_full_size():
    """B=64 trees of 16 nodes, V=151936 bf16: every request."""
    got, ref = check_tree(synth.make_tree_inputs(W[TREE]), "tree recipe full")
    say(f"  mean committed depth {ref['accept_count'].mean():.2f} of 5")


# ------------------------------------------------------------ path commit

@pytest.mark.parametrize("batch", [12, 64])
def test_path_commit_matches_oracle(batch):
    """verify_tree on the device, then specdec_commit_kv with its path as the
    slot map (scratch of N slots, window = tree depth), against the oracle's
    tree verification and commit."""
    import torch
    wl = W[TREE] if batch == W[TREE].batch else W[TREE].scaled(batch, 20000)
    x = synth.make_tree_inputs(wl)
    kv = synth.make_kv_inputs(wl)
    K = wl.kv
    N = wl.gamma_max + 1
    depth = np.array([synth.kv_window(wl, b) for b in range(wl.batch)], np.int32)
    dev = "cuda"
    tdesc = sd.make_tree_desc(wl.batch, N, wl.vocab)
    ws = torch.zeros(sd.specdec_verify_tree_workspace_bytes(tdesc), dtype=torch.uint8, device=dev)
    acc = torch.empty(wl.batch, dtype=torch.int32, device=dev)
    out = torch.empty(wl.batch, N, dtype=torch.int32, device=dev)
    path = torch.empty(wl.batch, N, dtype=torch.int32, device=dev)
    sd.specdec_verify_tree(tdesc, to_dev(x["target"], dev), to_dev(x["tokens"], dev),
                           to_dev(x["parents"], dev), None, None, acc, None, out, path, None, ws)
    kdesc = sd.make_kv_desc(wl.batch, N - 1, K.layers, K.kv_heads, K.head_dim, K.block_size,
                            kv.block_table.shape[1], kv.num_blocks, scratch_slots=N)
    kws = torch.zeros(sd.specdec_commit_kv_workspace_bytes(kdesc), dtype=torch.uint8, device=dev)
    pool = to_dev(kv.pool, dev)
    seq = to_dev(kv.seq_lens, dev)
    fl = torch.zeros(wl.batch, dtype=torch.int32, device=dev)
    sd.specdec_commit_kv(kdesc, to_dev(kv.scratch, dev), pool, to_dev(kv.block_table, dev), acc,
                         to_dev(depth, dev), path, seq, fl, kws)
    torch.cuda.synchronize()
    ref = oracle.verify_tree(x["target"], x["tokens"], x["parents"])
    want_pool, want_seq = kv.pool.copy(), kv.seq_lens.copy()
    oracle.commit_kv(kv.scratch, want_pool, kv.block_table, ref["accept_count"], want_seq, depth,
                     slot_map=ref["path"].clip(min=0))
    assert np.array_equal(acc.cpu().numpy(), ref["accept_count"])
    assert np.array_equal(path.cpu().numpy(), ref["path"])
    assert np.all(fl.cpu().numpy() == 0)
    assert np.array_equal(seq.cpu().numpy(), want_seq)
    got_pool = pool.cpu().numpy().view(np.uint16)
    bad = np.argwhere(got_pool != want_pool)
    assert bad.size == 0, f"pool differs at {bad[:5].tolist()}"
    say(f"[tree commit] B={wl.batch}: mean path depth {ref['accept_count'].mean():.2f}")
