"""Seeded synthetic inputs for the speculative-decoding verify-and-commit step.

This module only *produces inputs*: logits rows, draft tokens, per-request draft
lengths and the paged-KV fixtures.  It holds none of the verify arithmetic (no
temperature scaling, softmax, acceptance test, residual or inverse CDF), so the
CPU oracle and the HIP path can both be fed from it without sharing any of the
method's code.

Every request draws from its own counter-keyed streams
(``SeedSequence([data_seed, request, tag])``), so any subset of requests can be
regenerated bit-identically on its own and the full batch can be generated in
parallel threads.

Workloads (the shapes and value recipes of the verify step as studied on the
pages; sizes are the full-scale cases used for parity and timing):

* ``b8_g4_v32000_f32``       B=8,   gamma=4, V=32000, fp32, T=1.0 sampling
                              (greedy re-run uses the same logits).
* ``b64_g4_v128256_bf16``    B=64,  gamma=4, V=128256, bf16, T=0.8 sampling.
* ``b256_g7_v151936_greedy_kv``  B=256, gamma=7, V=151936, bf16 greedy + paged
                              KV commit (28 layers x 4 heads x 128, block 16).
* ``b128_g4_v128256_topk50_topp09``  B=128, gamma=4, V=128256, bf16, T=0.7,
                              top-k 50 then top-p 0.9.
* ``b512_ragged_v262144_kv`` B=512, gamma_i in U{1..8}, V=262144, bf16, T=1.0,
                              paged KV commit (32 layers x 8 heads x 128).
* ``b64_g4_v128256_topp09``  the b64_g4_v128256_bf16 recipe with top-p 0.9 and
                              no top-k (kept sets of hundreds to thousands of
                              tokens, too many to list).

* ``tree_b64_n16_v151936_greedy_kv``  B=64 draft trees of 16 nodes (depth 5,
                              the fixed topology TREE16 below), V=151936, bf16,
                              greedy tree verification + path commit into the
                              28 x 4 x 128 paged cache.  The k children of a
                              node carry the target's k top-ranked tokens
                              after it, the first child (the deepest branch)
                              the top-1, except that at rate 0.25 the top-1
                              sits at another child (or, for a single child,
                              is replaced by the second-ranked token).

* ``ngram_b512_ctx1k8k_g8``  prompt-lookup drafting over B=512 histories of
                              U{1024..8192} tokens (the ragged recipe's context
                              lengths), ids below 262144, n from 4 down to 2,
                              up to 8 tokens proposed.  A history is built
                              from segments of U{8..64} tokens: with
                              probability 1/2 a copy of an earlier span,
                              otherwise fresh Zipf(1.1)-ranked tokens (a
                              per-request random rank order), so n-grams recur
                              as in repetitive text.

The two KV workloads also carry a draft model's cache shape for the draft-cache
rollback (the pages give none; a small model of the same family is assumed):
24 layers x 2 heads x 64 beside the 28 x 4 x 128 target, and 18 layers x
1 head x 256 beside the 32 x 8 x 128 target.

The proposer itself is outside the verify step; draft tokens are emulated here
by a Gumbel-max draw from the draft logits at the workload temperature
(``argmax(z/T + G)``, G standard Gumbel), which is an exact categorical sample
of the draft's tempered distribution without computing it.  For the top-k/top-p
workload the draw is restricted to the draft's 50 largest raw logits.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Sequence

import numpy as np

# Stream tags: one independent stream per (request, purpose).
_TAG_TARGET, _TAG_DRAFT, _TAG_TOKENS, _TAG_SIGMA, _TAG_GAMMA = 0, 1, 2, 3, 4
_TAG_KV, _TAG_CTX, _TAG_ZIPF, _TAG_SWAP = 5, 6, 7, 8
_TAG_DRAFT_KV = 9
_TAG_TREE = 10
_TAG_HIST = 11

# A 16-node draft tree of depth 5 (node 0 = the pending token): four
# candidates for the first position, then narrowing branches, the shape of
# the multi-candidate trees that tree speculation verifies in one forward.
TREE16 = (-1, 0, 0, 0, 0, 1, 1, 1, 2, 2, 5, 5, 8, 10, 12, 13)

BF16_QNAN = np.uint16(0x7FC0)      # fill for padded (never used) logits rows
KV_POISON = np.uint16(0x7FA5)      # fill for untouched KV-pool entries (a NaN)
NO_BLOCK = -1                      # block-table entry that the step never reads


@dataclasses.dataclass(frozen=True)
class KVShape:
    layers: int
    kv_heads: int
    head_dim: int
    block_size: int
    ctx_lo: int
    ctx_hi: int


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    gamma_max: int
    vocab: int
    dtype: str                  # "bf16" or "f32"
    mode: str                   # "sample" or "greedy"
    temperature: float
    target_sigma: float
    draft_recipe: str           # "noise_fixed", "noise_per_request", "top_swap"
    draft_sigma: float = 0.0    # fixed noise sigma ("noise_fixed")
    sigma_lo: float = 0.0       # per-request sigma range ("noise_per_request")
    sigma_hi: float = 0.0
    swap_rate: float = 0.0      # "top_swap": draft top-1 is target's 2nd token
    zipf_s: float = 0.0         # rank bias -s*ln(rank) on both rows
    top_k: int = 0
    top_p: float = 1.0
    ragged: bool = False        # gamma_i ~ U{1..gamma_max}
    kv: Optional[KVShape] = None
    draft_kv: Optional[KVShape] = None   # the draft model's cache (rollback)
    tree: Optional[tuple] = None         # tree workloads: parent of each node (node 0 = root)
    ngram: Optional[tuple] = None        # n-gram workloads: (n_min, n_max, ctx_lo, ctx_hi)
    data_seed: int = 0
    verify_seed: int = 0

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def scaled(self, batch: int, vocab: Optional[int] = None, **kw) -> "Workload":
        """Same recipe at a smaller size (for fast parity cases)."""
        return dataclasses.replace(self, batch=batch, vocab=vocab or self.vocab,
                                   name=f"{self.name}@b{batch}v{vocab or self.vocab}", **kw)


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("b8_g4_v32000_f32", 8, 4, 32000, "f32", "sample", 1.0, 2.0,
             "noise_fixed", draft_sigma=0.5, data_seed=1001, verify_seed=43),
    Workload("b64_g4_v128256_bf16", 64, 4, 128256, "bf16", "sample", 0.8, 3.0,
             "noise_per_request", sigma_lo=0.2, sigma_hi=1.5,
             data_seed=1002, verify_seed=44),
    Workload("b256_g7_v151936_greedy_kv", 256, 7, 151936, "bf16", "greedy", 1.0, 3.0,
             "top_swap", swap_rate=0.25,
             kv=KVShape(28, 4, 128, 16, 512, 4096), draft_kv=KVShape(24, 2, 64, 16, 512, 4096),
             data_seed=1003, verify_seed=45),
    Workload("b128_g4_v128256_topk50_topp09", 128, 4, 128256, "bf16", "sample", 0.7, 4.0,
             "noise_fixed", draft_sigma=0.8, zipf_s=1.1, top_k=50, top_p=0.9,
             data_seed=1004, verify_seed=46),
    Workload("tree_b64_n16_v151936_greedy_kv", 64, 15, 151936, "bf16", "greedy", 1.0, 3.0,
             "top_swap", swap_rate=0.25, tree=TREE16,
             kv=KVShape(28, 4, 128, 16, 512, 4096), data_seed=1006, verify_seed=48),
    Workload("ngram_b512_ctx1k8k_g8", 512, 8, 262144, "bf16", "greedy", 1.0, 0.0,
             "history", zipf_s=1.1, ngram=(2, 4, 1024, 8192), data_seed=1007, verify_seed=49),
    Workload("b64_g4_v128256_topp09", 64, 4, 128256, "bf16", "sample", 0.8, 3.0,
             "noise_per_request", sigma_lo=0.2, sigma_hi=1.5, top_p=0.9,
             data_seed=1008, verify_seed=50),
    Workload("b512_ragged_v262144_kv", 512, 8, 262144, "bf16", "sample", 1.0, 3.0,
             "noise_fixed", draft_sigma=0.6, ragged=True,
             kv=KVShape(32, 8, 128, 16, 1024, 8192), draft_kv=KVShape(18, 1, 256, 16, 1024, 8192),
             data_seed=1005, verify_seed=47),
]}

HEADLINE = "b64_g4_v128256_bf16"


def _rng(seed: int, b: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b, tag])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _gumbel_argmax(z: np.ndarray, temperature: float, rng: np.random.Generator,
                   candidates: Optional[np.ndarray] = None) -> int:
    """Categorical draw of the draft's proposal via Gumbel-max (proposer stand-in)."""
    zz = z.astype(np.float64) if candidates is None else z[candidates].astype(np.float64)
    u = rng.random(zz.shape[0])
    u = np.maximum(u, np.finfo(np.float64).tiny)
    g = -np.log(-np.log(u))
    k = int(np.argmax(zz / temperature + g))
    return k if candidates is None else int(candidates[k])


def request_gamma(wl: Workload, b: int) -> int:
    if not wl.ragged:
        return wl.gamma_max
    return int(_rng(wl.data_seed, b, _TAG_GAMMA).integers(1, wl.gamma_max + 1))


def _request_logits(wl: Workload, b: int, need_draft_logits: bool):
    """Target rows [gmax+1][V], draft rows [gmax][V] (or None), draft tokens [gmax]."""
    V, G = wl.vocab, wl.gamma_max
    g_b = request_gamma(wl, b)
    rt = _rng(wl.data_seed, b, _TAG_TARGET)
    tgt32 = rt.standard_normal((g_b + 1, V), dtype=np.float32) * np.float32(wl.target_sigma)
    if wl.zipf_s:
        ranks = _rng(wl.data_seed, b, _TAG_ZIPF).permutation(V).astype(np.float64) + 1.0
        bias = (-wl.zipf_s * np.log(ranks)).astype(np.float32)
        tgt32 += bias[None, :]
    if wl.dtype == "bf16":
        tgt_store = f32_to_bf16_bits(tgt32)
        tgt_val = bf16_bits_to_f32(tgt_store)
    else:
        tgt_store = tgt32
        tgt_val = tgt32

    tokens = np.full(G, -1, dtype=np.int32)
    rtok = _rng(wl.data_seed, b, _TAG_TOKENS)
    drf_store = None
    if wl.draft_recipe == "top_swap":
        # The draft agrees with the target's top-1 except, at rate swap_rate, it
        # ranks the target's second token first (top-1/top-2 values swapped).
        coins = _rng(wl.data_seed, b, _TAG_SWAP).random(G)
        if need_draft_logits:
            drf_val = tgt_val[:g_b].copy()
        for i in range(g_b):
            row = tgt_val[i]
            first = int(np.argmax(row))
            masked = row.copy()
            masked[first] = -np.inf
            second = int(np.argmax(masked))
            if coins[i] < wl.swap_rate:
                tokens[i] = second
                if need_draft_logits:
                    drf_val[i, first], drf_val[i, second] = row[second], row[first]
            else:
                tokens[i] = first
        if need_draft_logits:
            drf_store = f32_to_bf16_bits(drf_val) if wl.dtype == "bf16" else drf_val
        return tgt_store, drf_store, tokens, g_b

    if wl.draft_recipe == "noise_per_request":
        sigma = float(_rng(wl.data_seed, b, _TAG_SIGMA).uniform(wl.sigma_lo, wl.sigma_hi))
    else:
        sigma = wl.draft_sigma
    rd = _rng(wl.data_seed, b, _TAG_DRAFT)
    drf32 = tgt_val[:g_b] + rd.standard_normal((g_b, V), dtype=np.float32) * np.float32(sigma)
    if wl.dtype == "bf16":
        drf_store = f32_to_bf16_bits(drf32)
        drf_val = bf16_bits_to_f32(drf_store)
    else:
        drf_store = drf32
        drf_val = drf32
    for i in range(g_b):
        cand = None
        if wl.top_k:
            cand = np.argpartition(drf_val[i], V - wl.top_k)[V - wl.top_k:]
        tokens[i] = _gumbel_argmax(drf_val[i], wl.temperature, rtok, cand)
    return tgt_store, drf_store, tokens, g_b


def _pool_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_verify_inputs(wl: Workload, need_draft_logits: Optional[bool] = None,
                       threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Full batch of verify inputs in the padded device layout.

    Returns ``target`` [B][gmax+1][V], ``draft`` [B][gmax][V] (bf16 bit patterns
    as uint16, or float32), ``draft_tokens`` [B][gmax] int32 (-1 past gamma_i)
    and ``gamma`` [B] int32.  Rows past a request's gamma_i hold a NaN pattern.
    """
    if need_draft_logits is None:
        need_draft_logits = wl.mode == "sample"
    B, G, V = wl.batch, wl.gamma_max, wl.vocab
    st = np.uint16 if wl.dtype == "bf16" else np.float32
    fill = BF16_QNAN if wl.dtype == "bf16" else np.float32(np.nan)
    target = np.empty((B, G + 1, V), dtype=st)
    draft = np.empty((B, G, V), dtype=st) if need_draft_logits else None
    tokens = np.empty((B, G), dtype=np.int32)
    gamma = np.empty(B, dtype=np.int32)

    def one(b: int) -> None:
        t, d, tok, g_b = _request_logits(wl, b, need_draft_logits)
        target[b, :g_b + 1] = t
        target[b, g_b + 1:] = fill
        if draft is not None:
            draft[b, :g_b] = d
            draft[b, g_b:] = fill
        tokens[b] = tok
        gamma[b] = g_b

    with ThreadPoolExecutor(threads or _pool_threads()) as ex:
        list(ex.map(one, range(B)))
    return {"target": target, "draft": draft, "draft_tokens": tokens, "gamma": gamma}


def make_request_inputs(wl: Workload, b: int, need_draft_logits: Optional[bool] = None):
    """One request's rows, bit-identical to row b of :func:`make_verify_inputs`."""
    if need_draft_logits is None:
        need_draft_logits = wl.mode == "sample"
    t, d, tok, g_b = _request_logits(wl, b, need_draft_logits)
    return {"target": t, "draft": d, "draft_tokens": tok, "gamma": g_b}


# ---------------------------------------------------------------- paged KV

@dataclasses.dataclass
class KVInputs:
    scratch: np.ndarray       # uint16 [B][gmax+1][L][2][H][D]
    pool: np.ndarray          # uint16 [L][2][num_blocks][block][H][D], poison-filled
    block_table: np.ndarray   # int32 [B][max_blocks_per_req]
    seq_lens: np.ndarray      # int32 [B] (t_i: valid cache entries before the round)
    num_blocks: int


def kv_pool_shape(wl: Workload, num_blocks: int):
    kv = wl.kv
    return (kv.layers, 2, num_blocks, kv.block_size, kv.kv_heads, kv.head_dim)


def tree_depths(parents: Sequence[int]) -> np.ndarray:
    """Depth of every node of a parent array (node 0 = root)."""
    d = np.zeros(len(parents), np.int32)
    for j in range(1, len(parents)):
        d[j] = d[parents[j]] + 1
    return d


def kv_window(wl: Workload, b: int) -> int:
    """Last window offset the commit of request b may touch: gamma_b for a
    chain, the tree's depth for a tree."""
    if wl.tree is not None:
        return int(tree_depths(wl.tree).max())
    return request_gamma(wl, b)


def make_tree_inputs(wl: Workload, threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Greedy tree verification inputs: ``target`` [B][N][V] (row j = the
    target after the path to node j), ``tokens`` [B][N], ``parents`` [B][N]
    (wl.tree for every request), ``num_nodes`` [B]."""
    par = np.array(wl.tree, np.int32)
    N, V, B = len(par), wl.vocab, wl.batch
    assert N == wl.gamma_max + 1
    kids = [[j for j in range(1, N) if par[j] == p] for p in range(N)]
    target = np.empty((B, N, V), dtype=np.uint16 if wl.dtype == "bf16" else np.float32)
    tokens = np.zeros((B, N), np.int32)

    def one(b: int) -> None:
        rt = _rng(wl.data_seed, b, _TAG_TARGET)
        z = rt.standard_normal((N, V), dtype=np.float32) * np.float32(wl.target_sigma)
        if wl.dtype == "bf16":
            target[b] = f32_to_bf16_bits(z)
            zv = bf16_bits_to_f32(target[b])
        else:
            target[b] = z
            zv = z
        rtree = _rng(wl.data_seed, b, _TAG_TREE)
        coins = rtree.random(N)
        for p in range(N):
            k = len(kids[p])
            if k == 0:
                continue
            top = np.argpartition(zv[p], V - (k + 1))[V - (k + 1):]
            top = top[np.lexsort((top, -zv[p][top]))]     # rank order, lowest index first
            ranked = list(top[:k])
            if coins[p] < wl.swap_rate:
                # the draft's first candidate is not the target's choice: the
                # target's token sits at another child, or nowhere when the
                # node has a single child
                if k > 1:
                    c = int(rtree.integers(1, k))
                    ranked[0], ranked[c] = ranked[c], ranked[0]
                else:
                    ranked[0] = top[k]
            for c, j in enumerate(kids[p]):
                tokens[b, j] = ranked[c]

    with ThreadPoolExecutor(threads or _pool_threads()) as ex:
        list(ex.map(one, range(B)))
    return {"target": target, "tokens": tokens, "parents": np.tile(par, (B, 1)),
            "num_nodes": np.full(B, N, np.int32)}


def make_ngram_inputs(wl: Workload, threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Token histories for prompt-lookup drafting: ``history`` [B][max_len]
    int32 (-1 past a row's length) and ``hist_len`` [B].  Lengths follow the
    workload's context range (``ngram[2] .. ngram[3]``)."""
    B, V = wl.batch, wl.vocab
    lo, hi = wl.ngram[2], wl.ngram[3]
    lens = np.array([int(_rng(wl.data_seed, b, _TAG_CTX).integers(lo, hi + 1)) for b in range(B)],
                    np.int32)
    hist = np.full((B, hi), -1, np.int32)
    # Zipf(s) over token ranks 1..V, by inverse CDF on a shared table
    w = 1.0 / np.arange(1, V + 1, dtype=np.float64) ** wl.zipf_s
    cdf = np.cumsum(w / w.sum())

    def one(b: int) -> None:
        r = _rng(wl.data_seed, b, _TAG_HIST)
        perm = r.permutation(V).astype(np.int32)
        L = int(lens[b])
        out = np.empty(L, np.int32)
        n = 0
        while n < L:
            seg = int(r.integers(8, 65))
            seg = min(seg, L - n)
            if n >= seg and r.random() < 0.5:
                st = int(r.integers(0, n - seg + 1))
                out[n:n + seg] = out[st:st + seg]
            else:
                ranks = np.searchsorted(cdf, r.random(seg), side="right")
                out[n:n + seg] = perm[np.minimum(ranks, V - 1)]
            n += seg
        hist[b, :L] = out

    with ThreadPoolExecutor(threads or _pool_threads()) as ex:
        list(ex.map(one, range(B)))
    return {"history": hist, "hist_len": lens}


def make_kv_inputs(wl: Workload, with_pool: bool = True,
                   threads: Optional[int] = None, with_scratch: bool = True) -> KVInputs:
    """Scratch K/V for the gamma+1 verified slots, block table and context lengths.

    Only the (at most two) physical blocks that a request's commit window
    [t_i, t_i + gamma_i] touches are backed; all other block-table entries are
    NO_BLOCK.  The window blocks are a seeded random permutation of the pool so
    that writes scatter across it.
    """
    kv = wl.kv
    assert kv is not None
    B, G = wl.batch, wl.gamma_max
    L, H, D, bs = kv.layers, kv.kv_heads, kv.head_dim, kv.block_size
    seq = np.array([int(_rng(wl.data_seed, b, _TAG_CTX).integers(kv.ctx_lo, kv.ctx_hi + 1))
                    for b in range(B)], dtype=np.int32)
    gam = np.array([kv_window(wl, b) for b in range(B)], dtype=np.int32)
    max_blocks = (kv.ctx_hi + G + 1 + bs - 1) // bs
    first = seq // bs
    last = (seq + gam) // bs
    n_window = (last - first + 1).astype(np.int64)
    num_blocks = int(n_window.sum())
    perm = _rng(wl.data_seed, 0, _TAG_KV + 100).permutation(num_blocks).astype(np.int32)
    table = np.full((B, max_blocks), NO_BLOCK, dtype=np.int32)
    k = 0
    for b in range(B):
        for blk in range(first[b], last[b] + 1):
            table[b, blk] = perm[k]
            k += 1
    scratch = np.empty((B, G + 1, L, 2, H, D) if with_scratch else (0,), dtype=np.uint16)

    def one(b: int) -> None:
        r = _rng(wl.data_seed, b, _TAG_KV)
        scratch[b] = f32_to_bf16_bits(r.standard_normal((G + 1, L, 2, H, D), dtype=np.float32))

    if with_scratch:
        with ThreadPoolExecutor(threads or _pool_threads()) as ex:
            list(ex.map(one, range(B)))
    pool = None
    if with_pool:
        pool = np.full(kv_pool_shape(wl, num_blocks), KV_POISON, dtype=np.uint16)
    return KVInputs(scratch, pool, table, seq, num_blocks)


def make_draft_kv_inputs(wl: Workload, kv: Optional[KVInputs] = None,
                         threads: Optional[int] = None):
    """The draft model's paged cache at the end of proposing.

    It shares the target's block table and context lengths (one table per
    request for both models) and has its own pool of the same number of
    blocks, shaped by ``wl.draft_kv``.  Positions t_i .. t_i + gamma_i - 1 hold
    the draft's own K/V, written while it proposed (random bf16); every other
    entry is poison.  Returns (pool, block_table, seq_lens, num_blocks).
    """
    if kv is None:
        kv = make_kv_inputs(wl, with_pool=False, threads=threads, with_scratch=False)
    dk = wl.draft_kv
    assert dk is not None and dk.block_size == wl.kv.block_size
    shape = (dk.layers, 2, kv.num_blocks, dk.block_size, dk.kv_heads, dk.head_dim)
    pool = np.full(shape, KV_POISON, dtype=np.uint16)
    bs = dk.block_size
    for b in range(wl.batch):
        g = request_gamma(wl, b)
        if g == 0:
            continue
        r = _rng(wl.data_seed, b, _TAG_DRAFT_KV)
        vals = f32_to_bf16_bits(r.standard_normal((g, dk.layers, 2, dk.kv_heads, dk.head_dim),
                                                  dtype=np.float32))
        for j in range(g):
            pos = int(kv.seq_lens[b]) + j
            blk = int(kv.block_table[b, pos // bs])
            pool[:, :, blk, pos % bs] = vals[j]
    return pool, kv.block_table, kv.seq_lens.copy(), kv.num_blocks


def logits_bytes(wl: Workload, gamma: Optional[Sequence[int]] = None) -> int:
    """Bytes of the logits rows a verify call must read once (used rows only)."""
    if gamma is None:
        gamma = [wl.gamma_max] * wl.batch
    rows = 0
    for g in gamma:
        g = int(g)
        rows += (g + 1) + (g if wl.mode == "sample" else 0)
    return int(rows) * int(wl.vocab) * int(wl.elem_bytes)
