"""CPU oracle of the speculative-decoding verify-and-commit step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  It wraps ``liboracle.so``, a
plain single-threaded double-precision C restatement of the step (see
``specdec_oracle.c`` for the passages it follows), and shares no code with the
HIP path.  Its inputs come from the seeded generator; its outputs are never fed
back into the device path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "specdec_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FLAG_RESIDUAL_FALLBACK = 0x2
FLAG_NONFINITE = 0x4
FLAG_TOKEN_RANGE = 0x8
FLAG_EOS = 0x80
FLAG_LENGTH = 0x100
FLAG_BAD_TREE = 0x200


def _compile(src: str, out: str) -> None:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", "-I", HERE, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)


def build_sanitized(out: str) -> str:
    """Compile a copy of liboracle.so instrumented with AddressSanitizer and
    UndefinedBehaviorSanitizer (every report fatal), for the test that runs
    the pins against it in a process that preloads the ASan runtime."""
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", HERE, "-o", out, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def build() -> str:
    """Compile liboracle.so with gcc (-O2, no fast-math: IEEE double)."""
    _compile(SRC, LIB)
    return LIB


def build_copy(source_text: str, workdir: str) -> "Oracle":
    """Compile a (test-modified) copy of the oracle source and load it.

    Used only by tests that plant a mistake in the oracle to show that its
    pins catch it."""
    os.makedirs(workdir, exist_ok=True)
    src = os.path.join(workdir, "oracle_copy.c")
    with open(src, "w") as f:
        f.write(source_text)
    out = os.path.join(workdir, "liboracle_copy.so")
    _compile(src, out)
    return Oracle(out)


class _Args(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("gamma_max", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("is_bf16", ctypes.c_int32),
                ("greedy", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("temperature", ctypes.c_double), ("top_p", ctypes.c_double),
                ("seed", ctypes.c_uint64), ("round", ctypes.c_uint32),
                ("eos_token", ctypes.c_int32)]


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """A loaded oracle library (the default one, or a test build of a copy)."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        L.oracle_verify.argtypes = [ctypes.POINTER(_Args), P, P, P, P, P, P, ctypes.c_int32,
                                    P, P, P, P, P, P, P, P, P, P]
        L.oracle_verify.restype = ctypes.c_int
        L.oracle_row_distribution.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                              ctypes.c_int32, ctypes.c_double, P, P]
        L.oracle_row_distribution.restype = ctypes.c_int
        L.oracle_philox4x32_10.argtypes = [P, P, P]
        L.oracle_philox4x32_10.restype = None
        L.oracle_commit_kv.argtypes = ([ctypes.c_int32] * 7 + [ctypes.c_int64, ctypes.c_int32]
                                       + [P] * 7)
        L.oracle_commit_kv.restype = ctypes.c_int
        L.oracle_rollback_kv.argtypes = [ctypes.c_int32] * 7 + [ctypes.c_int64, P, P, P, P, P]
        L.oracle_rollback_kv.restype = ctypes.c_int
        L.oracle_verify_tree.argtypes = [ctypes.c_int32] * 4 + [P, P, P, P, ctypes.c_int32] + [P] * 6
        L.oracle_verify_tree.restype = ctypes.c_int
        L.oracle_propose_ngram.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, P, P, P]
        L.oracle_propose_ngram.restype = ctypes.c_int
        self.lib = L
        self.path = path

    def philox4x32_10(self, ctr, key) -> np.ndarray:
        c = np.ascontiguousarray(ctr, dtype=np.uint32)
        k = np.ascontiguousarray(key, dtype=np.uint32)
        out = np.zeros(4, dtype=np.uint32)
        self.lib.oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
        return out

    def row_distribution(self, row: np.ndarray, temperature: float = 1.0, top_k: int = 0,
                         top_p: float = 1.0):
        """Dense sampling distribution of one row; returns (prob, kept, near_cut)."""
        row = np.ascontiguousarray(row)
        is_bf16 = row.dtype == np.uint16
        if not is_bf16:
            row = row.astype(np.float32)
        prob = np.zeros(row.shape[0], dtype=np.float64)
        near = np.zeros(1, dtype=np.int32)
        kept = self.lib.oracle_row_distribution(_ptr(row), int(is_bf16), row.shape[0],
                                             float(temperature), int(top_k), float(top_p),
                                             _ptr(prob), _ptr(near))
        return prob, kept, bool(near[0])

    def verify(self, target: np.ndarray, draft: Optional[np.ndarray], draft_tokens: np.ndarray,
               gamma: Optional[np.ndarray] = None, *, greedy: bool = False,
               temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0,
               seed: int = 0, round: int = 0, requests=None,
               u_accept: Optional[np.ndarray] = None, u_sample: Optional[np.ndarray] = None,
               eos_token: int = -1, max_tokens: Optional[np.ndarray] = None):
        """Run the oracle on (a subset of) a padded batch.  Returns a dict of arrays.

        eos_token (-1: none) and max_tokens ([B] per-request token budget, or
        None) cut the committed list; accept_count is then the number of
        drafts left in it and num_tokens its length."""
        target = np.ascontiguousarray(target)
        B, G1, V = target.shape
        G = G1 - 1
        is_bf16 = target.dtype == np.uint16
        if draft is not None:
            draft = np.ascontiguousarray(draft)
            assert draft.dtype == target.dtype and draft.shape == (B, G, V)
        tokens = np.ascontiguousarray(draft_tokens, dtype=np.int32)
        assert tokens.shape == (B, G)
        if gamma is not None:
            gamma = np.ascontiguousarray(gamma, dtype=np.int32)
        ids = None
        n = B
        if requests is not None:
            ids = np.ascontiguousarray(requests, dtype=np.int32)
            n = ids.shape[0]
        if u_accept is not None:
            u_accept = np.ascontiguousarray(u_accept, dtype=np.float64)
            u_sample = np.ascontiguousarray(u_sample, dtype=np.float64)
            assert u_accept.shape == (n, G + 1) and u_sample.shape == (n, G + 1)
        if max_tokens is not None:
            max_tokens = np.ascontiguousarray(max_tokens, dtype=np.int32)
            assert max_tokens.shape == (B,)
        a = _Args(B, G, V, int(is_bf16), int(greedy), int(top_k), float(temperature),
                  float(top_p), int(seed) & (2**64 - 1), int(round) & 0xFFFFFFFF, int(eos_token))
        out = {
            "accept_count": np.zeros(n, np.int32),
            "num_tokens": np.zeros(n, np.int32),
            "out_tokens": np.zeros((n, G + 1), np.int32),
            "p_draft": np.zeros((n, G), np.float64),
            "q_draft": np.zeros((n, G), np.float64),
            "residual_mass": np.zeros(n, np.float64),
            "flags": np.zeros(n, np.uint32),
            "near_pos": np.zeros(n, np.int32),
        }
        rc = self.lib.oracle_verify(ctypes.byref(a), _ptr(target), _ptr(draft), _ptr(tokens),
                                 _ptr(gamma), _ptr(max_tokens), _ptr(ids), n, _ptr(u_accept),
                                 _ptr(u_sample), _ptr(out["accept_count"]),
                                 _ptr(out["num_tokens"]), _ptr(out["out_tokens"]),
                                 _ptr(out["p_draft"]), _ptr(out["q_draft"]),
                                 _ptr(out["residual_mass"]), _ptr(out["flags"]),
                                 _ptr(out["near_pos"]))
        if rc != 0:
            raise ValueError(f"oracle_verify rejected its arguments (code {rc})")
        return out

    def commit_kv(self, scratch: np.ndarray, pool: np.ndarray, block_table: np.ndarray,
                  accept_count: np.ndarray, seq_lens: np.ndarray, gamma=None, slot_map=None,
                  gamma_max: Optional[int] = None):
        """Apply the commit to ``pool`` and ``seq_lens`` in place (numpy uint16/int32).

        slot_map [B][G+1] (tree paths) names the scratch slot of each window
        position; gamma_max (G) then defaults to slot_map's width - 1."""
        B, S, L, two, H, D = scratch.shape
        assert two == 2 and pool.dtype == np.uint16 and scratch.dtype == np.uint16
        smap = None
        if slot_map is not None:
            smap = np.ascontiguousarray(slot_map, dtype=np.int32)
            G1 = smap.shape[1] if gamma_max is None else gamma_max + 1
            assert smap.shape == (B, G1)
        else:
            G1 = S if gamma_max is None else gamma_max + 1
        Lp, two2, NB, BS, Hp, Dp = pool.shape
        assert (Lp, two2, Hp, Dp) == (L, 2, H, D)
        assert pool.flags.c_contiguous and seq_lens.flags.c_contiguous
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        acc = np.ascontiguousarray(accept_count, dtype=np.int32)
        gam = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.int32)
        assert seq_lens.dtype == np.int32
        rc = self.lib.oracle_commit_kv(B, G1 - 1, L, H, D, BS, bt.shape[1], NB, S,
                                    _ptr(np.ascontiguousarray(scratch)), _ptr(smap), _ptr(pool),
                                    _ptr(bt), _ptr(acc), _ptr(gam), _ptr(seq_lens))
        if rc != 0:
            raise ValueError(f"oracle_commit_kv rejected its arguments (code {rc})")


    def verify_tree(self, target: np.ndarray, tokens: np.ndarray, parents: np.ndarray,
                    num_nodes: Optional[np.ndarray] = None, *, eos_token: int = -1,
                    max_tokens: Optional[np.ndarray] = None):
        """Greedy tree verification; returns a dict of arrays."""
        target = np.ascontiguousarray(target)
        B, N, V = target.shape
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        par = np.ascontiguousarray(parents, dtype=np.int32)
        assert tok.shape == (B, N) and par.shape == (B, N)
        nn = None if num_nodes is None else np.ascontiguousarray(num_nodes, dtype=np.int32)
        mt = None if max_tokens is None else np.ascontiguousarray(max_tokens, dtype=np.int32)
        out = {"accept_count": np.zeros(B, np.int32), "num_tokens": np.zeros(B, np.int32),
               "out_tokens": np.zeros((B, N), np.int32), "path": np.zeros((B, N), np.int32),
               "flags": np.zeros(B, np.uint32)}
        rc = self.lib.oracle_verify_tree(B, N, V, int(target.dtype == np.uint16), _ptr(target),
                                         _ptr(tok), _ptr(par), _ptr(nn), int(eos_token), _ptr(mt),
                                         _ptr(out["accept_count"]), _ptr(out["num_tokens"]),
                                         _ptr(out["out_tokens"]), _ptr(out["path"]),
                                         _ptr(out["flags"]))
        if rc != 0:
            raise ValueError(f"oracle_verify_tree rejected its arguments (code {rc})")
        return out

    def propose_ngram(self, history: np.ndarray, hist_len: np.ndarray, n_min: int, n_max: int,
                      gamma_max: int):
        """Prompt-lookup proposal; returns (draft_tokens [B][G], num_drafts [B], match_len [B])."""
        h = np.ascontiguousarray(history, dtype=np.int32)
        ln = np.ascontiguousarray(hist_len, dtype=np.int32)
        B, Lmax = h.shape
        toks = np.zeros((B, gamma_max), np.int32)
        nd = np.zeros(B, np.int32)
        ml = np.zeros(B, np.int32)
        rc = self.lib.oracle_propose_ngram(B, Lmax, _ptr(h), _ptr(ln), int(n_min), int(n_max),
                                           int(gamma_max), _ptr(toks), _ptr(nd), _ptr(ml))
        if rc != 0:
            raise ValueError(f"oracle_propose_ngram rejected its arguments (code {rc})")
        return toks, nd, ml

    def rollback_kv(self, pool: np.ndarray, block_table: np.ndarray, accept_count: np.ndarray,
                    seq_lens: np.ndarray, gamma_max: int, gamma=None):
        """Roll back a draft cache in place (``pool`` uint16, ``seq_lens`` int32)."""
        Lp, two, NB, BS, H, D = pool.shape
        assert two == 2 and pool.dtype == np.uint16 and pool.flags.c_contiguous
        assert seq_lens.dtype == np.int32 and seq_lens.flags.c_contiguous
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        acc = np.ascontiguousarray(accept_count, dtype=np.int32)
        gam = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.int32)
        rc = self.lib.oracle_rollback_kv(bt.shape[0], int(gamma_max), Lp, H, D, BS, bt.shape[1],
                                      NB, _ptr(pool), _ptr(bt), _ptr(acc), _ptr(gam),
                                      _ptr(seq_lens))
        if rc != 0:
            raise ValueError(f"oracle_rollback_kv rejected its arguments (code {rc})")


_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle built from this directory's source (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _default = Oracle(LIB)
    return _default


def philox4x32_10(ctr, key):
    return default().philox4x32_10(ctr, key)


def row_distribution(row, temperature=1.0, top_k=0, top_p=1.0):
    return default().row_distribution(row, temperature, top_k, top_p)


def verify(*args, **kw):
    return default().verify(*args, **kw)


def commit_kv(*args, **kw):
    return default().commit_kv(*args, **kw)


def rollback_kv(*args, **kw):
    return default().rollback_kv(*args, **kw)


def verify_tree(*args, **kw):
    return default().verify_tree(*args, **kw)


def propose_ngram(*args, **kw):
    return default().propose_ngram(*args, **kw)
