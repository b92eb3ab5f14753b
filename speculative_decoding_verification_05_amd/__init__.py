"""Speculative-decoding verify-and-commit on one MI355X (gfx950).

Thin Python binding of ``libspecdec.so`` (C ABI declared in
``include/specdec.h``).  The functions keep the C names and only marshal
arguments: torch tensors become device pointers, the current torch stream
becomes the HIP stream.  Every step of the computation runs in the HIP
kernels; there is no CPU fallback, and the functions raise if the library is
missing or refuses a call.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libspecdec.so")
# the same kernels built with the environment switches of the tests and
# tuning sweeps (SPECDEC_FUSED, SPECDEC_FUSED_WAIT_TICKS, ...); see debug_library()
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libspecdec_debug.so")

SPECDEC_OK = 0
SPECDEC_ERR_INVALID_ARGUMENT = 1
SPECDEC_ERR_WORKSPACE_TOO_SMALL = 2
SPECDEC_ERR_UNSUPPORTED = 3
SPECDEC_ERR_DEVICE = 4

SPECDEC_F32, SPECDEC_BF16 = 0, 1
SPECDEC_SAMPLE, SPECDEC_GREEDY = 0, 1

FLAG_RESIDUAL_FALLBACK = 0x2
FLAG_NONFINITE = 0x4
FLAG_TOKEN_RANGE = 0x8
FLAG_BAD_BLOCK = 0x10
FLAG_BAD_GAMMA = 0x20
FLAG_TRUNC_OVERFLOW = 0x40
FLAG_EOS = 0x80
FLAG_LENGTH = 0x100
FLAG_BAD_TREE = 0x200
FLAG_WAIT_TIMEOUT = 0x400

# exported symbols of include/specdec.h
EXPORTS = ("specdec_verify_workspace_bytes", "specdec_verify", "specdec_verify_profiled",
           "specdec_commit_kv_workspace_bytes", "specdec_commit_kv", "specdec_rollback_kv",
           "specdec_commit_and_rollback_kv",
           "specdec_verify_tree_workspace_bytes", "specdec_verify_tree",
           "specdec_verify_tree_profiled", "specdec_propose_ngram",
           "specdec_propose_ngram_workspace_bytes",
           "specdec_workspace_clear", "specdec_status_string", "specdec_abi_version",
           "specdec_verify_noalloc")


class VerifyDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("gamma_max", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("temperature", ctypes.c_float), ("top_p", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("round", ctypes.c_uint32),
                ("eos_plus1", ctypes.c_int32)]


class KVDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("gamma_max", ctypes.c_int32),
                ("num_layers", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks_per_req", ctypes.c_int32), ("scratch_slots", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64)]


class NgramDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_len", ctypes.c_int32),
                ("n_min", ctypes.c_int32), ("n_max", ctypes.c_int32),
                ("gamma_max", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class TreeDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_nodes", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("eos_plus1", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SpecdecError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


_lib = None
_loaded = {}


def lib() -> ctypes.CDLL:
    """The loaded libspecdec.so (build it with ``__graft_entry__.build()``),
    or the debug build inside ``debug_library()``."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def debug_library():
    """Every call in the block goes to libspecdec_debug.so: the same kernels,
    whose host code also reads the environment switches SPECDEC_FUSED (0: the
    two-kernel paths), SPECDEC_FUSED_WAIT_TICKS, SPECDEC_FUSED_LAG,
    SPECDEC_STATS_TILES, SPECDEC_SAMPLE_WPR and SPECDEC_TRUNC_CUT.  For tests and sweeps only."""
    global _lib
    old = _lib
    _lib = _load(DEBUG_LIB_PATH)
    try:
        yield _lib
    finally:
        _lib = old


def _hip_runtimes() -> set:
    """Files of the HIP runtime (libamdhip64) mapped into this process."""
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                p = line.split(None, 5)[-1].strip()
                if os.path.basename(p).startswith("libamdhip64.so"):
                    found.add(os.path.realpath(p))
    except OSError:
        pass
    return found


def _load(path: str) -> ctypes.CDLL:
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise ImportError(f"{os.path.basename(path)} is not built ({path}); run __graft_entry__.build()")
    # One HIP runtime per process.  torch ships its own libamdhip64 (soname
    # libamdhip64.so.7) and asks for it by the unversioned name; the library
    # asks for libamdhip64.so.7.  Loaded after torch, the library binds to
    # torch's copy by its soname.  Loaded first, it would bind the system
    # copy, and torch would then load its own beside it: the runtime that
    # initialises second finds no device it can open, and the process's
    # pinned host allocations fail from then on.
    try:
        import torch  # noqa: F401  (for its HIP runtime, loaded with it)
    except ImportError:
        pass
    L = ctypes.CDLL(path)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded in this process (" + ", ".join(sorted(runtimes))
                          + "); import torch before anything that loads a HIP runtime")
    P, S = ctypes.c_void_p, ctypes.c_size_t
    L.specdec_verify_workspace_bytes.argtypes = [ctypes.POINTER(VerifyDesc)]
    L.specdec_verify_workspace_bytes.restype = S
    L.specdec_verify.argtypes = [ctypes.POINTER(VerifyDesc)] + [P] * 13 + [S, P]
    L.specdec_verify.restype = ctypes.c_int
    L.specdec_verify_profiled.argtypes = [ctypes.POINTER(VerifyDesc)] + [P] * 13 + [S, P, P]
    L.specdec_verify_profiled.restype = ctypes.c_int
    L.specdec_verify_noalloc.argtypes = [ctypes.POINTER(VerifyDesc)] + [P] * 12 + [P]
    L.specdec_verify_noalloc.restype = ctypes.c_int
    L.specdec_commit_kv_workspace_bytes.argtypes = [ctypes.POINTER(KVDesc)]
    L.specdec_commit_kv_workspace_bytes.restype = S
    L.specdec_commit_kv.argtypes = [ctypes.POINTER(KVDesc)] + [P] * 9 + [S, P]
    L.specdec_commit_kv.restype = ctypes.c_int
    L.specdec_rollback_kv.argtypes = [ctypes.POINTER(KVDesc)] + [P] * 7 + [S, P]
    L.specdec_rollback_kv.restype = ctypes.c_int
    L.specdec_commit_and_rollback_kv.argtypes = (
        [ctypes.POINTER(KVDesc)] + [P] * 7 + [S] + [ctypes.POINTER(KVDesc)] + [P] * 5 + [S]
        + [P] * 3)
    L.specdec_commit_and_rollback_kv.restype = ctypes.c_int
    L.specdec_verify_tree_workspace_bytes.argtypes = [ctypes.POINTER(TreeDesc)]
    L.specdec_verify_tree_workspace_bytes.restype = S
    L.specdec_verify_tree.argtypes = [ctypes.POINTER(TreeDesc)] + [P] * 11 + [S, P]
    L.specdec_verify_tree.restype = ctypes.c_int
    L.specdec_verify_tree_profiled.argtypes = [ctypes.POINTER(TreeDesc)] + [P] * 11 + [S, P, P]
    L.specdec_verify_tree_profiled.restype = ctypes.c_int
    L.specdec_propose_ngram.argtypes = [ctypes.POINTER(NgramDesc)] + [P] * 6 + [S, P]
    L.specdec_propose_ngram.restype = ctypes.c_int
    L.specdec_propose_ngram_workspace_bytes.argtypes = [ctypes.POINTER(NgramDesc)]
    L.specdec_propose_ngram_workspace_bytes.restype = S
    L.specdec_workspace_clear.argtypes = [P, S, P]
    L.specdec_workspace_clear.restype = ctypes.c_int
    L.specdec_status_string.argtypes = [ctypes.c_int]
    L.specdec_status_string.restype = ctypes.c_char_p
    L.specdec_abi_version.argtypes = []
    L.specdec_abi_version.restype = ctypes.c_int32
    _loaded[path] = L
    return L


def status_string(status: int) -> str:
    return lib().specdec_status_string(int(status)).decode()


def _ptr(x) -> Optional[int]:
    """Device address of a tensor (or an int address); None stays NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("specdec arguments must be device tensors")
    if not x.is_contiguous():
        raise ValueError("specdec arguments must be contiguous")
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_verify_desc(batch, gamma_max, vocab, *, bf16=True, greedy=False, temperature=1.0,
                     top_k=0, top_p=1.0, seed=0, round=0, eos_token=-1) -> VerifyDesc:
    return VerifyDesc(int(batch), int(gamma_max), int(vocab),
                      SPECDEC_BF16 if bf16 else SPECDEC_F32,
                      SPECDEC_GREEDY if greedy else SPECDEC_SAMPLE, int(top_k),
                      float(temperature), float(top_p), int(seed) & (2 ** 64 - 1),
                      int(round) & 0xFFFFFFFF, int(eos_token) + 1)


def make_kv_desc(batch, gamma_max, num_layers, num_kv_heads, head_dim, block_size,
                 max_blocks_per_req, num_blocks, scratch_slots=0) -> KVDesc:
    return KVDesc(int(batch), int(gamma_max), int(num_layers), int(num_kv_heads),
                  int(head_dim), int(block_size), int(max_blocks_per_req), int(scratch_slots),
                  int(num_blocks))


def make_tree_desc(batch, num_nodes, vocab, *, bf16=True, eos_token=-1) -> TreeDesc:
    return TreeDesc(int(batch), int(num_nodes), int(vocab), SPECDEC_BF16 if bf16 else SPECDEC_F32,
                    int(eos_token) + 1, 0)


def make_ngram_desc(batch, max_len, n_min, n_max, gamma_max) -> NgramDesc:
    return NgramDesc(int(batch), int(max_len), int(n_min), int(n_max), int(gamma_max), 0)


def specdec_propose_ngram_workspace_bytes(desc: NgramDesc) -> int:
    return int(lib().specdec_propose_ngram_workspace_bytes(ctypes.byref(desc)))


def specdec_propose_ngram(desc: NgramDesc, history, hist_len, draft_tokens, num_drafts,
                          match_len, workspace, workspace_bytes: Optional[int] = None,
                          stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().specdec_propose_ngram(ctypes.byref(desc), _ptr(history), _ptr(hist_len),
                                     _ptr(draft_tokens), _ptr(num_drafts), _ptr(match_len),
                                     _ptr(workspace), int(workspace_bytes), _stream(stream))
    if st != SPECDEC_OK:
        raise SpecdecError(st, "specdec_propose_ngram")


def specdec_verify_tree_workspace_bytes(desc: TreeDesc) -> int:
    return int(lib().specdec_verify_tree_workspace_bytes(ctypes.byref(desc)))


def specdec_verify_tree(desc: TreeDesc, target_logits, node_tokens, parents, num_nodes,
                        max_tokens, accept_count, num_tokens, out_tokens, path, flags, workspace,
                        workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().specdec_verify_tree(ctypes.byref(desc), _ptr(target_logits), _ptr(node_tokens),
                                   _ptr(parents), _ptr(num_nodes), _ptr(max_tokens),
                                   _ptr(accept_count), _ptr(num_tokens), _ptr(out_tokens),
                                   _ptr(path), _ptr(flags), _ptr(workspace),
                                   int(workspace_bytes), _stream(stream))
    if st != SPECDEC_OK:
        raise SpecdecError(st, "specdec_verify_tree")


def specdec_verify_tree_profiled(desc: TreeDesc, target_logits, node_tokens, parents, num_nodes,
                                 max_tokens, accept_count, num_tokens, out_tokens, path, flags,
                                 workspace, stage_events, workspace_bytes: Optional[int] = None,
                                 stream=None) -> None:
    """stage_events: four raw hipEvent_t handles (ints; None entries allowed)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    handles = (ctypes.c_void_p * 4)(*[None if e is None else int(e) for e in stage_events])
    st = lib().specdec_verify_tree_profiled(ctypes.byref(desc), _ptr(target_logits),
                                            _ptr(node_tokens), _ptr(parents), _ptr(num_nodes),
                                            _ptr(max_tokens), _ptr(accept_count),
                                            _ptr(num_tokens), _ptr(out_tokens), _ptr(path),
                                            _ptr(flags), _ptr(workspace), int(workspace_bytes),
                                            _stream(stream), handles)
    if st != SPECDEC_OK:
        raise SpecdecError(st, "specdec_verify_tree_profiled")


def specdec_verify_workspace_bytes(desc: VerifyDesc) -> int:
    return int(lib().specdec_verify_workspace_bytes(ctypes.byref(desc)))


def specdec_commit_kv_workspace_bytes(desc: KVDesc) -> int:
    return int(lib().specdec_commit_kv_workspace_bytes(ctypes.byref(desc)))


def specdec_verify(desc: VerifyDesc, target_logits, draft_logits, draft_tokens, gamma,
                   max_tokens, accept_count, num_tokens, out_tokens, p_draft, q_draft,
                   residual_mass, flags, workspace, workspace_bytes: Optional[int] = None,
                   stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().specdec_verify(ctypes.byref(desc), _ptr(target_logits), _ptr(draft_logits),
                              _ptr(draft_tokens), _ptr(gamma), _ptr(max_tokens),
                              _ptr(accept_count), _ptr(num_tokens),
                              _ptr(out_tokens), _ptr(p_draft), _ptr(q_draft),
                              _ptr(residual_mass), _ptr(flags), _ptr(workspace),
                              int(workspace_bytes), _stream(stream))
    if st != SPECDEC_OK:
        raise SpecdecError(st, "specdec_verify")


def specdec_verify_noalloc(desc: VerifyDesc, target_logits, draft_logits, draft_tokens, gamma,
                           max_tokens, accept_count, num_tokens, out_tokens, p_draft, q_draft,
                           residual_mass, flags, stream=None) -> None:
    """specdec_verify with the library's own per-GPU workspace (no allocation)."""
    st = lib().specdec_verify_noalloc(ctypes.byref(desc), _ptr(target_logits), _ptr(draft_logits),
                                      _ptr(draft_tokens), _ptr(gamma), _ptr(max_tokens),
                                      _ptr(accept_count), _ptr(num_tokens),
                                      _ptr(out_tokens), _ptr(p_draft), _ptr(q_draft),
                                      _ptr(residual_mass), _ptr(flags), _stream(stream))
    if st != SPECDEC_OK:
        raise SpecdecError(st, "specdec_verify_noalloc")


def specdec_verify_profiled(desc: VerifyDesc, target_logits, draft_logits, draft_tokens, gamma,
                            max_tokens, accept_count, num_tokens, out_tokens, p_draft, q_draft,
                            residual_mass, flags, workspace, stage_events,
                            workspace_bytes: Optional[int] = None, stream=None) -> None:
    """stage_events: four raw hipEvent_t handles (ints; None entries allowed)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    handles = (ctypes.c_void_p * 4)(*[None if e is None else int(e) for e in stage_events])
    st = lib().specdec_verify_profiled(ctypes.byref(desc), _ptr(target_logits), _ptr(draft_logits),
                                       _ptr(draft_tokens), _ptr(gamma), _ptr(max_tokens),
                                       _ptr(accept_count), _ptr(num_tokens),
                                       _ptr(out_tokens), _ptr(p_draft), _ptr(q_draft),
                                       _ptr(residual_mass), _ptr(flags), _ptr(workspace),
                                       int(workspace_bytes), _stream(stream), handles)
    if st != SPECDEC_OK:
        raise SpecdecError(st, "specdec_verify_profiled")


def specdec_commit_kv(desc: KVDesc, scratch_kv, kv_pool, block_table, accept_count, gamma,
                      slot_map, seq_lens, flags, workspace, workspace_bytes: Optional[int] = None,
                      stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().specdec_commit_kv(ctypes.byref(desc), _ptr(scratch_kv), _ptr(kv_pool),
                                 _ptr(block_table), _ptr(accept_count), _ptr(gamma),
                                 _ptr(slot_map), _ptr(seq_lens), _ptr(flags), _ptr(workspace),
                                 int(workspace_bytes), _stream(stream))
    if st != SPECDEC_OK:
        raise SpecdecError(st, "specdec_commit_kv")


def specdec_rollback_kv(desc: KVDesc, kv_pool, block_table, accept_count, gamma, seq_lens,
                        flags, workspace, workspace_bytes: Optional[int] = None,
                        stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().specdec_rollback_kv(ctypes.byref(desc), _ptr(kv_pool), _ptr(block_table),
                                   _ptr(accept_count), _ptr(gamma), _ptr(seq_lens), _ptr(flags),
                                   _ptr(workspace), int(workspace_bytes), _stream(stream))
    if st != SPECDEC_OK:
        raise SpecdecError(st, "specdec_rollback_kv")


def specdec_commit_and_rollback_kv(desc: KVDesc, scratch_kv, kv_pool, block_table, slot_map,
                                   seq_lens, flags, workspace, draft_desc: KVDesc, draft_pool,
                                   draft_block_table, draft_seq_lens, draft_flags,
                                   draft_workspace, accept_count, gamma, stream=None) -> None:
    st = lib().specdec_commit_and_rollback_kv(
        ctypes.byref(desc), _ptr(scratch_kv), _ptr(kv_pool), _ptr(block_table), _ptr(slot_map),
        _ptr(seq_lens), _ptr(flags), _ptr(workspace), workspace.numel() * workspace.element_size(),
        ctypes.byref(draft_desc), _ptr(draft_pool), _ptr(draft_block_table), _ptr(draft_seq_lens),
        _ptr(draft_flags), _ptr(draft_workspace),
        draft_workspace.numel() * draft_workspace.element_size(),
        _ptr(accept_count), _ptr(gamma), _stream(stream))
    if st != SPECDEC_OK:
        raise SpecdecError(st, "specdec_commit_and_rollback_kv")


def specdec_workspace_clear(workspace, nbytes: Optional[int] = None, stream=None) -> None:
    if nbytes is None:
        nbytes = workspace.numel() * workspace.element_size()
    st = lib().specdec_workspace_clear(_ptr(workspace), int(nbytes), _stream(stream))
    if st != SPECDEC_OK:
        raise SpecdecError(st, "specdec_workspace_clear")


def specdec_abi_version() -> int:
    return int(lib().specdec_abi_version())


class HipEvents:
    """Raw timing events of the HIP runtime (for specdec_verify_profiled)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles.append(h.value)

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[a], self.handles[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self) -> None:
        for h in self.handles:
            self.hip.hipEventDestroy(h)
        self.handles = []


class Verifier:
    """Owns the outputs and the zero-initialised workspace of one verify shape.

    ``verifier(target, draft, draft_tokens, gamma)`` enqueues specdec_verify
    on the current stream and returns the output tensors (still on device).
    """

    def __init__(self, desc: VerifyDesc, device="cuda"):
        import torch
        self.desc = desc
        B, G = desc.batch, desc.gamma_max
        nbytes = specdec_verify_workspace_bytes(desc)
        if nbytes == 0:
            raise SpecdecError(SPECDEC_ERR_INVALID_ARGUMENT, "specdec_verify_workspace_bytes")
        self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        i32, f32 = torch.int32, torch.float32
        self.accept_count = torch.empty(B, dtype=i32, device=device)
        self.num_tokens = torch.empty(B, dtype=i32, device=device)
        self.out_tokens = torch.empty(B, G + 1, dtype=i32, device=device)
        self.p_draft = torch.empty(B, G, dtype=f32, device=device)
        self.q_draft = torch.empty(B, G, dtype=f32, device=device)
        self.residual_mass = torch.empty(B, dtype=f32, device=device)
        self.flags = torch.empty(B, dtype=torch.int32, device=device)

    def __call__(self, target, draft, draft_tokens, gamma=None, max_tokens=None, stream=None):
        specdec_verify(self.desc, target, draft, draft_tokens, gamma, max_tokens,
                       self.accept_count, self.num_tokens, self.out_tokens, self.p_draft,
                       self.q_draft, self.residual_mass, self.flags, self.workspace,
                       stream=stream)
        return {"accept_count": self.accept_count, "num_tokens": self.num_tokens,
                "out_tokens": self.out_tokens,
                "p_draft": self.p_draft, "q_draft": self.q_draft,
                "residual_mass": self.residual_mass, "flags": self.flags}
