"""The C ABI library loads, exports every entry point include/specdec.h
declares, and rejects bad arguments on the host before touching a device
(no GPU needed: these calls return before any HIP call)."""
import ctypes
import os
import re

import pytest

import speculative_decoding_verification_05_amd as sd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(specdec_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_function():
    L = sd.lib()
    declared = declared_functions()
    assert declared == set(sd.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_abi_version_and_status_strings():
    assert sd.specdec_abi_version() == 3
    for s in range(5):
        assert sd.status_string(s).startswith("SPECDEC_")


def test_struct_layouts_match_header():
    assert ctypes.sizeof(sd.VerifyDesc) == 48
    assert sd.VerifyDesc.seed.offset == 32
    assert ctypes.sizeof(sd.KVDesc) == 40
    assert sd.KVDesc.num_blocks.offset == 32


def good_desc(**kw):
    args = dict(batch=4, gamma_max=4, vocab=1000, bf16=True, temperature=0.8, seed=1)
    args.update(kw)
    return sd.make_verify_desc(**args)


def call_verify(desc, ws_bytes=None, **ptrs):
    p = dict(target=0x1000, draft=0x2000, tokens=0x3000, gamma=None, acc=0x4000, out=0x5000,
             ws=0x10000)
    p.update(ptrs)
    nbytes = sd.specdec_verify_workspace_bytes(desc) if ws_bytes is None else ws_bytes
    return sd.lib().specdec_verify(ctypes.byref(desc), p["target"], p["draft"], p["tokens"],
                                   p["gamma"], None, p["acc"], None, p["out"], None, None, None,
                                   None, p["ws"], nbytes, None)


@pytest.mark.parametrize("bad", [
    dict(batch=-1), dict(gamma_max=64), dict(gamma_max=-1), dict(vocab=0),
    dict(temperature=0.0), dict(temperature=-1.0), dict(temperature=float("nan")),
    dict(top_p=0.0), dict(top_p=1.5), dict(top_k=-3), dict(batch=70000),
])
def test_bad_descriptors_are_rejected(bad):
    d = good_desc(**bad)
    assert sd.specdec_verify_workspace_bytes(d) == 0
    assert call_verify(d, ws_bytes=1 << 30) == sd.SPECDEC_ERR_INVALID_ARGUMENT


def test_bad_dtype_mode_eos():
    for field, val in (("dtype", 7), ("mode", 5), ("eos_plus1", -1), ("eos_plus1", 1001)):
        d = good_desc()
        setattr(d, field, val)
        assert call_verify(d, ws_bytes=1 << 30) == sd.SPECDEC_ERR_INVALID_ARGUMENT


def test_null_pointers_and_workspace():
    d = good_desc()
    # (a NULL draft is valid in sampling mode: point-mass drafts)
    for name in ("target", "tokens", "acc", "out", "ws"):
        assert call_verify(d, **{name: None}) == sd.SPECDEC_ERR_INVALID_ARGUMENT, name
    assert call_verify(d, ws=0x10010) == sd.SPECDEC_ERR_INVALID_ARGUMENT  # misaligned
    n = sd.specdec_verify_workspace_bytes(d)
    assert n > 0 and n % 256 == 0
    assert call_verify(d, ws_bytes=n - 1) == sd.SPECDEC_ERR_WORKSPACE_TOO_SMALL


def test_greedy_needs_no_draft_logits():
    d = good_desc(greedy=True, batch=0)
    assert call_verify(d, draft=None) == sd.SPECDEC_OK  # B = 0: nothing to enqueue


def test_workspace_grows_with_batch():
    a = sd.specdec_verify_workspace_bytes(good_desc(batch=8))
    b = sd.specdec_verify_workspace_bytes(good_desc(batch=64))
    assert b > a


def test_commit_descriptor_checks():
    ok = sd.make_kv_desc(4, 7, 28, 4, 128, 16, 300, 8)
    assert sd.specdec_commit_kv_workspace_bytes(ok) >= 16
    for field, val in (("num_layers", 0), ("block_size", 0), ("num_blocks", 0),
                       ("gamma_max", 64), ("scratch_slots", -1)):
        d = sd.make_kv_desc(4, 7, 28, 4, 128, 16, 300, 8)
        setattr(d, field, val)
        assert sd.specdec_commit_kv_workspace_bytes(d) == 0
        st = sd.lib().specdec_commit_kv(ctypes.byref(d), 1, 1, 1, 1, None, None, 1, None, 16,
                                        1 << 20, None)
        assert st == sd.SPECDEC_ERR_INVALID_ARGUMENT
    st = sd.lib().specdec_commit_kv(ctypes.byref(ok), 16, 16, 16, 16, None, None, 16, None, 16, 0,
                                    None)
    assert st == sd.SPECDEC_ERR_WORKSPACE_TOO_SMALL
    assert sd.lib().specdec_workspace_clear(None, 16, None) == sd.SPECDEC_ERR_INVALID_ARGUMENT


def test_rollback_descriptor_checks():
    ok = sd.make_kv_desc(4, 7, 24, 2, 64, 16, 300, 8)
    for field, val in (("num_layers", 0), ("head_dim", 0), ("gamma_max", 64)):
        d = sd.make_kv_desc(4, 7, 24, 2, 64, 16, 300, 8)
        setattr(d, field, val)
        st = sd.lib().specdec_rollback_kv(ctypes.byref(d), 16, 16, 16, None, 16, None, 16,
                                          1 << 20, None)
        assert st == sd.SPECDEC_ERR_INVALID_ARGUMENT
    for args in ((None, 16, 16, 16), (16, None, 16, 16), (16, 16, None, 16), (16, 16, 16, None)):
        pool, table, acc, seq = args
        st = sd.lib().specdec_rollback_kv(ctypes.byref(ok), pool, table, acc, None, seq, None, 16,
                                          1 << 20, None)
        assert st == sd.SPECDEC_ERR_INVALID_ARGUMENT
    st = sd.lib().specdec_rollback_kv(ctypes.byref(ok), 16, 16, 16, None, 16, None, 16, 0, None)
    assert st == sd.SPECDEC_ERR_WORKSPACE_TOO_SMALL


def test_tree_descriptor_checks():
    ok = sd.make_tree_desc(4, 16, 1000)
    assert sd.specdec_verify_tree_workspace_bytes(ok) > 0
    for field, val in (("num_nodes", 0), ("num_nodes", 65), ("vocab", 0), ("dtype", 3),
                       ("eos_plus1", 1001), ("eos_plus1", -1), ("reserved", 1), ("batch", -1)):
        d = sd.make_tree_desc(4, 16, 1000)
        setattr(d, field, val)
        assert sd.specdec_verify_tree_workspace_bytes(d) == 0
        st = sd.lib().specdec_verify_tree(ctypes.byref(d), 16, 16, 16, None, None, 16, None, 16, 16,
                                          None, 256, 1 << 20, None)
        assert st == sd.SPECDEC_ERR_INVALID_ARGUMENT, (field, val)
    n = sd.specdec_verify_tree_workspace_bytes(ok)
    for i in range(5):
        args = [16, 16, 16, None, None, 16, None, 16, 16, None, 256]
        args[[0, 1, 2, 5, 7][i]] = None
        st = sd.lib().specdec_verify_tree(ctypes.byref(ok), *args[:10], 256, n, None)
        assert st == sd.SPECDEC_ERR_INVALID_ARGUMENT
    st = sd.lib().specdec_verify_tree(ctypes.byref(ok), 16, 16, 16, None, None, 16, None, 16, 16,
                                      None, 256, n - 1, None)
    assert st == sd.SPECDEC_ERR_WORKSPACE_TOO_SMALL


def test_commit_slot_count_must_cover_the_window():
    d = sd.make_kv_desc(4, 7, 2, 2, 64, 16, 300, 8, scratch_slots=4)
    st = sd.lib().specdec_commit_kv(ctypes.byref(d), 16, 16, 16, 16, None, None, 16, None, 16,
                                    1 << 20, None)
    assert st == sd.SPECDEC_ERR_INVALID_ARGUMENT     # no slot map: needs G+1 = 8 slots
    st = sd.lib().specdec_rollback_kv(ctypes.byref(d), 16, 16, 16, None, 16, None, 16, 1 << 20,
                                      None)
    assert st == sd.SPECDEC_ERR_INVALID_ARGUMENT     # rollback takes no scratch


def test_point_mass_drafts_with_truncation_pass_the_host_checks():
    """Truncation with point-mass drafts is served (by the cut path): the
    host checks go on to the workspace size instead of refusing the request
    (a too-small workspace stops the call before any launch)."""
    for kw in (dict(top_k=50), dict(top_p=0.9), dict(top_k=5000, top_p=0.5)):
        d = good_desc(**kw)
        assert call_verify(d, draft=None, ws_bytes=256) == sd.SPECDEC_ERR_WORKSPACE_TOO_SMALL


def test_workspace_covers_point_mass_layout():
    for G in (1, 4, 8):
        d = good_desc(gamma_max=G, vocab=262144, batch=512)
        assert sd.specdec_verify_workspace_bytes(d) > 0


def test_ngram_descriptor_checks():
    ok = sd.make_ngram_desc(4, 100, 1, 4, 8)
    for field, val in (("batch", -1), ("max_len", 0), ("max_len", 1 << 24), ("n_min", 0),
                       ("n_max", 33), ("gamma_max", 64), ("gamma_max", -1), ("reserved", 1)):
        d = sd.make_ngram_desc(4, 100, 1, 4, 8)
        setattr(d, field, val)
        assert sd.specdec_propose_ngram_workspace_bytes(d) == 0
        st = sd.lib().specdec_propose_ngram(ctypes.byref(d), 16, 16, 16, 16, None, 256, 1 << 20,
                                            None)
        assert st == sd.SPECDEC_ERR_INVALID_ARGUMENT, (field, val)
    d = sd.make_ngram_desc(4, 100, 3, 2, 8)     # n_max < n_min
    assert sd.lib().specdec_propose_ngram(ctypes.byref(d), 16, 16, 16, 16, None, 256, 1 << 20,
                                          None) == sd.SPECDEC_ERR_INVALID_ARGUMENT
    n = sd.specdec_propose_ngram_workspace_bytes(ok)
    assert n >= 32
    for args in ((None, 16, 16, 16), (16, None, 16, 16), (16, 16, None, 16), (16, 16, 16, None)):
        st = sd.lib().specdec_propose_ngram(ctypes.byref(ok), *args, None, 256, n, None)
        assert st == sd.SPECDEC_ERR_INVALID_ARGUMENT
    assert sd.lib().specdec_propose_ngram(ctypes.byref(ok), 16, 16, 16, 16, None, None, n, None) == \
        sd.SPECDEC_ERR_INVALID_ARGUMENT
    assert sd.lib().specdec_propose_ngram(ctypes.byref(ok), 16, 16, 16, 16, None, 256, n - 1,
                                          None) == sd.SPECDEC_ERR_WORKSPACE_TOO_SMALL
    empty = sd.make_ngram_desc(0, 100, 1, 4, 8)
    assert sd.lib().specdec_propose_ngram(ctypes.byref(empty), 16, 16, 16, 16, None, 256, 256,
                                          None) == sd.SPECDEC_OK


def test_flag_and_status_constants_match_header():
    """The binding's flag bits and status codes are the header's."""
    text = open(os.path.join(ROOT, "include", "specdec.h")).read()
    flags = dict(re.findall(r"#define\s+SPECDEC_FLAG_([A-Z_]+)\s+(0x[0-9a-fA-F]+)u", text))
    assert flags, "no SPECDEC_FLAG_ definitions found"
    for name, val in flags.items():
        assert getattr(sd, "FLAG_" + name) == int(val, 16), name
    assert len(set(int(v, 16) for v in flags.values())) == len(flags)  # distinct bits
    codes = dict(re.findall(r"SPECDEC_(OK|ERR_[A-Z_]+)\s*=\s*(\d+)", text))
    for name, val in codes.items():
        assert getattr(sd, "SPECDEC_" + name) == int(val), name


def test_noalloc_refuses_oversized_descriptors_before_any_launch():
    """specdec_verify_noalloc checks the descriptor and its workspace size on
    the host: a request above the library's 16 MiB array is refused without
    touching any argument (here, addresses nothing may dereference)."""
    L = sd.lib()
    desc = sd.make_verify_desc(512, 8, 262144, top_k=50, temperature=1.0)
    assert sd.specdec_verify_workspace_bytes(desc) > 16 << 20
    st = L.specdec_verify_noalloc(ctypes.byref(desc), *([16] * 12), None)
    assert st == sd.SPECDEC_ERR_WORKSPACE_TOO_SMALL
    bad = sd.make_verify_desc(4, 2, 1000, temperature=0.0)
    assert L.specdec_verify_noalloc(ctypes.byref(bad), *([16] * 12), None) == sd.SPECDEC_ERR_INVALID_ARGUMENT


def test_commit_and_rollback_refuses_shared_workspace_and_lengths():
    """The one-launch commit + rollback runs both halves side by side, each
    with its own arrival counters and lengths: a shared (or overlapping)
    workspace or length array is refused on the host, as is a batch or
    gamma_max mismatch, before anything is enqueued (the addresses below are
    never dereferenced)."""
    L = sd.lib()
    d = sd.make_kv_desc(4, 7, 28, 4, 128, 16, 300, 8)
    dd = sd.make_kv_desc(4, 7, 24, 2, 64, 16, 300, 8)
    nw = sd.specdec_commit_kv_workspace_bytes(d)
    ws, dws = 1 << 24, 1 << 25
    seq, dseq = 1 << 26, 1 << 27

    def call(desc, ddesc, ws_, dws_, seq_, dseq_):
        return L.specdec_commit_and_rollback_kv(
            ctypes.byref(desc), 1 << 28, 1 << 29, 1 << 30, None, seq_, None, ws_, nw,
            ctypes.byref(ddesc), 1 << 31, 1 << 30, dseq_, None, dws_, nw, 1 << 32, None, None)

    bad = sd.SPECDEC_ERR_INVALID_ARGUMENT
    assert call(d, dd, ws, ws, seq, dseq) == bad            # one workspace for both
    assert call(d, dd, ws, ws + 4, seq, dseq) == bad        # overlapping workspaces
    assert call(d, dd, ws, dws, seq, seq) == bad            # one length array for both
    assert call(d, dd, ws, dws, seq, seq + 8) == bad        # overlapping length arrays
    d2 = sd.make_kv_desc(5, 7, 28, 4, 128, 16, 300, 8)
    assert call(d2, dd, ws, dws, seq, dseq) == bad          # batch mismatch
    dd2 = sd.make_kv_desc(4, 6, 24, 2, 64, 16, 300, 8)
    assert call(d, dd2, ws, dws, seq, dseq) == bad          # gamma_max mismatch


def test_zero_filled_descriptor_has_no_eos():
    """A C caller that zero-fills the descriptors gets no end-of-sequence
    handling (eos_plus1 = 0), not EOS = token 0; the Python helpers take the
    token id itself (-1: none) and store id + 1; the largest id V - 1 is
    valid and V is not."""
    assert sd.VerifyDesc().eos_plus1 == 0 and sd.TreeDesc().eos_plus1 == 0
    assert sd.make_verify_desc(4, 2, 1000).eos_plus1 == 0
    assert sd.make_verify_desc(4, 2, 1000, eos_token=0).eos_plus1 == 1
    assert sd.make_tree_desc(4, 16, 1000, eos_token=7).eos_plus1 == 8
    d = sd.make_verify_desc(4, 2, 1000, eos_token=999)
    assert sd.specdec_verify_workspace_bytes(d) > 0
    d.eos_plus1 = 1001
    assert sd.specdec_verify_workspace_bytes(d) == 0
    assert sd.specdec_abi_version() == 3


def _fresh_python(code):
    import subprocess
    import sys
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                          timeout=300)


def test_loading_first_keeps_a_single_hip_runtime():
    """A process that loads the library before it imports torch still maps
    one HIP runtime, torch's: two (the system copy and torch's) leave the
    one that initialises second without a device, and pinned host
    allocations failing.  The debug build is loaded the way the tests'
    environment switches load it."""
    r = _fresh_python(
        "import speculative_decoding_verification_05_amd as sd\n"
        "sd._load(sd.DEBUG_LIB_PATH); sd.lib()\n"
        "rt = sd._hip_runtimes()\n"
        "print(len(rt), *sorted(rt))\n")
    assert r.returncode == 0, r.stderr
    n, *paths = r.stdout.split()
    assert n == "1", r.stdout
    assert "torch" in paths[0], paths


def test_a_second_hip_runtime_is_refused():
    """With the system's HIP runtime already loaded when torch brings its
    own, the loader refuses instead of handing out calls that would fail
    later with unrelated-looking errors."""
    r = _fresh_python(
        "import ctypes, glob\n"
        "cands = sorted(glob.glob('/opt/rocm*/lib/libamdhip64.so.*'))\n"
        "if not cands: raise SystemExit(3)\n"
        "ctypes.CDLL(cands[0])\n"
        "import speculative_decoding_verification_05_amd as sd\n"
        "try:\n"
        "    sd.lib()\n"
        "except ImportError as e:\n"
        "    print('refused', e)\n")
    if r.returncode == 3:
        pytest.skip("no system HIP runtime here")
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("refused two HIP runtimes"), r.stdout
