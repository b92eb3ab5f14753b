#!/usr/bin/env python3
"""Throughput of the speculative-decoding verify step on one MI355X.

Default workload: B=64 requests, gamma=4 drafts, V=128256, bf16 logits,
T=0.8 sampling with a bonus token on full acceptance (the headline case).
A step is one specdec_verify call over one batch: the statistics pass over
every used logits row, the acceptance tests and ballot, and the correction /
bonus draw.  Inputs are synthetic (seeded generator), resident in HBM before
timing, and rotate over several independent input sets whose total exceeds the
256 MB Infinity Cache, so every step reads its logits from HBM.

Timing: W warmup steps, then exactly K steps bracketed by
torch.cuda.synchronize(); value = verified positions / second.  The K steps
are replayed from HIP graphs (each holds whole passes over the input sets, at
least 16 steps, so that the launch gap between replays is amortized) or
launched eagerly, whichever ran a window of K steps faster in untimed
calibration after the warmup (a short window pays a graph replay's start-up
in full); the JSON's config.launch names the mode.
The roofline entry is the dominant kernel: the one-kernel verify of the
sampling, greedy and tree paths (statistics and decision workgroups in one
launch), or the selection kernel on the truncation path.  It is
the kernel's algorithmic bytes per launch (every used logits row read once,
plus draft tokens and outputs) over its average duration, timed live with
start/stop events that bracket the kernel itself (specdec_verify_profiled).
cpu_baseline: the CPU oracle (single-threaded C, double precision) run on the
same input set for a bounded time; cpu_baseline_all_cores: the same oracle on
every host core this process may use (at most 16), one thread per core over
its own slice of the requests.

Other workloads (--workload) print the same JSON line for that recipe; the
ones with a paged KV cache time a whole round: verify, the target's commit
and the draft cache's rollback (one specdec_commit_and_rollback_kv launch;
--separate-kv-calls times the two calls instead).  Each step of a graph has its own cache
lengths, all restored by one small copy at the graph's start, so that every
step commits into the same window.  Their JSON line also lists each kernel's average time
and algorithmic bandwidth.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E
METRIC = "verified positions/sec + achieved HBM GB/s (% of peak), B=64 γ=4 V=128256"


def steps_per_graph(sets: int, at_least: int) -> int:
    """Whole passes over the input sets, at least `at_least` steps.  A graph
    replay starts ~9 us after the previous one ends and its first kernel runs a
    few us longer, so a graph holds many steps to keep that out of the
    per-step time."""
    return sets * max(1, -(-at_least // sets))


class GraphSteps:
    """Runs exactly n steps.  enqueue(n) puts steps 0..n-1 on the current stream
    (step i reads input set i % sets); it is captured once per length used: a
    graph of `per` steps replayed n // per times, then one of the n % per
    remaining steps.  Each graph is replayed three times after capture, and each
    replay must reproduce the eager outputs of its last step (check(i)); if one
    does not, every run launches eagerly and `graphed` is False."""

    def __init__(self, enqueue, per: int, check, use_graphs: bool = True):
        self.enqueue, self.per, self.check = enqueue, per, check
        self.graphs = {}
        self.graphed = use_graphs

    def _capture(self, n: int) -> bool:
        import torch
        if n == 0 or n in self.graphs:
            return True
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.enqueue(n)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.enqueue(n)
        for _ in range(3):
            g.replay()
            torch.cuda.synchronize()
            if not self.check(n - 1):
                return False
        self.graphs[n] = g
        return True

    def prepare(self, *counts: int) -> None:
        """Capture and check every graph the given step counts need."""
        for n in counts:
            for size in ((self.per if n >= self.per else 0), n % self.per):
                if self.graphed and not self._capture(size):
                    log(f"graph replay of {size} steps differs from eager launches; "
                        "timing eager launches")
                    self.graphed = False

    def pick_faster(self, n: int, rounds: int = 5) -> str:
        """Untimed windows of n steps, launched from the graphs and eagerly
        in turn; the faster by median becomes the launch mode of the timed
        run (a graph replay's start-up is paid once per window, which a short
        window feels, while eager launches overlap the host's enqueue with the
        first kernels).  Returns the mode's name."""
        import torch
        if self.graphed:
            times = {True: [], False: []}
            for _ in range(rounds):
                for g in (True, False):
                    self.graphed = g
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    self.run(n)
                    torch.cuda.synchronize()
                    times[g].append(time.perf_counter() - t0)
            self.graphed = bool(np.median(times[True]) <= np.median(times[False]))
        return "hipgraph" if self.graphed else "eager"

    def run(self, n: int) -> None:
        full, rem = divmod(n, self.per)
        for size, count in ((self.per, full), (rem, 1 if rem else 0)):
            for _ in range(count):
                if self.graphed:
                    self.graphs[size].replay()
                else:
                    self.enqueue(size)


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def measured_traffic(kernel_workload: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or None if there is none or the kernel sources have
    changed since the counters were taken (sha256 recorded with them)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel_workload}__pmc_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if "kernel_source_sha256" not in fields or "traffic_bytes_per_launch" not in fields:
        return None
    h = hashlib.sha256()
    for f in fields["kernel_sources"].split():
        h.update(open(os.path.join(ROOT, "speculative_decoding_verification_05_amd", "csrc", f), "rb").read())
    if h.hexdigest() != fields["kernel_source_sha256"]:
        return None
    return float(fields["traffic_bytes_per_launch"])


def oracle_all_cores(run_slice, weights, seconds, firsts=None):
    """The oracle, as it stands, on every host core this process may use (at
    most 16, one GPU's share of the box): one thread per core, each running
    the oracle again and again over its own slice of the items (the oracle is
    C behind ctypes, which releases the GIL).  Returns (weight per second,
    threads, seconds, passes); firsts (a list), if given, receives
    (slice, output of its first pass) per thread."""
    from concurrent.futures import ThreadPoolExecutor
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    n = len(weights)
    nt = max(1, min(16, ncpu, n))
    slices = np.array_split(np.arange(n), nt)
    stop = time.perf_counter() + seconds

    def worker(ix):
        done, passes = 0.0, 0
        while True:
            r = run_slice(ix)
            if passes == 0 and firsts is not None:
                firsts.append((ix, r))
            done += float(np.sum(weights[ix]))
            passes += 1
            if time.perf_counter() >= stop:
                return done, passes

    t0 = time.perf_counter()
    with ThreadPoolExecutor(nt) as ex:
        out = list(ex.map(worker, slices))
    t = time.perf_counter() - t0
    return sum(d for d, _ in out) / t, nt, t, min(p for _, p in out)


PROB_ABS, PROB_REL = 1e-5, 1e-4  # probabilities: 1e-5 absolute or 1e-4 relative


def parity(ref, got, gamma, greedy):
    """GPU outputs against the oracle's, request by request: accept count,
    tokens, token count and flags bit-exact, p(d), q(d) and the residual mass
    within tolerance.  A request whose oracle run met a draw within 1e-6 of
    its threshold (near_pos >= 0) is compared up to that decision only and
    counted.  Returns (requests compared, near-threshold requests, ids of
    mismatching requests)."""
    bad, near = [], 0
    B = len(ref["accept_count"])
    for b in range(B):
        g, npos = int(gamma[b]), int(ref["near_pos"][b])
        m_ref, m_got = int(ref["accept_count"][b]), int(got["accept_count"][b])
        ok = True
        if npos >= 0:
            near += 1
            ok &= not (m_got < npos <= m_ref)
            ok &= list(got["out_tokens"][b][:npos]) == list(ref["out_tokens"][b][:npos])
        else:
            ok &= m_got == m_ref
            ok &= list(got["out_tokens"][b]) == list(ref["out_tokens"][b])
            ok &= int(got["num_tokens"][b]) == int(ref["num_tokens"][b])
            ok &= (int(got["flags"][b]) & 0x18F) == (int(ref["flags"][b]) & 0x18F)
        if not greedy:
            for i in range(g if npos < 0 else min(g, npos)):
                for k in ("p_draft", "q_draft"):
                    a, r = float(got[k][b, i]), float(ref[k][b, i])
                    ok &= abs(a - r) <= max(PROB_ABS, PROB_REL * abs(r))
            if npos < 0:
                a, r = float(got["residual_mass"][b]), float(ref["residual_mass"][b])
                ok &= abs(a - r) <= max(PROB_ABS, PROB_REL * abs(r)) if m_ref < g else a == 0.0
        if not ok:
            bad.append(b)
    return B, near, bad


def quantiles(t_s):
    """p10 / median / p90 of durations in seconds, as microseconds."""
    t = np.asarray(t_s) * 1e6
    return {"p10": float(np.percentile(t, 10)), "median": float(np.median(t)),
            "p90": float(np.percentile(t, 90)), "n": int(t.size)}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None, help="generator workload name")
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0: auto)")
    ap.add_argument("--profile-steps", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches, no graph")
    ap.add_argument("--separate-kv-calls", action="store_true",
                    help="KV recipes: commit and rollback as two calls instead of one launch")
    ap.add_argument("--debug-library", action="store_true",
                    help="use libspecdec_debug.so, which reads the SPECDEC_* tuning switches "
                         "from the environment (sweeps; the product library reads none)")
    ap.add_argument("--pmc-copy-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a dispatch of "
                         "known size to calibrate FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")
    return args


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py measures the verify-and-commit step on one GPU; there is no multi-GPU "
            "path (requests would shard across GPUs with no exchange). "
            "Run it with --gpus 1.")
        return 2

    import torch
    import speculative_decoding_verification_05_amd as sd
    from speculative_decoding_verification_05_amd import synth

    dev = torch.device("cuda:0")
    # every call of this run goes to the debug build (the context object is
    # kept for the whole run: dropping it would close the context and bring
    # the product library back)
    debug_ctx = sd.debug_library() if args.debug_library else None
    if debug_ctx is not None:
        debug_ctx.__enter__()
    lib = sd.lib()
    if args.debug_library and getattr(lib, "_name", "") != sd.DEBUG_LIB_PATH:
        raise RuntimeError("--debug-library: the debug build is not the library in use")
    if args.pmc_copy_mib:
        src = torch.ones(args.pmc_copy_mib << 18, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.pmc_copy_mib} MiB read + {args.pmc_copy_mib} MiB written")
        del src, dst
    wl0 = synth.WORKLOADS[args.workload or synth.HEADLINE]
    if wl0.tree is not None:
        return bench_tree(args, wl0)
    if wl0.ngram is not None:
        return bench_ngram(args, wl0)
    greedy = wl0.mode == "greedy"
    bf16 = wl0.dtype == "bf16"
    per_set = synth.logits_bytes(wl0)
    sets = args.sets or max(1, min(8, int(np.ceil(2 * 256e6 / per_set)) + (1 if per_set < 512e6 else 0)))
    log(f"workload {wl0.name}: {per_set / 1e6:.2f} MB of logits per set, {sets} rotating sets")

    # ---- inputs, resident in HBM
    host, dev_in = [], []
    for k in range(sets):
        wl = dataclasses.replace(wl0, data_seed=wl0.data_seed + 100 * k)
        x = synth.make_verify_inputs(wl)
        host.append(x)
        d = {"target": torch.from_numpy(x["target"].view(np.int16) if bf16 else x["target"]).to(dev),
             "draft": None if greedy else torch.from_numpy(
                 x["draft"].view(np.int16) if bf16 else x["draft"]).to(dev),
             "tokens": torch.from_numpy(x["draft_tokens"]).to(dev),
             "gamma": torch.from_numpy(x["gamma"]).to(dev)}
        dev_in.append(d)
        log(f"  input set {k} uploaded")
    per = steps_per_graph(sets, 16)
    kv = None
    if wl0.kv is not None:
        kvin = synth.make_kv_inputs(wl0)
        K = wl0.kv
        kdesc = sd.make_kv_desc(wl0.batch, wl0.gamma_max, K.layers, K.kv_heads, K.head_dim,
                                K.block_size, kvin.block_table.shape[1], kvin.num_blocks)
        kv = {"desc": kdesc, "in": kvin,
              "scratch": torch.from_numpy(kvin.scratch.view(np.int16)).to(dev),
              "pool": torch.from_numpy(kvin.pool.view(np.int16)).to(dev),
              "table": torch.from_numpy(kvin.block_table).to(dev),
              "ws": torch.zeros(sd.specdec_commit_kv_workspace_bytes(kdesc), dtype=torch.uint8,
                                device=dev)}
        log(f"  paged KV pool {kvin.pool.nbytes / 1e6:.1f} MB uploaded")
        dpool, _, dseq, nb = synth.make_draft_kv_inputs(wl0, kvin)
        DK = wl0.draft_kv
        ddesc = sd.make_kv_desc(wl0.batch, wl0.gamma_max, DK.layers, DK.kv_heads, DK.head_dim,
                                DK.block_size, kvin.block_table.shape[1], nb)
        # cache lengths per step of a graph: [step][target | draft][B], all
        # restored by one copy at the graph's start, so that every step
        # commits into the same window
        seqs0 = np.stack([np.stack([kvin.seq_lens, dseq])] * per).astype(np.int32)
        kv.update({"ddesc": ddesc, "dpool": torch.from_numpy(dpool.view(np.int16)).to(dev),
                   "seqs0": torch.from_numpy(seqs0).to(dev),
                   "seqs": torch.from_numpy(seqs0.copy()).to(dev),
                   "dws": torch.zeros(sd.specdec_commit_kv_workspace_bytes(ddesc),
                                      dtype=torch.uint8, device=dev)})
        log(f"  draft KV pool {dpool.nbytes / 1e6:.1f} MB uploaded")

    desc = sd.make_verify_desc(wl0.batch, wl0.gamma_max, wl0.vocab, bf16=bf16, greedy=greedy,
                               temperature=wl0.temperature, top_k=wl0.top_k, top_p=wl0.top_p,
                               seed=wl0.verify_seed)
    ver = sd.Verifier(desc, dev)

    # step i reads input set i % sets and commits with the cache lengths of slot i
    def commit(i: int) -> None:
        sd.specdec_commit_kv(kv["desc"], kv["scratch"], kv["pool"], kv["table"],
                             ver.accept_count, dev_in[i % sets]["gamma"], None, kv["seqs"][i, 0],
                             None, kv["ws"])

    def rollback(i: int) -> None:
        sd.specdec_rollback_kv(kv["ddesc"], kv["dpool"], kv["table"], ver.accept_count,
                               dev_in[i % sets]["gamma"], kv["seqs"][i, 1], None, kv["dws"])

    def reset() -> None:
        if kv is not None:
            kv["seqs"].copy_(kv["seqs0"])

    def commit_and_rollback(i: int) -> None:
        sd.specdec_commit_and_rollback_kv(kv["desc"], kv["scratch"], kv["pool"], kv["table"], None,
                                          kv["seqs"][i, 0], None, kv["ws"], kv["ddesc"], kv["dpool"],
                                          kv["table"], kv["seqs"][i, 1], None, kv["dws"],
                                          ver.accept_count, dev_in[i % sets]["gamma"])

    def step(i: int) -> None:
        d = dev_in[i % sets]
        ver(d["target"], d["draft"], d["tokens"], d["gamma"])
        if kv is not None:
            if args.separate_kv_calls:
                commit(i)
                rollback(i)
            else:
                # the target's commit and the draft's rollback in one launch
                commit_and_rollback(i)

    def enqueue(n: int) -> None:
        reset()
        for i in range(n):
            step(i)

    # ---- eager reference outputs, then the graphs
    eager = []
    names = ("accept_count", "num_tokens", "out_tokens", "p_draft", "q_draft", "residual_mass", "flags")
    reset()
    for k in range(sets):
        step(k)
        torch.cuda.synchronize()
        eager.append({n: getattr(ver, n).clone() for n in names})
    torch.cuda.synchronize()

    def check(i: int) -> bool:
        return all(torch.equal(getattr(ver, n), eager[i % sets][n])
                   for n in ("accept_count", "out_tokens"))

    runner = GraphSteps(enqueue, per, check, use_graphs=not args.eager)
    runner.prepare(args.warmup, args.steps)
    steps = args.steps
    runner.run(args.warmup)
    log(f"  timed launches: {runner.pick_faster(steps)}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    runner.run(steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec_per_step = (t1 - t0) / steps

    # ---- per-step durations: each step timed alone (eager launches, events
    # on the stream the calls use) for the median and p10 / p90
    n_q = max(sets, (min(args.profile_steps, 400) // sets) * sets)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_q)]
    for j in range(n_q):
        if j % per == 0:
            reset()  # (each slot's cache lengths once per pass, as in the graphs)
        evs[j][0].record()
        step(j % per)
        evs[j][1].record()
    torch.cuda.synchronize()
    t_step = np.array([a.elapsed_time(b) for a, b in evs]) * 1e-3

    gam_sets = [h["gamma"] for h in host]
    positions = float(np.mean([g.sum() for g in gam_sets]))
    value = positions / sec_per_step
    acc = [e["accept_count"].cpu().numpy() for e in eager]
    committed = float(np.mean([(a + 1).sum() for a in acc]))

    # ---- live per-kernel timing with events around the kernels themselves
    n_prof = max(sets, (args.profile_steps // sets) * sets)
    ev = sd.HipEvents(4 * n_prof)
    for j in range(n_prof):
        d = dev_in[j % sets]
        h = ev.handles[4 * j:4 * j + 4]
        e = h
        sd.specdec_verify_profiled(desc, d["target"], d["draft"], d["tokens"], d["gamma"], None,
                                   ver.accept_count, ver.num_tokens, ver.out_tokens, ver.p_draft,
                                   ver.q_draft, ver.residual_mass, ver.flags, ver.workspace, e)
    torch.cuda.synchronize()
    k1 = np.array([ev.elapsed_ms(4 * j, 4 * j + 1) for j in range(n_prof)]) * 1e-3  # seconds
    k2 = np.array([ev.elapsed_ms(4 * j + 2, 4 * j + 3) for j in range(n_prof)]) * 1e-3
    ev.close()
    k1_avg = float(k1.mean())
    kernels = {}
    if kv is not None:
        # commit and rollback run on torch's current stream: torch events bracket them
        tc = []
        for j in range(n_prof):
            k = j % sets
            d = dev_in[k]
            ver(d["target"], d["draft"], d["tokens"], d["gamma"])
            reset()  # step k below commits with slot k's restored lengths
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record()
            commit(k)
            e[1].record()
            e[2].record()
            rollback(k)
            e[3].record()
            tc.append(e)
        torch.cuda.synchronize()
        t_commit = np.array([e[0].elapsed_time(e[1]) for e in tc]) * 1e-3
        t_roll = np.array([e[2].elapsed_time(e[3]) for e in tc]) * 1e-3
        K, DK = wl0.kv, wl0.draft_kv
        slot_t = K.layers * 2 * K.kv_heads * K.head_dim * 2
        slot_d = DK.layers * 2 * DK.kv_heads * DK.head_dim * 2
        cb, rb = [], []
        for k in range(sets):
            m = eager[k]["accept_count"].cpu().numpy().astype(np.int64)
            g = host[k]["gamma"].astype(np.int64)
            # copy: read + write per kept slot; zero-fill: write per rejected slot
            cb.append(float(((m + 1) * 2 + (g - m)).sum() * slot_t))
            rb.append(float(np.maximum(g - 1 - m, 0).sum() * slot_d))
        for name, t, by in (("k_commit", t_commit, cb), ("k_rollback", t_roll, rb)):
            avg = float(t.mean())
            b_avg = float(np.mean(by))
            kernels[name] = {"avg_us": avg * 1e6, "bytes_per_launch": b_avg,
                             "GBps": b_avg / avg / 1e9, "frac": b_avg / avg / 1e9 / HBM_PEAK_GBPS}
            log(f"{name}: avg {avg * 1e6:.2f} us, {b_avg / 1e6:.2f} MB algorithmic, "
                f"{b_avg / avg / 1e9:.1f} GB/s")

    # algorithmic bytes of one statistics launch: used rows read once, draft
    # tokens read, per-request outputs written
    B, G = wl0.batch, wl0.gamma_max
    out_bytes = B * 4 + B * (G + 1) * 4 + (0 if greedy else B * G * 8 + B * 4) + B * 4
    alg_k1 = float(np.mean([synth.logits_bytes(wl0, g) for g in gam_sets])) + B * G * 4 + out_bytes
    achieved = alg_k1 / k1_avg / 1e9
    trunc = bool(wl0.top_k) or wl0.top_p < 1.0
    # sampling without truncation and greedy verification run as one kernel
    # (statistics + decision); with --debug-library, SPECDEC_FUSED=0 selects
    # the two-kernel paths
    fused = not trunc and not (args.debug_library and os.environ.get("SPECDEC_FUSED", "1")[:1] == "0")
    # truncation lists each row's kept tokens (top_k <= 1024, or top-p alone
    # on V <= 2048) or finds each row's cut (k_trunc_cut) otherwise
    use_k = 0 < wl0.top_k < wl0.vocab
    cut = trunc and (wl0.top_k > 1024 if use_k else wl0.vocab > 2048)
    if greedy:
        kname = "k_greedy_fused" if fused else "k_stats_greedy"
    else:
        kname = ("k_trunc_cut" if cut else "k_trunc_select") if trunc else \
            "k_verify_fused" if fused else "k_stats_sample"
    if fused:
        log(f"step {sec_per_step * 1e6:.2f} us ({'graph' if runner.graphed else 'eager'}); "
            f"one-kernel verify avg {k1_avg * 1e6:.2f} us (p10 {np.percentile(k1, 10) * 1e6:.2f}, "
            f"p90 {np.percentile(k1, 90) * 1e6:.2f})")
        log(f"one-kernel verify {achieved:.1f} GB/s = {100 * achieved / HBM_PEAK_GBPS:.1f}% of "
            f"{HBM_PEAK_GBPS:.0f} GB/s; whole step {alg_k1 / sec_per_step / 1e9:.1f} GB/s")
    else:
        log(f"step {sec_per_step * 1e6:.2f} us ({'graph' if runner.graphed else 'eager'}); "
            f"{kname} avg {k1_avg * 1e6:.2f} us (p10 {np.percentile(k1, 10) * 1e6:.2f}, "
            f"p90 {np.percentile(k1, 90) * 1e6:.2f}); decision kernel avg {k2.mean() * 1e6:.2f} us")
        log(f"{kname} {achieved:.1f} GB/s = {100 * achieved / HBM_PEAK_GBPS:.1f}% of "
            f"{HBM_PEAK_GBPS:.0f} GB/s; whole step {alg_k1 / sec_per_step / 1e9:.1f} GB/s")
    log(f"mean accepted {np.mean([a.mean() for a in acc]):.3f} of {G}; histogram of m: "
        f"{np.bincount(np.concatenate(acc), minlength=G + 1).tolist()}; "
        f"committed tokens/s {committed / sec_per_step:.3e}")

    # ---- CPU baseline: the oracle on the host copy of input set 0
    cpu = cpu_all = par = None
    if not args.no_cpu_baseline:
        import oracle
        x = host[0]
        ref = None
        reps_c, t_c = 0, 0.0
        n_req = B
        # bounded sample: whole batches while under the time budget, else fewer requests
        t_s = time.perf_counter()
        while True:
            r = oracle.verify(x["target"], None if greedy else x["draft"], x["draft_tokens"],
                              x["gamma"], greedy=greedy, temperature=wl0.temperature,
                              top_k=wl0.top_k, top_p=wl0.top_p, seed=wl0.verify_seed,
                              requests=np.arange(n_req))
            ref = ref or r
            reps_c += 1
            t_c = time.perf_counter() - t_s
            if t_c >= args.cpu_seconds or reps_c >= 50:
                break
        cpu_pos = reps_c * float(x["gamma"][:n_req].sum()) / t_c
        m_ok = np.array_equal(ref["accept_count"][ref["near_pos"] < 0],
                              eager[0]["accept_count"].cpu().numpy()[ref["near_pos"] < 0])
        log(f"oracle: {reps_c} x {n_req} requests in {t_c:.2f} s on 1 core; GPU accept counts "
            f"{'match' if m_ok else 'DIFFER FROM'} the oracle's on set 0")
        cpu = {"value": cpu_pos, "unit": "positions/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps_c} pass(es) over all {n_req} requests of input set 0 "
                         f"({t_c:.1f} s, single-threaded C, double precision)"}
        firsts = []
        rate, nt, t_a, passes = oracle_all_cores(
            lambda ix: oracle.verify(x["target"], None if greedy else x["draft"], x["draft_tokens"],
                                     x["gamma"], greedy=greedy, temperature=wl0.temperature,
                                     top_k=wl0.top_k, top_p=wl0.top_p, seed=wl0.verify_seed,
                                     requests=ix),
            x["gamma"].astype(np.float64), args.cpu_seconds / 2, firsts)
        # every request of input set 0: the oracle's outputs (the first pass of
        # each thread) against the GPU's
        full = {}
        for ix, r in firsts:
            for k, v in r.items():
                if k not in full:
                    full[k] = np.zeros((B,) + v.shape[1:], v.dtype)
                full[k][ix] = v
        got = {k: v.cpu().numpy() for k, v in eager[0].items()}
        n_cmp, n_near, bad = parity(full, got, x["gamma"], greedy)
        par = {"input_set": 0, "requests": n_cmp, "near_threshold": n_near, "mismatches": len(bad),
               "rule": "accept counts, tokens, token counts and flags bit-exact; p(d), q(d) and "
                       "the residual mass within 1e-5 abs or 1e-4 rel; a request with a draw "
                       "within 1e-6 of its threshold is compared up to that draw and counted"}
        log(f"parity on input set 0: {n_cmp} requests, {len(bad)} mismatches, {n_near} near-threshold"
            + (f"; mismatching requests {bad[:16]}" if bad else ""))
        log(f"oracle on {nt} threads: {rate:.1f} positions/s ({t_a:.1f} s, at least {passes} "
            f"pass(es) per thread)")
        cpu_all = {"value": rate, "unit": "positions/s", "cores": nt, "kind": "oracle",
                   "sample": f"input set 0's {n_req} requests split over {nt} threads, each "
                             f"repeating its slice for {t_a:.1f} s (at least {passes} passes)"}

    res = {
        "metric": METRIC if wl0.name == synth.HEADLINE else f"verified positions/sec ({wl0.name})",
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": sec_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl0.name, "batch": B, "gamma_max": G, "vocab": wl0.vocab,
                   "logits": wl0.dtype, "mode": wl0.mode, "temperature": wl0.temperature,
                   "top_k": wl0.top_k, "top_p": wl0.top_p, "kv_commit": wl0.kv is not None,
                   "draft_rollback": wl0.draft_kv is not None,
                   "commit_and_rollback": ("two launches" if args.separate_kv_calls else "one launch")
                   if wl0.kv is not None else None,
                   "rotating_input_sets": sets, "steps_per_graph": per,
                   "launch": "hipgraph" if runner.graphed else "eager",
                   "committed_tokens_per_s": committed / sec_per_step,
                   "step_GBps": alg_k1 / sec_per_step / 1e9},
        "kernels": dict(({kname[2:]: {"avg_us": k1_avg * 1e6, "bytes_per_launch": alg_k1,
                                      "GBps": achieved, "frac": achieved / HBM_PEAK_GBPS}}
                          if fused else
                          {kname[2:]: {"avg_us": k1_avg * 1e6, "bytes_per_launch": alg_k1,
                                       "GBps": achieved, "frac": achieved / HBM_PEAK_GBPS},
                           "decision": {"avg_us": float(k2.mean()) * 1e6}}), **kernels),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(f"{kname}__{wl0.name}"),
                     "kernel": kname,
                     "kernel_avg_us": k1_avg * 1e6, "bytes_per_launch": alg_k1},
        "quantiles_us": {"step_eager": quantiles(t_step), "kernel": quantiles(k1)},
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "parity": par,
    }
    print(json.dumps(res), flush=True)
    # a GPU result that differs from the oracle's outside the counted
    # near-threshold draws fails the run
    return 3 if par is not None and par["mismatches"] else 0


def bench_tree(args, wl0) -> int:
    """Greedy tree verification + path commit: a step is specdec_verify_tree
    (statistics pass over every node's row, the tree decision) followed by
    specdec_commit_kv with the kept path as the slot map."""
    import torch
    import speculative_decoding_verification_05_amd as sd
    from speculative_decoding_verification_05_amd import synth

    dev = torch.device("cuda:0")
    B, N, V = wl0.batch, wl0.gamma_max + 1, wl0.vocab
    per_set = B * N * V * wl0.elem_bytes
    sets = args.sets or max(1, int(np.ceil(2 * 256e6 / per_set)) + 1)
    log(f"workload {wl0.name}: {per_set / 1e6:.2f} MB of logits per set, {sets} rotating sets")
    host, dev_in = [], []
    for k in range(sets):
        x = synth.make_tree_inputs(dataclasses.replace(wl0, data_seed=wl0.data_seed + 100 * k))
        host.append(x)
        dev_in.append({n: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).to(dev)
                       for n, v in x.items()})
        log(f"  input set {k} uploaded")
    kvin = synth.make_kv_inputs(wl0)
    K = wl0.kv
    kdesc = sd.make_kv_desc(B, N - 1, K.layers, K.kv_heads, K.head_dim, K.block_size,
                            kvin.block_table.shape[1], kvin.num_blocks, scratch_slots=N)
    depth = np.array([synth.kv_window(wl0, b) for b in range(B)], np.int32)
    scratch = torch.from_numpy(kvin.scratch.view(np.int16)).to(dev)
    pool = torch.from_numpy(kvin.pool.view(np.int16)).to(dev)
    table = torch.from_numpy(kvin.block_table).to(dev)
    # cache lengths per step of a graph, all restored by one copy at its start
    per = steps_per_graph(sets, 16)
    seqs0 = torch.from_numpy(np.stack([kvin.seq_lens] * per).astype(np.int32)).to(dev)
    seqs = seqs0.clone()
    depth_d = torch.from_numpy(depth).to(dev)
    kws = torch.zeros(sd.specdec_commit_kv_workspace_bytes(kdesc), dtype=torch.uint8, device=dev)
    tdesc = sd.make_tree_desc(B, N, V, bf16=wl0.dtype == "bf16")
    ws = torch.zeros(sd.specdec_verify_tree_workspace_bytes(tdesc), dtype=torch.uint8, device=dev)
    i32 = torch.int32
    acc = torch.zeros(B, dtype=i32, device=dev)
    ntok = torch.zeros(B, dtype=i32, device=dev)
    out = torch.zeros(B, N, dtype=i32, device=dev)
    path = torch.zeros(B, N, dtype=i32, device=dev)
    flags = torch.zeros(B, dtype=i32, device=dev)

    def verify(k, ev=None):
        d = dev_in[k % sets]
        if ev is None:
            sd.specdec_verify_tree(tdesc, d["target"], d["tokens"], d["parents"], d["num_nodes"],
                                   None, acc, ntok, out, path, flags, ws)
        else:
            sd.specdec_verify_tree_profiled(tdesc, d["target"], d["tokens"], d["parents"],
                                            d["num_nodes"], None, acc, ntok, out, path, flags, ws,
                                            ev)

    # step i reads input set i % sets and commits with the cache lengths of slot i
    def commit(i):
        sd.specdec_commit_kv(kdesc, scratch, pool, table, acc, depth_d, path, seqs[i], None, kws)

    def step(i):
        verify(i)
        commit(i)

    def enqueue(n):
        seqs.copy_(seqs0)
        for i in range(n):
            step(i)

    eager = []
    seqs.copy_(seqs0)
    for k in range(sets):
        step(k)
        torch.cuda.synchronize()
        eager.append((acc.clone(), out.clone()))

    def check(i):
        return torch.equal(acc, eager[i % sets][0]) and torch.equal(out, eager[i % sets][1])

    runner = GraphSteps(enqueue, per, check)
    runner.prepare(args.warmup, args.steps)
    if not runner.graphed:
        return 1
    steps = args.steps
    runner.run(args.warmup)
    log(f"  timed launches: {runner.pick_faster(steps)}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    runner.run(steps)
    torch.cuda.synchronize()
    sec_per_step = (time.perf_counter() - t0) / steps

    # live per-kernel times
    n_prof = max(sets, (args.profile_steps // sets) * sets)
    ev = sd.HipEvents(4 * n_prof)
    tc = []
    for j in range(n_prof):
        verify(j % sets, ev.handles[4 * j:4 * j + 4])
        seqs.copy_(seqs0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        commit(j % sets)
        e1.record()
        tc.append((e0, e1))
    torch.cuda.synchronize()
    k1 = np.array([ev.elapsed_ms(4 * j, 4 * j + 1) for j in range(n_prof)]) * 1e-3
    k2 = np.array([ev.elapsed_ms(4 * j + 2, 4 * j + 3) for j in range(n_prof)]) * 1e-3
    kc = np.array([a.elapsed_time(b) for a, b in tc]) * 1e-3
    ev.close()
    # algorithmic bytes: every node's row once + tokens and parents + outputs
    alg_k1 = float(per_set + B * N * 8 + B * (2 * N + 3) * 4)
    achieved = alg_k1 / float(k1.mean()) / 1e9
    slot = K.layers * 2 * K.kv_heads * K.head_dim * 2
    cbytes = []
    for a, _ in eager:
        m = a.cpu().numpy().astype(np.int64)
        cbytes.append(float(((m + 1) * 2 + (depth - m)).sum() * slot))
    cb = float(np.mean(cbytes))
    depth_mean = float(np.mean([a.float().mean().item() for a, _ in eager]))
    # the statistics and the tree decision run as one kernel (with
    # --debug-library, SPECDEC_FUSED=0 selects the two-kernel path)
    fused = not (args.debug_library and os.environ.get("SPECDEC_FUSED", "1")[:1] == "0")
    kname = "k_tree_fused" if fused else "k_stats_greedy"
    if fused:
        log(f"step {sec_per_step * 1e6:.2f} us (graph); one-kernel tree verify avg "
            f"{k1.mean() * 1e6:.2f} us; path commit {kc.mean() * 1e6:.2f} us")
    else:
        log(f"step {sec_per_step * 1e6:.2f} us (graph); stats kernel avg {k1.mean() * 1e6:.2f} us; "
            f"tree decision {k2.mean() * 1e6:.2f} us; path commit {kc.mean() * 1e6:.2f} us")
    log(f"{'one-kernel tree verify' if fused else 'stats kernel'} {achieved:.1f} GB/s = "
        f"{100 * achieved / HBM_PEAK_GBPS:.1f}% of {HBM_PEAK_GBPS:.0f} GB/s; commit "
        f"{cb / kc.mean() / 1e9:.1f} GB/s; mean kept depth {depth_mean:.3f}")

    cpu = cpu_all = par = None
    if not args.no_cpu_baseline:
        import oracle
        x = host[0]
        reps_c, t_s = 0, time.perf_counter()
        while True:
            oracle.verify_tree(x["target"], x["tokens"], x["parents"], x["num_nodes"])
            reps_c += 1
            t_c = time.perf_counter() - t_s
            if t_c >= args.cpu_seconds or reps_c >= 50:
                break
        cpu = {"value": reps_c * B * (N - 1) / t_c, "unit": "tree nodes/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{reps_c} pass(es) over all {B} trees of input set 0 ({t_c:.1f} s, "
                         f"single-threaded C, double precision)"}
        nn = x["num_nodes"]
        rate, nt, t_a, passes = oracle_all_cores(
            lambda ix: oracle.verify_tree(x["target"][ix], x["tokens"][ix], x["parents"][ix],
                                          None if nn is None else nn[ix]),
            np.full(B, float(N - 1)), args.cpu_seconds / 2)
        log(f"oracle on {nt} threads: {rate:.1f} tree nodes/s ({t_a:.1f} s)")
        cpu_all = {"value": rate, "unit": "tree nodes/s", "cores": nt, "kind": "oracle",
                   "sample": f"input set 0's {B} trees split over {nt} threads, each repeating "
                             f"its slice for {t_a:.1f} s (at least {passes} passes)"}
    res = {
        "metric": f"verified tree nodes/sec ({wl0.name})",
        "value": B * (N - 1) / sec_per_step,
        "unit": "tree nodes/s",
        "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": sec_per_step * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl0.name, "batch": B, "tree_nodes": N, "vocab": V,
                   "logits": wl0.dtype, "mode": "greedy tree", "kv_commit": True,
                   "rotating_input_sets": sets, "steps_per_graph": per, "launch": "hipgraph" if runner.graphed else "eager",
                   "committed_tokens_per_s": B * (depth_mean + 1) / sec_per_step},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(f"{kname}__{wl0.name}"),
                     "kernel": kname,
                     "kernel_avg_us": float(k1.mean()) * 1e6, "bytes_per_launch": alg_k1},
        "kernels": dict(({"tree_fused": {"avg_us": float(k1.mean()) * 1e6, "bytes_per_launch": alg_k1,
                                         "GBps": achieved, "frac": achieved / HBM_PEAK_GBPS}}
                         if fused else
                         {"stats": {"avg_us": float(k1.mean()) * 1e6, "bytes_per_launch": alg_k1,
                                    "GBps": achieved, "frac": achieved / HBM_PEAK_GBPS},
                          "k_decide_tree": {"avg_us": float(k2.mean()) * 1e6}}),
                        k_commit={"avg_us": float(kc.mean()) * 1e6, "bytes_per_launch": cb,
                                  "GBps": cb / kc.mean() / 1e9,
                                  "frac": cb / kc.mean() / 1e9 / HBM_PEAK_GBPS}),
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
    }
    print(json.dumps(res), flush=True)
    return 0


def bench_ngram(args, wl0) -> int:
    """Prompt-lookup drafting: a step is one specdec_propose_ngram call over the
    batch of token histories (one read of every history row)."""
    import torch
    import speculative_decoding_verification_05_amd as sd
    from speculative_decoding_verification_05_amd import synth

    dev = torch.device("cuda:0")
    B, G = wl0.batch, wl0.gamma_max
    n_min, n_max = wl0.ngram[:2]
    sets = args.sets or 4
    host, dev_in = [], []
    for k in range(sets):
        x = synth.make_ngram_inputs(dataclasses.replace(wl0, data_seed=wl0.data_seed + 100 * k))
        host.append(x)
        dev_in.append({n: torch.from_numpy(v).to(dev) for n, v in x.items()})
    Lmax = host[0]["history"].shape[1]
    log(f"workload {wl0.name}: {sets} input sets of {B} histories "
        f"({np.mean([h['hist_len'].mean() for h in host]):.0f} tokens on average)")
    desc = sd.make_ngram_desc(B, Lmax, n_min, n_max, G)
    ws = torch.zeros(sd.specdec_propose_ngram_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    toks = torch.empty(B, G, dtype=torch.int32, device=dev)
    nd = torch.empty(B, dtype=torch.int32, device=dev)
    ml = torch.empty(B, dtype=torch.int32, device=dev)

    def step(i):  # step i reads input set i % sets
        k = i % sets
        sd.specdec_propose_ngram(desc, dev_in[k]["history"], dev_in[k]["hist_len"], toks, nd, ml,
                                 ws)

    def enqueue(n):
        for i in range(n):
            step(i)

    eager = []
    for k in range(sets):
        step(k)
        torch.cuda.synchronize()
        eager.append((toks.clone(), nd.clone()))

    def check(i):
        return torch.equal(toks, eager[i % sets][0]) and torch.equal(nd, eager[i % sets][1])

    per = steps_per_graph(sets, 64)
    runner = GraphSteps(enqueue, per, check)
    runner.prepare(args.warmup, args.steps)
    if not runner.graphed:
        return 1
    steps = args.steps
    runner.run(args.warmup)
    log(f"  timed launches: {runner.pick_faster(steps)}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    runner.run(steps)
    torch.cuda.synchronize()
    sec_per_step = (time.perf_counter() - t0) / steps
    # kernel time alone: events around each launch on the launching stream
    n_prof = max(sets, (args.profile_steps // sets) * sets)
    evs = []
    for j in range(n_prof):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step(j % sets)
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    kt = np.array([a.elapsed_time(b) for a, b in evs]) * 1e-3
    alg = float(np.mean([h["hist_len"].sum() for h in host])) * 4 + B * 4 + B * (G + 2) * 4
    # the step is this one kernel: its graph-replayed time per launch is the
    # kernel duration plus the dispatch gap, the events' also the event overhead
    k_us = min(float(kt.mean()), sec_per_step)
    kname = "k_propose_ngram_whole" if Lmax <= 8192 else "k_propose_ngram"
    achieved = alg / k_us / 1e9
    proposed = float(np.mean([e[1].sum().item() for e in eager]))
    log(f"step {sec_per_step * 1e6:.2f} us (graph); propose kernel avg {kt.mean() * 1e6:.2f} us "
        f"(events); {achieved:.1f} GB/s = {100 * achieved / HBM_PEAK_GBPS:.1f}% of "
        f"{HBM_PEAK_GBPS:.0f} GB/s; {proposed:.0f} tokens proposed per step")
    cpu = cpu_all = par = None
    if not args.no_cpu_baseline:
        import oracle
        x = host[0]
        reps_c, t_s = 0, time.perf_counter()
        while True:
            oracle.propose_ngram(x["history"], x["hist_len"], n_min, n_max, G)
            reps_c += 1
            t_c = time.perf_counter() - t_s
            if t_c >= args.cpu_seconds or reps_c >= 2000:
                break
        cpu = {"value": reps_c * B / t_c, "unit": "requests/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps_c} pass(es) over all {B} histories of input set 0 ({t_c:.1f} s, "
                         f"single-threaded C)"}
        rate, nt, t_a, passes = oracle_all_cores(
            lambda ix: oracle.propose_ngram(x["history"][ix], x["hist_len"][ix], n_min, n_max, G),
            np.ones(B), args.cpu_seconds / 2)
        log(f"oracle on {nt} threads: {rate:.1f} requests/s ({t_a:.1f} s)")
        cpu_all = {"value": rate, "unit": "requests/s", "cores": nt, "kind": "oracle",
                   "sample": f"input set 0's {B} histories split over {nt} threads, each "
                             f"repeating its slice for {t_a:.1f} s (at least {passes} passes)"}
    res = {
        "metric": f"proposing requests/sec ({wl0.name})", "value": B / sec_per_step,
        "unit": "requests/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": sec_per_step * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": wl0.name, "batch": B, "max_len": Lmax, "n_min": n_min,
                   "n_max": n_max, "gamma_max": G, "rotating_input_sets": sets,
                   "steps_per_graph": per,
                   "launch": "hipgraph" if runner.graphed else "eager", "proposed_tokens_per_s": proposed / sec_per_step},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(f"{kname}__{wl0.name}"),
                     "kernel": kname,
                     "kernel_avg_us": k_us * 1e6,
                     "bytes_per_launch": alg},
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
