"""Host-side logic of bench.py (CPU): the step runner times exactly the
requested number of steps, and the graph length covers whole passes over the
input sets."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("sets,at_least,want", [(1, 16, 16), (5, 16, 20), (3, 16, 18), (4, 64, 64),
                                                 (7, 16, 21), (20, 16, 20)])
def test_steps_per_graph_is_whole_passes(sets, at_least, want):
    per = bench.steps_per_graph(sets, at_least)
    assert per == want
    assert per % sets == 0 and per >= at_least


@pytest.mark.parametrize("per", [1, 16, 18, 64])
@pytest.mark.parametrize("n", [1, 5, 17, 18, 100, 2000])
def test_runner_enqueues_exactly_n_steps(per, n):
    """Without graphs the runner enqueues the graphs' step sequences itself:
    n // per full groups, then one group of the n % per remaining steps, each
    group starting again at step 0 (the cache lengths are restored per group)."""
    calls = []
    runner = bench.GraphSteps(lambda k: calls.append(k), per, lambda i: True, use_graphs=False)
    runner.prepare(n)
    runner.run(n)
    assert sum(calls) == n
    assert calls == [per] * (n // per) + ([n % per] if n % per else [])
    assert not runner.graphed


@pytest.mark.parametrize("graph_s,eager_s,want", [(0.002, 0.0, "eager"), (0.0, 0.002, "hipgraph")])
def test_runner_picks_the_faster_launch_mode(monkeypatch, graph_s, eager_s, want):
    """pick_faster times untimed windows both ways and keeps the faster
    mode; the timed run then launches only that way."""
    import time
    import torch
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)

    class FakeGraph:
        replays = 0

        def replay(self):
            FakeGraph.replays += 1
            time.sleep(graph_s)

    calls = []

    def enqueue(k):
        calls.append(k)
        time.sleep(eager_s)

    runner = bench.GraphSteps(enqueue, 4, lambda i: True)
    runner.graphs = {4: FakeGraph()}
    assert runner.pick_faster(8, rounds=3) == want
    assert runner.graphed == (want == "hipgraph")
    calls.clear()
    FakeGraph.replays = 0
    runner.run(8)
    assert (FakeGraph.replays, sum(calls)) == ((2, 0) if want == "hipgraph" else (0, 8))


def test_runner_without_graphs_stays_eager():
    calls = []
    runner = bench.GraphSteps(lambda k: calls.append(k), 4, lambda i: True, use_graphs=False)
    assert runner.pick_faster(8) == "eager"
    assert calls == []  # nothing run: there is no choice to make
