"""Host-side helpers of bench.py: the warm-up loop and the choice of the dense-causal comparator's
block (the faster one is kept).  No GPU: torch's synchronize is replaced by a stand-in."""
import os
import sys
import time

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


class _Cuda:
    def __init__(self):
        self.syncs = 0

    def synchronize(self):
        self.syncs += 1


class _Torch:
    def __init__(self):
        self.cuda = _Cuda()


def test_warm_runs_at_least_n_calls():
    calls = []
    n = bench._warm(_Torch(), lambda t: calls.append(t), 5)
    assert n == 5 and calls == [None] * 5


def test_warm_keeps_going_until_the_time_floor():
    calls = []

    def fn(t):
        calls.append(t)
        time.sleep(0.002)

    n = bench._warm(_Torch(), fn, 1, min_ms=20.0)
    assert n == len(calls) and n >= 5  # at least 20 ms of 2 ms calls


def test_time_dense_keeps_the_fastest_block():
    cost = {64: 0.004, 128: 0.001}
    seen = []

    def run(block, timer):
        seen.append((block, timer))
        time.sleep(cost[block])

    ms, best, by_block, timer = bench.time_dense(_Torch(), run, (64, 128), steps=3, warmup=1)
    assert best == 128 and timer is None
    assert set(by_block) == {64, 128} and by_block[128] < by_block[64]
    assert abs(ms - by_block[128]) < 1e-3
    assert [b for b, _ in seen].count(64) == 4 and [b for b, _ in seen].count(128) == 4


class _Event:
    clock = [0.0]

    def __init__(self, enable_timing=True):
        self.t = None

    def record(self):
        _Event.clock[0] += 1.0
        self.t = _Event.clock[0]

    def elapsed_time(self, other):
        return other.t - self.t


class _CudaEv(_Cuda):
    Event = _Event


class _TorchEv:
    def __init__(self):
        self.cuda = _CudaEv()


def _step(timer, n_calls):
    timer.begin()
    for _ in range(n_calls):
        timer.mark()


def test_timer_records_every_boundary_by_default():
    t = bench.Timer(_TorchEv(), ["a", "b", "c"])
    _step(t, 3)
    assert sorted(t.pending[0]) == [0, 1, 2, 3]  # begin + one event after each call
    t.collect()
    assert all(t.samples[n] == [1.0] for n in ("a", "b", "c"))


def test_timer_only_records_around_the_chosen_call():
    t = bench.Timer(_TorchEv(), ["a", "b", "c"], only=("b",))
    _step(t, 3)
    _step(t, 3)
    assert [sorted(p) for p in t.pending] == [[1, 2], [1, 2]]  # two events per step, around call b
    t.collect()
    assert t.samples["b"] == [1.0, 1.0] and t.samples["a"] == [] and t.samples["c"] == []
    none = bench.Timer(_TorchEv(), ["a", "b"], only=())
    _step(none, 2)
    assert none.pending == [{}]  # no events at all


def test_time_with_breakdown_runs_breakdown_then_exactly_the_timed_steps(monkeypatch):
    monkeypatch.setattr(bench, "SETTLE_MS", 0.0)
    seen = []

    def fn(timer):
        seen.append(None if timer is None else id(timer))
        if timer is not None:
            _step(timer, 3)
        return len(seen)

    ms, out, bd, timed = bench.time_with_breakdown(_TorchEv(), fn, ["a", "b", "c"], steps=4, warmup=2,
                                                   timed_only=("c",))
    assert seen[:2] == [None, None]  # warm-up without events
    assert seen[2:6] == [id(bd)] * 4 and seen[6:] == [id(timed)] * 4  # nothing between the two passes
    assert out == 10 and ms >= 0.0
    assert all(len(bd.samples[n]) == 4 for n in "abc")
    assert timed.samples["c"] == [1.0] * 4 and timed.samples["a"] == [] and timed.samples["b"] == []
