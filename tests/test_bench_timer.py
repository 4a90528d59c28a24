"""Host logic of bench.py's chained step timer: with one event before each
kernel and one closing event, every kernel's span must run from its own
event to the next one (CPU only; the events are stand-ins that count)."""
import importlib.util
import os

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


class _Clock:
    t = 0


class _Event:
    """Records the running clock; elapsed_time is the difference."""

    def __init__(self, enable_timing=False):
        self.at = None

    def record(self):
        self.at = _Clock.t

    def elapsed_time(self, other):
        return float(other.at - self.at)


def test_chain_timer_pairs_each_kernel_with_the_next_event(monkeypatch):
    monkeypatch.setattr(torch.cuda, "Event", _Event)
    bench = _bench()
    kt = bench.ChainTimer()
    durations = {"quant_act_w": [3, 5, 4], "gemm": [40, 41, 39]}

    def kernel(name, k):
        def fn():
            _Clock.t += durations[name][k]   # the kernel's time on the stream
        return fn

    _Clock.t = 0
    for k in range(3):
        kt.run("quant_act_w", kernel("quant_act_w", k))
        kt.run("gemm", kernel("gemm", k))
    kt.close()
    assert kt.times_ms("quant_act_w") == [3.0, 5.0, 4.0]
    assert kt.times_ms("gemm") == [40.0, 41.0, 39.0]
    st = kt.stats_us("gemm")
    assert st["calls"] == 3 and st["us_min"] == 39e3 and st["us_median"] == 40e3
    kt.reset()
    assert kt.events == {} and kt.marks == []
