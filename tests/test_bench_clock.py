"""bench.py's clock reading, on the host: a stand-in for the metrics table
that refreshes on a timer, and a stand-in graph, check that only refreshes
seen after the settle time count, each once, averaged over the XCDs."""
import time

import pytest

import bench


class _Table:
    """Refreshes every `period` seconds; refresh i reports clocks base + i."""

    def __init__(self, period, base, xcds=8):
        self.t0, self.period, self.base, self.xcds = time.perf_counter(), period, base, xcds

    def read(self):
        i = int((time.perf_counter() - self.t0) / self.period)
        return 1000 + i, [float(self.base + i + (x % 2)) for x in range(self.xcds)]


class _Graph:
    def __init__(self):
        self.replays = 0

    def replay(self):
        self.replays += 1
        time.sleep(0.001)


class _Stream:
    def synchronize(self):
        pass


def test_clock_refreshes_after_settle(monkeypatch):
    table, closed = _Table(period=0.1, base=1900), []
    monkeypatch.setattr(bench, "gfx_clock_reader", lambda: (table.read, lambda: closed.append(1)))
    g = _Graph()
    c = bench.clock_under_load(g, _Stream(), replay_s=0.001, seconds=0.55, settle_s=0.15, period_s=0.005)
    assert closed == [1] and g.replays > 0
    # refresh i (mean clock 1900.5 + i) appears at 0.1 i s: 0 precedes the
    # load, 0 and 1 the settle time (1 may be first seen late, on a busy
    # host); each later one counts once
    assert 3 <= c["refreshes"] <= 5
    assert c["gfx_mhz_min"] in (pytest.approx(1901.5), pytest.approx(1902.5))
    assert c["gfx_mhz_max"] <= 1905.5
    assert c["gfx_mhz_min"] <= c["gfx_mhz_mean"] <= c["gfx_mhz_max"]
    assert c["spec_mhz"] == 2400.0


def test_clock_none_without_reader(monkeypatch):
    monkeypatch.setattr(bench, "gfx_clock_reader", lambda: None)
    assert bench.clock_under_load(_Graph(), _Stream(), replay_s=0.001, seconds=0.05) is None


def test_clock_none_without_refresh(monkeypatch):
    table = _Table(period=100.0, base=1700)  # never refreshes during the load
    monkeypatch.setattr(bench, "gfx_clock_reader", lambda: (table.read, lambda: None))
    assert bench.clock_under_load(_Graph(), _Stream(), replay_s=0.001, seconds=0.1, settle_s=0.01) is None
