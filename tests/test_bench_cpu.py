"""Host logic of bench.py that runs without a GPU: the untimed settle phase every
workload runs before its tuning, warm-up and timed region, and the command line."""
import sys
import types

import bench


def fake_torch(log):
    return types.SimpleNamespace(cuda=types.SimpleNamespace(synchronize=lambda: log.append("sync")))


def test_settle_calls_until_the_time_has_passed():
    log = []
    n = bench.settle(fake_torch(log), lambda i: log.append(i), 0.05)
    assert n > 0 and n % 8 == 0                       # whole groups of eight calls
    assert [x for x in log if x != "sync"] == list(range(n))
    assert log.count("sync") == n // 8                # one synchronisation per group


def test_settle_of_zero_seconds_calls_nothing():
    log = []
    assert bench.settle(fake_torch(log), lambda i: log.append(i), 0.0) == 0
    assert bench.settle(fake_torch(log), lambda i: log.append(i), -1.0) == 0
    assert log == []


def test_settle_seconds_option(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    assert bench.parse().settle_seconds == 5.0
    monkeypatch.setattr(sys, "argv", ["bench.py", "--settle-seconds", "0"])
    assert bench.parse().settle_seconds == 0.0
