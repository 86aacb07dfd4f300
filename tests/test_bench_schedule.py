"""The step schedule of bench.py (host side, no GPU): every step is issued and
committed exactly once, in order, with at most two steps in flight, and --
with instances used round-robin -- each instance's commit of step s is issued
before that instance's next step s + R."""
import pytest

import bench


@pytest.mark.parametrize("serial", [False, True])
@pytest.mark.parametrize("first,last", [(0, 0), (0, 1), (0, 2), (3, 11), (0, 40)])
def test_schedule_orders_issue_and_commit(serial, first, last):
    log = []
    bench.schedule_steps(first, last, lambda s: log.append(("launch", s)), lambda s: log.append(("finish", s)),
                         serial=serial)
    steps = list(range(first, last))
    assert [s for op, s in log if op == "launch"] == steps
    assert [s for op, s in log if op == "finish"] == steps
    pos = {e: i for i, e in enumerate(log)}
    in_flight = 0
    for op, s in log:
        in_flight += 1 if op == "launch" else -1
        assert 0 <= in_flight <= (1 if serial else 2)
    for s in steps:
        assert pos[("launch", s)] < pos[("finish", s)]
        for R in (2, 3, 8):                       # instance of step s is s % R
            if s + R < last:
                assert pos[("finish", s)] < pos[("launch", s + R)]
