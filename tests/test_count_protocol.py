"""The row count that picks each row's merging workgroup, restated on the CPU and run over
random arrival orders: exactly one of a row's ns workgroups sees the count complete, it is
the last to arrive at the row counter, every group counter and the row counter are back at
zero afterwards, and (for rows of more than 128 splits, counted 16 per group first) the
merging workgroup arrives only after every workgroup of the row has counted in. The
kernels' count_in follows these rules: one increment per workgroup on its group counter
(groups of 16 consecutive splits), then, by a group's last workgroup, one on the row
counter; rows of at most 128 splits use the row counter alone."""
import numpy as np
import pytest

GROUP, TWO_LEVEL = 16, 128


def count_in(counters, s, ns):
    """counters: dict of counter name -> value (the row counter 'row', groups ('g', k))."""
    if ns > TWO_LEVEL:
        g = s // GROUP
        members = min(GROUP, ns - g * GROUP)
        prev = counters[("g", g)]
        counters[("g", g)] = prev + 1
        if prev != members - 1:
            return False
        counters[("g", g)] = 0
        ns = -(-ns // GROUP)
    prev = counters["row"]
    counters["row"] = prev + 1
    if prev != ns - 1:
        return False
    counters["row"] = 0
    return True


@pytest.mark.parametrize("ns", [1, 2, 16, 17, 64, 128, 129, 130, 144, 200, 255, 256])
def test_one_merger_after_everyone(ns):
    rng = np.random.default_rng(ns)
    for _ in range(200):
        counters = {"row": 0, **{("g", k): 0 for k in range(16)}}
        order = rng.permutation(ns)
        winners = [i for i, s in enumerate(order) if count_in(counters, int(s), ns)]
        assert len(winners) == 1
        # The last split to arrive completes its group, and every other group is complete
        # by then, so in both schemes it is the one that merges: all lists are published.
        assert winners[0] == ns - 1
        assert all(v == 0 for v in counters.values())
