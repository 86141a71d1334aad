"""The pruning the merge relies on, restated on the CPU and checked over random list sets:
for lists sorted best first (zero padded, all keys distinct), the 16 largest keys of their
union lie in the 16 lists with the largest heads, so merging only those lists gives the
same top 16 (and therefore the same first m <= 16) as merging all of them. The kernels'
merge_top16 prunes this way for many short lists (e.g. 256 splits of 4 blocks)."""
import numpy as np
import pytest


def top16(keys):
    return sorted(keys, reverse=True)[:16]


def make_lists(rng, ns, lk, fill):
    """ns lists of lk slots, distinct positive keys best first, each with 1..lk real keys."""
    keys = np.unique(rng.integers(1, 1 << 40, size=2 * ns * lk))[: ns * lk]  # distinct
    assert keys.size == ns * lk
    rng.shuffle(keys)
    lists = []
    for i in range(ns):
        real = lk if fill else int(rng.integers(1, lk + 1))
        k = sorted(keys[i * lk:i * lk + real].tolist(), reverse=True)
        lists.append(k + [0] * (lk - real))
    return lists


@pytest.mark.parametrize("ns,lk", [(17, 1), (64, 4), (129, 4), (256, 4), (200, 3), (128, 8),
                                   (65, 8), (64, 16), (33, 16), (256, 2)])
def test_top16_lies_in_the_lists_with_the_best_heads(ns, lk):
    rng = np.random.default_rng(ns * 31 + lk)
    for trial in range(60):
        lists = make_lists(rng, ns, lk, fill=trial % 2 == 0)
        if trial % 3 == 0:  # adversarial: one list holds all the large keys
            big = sorted(np.unique(rng.integers(1 << 41, 1 << 42, size=4 * lk))[:lk].tolist(), reverse=True)
            lists[int(rng.integers(ns))] = big
        everything = [k for l in lists for k in l if k]
        best = sorted(range(ns), key=lambda i: lists[i][0], reverse=True)[:16]
        pruned = [k for i in best for k in lists[i] if k]
        assert top16(pruned) == top16(everything)


@pytest.mark.parametrize("ns,lk", [(129, 4), (200, 4), (256, 4), (256, 2), (193, 1)])
def test_best_heads_lie_in_the_lanes_with_the_best_maxima(ns, lk):
    # The same argument one level up, as merge_top16 applies it before ranking the heads of
    # more than 64 lists: lane l holds the heads of lists l, l + 64, l + 128, l + 192, and the
    # 16 best heads lie among the heads of the 16 lanes whose largest head is best, so those
    # (at most 64) heads ranked alone give the same 16 lists.
    rng = np.random.default_rng(ns * 7 + lk)
    for trial in range(60):
        lists = make_lists(rng, ns, lk, fill=trial % 2 == 0)
        if trial % 3 == 0:  # adversarial: one lane holds the four best heads
            lane = int(rng.integers(64))
            for t in range(4):
                if lane + 64 * t < ns:
                    lists[lane + 64 * t][0] = (1 << 45) + t
        heads = [l[0] for l in lists]
        lanes = {}
        for i, h in enumerate(heads):
            lanes.setdefault(i % 64, []).append(h)
        best_lanes = sorted(lanes, key=lambda l: max(lanes[l]), reverse=True)[:16]
        gathered = [h for l in best_lanes for h in lanes[l]]
        assert top16(gathered) == top16(heads)

