"""The device plan's rules, checked on the CPU over random and adversarial length mixes.

For num_splits = 0, topk <= 16, 0 < W <= 4096 and batch * W >= 8192 blocks the kernels pick
the split width C from the row lengths: C = min(max(2^ceil(log2(ceil(N / 512))), C_min), 64),
N the blocks present, C_min the smallest of 4, 8, .., 64 at which every row's lists fit (at
most min(S * topk / Lk, 1024 / Lk2) splits of C blocks, S = min(64, ceil(W / 4)),
Lk = min(topk, C), Lk2 = Lk rounded up to a power of two). Row b then takes
max(1, ceil(nb_b / C)) workgroups of a 1-D grid of min(batch * ceil(W / 4),
max(512, ceil(batch * W / 64)) + batch) workgroups. These tests restate those rules and check
what the kernels rely on: the grid covers every row, each row's lists fit its S * topk
workspace keys per head and the merge network's 1024, and a fitting width always exists."""
import numpy as np
import pytest


def pow2_at_least(x):
    p = 1
    while p < x:
        p <<= 1
    return p


def max_splits(C, S, topk):
    lk = min(topk, C)
    return min(S * topk // lk, 1024 // pow2_at_least(lk))


def plan(nb, W, topk):
    B = len(nb)
    S = min(64, -(-W // 4))
    N = int(nb.sum())
    C_min = None
    for t in range(5):
        C = 4 << t
        if int(nb.max(initial=0)) <= max_splits(C, S, topk) * C:
            C_min = C
            break
    assert C_min is not None, "no width fits the longest row"
    C = min(max(pow2_at_least(max(1, -(-N // 512))), C_min), 64)
    grid = min(B * -(-W // 4), max(512, -(-B * W // 64)) + B)
    return S, C, grid


def check(nb, W, topk):
    S, C, grid = plan(nb, W, topk)
    ns = np.maximum(1, -(-nb // C))
    assert int(ns.sum()) <= grid
    lk = min(topk, C)
    real = -(-nb // C)
    assert np.all(real * lk <= S * topk)
    assert np.all(real * pow2_at_least(lk) <= 1024)
    assert 4 <= C <= 64


@pytest.mark.parametrize("topk", [1, 3, 4, 8, 15, 16])
def test_random_mixes(topk):
    rng = np.random.default_rng(topk)
    for _ in range(400):
        W = int(rng.choice([8, 60, 64, 100, 256, 1000, 1024, 2048, 4095, 4096]))
        B = max(1, int(rng.integers(-(-8192 // W), -(-8192 // W) + 300)))
        kind = rng.integers(4)
        if kind == 0:
            nb = rng.integers(0, W + 1, size=B)
        elif kind == 1:
            nb = np.full(B, W)
        elif kind == 2:
            nb = rng.integers(0, 9, size=B)
            nb[rng.integers(B)] = W
        else:
            nb = np.where(rng.random(B) < 0.1, W, 0)
        check(nb.astype(np.int64), W, topk)


@pytest.mark.parametrize("W", [32, 256, 1024, 1025, 2048, 2049, 4096])
@pytest.mark.parametrize("B", [2, 8, 64, 300])
def test_one_full_row_among_empty_ones(W, B):
    if B * W < 8192:
        pytest.skip("host plan")
    for topk in (1, 8, 16):
        nb = np.zeros(B, dtype=np.int64)
        nb[B // 2] = W
        check(nb, W, topk)
        check(np.full(B, W, dtype=np.int64), W, topk)


def workgroup_map(nb, C):
    """Workgroup g -> (row, split) for batch <= 64: row b takes max(1, ceil(nb_b / C))
    consecutive ids, starting with the first row of the most splits and wrapping around."""
    cnt = np.maximum(1, -(-nb // C))
    incl = np.cumsum(cnt)
    total = int(incl[-1])
    r0 = int(np.argmax(cnt))  # the first row of the most splits
    shift = int(incl[r0] - cnt[r0])
    out = {}
    for g in range(total):
        gr = (g + shift) % total
        b = int(np.searchsorted(incl, gr, side="right"))
        out[g] = (b, gr - int(incl[b] - cnt[b]))
    return out, cnt


@pytest.mark.parametrize("seed", range(40))
def test_the_longest_row_takes_the_first_workgroups(seed):
    # Every (row, split) gets exactly one workgroup, and the row of the most splits gets
    # workgroups 0, 1, ..: dispatched first, they never share a CU with an earlier workgroup.
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 65))
    W = int(rng.choice([64, 256, 1024, 4096]))
    nb = rng.integers(0, 9, size=B).astype(np.int64)
    nb[int(rng.integers(B))] = int(rng.integers(W // 2, W + 1))
    C = int(rng.choice([4, 8, 16]))
    m, cnt = workgroup_map(nb, C)
    pairs = sorted(m.values())
    assert pairs == sorted((b, s) for b in range(B) for s in range(int(cnt[b])))
    r0 = int(np.argmax(cnt))
    assert [m[g] for g in range(int(cnt[r0]))] == [(r0, s) for s in range(int(cnt[r0]))]


# ---------------------------------------------------------------------------------------
# Even splits (host plan; 4 <= batch <= 64 rows of W blocks split into S = 256 / batch splits
# of C = ceil(W / S) or C - 1 blocks): the first wide = W - S (C - 1) splits of a row are the
# C-block ones, and the linear workgroup id g = y * S + x (the dispatch order) gives every row's
# wide splits the first ids. Restated from the split kernel's arithmetic.

def even_map(g, batch, S, wide):
    if g < batch * wide:
        return g // wide, g % wide
    k = g - batch * wide
    narrow = S - wide
    return k // narrow, wide + k % narrow


def even_start(s, C, wide):
    return s * (C - 1) + min(s, wide)


def even_taking_part(nb, C, wide):
    if nb <= wide * C:
        return -(-nb // C)
    return wide + (nb - wide * C + C - 2) // (C - 1)


@pytest.mark.parametrize("batch,W", [(16, 68), (8, 150), (4, 300), (64, 17), (32, 40), (5, 251), (16, 80)])
def test_even_split_layout(batch, W):
    S = 256 // batch
    C = -(-W // S)
    wide = W - S * (C - 1)
    assert 1 <= wide <= S and C >= 2
    seen = set()
    order = []
    for g in range(batch * S):                      # every workgroup a distinct (row, split)
        b, s = even_map(g, batch, S, wide)
        assert 0 <= b < batch and 0 <= s < S and (b, s) not in seen
        seen.add((b, s))
        order.append(C if s < wide else C - 1)
    assert order == sorted(order, reverse=True)      # the wide splits first in dispatch order
    starts = [even_start(s, C, wide) for s in range(S + 1)]
    assert starts[0] == 0 and starts[S] == W        # the splits tile the row
    assert all(starts[s + 1] - starts[s] == (C if s < wide else C - 1) for s in range(S))
    for nb in range(W + 1):                          # splits that start below nb take part
        assert even_taking_part(nb, C, wide) == sum(1 for s in range(S) if starts[s] < nb), nb
