"""Host-side checks of a rank's share in the context-parallel layout (round-robin blocks
j = local * P + rank, vLLM PR #57832, Solution): the shares partition every row's blocks,
keep each block's page and valid-token count, and put the pinned blocks at the ends of the
ranks' local ranges, where the kernel's scalar pin counts find them."""
import numpy as np
import pytest

from sparse_attention_block_amd import shard


def local_view(bt_r, lens_r, b, P, r):
    nb_r = -(-int(lens_r[b]) // 128)
    return [(l * P + r, int(bt_r[b, l]), min(128, int(lens_r[b]) - l * 128)) for l in range(nb_r)]


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("L", [1, 127, 128, 129, 128 * 7, 128 * 37 + 5, 128 * 64])
def test_shares_partition_the_row(P, L):
    rng = np.random.default_rng(P * 1000 + L)
    B, W = 3, 70
    bt = rng.integers(0, 10_000, size=(B, W)).astype(np.int32)
    lens = np.full(B, L, dtype=np.int32)
    nb = -(-L // 128)
    n_init, n_local = 1, 2
    seen = {}
    pins = set()
    for r in range(P):
        bt_r, lens_r, ni, nl = shard.rank_share(bt, lens, P, r, n_init, n_local)
        assert bt_r.shape == (B, -(-W // P))
        for b in range(B):
            loc = local_view(bt_r, lens_r, b, P, r)
            for jl, (j, page, valid) in enumerate(loc):
                assert j % P == r and j < nb
                assert page == bt[b, j]
                assert valid == min(128, L - j * 128)        # same tokens as in the full row
                seen[(b, j)] = seen.get((b, j), 0) + 1
                if jl < ni or jl >= len(loc) - nl:
                    pins.add((b, j))
    assert all(seen.get((b, j)) == 1 for b in range(B) for j in range(nb))
    assert len(seen) == B * nb
    want = {(b, j) for b in range(B) for j in range(nb) if j < n_init or j >= nb - n_local}
    assert pins == want


def test_global_ids_and_padding():
    ids = np.array([[0, 3, -1], [5, -1, -1]], dtype=np.int32)
    assert np.array_equal(shard.global_ids(ids, 4, 2), [[2, 14, -1], [22, -1, -1]])


def test_rows_needing_different_pins_are_refused():
    bt = np.zeros((2, 8), dtype=np.int32)
    lens = np.array([128 * 8, 128 * 7], dtype=np.int32)   # rank 3 holds block 7 of row 0 only
    with pytest.raises(ValueError):
        shard.rank_share(bt, lens, 4, 3, 1, 2)


@pytest.mark.parametrize("P", [2, 3, 4])
@pytest.mark.parametrize("L", [128 * 12, 128 * 11 + 40, 128 * 5 + 1])
def test_oracle_on_the_shares_merges_to_the_oracle_on_the_rows(P, L):
    # The pages' exactness argument, run with the oracle: each rank's top-k of its share
    # (pins on the shard), merged per head with pins first, equals the top-k of the rows.
    import oracle
    from sparse_attention_block_amd import synth

    B, W, topk, n_init, n_local = 3, 12, 4, 1, 2
    inp = synth.paged_case(600 + P, [L] * B, W, poison=False, topk=topk, n_init=n_init,
                           n_local=n_local)
    want_ids, want_sc, _ = oracle.decode(inp)
    nb = -(-L // 128)
    cands = [[[] for _ in range(4)] for _ in range(B)]
    for r in range(P):
        bt_r, lens_r, ni, nl = shard.rank_share(inp.block_table, inp.seq_lens, P, r, n_init, n_local)
        sub = synth.Inputs("share", inp.q, inp.k_cache, bt_r, lens_r, topk=topk, n_init=ni,
                           n_local=nl)
        ids, sc, _ = oracle.decode(sub)
        gids = shard.global_ids(ids, P, r)
        for b in range(B):
            for h in range(4):
                cands[b][h] += [(int(j), float(s)) for j, s in zip(gids[b, h], sc[b, h]) if j >= 0]
    for b in range(B):
        for h in range(4):
            pinned = lambda j: j < n_init or j >= nb - n_local
            got = sorted(cands[b][h], key=lambda c: (not pinned(c[0]), -c[1], c[0]))[:min(topk, nb)]
            m = len(got)
            assert [j for j, _ in got] == list(want_ids[b, h, :m])
            assert [s for _, s in got] == list(want_sc[b, h, :m])
            assert np.all(want_ids[b, h, m:] == -1)
