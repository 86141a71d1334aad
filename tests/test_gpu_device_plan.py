"""GPU parity of the device plan: with num_splits = 0 (W <= 4096, topk <= 16, batch * W at
least 8192 blocks) the fused single-token pass, and the multi-token and FP8 passes, pick the
split width C and each workgroup's (row, split) on the device from the row lengths (about 512
workgroups in all; a row may have as many splits as its lists fit the workspace and the merge
network: at topk 16, 256 splits of 4 blocks, 128 of 8, or 64 of 16..64). Scores do not depend
on the plan, so the selection must equal the oracle's selection on the GPU's own block scores,
and the oracle's within the near-tie rule; exact-integer data must match bit for bit."""
import numpy as np
import pytest

import oracle
from sparse_attention_block_amd import synth

from gpu_util import check_selection_exact_given_scores, check_selection_vs_oracle, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_block_amd as m
    m.load()
    return m


def check(msa, inp, ids=None, sc=None):
    q, k, bt, lens = to_device(inp)
    assert msa.plan(inp.batch, inp.max_blocks, inp.topk)["blocks_per_split"] == 0  # device plan
    if ids is None:
        ids, sc = msa.msa_indexer_decode(q, k, bt, lens, inp.topk, inp.n_init, inp.n_local)
    gpu_s = msa.msa_indexer_block_scores(q, k, bt, lens).cpu().numpy()
    ids, sc = ids.cpu().numpy(), sc.cpu().numpy()
    check_selection_exact_given_scores(ids, sc, gpu_s, inp.seq_lens, inp.topk, inp.n_init, inp.n_local)
    ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, inp.seq_lens)
    check_selection_vs_oracle(ids, ref, inp.seq_lens, inp.topk, inp.n_init, inp.n_local)
    return ids


def test_many_rows_cross_the_wave_scan(msa):
    # 150 rows: the device prefix scan over row split counts runs in three 64-row chunks.
    rng = np.random.default_rng(401)
    lens = rng.integers(0, 128 * 20, size=150)
    lens[[3, 70, 149]] = [128 * 40, 128 * 33 + 5, 1]
    inp = synth.paged_case(401, lens.tolist(), 60)   # 150 x 60 blocks: the device plan
    check(msa, inp)


def test_long_row_among_empty_rows(msa):
    # One 1024-block row and 47 empty rows: each empty row still gets a workgroup for its
    # padding, and the long row gets 256 splits of 4 blocks.
    lens = [0] * 48
    lens[17] = 128 * 1024
    inp = synth.paged_case(402, lens, 1024)
    ids = check(msa, inp)
    assert np.all(ids[np.arange(48) != 17] == -1)


def test_widest_device_table(msa):
    # W = 4096: the longest row takes 64 splits of 64 blocks (the largest staged lists).
    inp = synth.paged_case(403, [128 * 4096, 128 * 100 + 7, 128 * 4095], 4096, poison=False)
    check(msa, inp)
    # one block wider: the host plan
    assert msa.plan(3, 4097, 16)["blocks_per_split"] > 0


def test_planted_exact_under_device_plan(msa):
    # The planted workload behind a table widened to 512 blocks, so that the decode call
    # takes the device plan (the rows still hold 68 blocks).
    inp = synth.config(5)
    want_ids, want_sc, _ = oracle.decode(inp)
    q, k, bt, lens = to_device(inp, extra_cols=512 - 68)
    assert msa.plan(16, 512, 16)["blocks_per_split"] == 0
    ids, sc = msa.msa_indexer_decode(q, k, bt, lens)
    assert np.array_equal(ids.cpu().numpy(), want_ids)
    assert np.array_equal(sc.cpu().numpy().astype(np.float64), want_sc)


def test_full_rows_take_the_full_row_plan(msa):
    # Every row W blocks long: the workgroups take the host's full-row plan from one ballot
    # instead of computing the general plan. The same rows with one row a block short take the
    # general plan; both (and the multi-token and FP8 passes on each) select as the oracle does.
    from test_gpu_fp8 import run_fp8
    from test_gpu_multi import run_multi

    W, B = 600, 16
    assert msa.plan(B, W, 16)["blocks_per_split"] == 0
    for name, lens in (("full", [128 * W] * B), ("one row short", [128 * W] * 5 + [128 * (W - 1)] + [128 * W] * 10)):
        check(msa, synth.paged_case(415, lens, W, poison=False))
        run_multi(msa, synth.multi_case(416, lens, W, 2, poison=False))
        run_fp8(msa, synth.fp8_case(417, lens, W, 1, k_scale=0.5, poison=False), 1e-3 * 4.0 * 0.5)


def test_split_width_changes_between_graph_replays(msa):
    # The captured grid covers any lengths; replays with lengths that move the device's
    # split width (C = 4 .. 64) and the long row's split count must match eager calls.
    inp = synth.paged_case(404, [128 * 512] * 32, 512, poison=False)
    q, k, bt, lens = to_device(inp)
    ws = msa.new_workspace(32, 512, 16)
    ids = torch.empty((32, 4, 16), dtype=torch.int32, device="cuda")
    sc = torch.empty((32, 4, 16), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        msa.msa_indexer_decode(q, k, bt, lens, out_ids=ids, out_scores=sc, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        msa.msa_indexer_decode(q, k, bt, lens, out_ids=ids, out_scores=sc, workspace=ws)
    rng = np.random.default_rng(5)
    for it, kind in enumerate(["all long", "one long", "all short", "mixed", "empty"]):
        if kind == "all long":
            new = np.full(32, 128 * 512)
        elif kind == "one long":
            new = np.zeros(32, np.int64); new[9] = 128 * 512
        elif kind == "all short":
            new = rng.integers(1, 300, size=32)
        elif kind == "mixed":
            new = rng.integers(0, 128 * 512 + 1, size=32)
        else:
            new = np.zeros(32, np.int64)
        lens.copy_(torch.from_numpy(new.astype(np.int32)))
        g.replay()
        torch.cuda.synchronize()
        eager_ids, eager_sc = msa.msa_indexer_decode(q, k, bt, lens)
        assert torch.equal(ids, eager_ids) and torch.equal(sc, eager_sc), kind
        cur = synth.Inputs("replay", inp.q, inp.k_cache, inp.block_table, new.astype(np.int32))
        gpu_s = msa.msa_indexer_block_scores(q, k, bt, lens).cpu().numpy()
        check_selection_exact_given_scores(ids.cpu().numpy(), sc.cpu().numpy(), gpu_s, cur.seq_lens,
                                           16, 1, 2)


def test_two_level_count_and_single_splits_under_graph_replays(msa):
    # Replays of one captured call whose lengths switch between rows of 256 splits (counted
    # in two levels), rows that fit one split (written without the merge) and a mix; each
    # replay equals an eager call, and every counter line is back at zero after it.
    B, W = 8, 1024
    inp = synth.paged_case(405, [128 * W] * B, W, poison=False)
    q, k, bt, lens = to_device(inp)
    ws = msa.new_workspace(B, W, 16)
    ids = torch.empty((B, 4, 16), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, 4, 16), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        msa.msa_indexer_decode(q, k, bt, lens, out_ids=ids, out_scores=sc, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        msa.msa_indexer_decode(q, k, bt, lens, out_ids=ids, out_scores=sc, workspace=ws)
    one_long = np.zeros(B, np.int64); one_long[3] = 128 * W
    two_long = np.zeros(B, np.int64); two_long[[0, 7]] = [128 * W, 128 * W - 5]
    short = np.array([1, 128, 129, 512, 0, 300, 511, 64])
    mixed = short.copy(); mixed[5] = 128 * W
    for it, new in enumerate([one_long, two_long, short, mixed, one_long, short, two_long]):
        lens.copy_(torch.from_numpy(new.astype(np.int32)))
        g.replay()
        torch.cuda.synchronize()
        counters = ws[256:256 + B * 17 * 256].view(torch.int32)
        assert int(counters.abs().sum()) == 0, it
        got_ids, got_sc = ids.clone(), sc.clone()
        eager_ids, eager_sc = msa.msa_indexer_decode(q, k, bt, lens)
        assert torch.equal(got_ids, eager_ids) and torch.equal(got_sc, eager_sc), it
        cur = synth.Inputs("replay", inp.q, inp.k_cache, inp.block_table, new.astype(np.int32))
        gpu_s = msa.msa_indexer_block_scores(q, k, bt, lens).cpu().numpy()
        check_selection_exact_given_scores(got_ids.cpu().numpy(), got_sc.cpu().numpy(), gpu_s,
                                           cur.seq_lens, 16, 1, 2)


# Rows at the edges of the per-row split limit (topk 16: C = 4 up to 1024 blocks, then C = 32
# up to 2048 and C = 64 up to 4096; topk 8: C = 16 up to 1024 blocks; topk 4: C = 4 up to 256
# blocks, C = 8 up to 512), for the single-token, multi-token and FP8 passes.
EDGE_CASES = [
    ("c4-256-splits", 1024, [128 * 1024, 1, 0, 128 * 1023 + 5, 7, 128 * 3, 129, 2], 16),
    ("c32-33-splits", 2048, [128 * 1024 + 1, 3, 128 * 700, 0], 16),
    ("c32-64-splits", 2048, [128 * 2048, 128 * 2047 + 1, 5, 128 * 1025], 16),
    ("c64", 4096, [128 * 2048 + 1, 5], 16),
    ("topk8-c16", 1024, [128 * 1024, 128 * 513, 9, 0, 128 * 512, 1, 2, 3], 8),
    ("topk4-c8", 1024, [128 * 512, 128 * 257, 9, 0, 128 * 256, 1, 2, 3], 4),
    # The merge is pruned to the 16 lists with the best heads past 8 registers of lists:
    # 128 lists of 4 keys (full network) against 129 (pruned) at C = 4, and 64 lists of 8
    # against 65 and 128 at C = 8.
    ("prune-c4-128-129", 1024, [128 * 512, 128 * 516, 5, 0, 128 * 3 + 7, 1, 2, 3], 16),
    ("prune-c8-64-65", 1024, [128 * 520, 128 * 512, 128 * 1024, 128 * 100 + 3, 0, 1, 2, 3], 16),
]


@pytest.mark.parametrize("name,W,lens,topk", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_split_limit_edges_single_token(msa, name, W, lens, topk):
    inp = synth.paged_case(410, lens, W, poison=False, topk=topk)
    check(msa, inp)


@pytest.mark.parametrize("name,W,lens,topk", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_split_limit_edges_multi_and_fp8(msa, name, W, lens, topk):
    from test_gpu_fp8 import run_fp8
    from test_gpu_multi import run_multi

    assert msa.plan(len(lens), W, topk)["blocks_per_split"] == 0
    run_multi(msa, synth.multi_case(411, lens, W, 4, poison=False, topk=topk))
    run_fp8(msa, synth.fp8_case(412, lens, W, 1, k_scale=0.5, poison=False, topk=topk), 1e-3 * 4.0 * 0.5)


# Several positions per row (the split kernel ranks the positions' keys side by side; the merge
# kernel merges each (row, position, head)): 2 and 3 positions, and FP8 with 2 to 4 positions,
# at the edges above.
@pytest.mark.parametrize("name,Q,fp8", [("c4-256-splits", 2, False), ("c4-256-splits", 3, True),
                                        ("prune-c8-64-65", 3, False), ("prune-c4-128-129", 2, True),
                                        ("c32-64-splits", 4, True), ("topk8-c16", 3, False)])
def test_multi_position_split_limit_edges(msa, name, Q, fp8):
    from test_gpu_fp8 import run_fp8
    from test_gpu_multi import run_multi

    _, W, lens, topk = [c for c in EDGE_CASES if c[0] == name][0]
    assert msa.plan(len(lens), W, topk)["blocks_per_split"] == 0
    if fp8:
        run_fp8(msa, synth.fp8_case(413, lens, W, Q, k_scale=0.5, poison=False, topk=topk), 1e-3 * 4.0 * 0.5)
    else:
        run_multi(msa, synth.multi_case(414, lens, W, Q, poison=False, topk=topk))
