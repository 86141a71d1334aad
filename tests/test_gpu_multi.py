"""GPU parity of the multi-token (draft verify) decode against the CPU oracle.

Bars, as in the single-token tests:
  * block scores of every (row, position, head): |fp32 GPU - fp64 oracle| <= 1e-3, same -inf
    pattern (a position's causal end decides which blocks it sees), bitwise equal across split
    counts; with one position they are bit-identical to the single-token MFMA engine (same
    instruction, same operand rows);
  * selections: exactly the oracle's selection on the GPU's own fp32 scores, and against the
    fp64 oracle exact unless the scores at the cut lie within 1e-3;
  * the planted workload (integer scores): ids and scores bit for bit.
"""
import numpy as np
import pytest

import oracle
from sparse_attention_block_amd import synth

from gpu_util import check_scores, check_selection_vs_oracle, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_block_amd as m
    m.load()
    return m


def to_device_multi(inp):
    """(q [B, Q, 4, 128], k_cache, block_table, seq_lens) device tensors."""
    q = torch.from_numpy(np.ascontiguousarray(inp.q).view(np.int16)).to("cuda").view(torch.bfloat16)
    k = torch.from_numpy(inp.k_cache.view(np.int16)).to("cuda").view(torch.bfloat16)
    bt = torch.from_numpy(np.ascontiguousarray(inp.block_table)).to("cuda")
    lens = torch.from_numpy(np.ascontiguousarray(inp.seq_lens)).to("cuda")
    return q, k, bt, lens


def position_lens(inp, p):
    Q = inp.qlen
    L = np.clip(inp.seq_lens.astype(np.int64), 0, inp.max_blocks * 128)
    return np.maximum(L - (Q - 1 - p), 0).astype(np.int32)


def feasible(splits, W):
    lo = max(1, -(-W // 64))
    return sorted({0 if s == 0 else max(s, lo) for s in splits})


def run_multi(msa, inp, splits=(0,)):
    """Scores and selections of the multi-token pass against the oracle; returns the last
    split count's (ids, scores)."""
    q, k, bt, lens = to_device_multi(inp)
    want_ids, want_sc, ref = oracle.decode(inp)
    s0 = None
    for ns in feasible(splits, inp.max_blocks):
        s = msa.msa_indexer_block_scores_multi(q, k, bt, lens, num_splits=ns).cpu().numpy()
        check_scores(s, ref)
        if s0 is None:
            s0 = s
        else:
            assert np.array_equal(s, s0)
    for ns in feasible(splits, inp.max_blocks):
        ids, sc = msa.msa_indexer_decode_multi(q, k, bt, lens, inp.topk, inp.n_init, inp.n_local,
                                               num_splits=ns)
        ids, sc = ids.cpu().numpy(), sc.cpu().numpy()
        for p in range(inp.qlen):
            lp = position_lens(inp, p)
            gi, gs = oracle.select(s0[:, p].astype(np.float64), lp, inp.topk, inp.n_init, inp.n_local)
            assert np.array_equal(ids[:, p], gi), (ns, p)
            sel = gi >= 0
            assert np.array_equal(sc[:, p][sel].astype(np.float64), gs[sel])
            assert np.all(np.isneginf(sc[:, p][~sel]))
            check_selection_vs_oracle(ids[:, p], ref[:, p], lp, inp.topk, inp.n_init, inp.n_local)
    return ids, sc


@pytest.mark.parametrize("seed,lens,W,Q", [
    (201, [300, 128, 1, 0, 1000, 257, 3, 129, 130], 8, 4),
    (202, [128 * 5, 77, 2], 5, 3),
    (203, [4000, 3000, 129, 4], 32, 2),
    (204, [128 * 300 + 2, 128 * 300 + 3, 128 * 64, 700], 301, 4),
    (205, [5, 17, 127, 128, 255, 256, 1000, 2000], 16, 1),
])
def test_multi_ragged(msa, seed, lens, W, Q):
    inp = synth.multi_case(seed, lens, W, Q)
    run_multi(msa, inp, splits=(0, 1, 3, W))


def test_multi_one_position_matches_single_token_mfma(msa):
    inp = synth.paged_case(206, [128 * 40 + 9, 128 * 7, 300, 0], 41)
    q, k, bt, lens = to_device(inp)
    single = msa.msa_indexer_block_scores(q, k, bt, lens, engine=2)
    multi = msa.msa_indexer_block_scores_multi(q[:, None].contiguous(), k, bt, lens)
    assert torch.equal(single, multi[:, 0])


@pytest.mark.parametrize("Q", [1, 2, 3, 4])
def test_multi_planted_bit_exact(msa, Q):
    inp = synth.multi_planted(Q)
    want_ids, want_sc, ref = oracle.decode(inp)
    q, k, bt, lens = to_device_multi(inp)
    s = msa.msa_indexer_block_scores_multi(q, k, bt, lens).cpu().numpy()
    assert np.array_equal(s.astype(np.float64), ref)
    for ns in (0, 2, 5, 17, 34, 68):
        ids, sc = msa.msa_indexer_decode_multi(q, k, bt, lens, num_splits=ns)
        assert np.array_equal(ids.cpu().numpy(), want_ids), ns
        assert np.array_equal(sc.cpu().numpy().astype(np.float64), want_sc), ns


@pytest.mark.parametrize("topk,n_init,n_local", [(1, 0, 1), (5, 2, 2), (16, 0, 0), (64, 3, 5),
                                                 (37, 5, 9)])
def test_multi_selection_parameters(msa, topk, n_init, n_local):
    inp = synth.multi_case(207, [128 * 90 + 3, 128 * 20, 128 * 3, 1, 2], 91, 4, topk=topk,
                           n_init=n_init, n_local=n_local)
    run_multi(msa, inp, splits=(0, 5))


def test_multi_edges(msa):
    inp = synth.multi_case(208, [0, 0, 128 * 5, 3], 5, 4)
    q, k, bt, lens = to_device_multi(inp)
    ids, sc = msa.msa_indexer_decode_multi(q, k, bt, lens)
    # lengths past the table width are clamped to it before the causal clamp
    lens_big = lens.clone()
    lens_big[2] = 10 ** 7
    ids2, sc2 = msa.msa_indexer_decode_multi(q, k, bt, lens_big)
    assert torch.equal(ids, ids2) and torch.equal(sc, sc2)
    ids, sc = ids.cpu().numpy(), sc.cpu().numpy()
    assert np.all(ids[:2] == -1) and np.all(np.isneginf(sc[:2]))
    # 3 tokens, 4 positions: position 0 sees nothing, positions 1..3 see block 0
    assert np.all(ids[3, 0] == -1)
    assert np.all(ids[3, 1:, :, 0] == 0) and np.all(ids[3, 1:, :, 1:] == -1)
    # all rows empty; a zero-width table; batch 0
    zero = torch.zeros_like(lens)
    ids, sc = msa.msa_indexer_decode_multi(q, k, bt, zero)
    assert torch.all(ids == -1) and torch.all(torch.isneginf(sc))
    bt0 = torch.zeros((4, 0), dtype=torch.int32, device="cuda")
    ids, _ = msa.msa_indexer_decode_multi(q, k, bt0, lens)
    assert torch.all(ids == -1)
    ids, _ = msa.msa_indexer_decode_multi(q[:0], k, bt[:0], lens[:0])
    assert ids.shape == (0, 4, 4, 16)


def test_multi_out_of_range_page_is_flagged_not_read(msa):
    inp = synth.multi_case(209, [128 * 6, 128 * 6], 6, 4)
    q, k, bt, lens = to_device_multi(inp)
    ws = torch.zeros(msa.workspace_bytes_multi(2, 6, 4, 16), dtype=torch.uint8, device="cuda")
    ids, _ = msa.msa_indexer_decode_multi(q, k, bt, lens, workspace=ws)
    assert msa.msa_indexer_read_error(ws) == 0
    bad = bt.clone()
    bad[1, 3] = inp.num_pages              # one past the last page
    bad[1, 4] = -5
    ids_bad, _ = msa.msa_indexer_decode_multi(q, k, bad, lens, workspace=ws)
    assert msa.msa_indexer_read_error(ws) == 1
    assert msa.msa_indexer_read_error(ws) == 0
    s = msa.msa_indexer_block_scores_multi(q, k, bad, lens).cpu().numpy()
    assert np.all(np.isneginf(s[1, :, :, 3:5]))      # every position, every head
    assert torch.equal(ids_bad[0], ids[0])


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_multi_full_size(msa):
    # The benchmark cache (batch 32 x 131072 tokens) with 4 draft positions per row.
    inp = synth.multi_config(4)
    ids, _ = run_multi(msa, inp)
    differ = [len({tuple(sorted(ids[b, 3, h])) for h in range(4)}) == 4 for b in range(inp.batch)]
    assert np.mean(differ) >= 0.9


@pytest.mark.parametrize("Q", [1, 4])
def test_multi_workspace_reuse_and_graph_replay(msa, Q):
    # With one position the pass merges in the same launch: each row's last split, found by
    # counting finished splits in the workspace, merges and resets the count. One workspace
    # must serve changing lengths (rows of length 0 included) and split counts, and a
    # captured graph must give the same result on every replay.
    inp = synth.multi_case(210, [128 * 40] * 5, 40, Q)
    q, k, bt, lens = to_device_multi(inp)
    plans = [0, 4, 13, 2, 40, 0]
    ws = torch.zeros(max(msa.workspace_bytes_multi(5, 40, Q, 16, ns) for ns in plans),
                     dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(3)
    for it, ns in enumerate(plans):
        new_lens = rng.integers(0, 128 * 40 + 1, size=5).astype(np.int32)
        new_lens[it % 5] = 0
        lens.copy_(torch.from_numpy(new_lens))
        ids, sc = msa.msa_indexer_decode_multi(q, k, bt, lens, num_splits=ns, workspace=ws)
        torch.cuda.synchronize()
        assert np.all(ws[:256 + 5 * 17 * 256].view(torch.int32).cpu().numpy() == 0), it  # header, 17 counter lines per row
        cur = synth.Inputs("reuse", inp.q, inp.k_cache, inp.block_table, new_lens)
        want_ids, _, ref = oracle.decode(cur)
        for p in range(Q):
            check_selection_vs_oracle(ids.cpu().numpy()[:, p], ref[:, p], position_lens(cur, p),
                                      16, 1, 2)
    # graph capture, then replays with lengths changed on the device in between
    ids = torch.empty((5, Q, 4, 16), dtype=torch.int32, device="cuda")
    sc = torch.empty((5, Q, 4, 16), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        msa.msa_indexer_decode_multi(q, k, bt, lens, out_ids=ids, out_scores=sc, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        msa.msa_indexer_decode_multi(q, k, bt, lens, out_ids=ids, out_scores=sc, workspace=ws)
    for it in range(4):
        new_lens = rng.integers(1, 128 * 40 + 1, size=5).astype(np.int32)
        lens.copy_(torch.from_numpy(new_lens))
        g.replay()
        torch.cuda.synchronize()
        eager_ids, eager_sc = msa.msa_indexer_decode_multi(q, k, bt, lens)
        assert torch.equal(ids, eager_ids) and torch.equal(sc, eager_sc), it


@pytest.mark.parametrize("Q", [2, 4])
def test_merge_kernel_full_row_guess(msa, Q):
    # The merge kernel reads a task's lists for a full row under the full-row plan before the row
    # lengths arrive, and keeps that read only when the row takes that plan. Host plan (4 rows of
    # 100 blocks, splits of 4): full rows (kept), a row ending inside its last split (kept, fewer
    # blocks than the table), rows of half the table (read again). Device plan (64 rows of 128
    # blocks): every row full (kept), then rows of mixed lengths (a general plan).
    W = 100
    for lens in ([128 * W] * 4, [128 * 98 + 5, 128 * W, 128 * 97 + 1, 128 * W], [128 * 50, 128 * 49 + 3, 128 * W, 0]):
        run_multi(msa, synth.multi_case(230 + Q, lens, W, Q, poison=False))
    W = 128
    rng = np.random.default_rng(231 + Q)
    mixed = rng.integers(0, 128 * W + 1, size=64)
    for lens in ([128 * W] * 64, mixed.tolist()):
        run_multi(msa, synth.multi_case(232 + Q, lens, W, Q, poison=False))
    from test_gpu_fp8 import run_fp8
    run_fp8(msa, synth.fp8_case(234 + Q, [128 * W] * 64, W, Q, k_scale=0.5, poison=False), 1e-3 * 4.0 * 0.5)
