"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the same seeded inputs.

Bars (the tolerance is written here, where it is used):
  * block scores: |fp32 GPU - fp64 oracle| <= 1e-3 absolute. The fp32 sum of 128 exact
    bf16 products in any order is within gamma_127 * sum|q_d k_d| ~ 7.6e-6 * sum|q_d k_d|
    of the exact value; sum|q_d k_d| stays near 80-130 for N(0,1) data, so the worst-case
    bound is below 1e-3 and typical errors are ~1e-5;
  * selected ids: exactly the oracle's selection computed on the GPU's own fp32 scores
    (same precision on both sides), and against the fp64 oracle exact unless the scores
    at the cut lie within 1e-3;
  * the planted workload (integer scores, exact in fp32 in any order): ids and scores
    bit for bit.
"""
import numpy as np
import pytest

import oracle
from sparse_attention_block_amd import synth

from gpu_util import (check_scores, check_selection_exact_given_scores, check_selection_vs_oracle,
                      to_device)

pytestmark = pytest.mark.gpu

CTR = 17 * 256  # workspace counter bytes per row (a row counter and 16 group counters)

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_block_amd as m
    m.load()
    return m


_CACHE = {}


def cfg(i):
    if i not in _CACHE:
        inp = synth.config(i)
        ids, sc, s = oracle.decode(inp)
        _CACHE[i] = (inp, ids, sc, s)
    return _CACHE[i]


ENGINES = [1, 2]  # VALU dot2, MFMA


def feasible(splits, W):
    """Requested split counts, raised where needed so a split holds at most 64 blocks."""
    lo = max(1, -(-W // 64))
    return sorted({0 if s == 0 else max(s, lo) for s in splits})


def run_case(msa, inp, ref_scores, engine_list=ENGINES, splits=(0,)):
    splits = feasible(splits, inp.max_blocks)
    q, k, bt, lens = to_device(inp)
    lens_np = inp.seq_lens
    for engine in engine_list:
        s0 = None
        for ns in splits:
            s = msa.msa_indexer_block_scores(q, k, bt, lens, num_splits=ns, engine=engine).cpu().numpy()
            check_scores(s, ref_scores)
            if s0 is None:
                s0 = s
            else:  # the split count cannot change a score (TensorRT-LLM PR #17008, Accuracy)
                assert np.array_equal(s, s0)
    # The decode pass (default engine) at each split count.
    gpu_s = msa.msa_indexer_block_scores(q, k, bt, lens).cpu().numpy()
    for ns in splits:
        ids, sc = msa.msa_indexer_decode(q, k, bt, lens, inp.topk, inp.n_init, inp.n_local, num_splits=ns)
        ids, sc = ids.cpu().numpy(), sc.cpu().numpy()
        check_selection_exact_given_scores(ids, sc, gpu_s, lens_np, inp.topk, inp.n_init, inp.n_local)
        check_selection_vs_oracle(ids, ref_scores, lens_np, inp.topk, inp.n_init, inp.n_local)
    return ids, sc


@pytest.mark.parametrize("i", [1, 2, 4])
def test_config_parity(msa, i):
    inp, _, _, ref = cfg(i)
    run_case(msa, inp, ref, splits=(0, 1, 3, 64))


def test_config5_planted_bit_exact(msa):
    inp, want_ids, want_sc, ref = cfg(5)
    q, k, bt, lens = to_device(inp)
    for engine in ENGINES:
        s = msa.msa_indexer_block_scores(q, k, bt, lens, engine=engine).cpu().numpy()
        assert np.array_equal(s.astype(np.float64), ref)   # integer scores: exact
    for ns in (0, 2, 4, 5, 17, 34, 68):   # split sizes 34 .. 1 blocks
        for engine in ENGINES:
            ws = msa.new_workspace(inp.batch, inp.max_blocks, 16, ns)
            msa.msa_indexer_split_topk(q, k, bt, lens, ws, 16, 1, 2, num_splits=ns, engine=engine)
            ids = torch.empty((inp.batch, 4, 16), dtype=torch.int32, device="cuda")
            sc = torch.empty((inp.batch, 4, 16), dtype=torch.float32, device="cuda")
            msa.msa_indexer_merge(lens, inp.max_blocks, ws, ids, sc, 16, num_splits=ns)
            assert np.array_equal(ids.cpu().numpy(), want_ids), (ns, engine)
            assert np.array_equal(sc.cpu().numpy().astype(np.float64), want_sc), (ns, engine)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_config3_full_size(msa):
    # The benchmark's workload at full size, decoded in the benchmark's launch configuration.
    inp, _, _, ref = cfg(3)
    ids, _ = run_case(msa, inp, ref, splits=(0,))
    # Heads must disagree (a merge that mixed heads would not), vLLM PR #57832, Test Plan.
    differ = [len({tuple(sorted(ids[b, h])) for h in range(4)}) == 4 for b in range(inp.batch)]
    assert np.mean(differ) >= 0.9


@pytest.mark.parametrize("seed,lens,W", [
    (101, [128 * 7 + 5, 1, 0, 128, 129, 128 * 40 - 1], 40),
    (102, [128 * 300 + 77] * 3, 301),
    (103, [5, 17, 127, 128, 255, 256, 1000, 2000], 16),
    (104, list(range(0, 128 * 70, 128 * 7 + 13)), 70),
])
def test_ragged_paged_cases(msa, seed, lens, W):
    inp = synth.paged_case(seed, lens, W)
    ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, inp.seq_lens)
    run_case(msa, inp, ref, splits=(0, 1, 2, 7, W))


@pytest.mark.parametrize("topk,n_init,n_local", [(1, 0, 0), (1, 1, 0), (4, 2, 2), (16, 0, 0),
                                                 (16, 0, 1), (64, 1, 2), (37, 5, 9)])
def test_selection_parameters(msa, topk, n_init, n_local):
    inp = synth.paged_case(105, [128 * 90 + 3, 128 * 20, 128 * 3, 1], 91, topk=topk,
                           n_init=n_init, n_local=n_local)
    ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, inp.seq_lens)
    run_case(msa, inp, ref, engine_list=[], splits=(0, 5))


def test_grid_bound_invariance(msa):
    # Scores and picks do not depend on how large the grid is sized (vLLM PR #57832, CUDA
    # graph capture: a grid for the batch and one for a bound 8x larger give equal scores).
    inp = synth.paged_case(106, [128 * 33 + 9, 128 * 12, 700], 34)
    q, k, bt, lens = to_device(inp)
    _, k8, bt8, _ = to_device(inp, extra_cols=34 * 7)
    a = msa.msa_indexer_block_scores(q, k, bt, lens).cpu().numpy()
    b = msa.msa_indexer_block_scores(q, k8, bt8, lens).cpu().numpy()
    assert np.array_equal(a, b[:, :, :34]) and np.all(np.isneginf(b[:, :, 34:]))
    ia, sa = msa.msa_indexer_decode(q, k, bt, lens)
    ib, sb = msa.msa_indexer_decode(q, k8, bt8, lens)
    assert torch.equal(ia, ib) and torch.equal(sa, sb)


def test_edges(msa):
    # Empty rows, seq_len past the table width (clamped), a table wider than used.
    inp = synth.paged_case(107, [0, 0, 128 * 5, 3], 5)
    q, k, bt, lens = to_device(inp)
    lens_big = lens.clone()
    lens_big[2] = 10 ** 7
    ids, sc = msa.msa_indexer_decode(q, k, bt, lens)
    ids2, sc2 = msa.msa_indexer_decode(q, k, bt, lens_big)
    assert torch.equal(ids, ids2) and torch.equal(sc, sc2)
    ids, sc = ids.cpu().numpy(), sc.cpu().numpy()
    assert np.all(ids[:2] == -1) and np.all(np.isneginf(sc[:2]))
    assert np.all(ids[3, :, 0] == 0) and np.all(ids[3, :, 1:] == -1)
    # All rows empty, and a zero-width table.
    zero = torch.zeros_like(lens)
    ids, sc = msa.msa_indexer_decode(q, k, bt, zero)
    assert torch.all(ids == -1) and torch.all(torch.isneginf(sc))
    bt0 = torch.zeros((4, 0), dtype=torch.int32, device="cuda")
    ids, _ = msa.msa_indexer_decode(q, k, bt0, lens)
    assert torch.all(ids == -1)
    # batch 0 is a no-op.
    ids, _ = msa.msa_indexer_decode(q[:0], k, bt[:0], lens[:0])
    assert ids.shape == (0, 4, 16)


def test_shared_pages_break_ties_by_id(msa):
    # Logical blocks backed by one physical page (prefix sharing) score bit for bit alike
    # whichever split, wave or engine reads them, and equal scores go to the lower block id.
    inp = synth.paged_case(112, [128 * 40, 128 * 40, 128 * 37 + 9], 40, poison=False)
    bt = inp.block_table.copy()
    bt[0, :] = bt[0, 0]
    bt[1, :] = bt[1, np.arange(40) % 10]
    bt[2, :20] = bt[1, :20]  # row 2 reads row 1's first 20 pages (with its own query)
    shared = synth.Inputs("shared pages", inp.q, inp.k_cache, bt, inp.seq_lens)
    ref = oracle.block_scores(shared.q, shared.k_cache, shared.block_table, shared.seq_lens)
    q, k, btd, lens = to_device(shared)
    for ns in feasible((0, 3, 10), 40):
        for engine in ENGINES:
            s = msa.msa_indexer_block_scores(q, k, btd, lens, num_splits=ns, engine=engine).cpu().numpy()
            check_scores(s, ref)
            assert np.all(s[0] == s[0, :, :1])
            assert np.array_equal(s[1], s[1][:, np.arange(40) % 10])
        ids, sc = msa.msa_indexer_decode(q, k, btd, lens, num_splits=ns)
        ids, sc = ids.cpu().numpy(), sc.cpu().numpy()
        for h in range(4):
            assert list(ids[0, h]) == [0, 38, 39] + list(range(1, 14)), (ns, h)
        s = msa.msa_indexer_block_scores(q, k, btd, lens, num_splits=ns).cpu().numpy()  # decode's engine
        check_selection_exact_given_scores(ids, sc, s, shared.seq_lens, 16, 1, 2)
        check_selection_vs_oracle(ids, ref, shared.seq_lens, 16, 1, 2)


def test_out_of_range_page_is_flagged_not_read(msa):
    inp = synth.paged_case(108, [128 * 6, 128 * 6], 6)
    q, k, bt, lens = to_device(inp)
    ws = msa.new_workspace(2, 6, 16)
    ids, _ = msa.msa_indexer_decode(q, k, bt, lens, workspace=ws)
    assert msa.msa_indexer_read_error(ws) == 0
    bad = bt.clone()
    bad[1, 3] = inp.num_pages          # one past the last page
    bad[1, 4] = -5
    ids_bad, sc_bad = msa.msa_indexer_decode(q, k, bad, lens, workspace=ws)
    assert msa.msa_indexer_read_error(ws) == 1
    assert msa.msa_indexer_read_error(ws) == 0  # cleared by the read
    s = msa.msa_indexer_block_scores(q, k, bad, lens).cpu().numpy()
    assert np.all(np.isneginf(s[1, :, 3:5]))
    assert torch.equal(ids_bad[0], ids[0])


def test_graph_replay_with_changing_lengths(msa):
    # Capture once, then change seq_lens and the block table on the device between
    # replays (SGLang PR #41488, Accuracy Tests: changed lengths after capture).
    big = synth.paged_case(109, [128 * 64] * 4, 64)
    q, k, bt, lens = to_device(big)
    ws = msa.new_workspace(4, 64, 16)
    ids = torch.empty((4, 4, 16), dtype=torch.int32, device="cuda")
    sc = torch.empty((4, 4, 16), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        msa.msa_indexer_decode(q, k, bt, lens, out_ids=ids, out_scores=sc, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        msa.msa_indexer_decode(q, k, bt, lens, out_ids=ids, out_scores=sc, workspace=ws)
    rng = np.random.default_rng(0)
    for rep in range(6):
        new_lens = rng.integers(0, 128 * 64 + 1, size=4).astype(np.int32)
        if rep == 0:
            new_lens[:] = [0, 1, 129, 128 * 64]
        perm = rng.permutation(big.num_pages).astype(np.int32)[: 4 * 64].reshape(4, 64)
        lens.copy_(torch.from_numpy(new_lens))
        bt.copy_(torch.from_numpy(perm))
        g.replay()
        torch.cuda.synchronize()
        got_ids, got_sc = ids.clone(), sc.clone()
        eager_ids, eager_sc = msa.msa_indexer_decode(q, k, bt, lens)
        assert torch.equal(got_ids, eager_ids) and torch.equal(got_sc, eager_sc), rep
        cur = synth.Inputs("replay", big.q, big.k_cache, perm, new_lens)
        ref = oracle.block_scores(cur.q, cur.k_cache, cur.block_table, cur.seq_lens)
        check_selection_vs_oracle(got_ids.cpu().numpy(), ref, new_lens, 16, 1, 2)


def test_unfused_plan_parity(msa):
    # Long rows at batch 2 in a table wider than the device plan's 4096 blocks: about 240
    # splits x 16 candidates per head do not fit the fused merge, so decode runs stage 1
    # and the separate merge kernel.
    lens = [128 * 3000 + 65, 128 * 4097]
    assert not msa.plan(2, 4097, 16)["fused"]
    inp = synth.paged_case(110, lens, 4097)
    ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, inp.seq_lens)
    run_case(msa, inp, ref, engine_list=[1], splits=(0,))


def test_pruned_merge_host_plans(msa):
    # Host plans whose lists go to the merge kernel: 128 lists of 4 keys (full network), 129
    # (pruned to the 16 lists with the best heads), 172 lists of 3 keys padded to 4, and 104
    # lists of 5 padded to 8 (pruned).
    for W, lens, cases in ((512, [128 * 512, 128 * 511 + 9, 128 * 300, 1], ((128, 4),)),
                           (516, [128 * 516, 128 * 515 + 9, 128 * 300, 1], ((129, 4), (172, 3), (128, 5)))):
        inp = synth.paged_case(113, lens, W)
        for ns, C in cases:
            assert msa.plan(4, W, 16, ns)["blocks_per_split"] == C
        ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, inp.seq_lens)
        run_case(msa, inp, ref, engine_list=[1], splits=tuple(ns for ns, _ in cases))
    # Smaller topk through the pruned path (the first m of its top 16): 256 splits of 4
    # blocks (automatic, or asked for) and 128 of 8; the short row fits one split.
    for topk, n_init, n_local in ((8, 1, 2), (3, 0, 1)):
        inp = synth.paged_case(116, [128 * 1024, 128 * 700 + 1, 5], 1024, topk=topk, n_init=n_init,
                               n_local=n_local)
        assert msa.plan(3, 1024, topk, 256)["blocks_per_split"] == 4
        ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, inp.seq_lens)
        run_case(msa, inp, ref, engine_list=[1], splits=(0, 129, 256))

@pytest.mark.parametrize("topk,n_init,n_local", [(16, 1, 2), (2, 1, 1), (3, 0, 0)])
def test_single_split_rows(msa, topk, n_init, n_local):
    # Every row fits one split (one split of the table's 4 blocks asked for; the FP8 call's
    # host plan takes 4-block splits by itself), so each workgroup writes its row's selection
    # and page table directly, without publishing its lists: the decode, page-table and FP8
    # calls against the oracle, with empty, partial and full rows, and fewer blocks than topk
    # as well as more. The automatic single-token plan of this small table (single-block
    # splits, spread layout) is checked too.
    from test_gpu_fp8 import run_fp8
    lens = [0, 1, 127, 128, 129, 300, 511, 512, 64, 256 + 3, 1, 0]
    inp = synth.paged_case(114, lens, 4, topk=topk, n_init=n_init, n_local=n_local)
    assert msa.plan(len(lens), 4, topk, 1)["blocks_per_split"] == 4
    assert msa.plan(len(lens), 4, topk)["blocks_per_split"] == 1
    ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, inp.seq_lens)
    ids, sc = run_case(msa, inp, ref, engine_list=[1], splits=(0, 1))
    q, k, bt, dl = to_device(inp)
    ids_p, sc_p, pages, tokens = msa.msa_indexer_decode_pages(q, k, bt, dl, topk, n_init, n_local,
                                                              num_splits=1)
    assert np.array_equal(ids_p.cpu().numpy(), ids) and np.array_equal(sc_p.cpu().numpy(), sc)
    want_p, want_t = oracle.expand_pages(ids, inp.block_table, inp.seq_lens)
    assert np.array_equal(pages.cpu().numpy(), want_p) and np.array_equal(tokens.cpu().numpy(), want_t)
    run_fp8(msa, synth.fp8_case(115, lens, 4, 1, k_scale=0.5, topk=topk, n_init=n_init, n_local=n_local),
            1e-3 * 4.0 * 0.5)


@pytest.mark.parametrize("B,W,seed", [(8, 150, 171), (16, 68, 172), (4, 300, 173), (64, 17, 174)])
def test_even_splits(msa, B, W, seed):
    # Tables whose 4-block splits would just exceed one workgroup per CU take 256 / B even
    # splits of 4 or 5 blocks (the spread layout, the first four blocks in flight and the fifth
    # after): full rows, empty and one-token rows, partial last blocks and rows that end inside
    # any split, against the oracle, and the same ids as an explicit 4-block plan.
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 128 * W + 1, size=B).astype(np.int32)
    lens[0], lens[1 % B] = 128 * W, 0
    if B > 2:
        lens[2] = 1
    inp = synth.paged_case(seed, lens.tolist(), W)
    p = msa.plan(B, W, 16)
    assert p["splits"] == 256 // B and p["blocks_per_split"] == -(-W // (256 // B))
    ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, inp.seq_lens)
    ids, _ = run_case(msa, inp, ref, engine_list=[1], splits=(0,))
    q, k, bt, dl = to_device(inp)
    ids4, _ = msa.msa_indexer_decode(q, k, bt, dl, num_splits=-(-W // 4))
    assert np.array_equal(ids, ids4.cpu().numpy())


def test_workspace_reuse_and_counter_reset(msa):
    # One workspace across calls with changing lengths and split counts: the per-row
    # counters must come back to zero after every fused call.
    inp = synth.paged_case(111, [128 * 200] * 6, 200)
    q, k, bt, lens = to_device(inp)
    plans = [0, 4, 13, 50, 200, 7, 0, 25]
    size = max(msa.workspace_bytes(6, 200, 16, ns) for ns in plans)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(1)
    for it, ns in enumerate(plans):
        new_lens = rng.integers(0, 128 * 200 + 1, size=6).astype(np.int32)
        new_lens[it % 6] = 0
        lens.copy_(torch.from_numpy(new_lens))
        ids, sc = msa.msa_indexer_decode(q, k, bt, lens, num_splits=ns, workspace=ws)
        torch.cuda.synchronize()
        # error word in the 256-byte header, then 17 256-byte counter lines per row
        header = ws[:256].view(torch.int32).cpu().numpy()
        counters = ws[256:256 + 6 * CTR].view(torch.int32).cpu().numpy().reshape(6, 17, 64)
        assert np.all(header == 0), (it, header[:4])
        assert np.all(counters == 0), (it, counters[:, :, 0])
        cur = synth.Inputs("reuse", inp.q, inp.k_cache, inp.block_table, new_lens)
        ref = oracle.block_scores(cur.q, cur.k_cache, cur.block_table, cur.seq_lens)
        gpu_s = msa.msa_indexer_block_scores(q, k, bt, lens).cpu().numpy()
        check_selection_exact_given_scores(ids.cpu().numpy(), sc.cpu().numpy(), gpu_s, new_lens, 16, 1, 2)
        check_selection_vs_oracle(ids.cpu().numpy(), ref, new_lens, 16, 1, 2)


def test_default_workspace_is_reused(msa):
    # Calls that pass no workspace share one per (device, stream); the library leaves its
    # counters at zero, so repeated calls with changing lengths stay exact.
    from sparse_attention_block_amd import _lib
    inp = synth.paged_case(112, [128 * 40] * 5, 40)
    q, k, bt, lens = to_device(inp)
    rng = np.random.default_rng(2)
    before = len(_lib._WS_CACHE)
    for it in range(4):
        new_lens = rng.integers(0, 128 * 40 + 1, size=5).astype(np.int32)
        lens.copy_(torch.from_numpy(new_lens))
        ids, sc = msa.msa_indexer_decode(q, k, bt, lens)
        gpu_s = msa.msa_indexer_block_scores(q, k, bt, lens).cpu().numpy()
        check_selection_exact_given_scores(ids.cpu().numpy(), sc.cpu().numpy(), gpu_s, new_lens, 16, 1, 2)
    assert len(_lib._WS_CACHE) <= before + 1
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        ids2, sc2 = msa.msa_indexer_decode(q, k, bt, lens)
    torch.cuda.synchronize()
    assert torch.equal(ids2, ids) and torch.equal(sc2, sc)
    for ws, rows, _ in _lib._WS_CACHE.values():  # every cached counter line is zero
        assert int(ws[256:256 + CTR * rows].view(torch.int32).abs().sum()) == 0


def test_decode_engines_agree_on_exact_data(msa):
    # Both engines through the whole pass on the planted workload: bit-exact ids and scores.
    inp, want_ids, want_sc, _ = cfg(5)
    q, k, bt, lens = to_device(inp)
    for engine in ENGINES:
        ids, sc = msa.msa_indexer_decode(q, k, bt, lens, engine=engine)
        assert np.array_equal(ids.cpu().numpy(), want_ids)
        assert np.array_equal(sc.cpu().numpy().astype(np.float64), want_sc)


@pytest.mark.parametrize("B", [1, 2, 4, 8, 15, 16, 32])
def test_split_width_sweep(msa, B):
    # The grid of TensorRT-LLM PR #17008 (Accuracy): scores identical at every split width
    # and the selected blocks identical, over batch x context length, with consecutive
    # decode lengths (8700 and 8701) in the grid.
    for kv in (256, 1000, 4096, 8700, 8701, 16384):
        nbk = -(-kv // 128)
        inp = synth.paged_case(1000 + B * 31 + kv, [kv] * B, nbk, poison=False, permute=True)
        q, k, bt, lens = to_device(inp)
        ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, inp.seq_lens)
        base_s, base_ids = None, None
        for ns in sorted({0, 1, 2, 3, 4, 7, nbk // 2, nbk}):
            try:
                msa.plan(B, nbk, 16, ns)
            except msa.MsaError:  # more than 64 blocks per split: refused by design
                continue
            s = msa.msa_indexer_block_scores(q, k, bt, lens, num_splits=ns).cpu().numpy()
            ids, sc = msa.msa_indexer_decode(q, k, bt, lens, num_splits=ns)
            ids, sc = ids.cpu().numpy(), sc.cpu().numpy()
            if base_s is None:
                base_s, base_ids = s, ids
                check_scores(s, ref)
                check_selection_exact_given_scores(ids, sc, s, inp.seq_lens, 16, 1, 2)
                check_selection_vs_oracle(ids, ref, inp.seq_lens, 16, 1, 2)
            assert np.array_equal(s, base_s), (B, kv, ns)
            assert np.array_equal(ids, base_ids), (B, kv, ns)


def test_heads_disagree_cfg2(msa):
    inp, _, _, _ = cfg(2)
    q, k, bt, lens = to_device(inp)
    ids, _ = msa.msa_indexer_decode(q, k, bt, lens)
    ids = ids.cpu().numpy()
    differ = [len({tuple(sorted(ids[b, h])) for h in range(4)}) == 4 for b in range(inp.batch)]
    assert np.mean(differ) >= 0.9
