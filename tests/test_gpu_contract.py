"""GPU tests at the edges of the C ABI's declared contract.

- One workspace shared, without clearing it again, by calls whose batch grows and shrinks
  (the persistent, allocation-free buffers of vLLM PR #57832, CUDA graph capture): row
  counters sit at fixed offsets and a call's keys at the buffer's end, so no call can leave
  stale counts for another.
- Negative seq_lens entries, which every decode call clamps to an empty row.
- The widest table the library takes (MSA_MAX_BLOCKS_PER_SEQ = 16384 blocks: a 2M-token row,
  512 MiB of bf16 index-K), through the decode call and the page-table call.

Bars as in test_gpu_parity.py: scores within 1e-3 of the fp64 oracle; ids equal to the oracle's
selection on the GPU's own fp32 scores and within the near-tie rule against fp64; page tables
bit for bit.
"""
import numpy as np
import pytest

import oracle
from sparse_attention_block_amd import synth

from gpu_util import check_scores, check_selection_exact_given_scores, check_selection_vs_oracle, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

HDR = 256
CTR = 17 * 256  # counter bytes per row


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_block_amd as m
    m.load()
    return m


def _check_single(msa, inp, rows, lens_np, ids, sc, q, k, bt, lens):
    cur = synth.Inputs("slice", inp.q[rows], inp.k_cache, inp.block_table[rows], lens_np)
    gpu_s = msa.msa_indexer_block_scores(q, k, bt, lens).cpu().numpy()
    ref = oracle.block_scores(cur.q, cur.k_cache, cur.block_table, cur.seq_lens)
    check_scores(gpu_s, ref)
    check_selection_exact_given_scores(ids, sc, gpu_s, lens_np, 16, 1, 2)
    check_selection_vs_oracle(ids, ref, lens_np, 16, 1, 2)


def test_workspace_shared_across_batch_sizes(msa):
    # Batch 4 -> 8 -> 2 -> 8 -> 3 on one buffer sized for batch 8, zeroed once. W = 1100 blocks:
    # batch 8 runs the device plan (8 x 1100 >= 8192 blocks), the smaller batches host plans,
    # so the calls' key regions differ as well as their counter lines.
    W = 1100
    rng = np.random.default_rng(41)
    full = rng.integers(1, 128 * W + 1, size=8).astype(np.int32)
    full[2] = 128 * W
    inp = synth.paged_case(141, full, W)
    q, k, bt, lens = to_device(inp)
    size = msa.workspace_bytes(8, W, 16)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    plans = []
    for it, (lo, hi) in enumerate([(0, 4), (0, 8), (4, 6), (0, 8), (5, 8)]):
        B = hi - lo
        new = rng.integers(0, 128 * W + 1, size=B).astype(np.int32)
        new = np.minimum(new, full[lo:hi])  # stay within each row's pages
        new[it % B] = full[lo + it % B]
        rl = torch.from_numpy(new).cuda()
        ids, sc = msa.msa_indexer_decode(q[lo:hi], k, bt[lo:hi], rl, workspace=ws)
        torch.cuda.synchronize()
        plans.append(msa.plan(B, W, 16)["blocks_per_split"])
        counters = ws[HDR:HDR + 8 * CTR].view(torch.int32)
        assert int(counters.abs().sum()) == 0, it  # every row's counters back at zero
        assert int(ws[:HDR].view(torch.int32).abs().sum()) == 0, it
        _check_single(msa, inp, slice(lo, hi), new, ids.cpu().numpy(), sc.cpu().numpy(),
                      q[lo:hi], k, bt[lo:hi], rl)
    assert 0 in plans and any(p > 0 for p in plans)  # device and host plans both ran


def test_workspace_shared_by_single_and_multi_token_calls(msa):
    # The general rule: a buffer that holds the largest batch's counter lines plus the largest
    # key region serves calls of different kinds and widths, in any order.
    W1, W2 = 300, 40
    inp1 = synth.paged_case(142, [128 * W1 - 3, 128 * 100, 5, 128 * W1, 0, 128 * 17 + 1], W1)
    inp2 = synth.multi_case(143, [128 * W2, 128 * 3 + 2, 7, 128 * W2 - 60], W2, 4)
    k1 = lambda B, W: msa.workspace_bytes(B, W, 16) - HDR - CTR * B
    k2 = lambda B, W: msa.workspace_bytes_multi(B, W, 4, 16) - HDR - CTR * B
    size = HDR + CTR * 6 + max(k1(6, W1), k2(4, W2), k1(2, W1))
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    q1, kc1, bt1, l1 = to_device(inp1)
    q2, kc2, bt2, l2 = to_device(inp2)
    s2 = msa.msa_indexer_block_scores_multi(q2, kc2, bt2, l2).cpu().numpy()
    for it in range(3):
        ids, sc = msa.msa_indexer_decode(q1, kc1, bt1, l1, workspace=ws)
        _check_single(msa, inp1, slice(0, 6), inp1.seq_lens, ids.cpu().numpy(), sc.cpu().numpy(),
                      q1, kc1, bt1, l1)
        ids2, sc2 = msa.msa_indexer_decode_multi(q2, kc2, bt2, l2, workspace=ws)
        got = ids2.cpu().numpy()
        for p in range(4):  # each position: the oracle's selection on the GPU's own scores
            sel, _ = oracle.select(s2[:, p].astype(np.float64),
                                   np.maximum(inp2.seq_lens - (3 - p), 0), 16, 1, 2)
            assert np.array_equal(got[:, p], sel), (it, p)
        idsb, _ = msa.msa_indexer_decode(q1[4:6], kc1, bt1[4:6], l1[4:6], workspace=ws)
        assert torch.equal(idsb, ids[4:6]), it
        torch.cuda.synchronize()
        assert int(ws[HDR:HDR + 6 * CTR].view(torch.int32).abs().sum()) == 0, it


def test_negative_seq_lens_are_empty_rows(msa):
    # seq_lens entries below zero clamp to 0 in every decode call: ids -1, scores -inf, an empty
    # page table; the other rows are unaffected.
    lens_np = np.array([128 * 29 + 9, 128 * 12, 77, 128 * 30], np.int32)
    inp = synth.paged_case(144, lens_np, 30)
    q, k, bt, lens = to_device(inp)
    neg = lens.clone()
    neg[1] = -5
    neg[3] = -(2 ** 31)
    zeroed = lens.clone()
    zeroed[1] = 0
    zeroed[3] = 0
    ref_ids, ref_sc = msa.msa_indexer_decode(q, k, bt, zeroed)
    ids, sc = msa.msa_indexer_decode(q, k, bt, neg)
    assert torch.equal(ids, ref_ids) and torch.equal(sc, ref_sc)
    idsn = ids.cpu().numpy()
    assert np.all(idsn[[1, 3]] == -1) and np.all(np.isneginf(sc.cpu().numpy()[[1, 3]]))
    want = inp.seq_lens.copy()
    want[[1, 3]] = 0
    gpu_s = msa.msa_indexer_block_scores(q, k, bt, neg).cpu().numpy()
    ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, want)
    check_scores(gpu_s, ref)
    check_selection_exact_given_scores(idsn, sc.cpu().numpy(), gpu_s, want, 16, 1, 2)
    # the page-table call
    ids_p, sc_p, pages, tokens = msa.msa_indexer_decode_pages(q, k, bt, neg)
    assert torch.equal(ids_p, ids) and torch.equal(sc_p, sc)
    wp, wt = oracle.expand_pages(ids.cpu().numpy(), inp.block_table, want)
    assert np.array_equal(pages.cpu().numpy(), wp) and np.array_equal(tokens.cpu().numpy(), wt)
    assert np.all(pages.cpu().numpy()[[1, 3]] == -1) and np.all(tokens.cpu().numpy()[[1, 3]] == 0)
    # the multi-token call (4 positions) and the FP8 call (1 and 4 positions)
    inpm = synth.multi_case(145, lens_np, 30, 4)
    qm, km, btm, _ = to_device(inpm)
    negm = neg.clone()
    wantm = inpm.seq_lens.copy()
    wantm[[1, 3]] = 0
    _, _, ref_m = oracle.decode_multi(inpm.q, inpm.k_cache, inpm.block_table, wantm, 16, 1, 2)
    s_m = msa.msa_indexer_block_scores_multi(qm, km, btm, negm).cpu().numpy()
    check_scores(s_m, ref_m)
    ids_m, _ = msa.msa_indexer_decode_multi(qm, km, btm, negm)
    ids_m = ids_m.cpu().numpy()
    assert np.all(ids_m[[1, 3]] == -1)
    for p in range(4):
        lp = np.maximum(wantm - (3 - p), 0)
        sel, _ = oracle.select(s_m[:, p].astype(np.float64), lp, 16, 1, 2)
        assert np.array_equal(ids_m[:, p], sel), p
        check_selection_vs_oracle(ids_m[:, p], ref_m[:, p], lp, 16, 1, 2)
    for Q in (1, 4):
        f8 = synth.fp8_case(146, lens_np, 30, Q, k_scale=0.5)
        q8 = torch.from_numpy(f8.q.view(np.int16)).cuda().view(torch.bfloat16)
        k8 = torch.from_numpy(f8.k_cache).cuda()
        bt8 = torch.from_numpy(f8.block_table).cuda()
        w8 = f8.seq_lens.copy()
        w8[[1, 3]] = 0
        s8 = msa.msa_indexer_block_scores_fp8(q8, k8, 0.5, bt8, negm).cpu().numpy()
        ref8 = oracle.default().decode_multi_fp8(f8.q, f8.k_cache, 0.5, f8.block_table, w8, 16, 1, 2)[2]
        check_scores(s8, ref8, 1e-3 * 4.0 * 0.5)
        ids8, sc8 = msa.msa_indexer_decode_fp8(q8, k8, 0.5, bt8, negm)
        ids8 = ids8.cpu().numpy()
        assert np.all(ids8[[1, 3]] == -1) and np.all(np.isneginf(sc8.cpu().numpy()[[1, 3]]))
        for p in range(Q):
            sel, _ = oracle.select(s8[:, p].astype(np.float64), np.maximum(w8 - (Q - 1 - p), 0), 16, 1, 2)
            assert np.array_equal(ids8[:, p], sel), (Q, p)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_widest_table_2m_token_row(msa):
    # MSA_MAX_BLOCKS_PER_SEQ = 16384: one row of 2M tokens less a partial block (512 MiB of
    # bf16 index-K) beside a short row, through the decode call and the page-table call.
    W = 16384
    lens_np = np.array([128 * W - 77, 1000], np.int32)
    inp = synth.paged_case(147, lens_np, W)
    q, k, bt, lens = to_device(inp)
    ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, inp.seq_lens)
    gpu_s = msa.msa_indexer_block_scores(q, k, bt, lens).cpu().numpy()
    check_scores(gpu_s, ref)
    ids, sc = msa.msa_indexer_decode(q, k, bt, lens)
    ids, sc = ids.cpu().numpy(), sc.cpu().numpy()
    check_selection_exact_given_scores(ids, sc, gpu_s, lens_np, 16, 1, 2)
    check_selection_vs_oracle(ids, ref, lens_np, 16, 1, 2)
    ids_p, sc_p, pages, tokens = msa.msa_indexer_decode_pages(q, k, bt, lens)
    assert np.array_equal(ids_p.cpu().numpy(), ids) and np.array_equal(sc_p.cpu().numpy(), sc)
    wp, wt = oracle.expand_pages(ids, inp.block_table, lens_np)
    assert np.array_equal(pages.cpu().numpy(), wp) and np.array_equal(tokens.cpu().numpy(), wt)
    # the last block (partial: 51 valid tokens) is pinned, so every head selects it
    assert all(W - 1 in ids[0, h] for h in range(4))


def test_bound_calls_match_the_binding(msa):
    # bind_decode / bind_decode_multi (arguments marshalled once, for timing loops) enqueue the
    # same C calls as the plain binding.
    inp = synth.paged_case(148, [128 * 40 - 5, 128 * 3, 0, 128 * 40], 40)
    q, k, bt, lens = to_device(inp)
    ws = msa.new_workspace(4, 40, 16)
    ids = torch.empty((4, 4, 16), dtype=torch.int32, device="cuda")
    sc = torch.empty((4, 4, 16), dtype=torch.float32, device="cuda")
    msa.bind_decode(q, k, bt, lens, 16, 1, 2, ids, sc, ws)()
    want_ids, want_sc = msa.msa_indexer_decode(q, k, bt, lens)
    torch.cuda.synchronize()
    assert torch.equal(ids, want_ids) and torch.equal(sc, want_sc)
    f8 = synth.fp8_case(149, [128 * 40 - 5, 128 * 3, 0, 128 * 40], 40, 4, k_scale=0.25)
    q8 = torch.from_numpy(f8.q.view(np.int16)).cuda().view(torch.bfloat16)
    k8 = torch.from_numpy(f8.k_cache).cuda()
    bt8 = torch.from_numpy(f8.block_table).cuda()
    l8 = torch.from_numpy(f8.seq_lens).cuda()
    ws8 = torch.zeros(msa.workspace_bytes_multi(4, 40, 4, 16), dtype=torch.uint8, device="cuda")
    ids8 = torch.empty((4, 4, 4, 16), dtype=torch.int32, device="cuda")
    sc8 = torch.empty((4, 4, 4, 16), dtype=torch.float32, device="cuda")
    msa.bind_decode_multi(q8, k8, bt8, l8, 16, 1, 2, ids8, sc8, ws8, k_scale=0.25)()
    w_ids, w_sc = msa.msa_indexer_decode_fp8(q8, k8, 0.25, bt8, l8)
    torch.cuda.synchronize()
    assert torch.equal(ids8, w_ids) and torch.equal(sc8, w_sc)


def test_an_earlier_failed_hip_call_is_not_reported_as_the_calls_error(msa):
    # A HIP call made by other code before the library's call fails and leaves its error for
    # hipGetLastError (here hipSetDevice with a device ordinal that does not exist, a host-side
    # argument error that changes nothing). The decode and multi-token calls still return ok
    # and their results equal those of calls made without the stale error.
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    inp = synth.paged_case(150, [128 * 40 - 5, 128 * 3, 0, 128 * 40], 40)
    q, k, bt, lens = to_device(inp)
    want_ids, want_sc = msa.msa_indexer_decode(q, k, bt, lens)
    torch.cuda.synchronize()
    assert hip.hipSetDevice(ctypes.c_int(1 << 20)) != 0
    ids, sc = msa.msa_indexer_decode(q, k, bt, lens)
    torch.cuda.synchronize()
    assert torch.equal(ids, want_ids) and torch.equal(sc, want_sc)
    q4 = torch.from_numpy(synth.normal_bf16(151, 3, (4, 2, 4, 128)).view(np.int16)).cuda().view(torch.bfloat16)
    want_ids4, want_sc4 = msa.msa_indexer_decode_multi(q4, k, bt, lens)
    torch.cuda.synchronize()
    assert hip.hipSetDevice(ctypes.c_int(1 << 20)) != 0
    ids4, sc4 = msa.msa_indexer_decode_multi(q4, k, bt, lens)
    torch.cuda.synchronize()
    assert torch.equal(ids4, want_ids4) and torch.equal(sc4, want_sc4)
    assert hip.hipGetLastError() == 0


@pytest.mark.parametrize("pattern,elem", [(0, 2), (1, 2), (0, 1), (1, 1)])
def test_streaming_probe_reads_exactly_the_tables_pages(pattern, elem):
    # The streaming-ceiling probe (msa_probe.h) folds every 16-byte chunk it loads into its
    # thread's word: the folds equal a host XOR over exactly the pages the table names, in the
    # decode kernels' assignment of blocks to waves and lanes.
    import ctypes
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    fn = bench.probe_lib()
    B, W, C, P = 3, 24, 8, 80
    page_bytes = 128 * 128 * elem
    rng = np.random.default_rng(150 + pattern + elem)
    cache = rng.integers(0, 2 ** 32, size=(P, page_bytes // 4), dtype=np.uint32)
    bt = rng.permutation(P)[:B * W].astype(np.int32).reshape(B, W)
    kd = torch.from_numpy(cache.view(np.int32)).cuda()
    btd = torch.from_numpy(bt).cuda()
    S = W // C
    out = torch.zeros(B * S * 256, dtype=torch.int32, device="cuda")
    rc = fn(kd.data_ptr(), page_bytes, btd.data_ptr(), B, W, W, C, pattern, out.data_ptr(), None)
    torch.cuda.synchronize()
    assert rc == 0
    got = out.cpu().numpy().view(np.uint32).reshape(B, S, 256)
    chunks = cache.reshape(P, -1, 4)  # [page][16-byte chunk][word]
    words = np.bitwise_xor.reduce(chunks, axis=2)  # x ^ y ^ z ^ w of each chunk
    for b in range(B):
        for s in range(S):
            for t in range(256):
                w, lane = t // 64, t % 64
                want = np.uint32(0)
                for j in range(s * C + w, s * C + C, 4):
                    want ^= np.bitwise_xor.reduce(words[bt[b, j], lane::64])
                assert got[b, s, t] == want, (b, s, t)
