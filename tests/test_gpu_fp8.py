"""GPU parity of the FP8 E4M3 index-cache pass against the CPU oracle.

Bars:
  * every non-NaN E4M3 code decodes exactly (one-token blocks score value(code) * k_scale,
    bit for bit, for scales whose products are exact in fp32);
  * block scores: |fp32 GPU - fp64 oracle| <= 1e-3 * amp * k_scale, same -inf pattern. The
    keys are amp * N(0,1) rounded to E4M3; an fp32 sum of 128 exact products q_d * k_d is
    within gamma_127 * sum|q_d k_d| ~ 7.6e-6 * 82 * amp of the exact sum (sum|q_d k_d| ~ 82 amp
    for this data), below the bar with margin, and the one rounding of the scale multiply
    adds ~6e-8 relative;
  * selections: exactly the oracle's selection on the GPU's own fp32 scores; against the fp64
    oracle exact unless the scores at the cut lie within the same bar;
  * exact-integer keys (-1, 0, 1): ids and scores bit for bit, equal to the bf16 pass's.
"""
import numpy as np
import pytest

import oracle
from sparse_attention_block_amd import synth

from gpu_util import check_scores, check_selection_vs_oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_block_amd as m
    m.load()
    return m


def to_device_fp8(inp):
    q = inp.q if inp.q.ndim == 4 else inp.q[:, None]
    q = torch.from_numpy(np.ascontiguousarray(q).view(np.int16)).to("cuda").view(torch.bfloat16)
    k = torch.from_numpy(np.ascontiguousarray(inp.k_cache)).to("cuda")
    bt = torch.from_numpy(np.ascontiguousarray(inp.block_table)).to("cuda")
    lens = torch.from_numpy(np.ascontiguousarray(inp.seq_lens)).to("cuda")
    return q, k, bt, lens


def position_lens(inp, p, Q):
    L = np.clip(inp.seq_lens.astype(np.int64), 0, inp.max_blocks * 128)
    return np.maximum(L - (Q - 1 - p), 0).astype(np.int32)


def run_fp8(msa, inp, tol, splits=(0,)):
    q, k, bt, lens = to_device_fp8(inp)
    Q = q.shape[1]
    _, _, ref = oracle.decode(inp)
    lo = max(1, -(-inp.max_blocks // 64))
    splits = sorted({0 if s == 0 else max(s, lo) for s in splits})
    s0 = None
    for ns in splits:
        s = msa.msa_indexer_block_scores_fp8(q, k, inp.k_scale, bt, lens, num_splits=ns).cpu().numpy()
        check_scores(s, ref, tol)
        if s0 is None:
            s0 = s
        else:
            assert np.array_equal(s, s0)
    for ns in splits:
        ids, sc = msa.msa_indexer_decode_fp8(q, k, inp.k_scale, bt, lens, inp.topk, inp.n_init,
                                             inp.n_local, num_splits=ns)
        ids, sc = ids.cpu().numpy(), sc.cpu().numpy()
        for p in range(Q):
            lp = position_lens(inp, p, Q)
            gi, gs = oracle.select(s0[:, p].astype(np.float64), lp, inp.topk, inp.n_init, inp.n_local)
            assert np.array_equal(ids[:, p], gi), (ns, p)
            sel = gi >= 0
            assert np.array_equal(sc[:, p][sel].astype(np.float64), gs[sel])
            check_selection_vs_oracle(ids[:, p], ref[:, p], lp, inp.topk, inp.n_init, inp.n_local,
                                      tol=tol)
    return ids, sc


def test_fp8_every_code_decodes_exactly(msa):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    B = len(codes)
    k = np.zeros((B, 128, 128), dtype=np.uint8)
    k[:, 0, 0] = codes
    q = np.zeros((B, 1, 4, 128), dtype=np.uint16)
    q[:, :, :, 0] = synth.bf16_bits(np.float32(1.0))
    bt = np.arange(B, dtype=np.int32).reshape(B, 1)
    lens = np.ones(B, dtype=np.int32)
    for scale in (1.0, 0.5, 3.0):
        inp = synth.Inputs("codes", q, k, bt, lens, k_scale=scale)
        qd, kd, btd, ld = to_device_fp8(inp)
        got = msa.msa_indexer_block_scores_fp8(qd, kd, scale, btd, ld).cpu().numpy()
        _, _, want = oracle.decode(inp)
        assert np.array_equal(got.astype(np.float64), want), scale


@pytest.mark.parametrize("seed,lens,W,Q,scale,amp", [
    (301, [300, 128, 1, 0, 1000, 257, 3, 129, 130], 8, 4, 0.5, 4.0),
    (302, [128 * 5, 77, 2], 5, 1, 1.0, 6.0),
    (303, [4000, 3000, 129, 4], 32, 2, 0.037, 4.0),
    (304, [128 * 300 + 2, 128 * 300 + 3, 128 * 64, 700], 301, 3, 2.5, 4.0),
    (305, [5, 17, 127, 128, 255, 256, 1000, 2000], 16, 1, 1.0, 1.0),
])
def test_fp8_ragged(msa, seed, lens, W, Q, scale, amp):
    inp = synth.fp8_case(seed, lens, W, Q, k_scale=scale, amp=amp)
    run_fp8(msa, inp, 1e-3 * amp * scale, splits=(0, 1, 3, W))


@pytest.mark.parametrize("Q", [1, 4])
def test_fp8_planted_bit_exact_and_equal_to_bf16(msa, Q):
    base = synth.multi_planted(Q)
    qb = torch.from_numpy(base.q.view(np.int16)).to("cuda").view(torch.bfloat16)
    kb = torch.from_numpy(base.k_cache.view(np.int16)).to("cuda").view(torch.bfloat16)
    btb = torch.from_numpy(base.block_table).to("cuda")
    lb = torch.from_numpy(base.seq_lens).to("cuda")
    ids_bf16, sc_bf16 = msa.msa_indexer_decode_multi(qb, kb, btb, lb)
    for scale in (1.0, 0.25):
        inp = synth.to_fp8(base, k_scale=scale)
        want_ids, want_sc, ref = oracle.decode(inp)
        q, k, bt, lens = to_device_fp8(inp)
        s = msa.msa_indexer_block_scores_fp8(q, k, scale, bt, lens).cpu().numpy()
        assert np.array_equal(s.astype(np.float64), ref)
        for ns in (0, 2, 17, 68):
            ids, sc = msa.msa_indexer_decode_fp8(q, k, scale, bt, lens, num_splits=ns)
            assert np.array_equal(ids.cpu().numpy(), want_ids), (scale, ns)
            assert np.array_equal(sc.cpu().numpy().astype(np.float64), want_sc), (scale, ns)
            assert torch.equal(ids, ids_bf16)
            assert torch.equal(sc, sc_bf16 * scale)


@pytest.mark.parametrize("topk,n_init,n_local", [(1, 0, 1), (16, 0, 0), (64, 3, 5)])
def test_fp8_selection_parameters(msa, topk, n_init, n_local):
    inp = synth.fp8_case(306, [128 * 90 + 3, 128 * 20, 128 * 3, 1, 2], 91, 2, k_scale=0.75,
                         topk=topk, n_init=n_init, n_local=n_local)
    run_fp8(msa, inp, 1e-3 * 4.0 * 0.75, splits=(0, 5))


def test_fp8_edges_and_out_of_range_page(msa):
    inp = synth.fp8_case(307, [0, 0, 128 * 5, 3], 5, 1)
    q, k, bt, lens = to_device_fp8(inp)
    ids, sc = msa.msa_indexer_decode_fp8(q, k, 1.0, bt, lens)
    ids = ids.cpu().numpy()
    assert np.all(ids[:2] == -1) and np.all(ids[3, 0, :, 0] == 0) and np.all(ids[3, 0, :, 1:] == -1)
    bt0 = torch.zeros((4, 0), dtype=torch.int32, device="cuda")
    ids0, _ = msa.msa_indexer_decode_fp8(q, k, 1.0, bt0, lens)
    assert torch.all(ids0 == -1)
    ids_b0, _ = msa.msa_indexer_decode_fp8(q[:0], k, 1.0, bt[:0], lens[:0])
    assert ids_b0.shape == (0, 1, 4, 16)
    ws = torch.zeros(msa.workspace_bytes_multi(4, 5, 1, 16), dtype=torch.uint8, device="cuda")
    bad = bt.clone()
    bad[2, 1] = inp.num_pages
    msa.msa_indexer_decode_fp8(q, k, 1.0, bad, lens, workspace=ws)
    assert msa.msa_indexer_read_error(ws) == 1
    s = msa.msa_indexer_block_scores_fp8(q, k, 1.0, bad, lens).cpu().numpy()
    assert np.all(np.isneginf(s[2, :, :, 1]))


@pytest.mark.parametrize("bf16", [False, True])
def test_single_position_merge_in_or_after_the_launch(msa, bf16):
    # One position merges inside the verify launch when each head's split lists fit four
    # registers of the merge network (16 splits of 17 blocks here) and in a second launch
    # otherwise (17 splits of 16): both must select exactly what the oracle selects on the
    # GPU's own scores, and agree with each other bit for bit.
    inp = synth.fp8_case(309, [128 * 272, 128 * 272 - 5, 128 * 200 + 1, 128 * 16, 3000, 0, 1],
                         272, 1, k_scale=0.5)
    if bf16:
        inp = synth.multi_case(309, inp.seq_lens.tolist(), 272, 1)
    q, k, bt, lens = (to_device_fp8(inp) if not bf16 else
                      (torch.from_numpy(np.ascontiguousarray(inp.q).view(np.int16)).cuda().view(torch.bfloat16),
                       torch.from_numpy(inp.k_cache.view(np.int16)).cuda().view(torch.bfloat16),
                       torch.from_numpy(inp.block_table).cuda(), torch.from_numpy(inp.seq_lens).cuda()))
    assert msa.plan(7, 272, 16, 16)["blocks_per_split"] == 17 and msa.plan(7, 272, 16, 17)["blocks_per_split"] == 16
    if bf16:
        s = msa.msa_indexer_block_scores_multi(q, k, bt, lens).cpu().numpy()
        run = lambda ns: msa.msa_indexer_decode_multi(q, k, bt, lens, num_splits=ns)
        tol = 1e-3
    else:
        s = msa.msa_indexer_block_scores_fp8(q, k, 0.5, bt, lens).cpu().numpy()
        run = lambda ns: msa.msa_indexer_decode_fp8(q, k, 0.5, bt, lens, num_splits=ns)
        tol = 1e-3 * 4.0 * 0.5
    _, _, ref = oracle.decode(inp)
    lp = position_lens(inp, 0, 1)
    gi, gs = oracle.select(s[:, 0].astype(np.float64), lp, 16, 1, 2)
    out = {}
    for ns in (16, 17, 0):
        ids, sc = run(ns)
        ids, sc = ids.cpu().numpy()[:, 0], sc.cpu().numpy()[:, 0]
        assert np.array_equal(ids, gi), ns
        assert np.array_equal(sc[gi >= 0].astype(np.float64), gs[gi >= 0]), ns
        check_selection_vs_oracle(ids, ref[:, 0], lp, 16, 1, 2, tol=tol)
        out[ns] = (ids, sc)
    assert np.array_equal(out[16][1], out[17][1])


def test_fp8_single_position_workspace_reuse(msa):
    # One position merges in the same launch through per-row counters in the workspace; they
    # must be back at zero after every call, whatever the lengths and split counts.
    inp = synth.fp8_case(308, [128 * 70] * 6, 70, 1, k_scale=0.5)
    q, k, bt, lens = to_device_fp8(inp)
    plans = [0, 3, 70, 2, 0]
    ws = torch.zeros(max(msa.workspace_bytes_multi(6, 70, 1, 16, ns) for ns in plans),
                     dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(5)
    for it, ns in enumerate(plans):
        new_lens = rng.integers(0, 128 * 70 + 1, size=6).astype(np.int32)
        new_lens[it % 6] = 0
        lens.copy_(torch.from_numpy(new_lens))
        ids, sc = msa.msa_indexer_decode_fp8(q, k, 0.5, bt, lens, num_splits=ns, workspace=ws)
        s = msa.msa_indexer_block_scores_fp8(q, k, 0.5, bt, lens, num_splits=ns).cpu().numpy()
        torch.cuda.synchronize()
        assert np.all(ws[:256 + 6 * 17 * 256].view(torch.int32).cpu().numpy() == 0), it  # header, 17 counter lines per row
        cur = synth.Inputs("reuse", inp.q, inp.k_cache, inp.block_table, new_lens, k_scale=0.5)
        gi, gs = oracle.select(s[:, 0].astype(np.float64), position_lens(cur, 0, 1), 16, 1, 2)
        assert np.array_equal(ids.cpu().numpy()[:, 0], gi), it
        _, _, ref = oracle.decode(cur)
        check_selection_vs_oracle(ids.cpu().numpy()[:, 0], ref[:, 0], position_lens(cur, 0, 1),
                                  16, 1, 2, tol=1e-3 * 4.0 * 0.5)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_fp8_full_size(msa):
    # The benchmark shape with an FP8 cache (512 MiB of E4M3 codes), one decode token per row.
    inp = synth.fp8_config(1, k_scale=0.5)
    ids, _ = run_fp8(msa, inp, 1e-3 * 4.0 * 0.5)
    differ = [len({tuple(sorted(ids[b, 0, h])) for h in range(4)}) == 4 for b in range(inp.batch)]
    assert np.mean(differ) >= 0.9
