"""GPU parity of the 16-token page table (vLLM blog "Following the Bottleneck", section 3,
Figure 5) against the CPU oracle's expansion.

The table is integer work, so the bar is bit-exact: msa_indexer_decode_pages must return
the same ids and scores as msa_indexer_decode and the oracle's expansion of those ids;
msa_indexer_expand_pages must equal the oracle's expansion of any id lists, including
unordered lists, -1 padding in the middle, ids past the row or the table, and repeats.
On the planted workload (exact scores) the table also equals the oracle's expansion of the
oracle's own selection.
"""
import numpy as np
import pytest

import oracle
from sparse_attention_block_amd import synth

from gpu_util import check_selection_vs_oracle, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_block_amd as m
    m.load()
    return m


def decode_both(msa, inp, splits=0, engine=0):
    q, k, bt, lens = to_device(inp)
    # the same engine on both sides: the engines sum the dot products in different orders
    ids0, sc0 = msa.msa_indexer_decode(q, k, bt, lens, inp.topk, inp.n_init, inp.n_local,
                                       num_splits=splits, engine=engine if engine else None)
    ids, sc, pages, tokens = msa.msa_indexer_decode_pages(q, k, bt, lens, inp.topk, inp.n_init,
                                                          inp.n_local, num_splits=splits,
                                                          engine=engine)
    torch.cuda.synchronize()
    return ids0.cpu().numpy(), sc0.cpu().numpy(), ids.cpu().numpy(), sc.cpu().numpy(), \
        pages.cpu().numpy(), tokens.cpu().numpy()


def check_decode_pages(msa, inp, splits=0, engine=0):
    ids0, sc0, ids, sc, pages, tokens = decode_both(msa, inp, splits, engine)
    assert np.array_equal(ids, ids0) and np.array_equal(sc.view(np.uint32), sc0.view(np.uint32))
    want_p, want_t = oracle.expand_pages(ids, inp.block_table, inp.seq_lens)
    assert np.array_equal(pages, want_p)
    assert np.array_equal(tokens, want_t)
    return ids, pages, tokens


@pytest.mark.parametrize("i", [1, 2, 4, 5])
def test_decode_pages_configs(msa, i):
    inp = synth.config(i)
    ids, pages, tokens = check_decode_pages(msa, inp)
    ref_ids, _, ref_scores = oracle.decode(inp)
    check_selection_vs_oracle(ids, ref_scores, inp.seq_lens, inp.topk, inp.n_init, inp.n_local)
    if i == 5:  # exact scores: the selection is the oracle's, and so is its table
        want_p, want_t = oracle.expand_pages(ref_ids, inp.block_table, inp.seq_lens)
        assert np.array_equal(pages, want_p) and np.array_equal(tokens, want_t)


@pytest.mark.parametrize("engine", [1, 2])
@pytest.mark.parametrize("splits", [16, 64, 256])
def test_decode_pages_plans_and_engines(msa, splits, engine):
    # 256 splits of a 1024-wide table are merged by the second kernel; the others are fused.
    inp = synth.paged_case(61, [128 * 1024, 128 * 300 + 5, 0, 77, 128 * 17], 1024, permute=True,
                           poison=True, extra_pages=3)
    check_decode_pages(msa, inp, splits=splits, engine=engine)


@pytest.mark.parametrize("topk,n_init,n_local", [(1, 0, 1), (5, 2, 2), (16, 0, 0), (64, 3, 5)])
def test_decode_pages_selection_parameters(msa, topk, n_init, n_local):
    inp = synth.paged_case(62, [128 * 200 + 3, 128 * 64, 700, 1, 128 * 70], 201, topk=topk,
                           n_init=n_init, n_local=n_local)
    check_decode_pages(msa, inp)


def test_decode_pages_empty_and_short_rows(msa):
    inp = synth.paged_case(63, [0, 1, 127, 128, 129, 0, 128 * 16, 128 * 16 + 1], 20)
    ids, pages, tokens = check_decode_pages(msa, inp)
    assert np.all(pages[0] == -1) and np.all(tokens[0] == 0) and np.all(tokens[1] == 1)


@pytest.mark.slow
def test_decode_pages_full_size(msa):
    inp = synth.config3()
    check_decode_pages(msa, inp)


def test_expand_pages_any_id_lists(msa):
    rng = np.random.default_rng(64)
    lens = np.array([128 * 40 + 9, 0, 128 * 3, 500, 128 * 64], np.int32)
    W = 64
    B = len(lens)
    bt = rng.integers(0, 1 << 27, size=(B, W), dtype=np.int32)
    bt[0, 5] = (1 << 28) - 1          # largest page id whose 16-token pages fit int32
    for topk in (1, 7, 16, 64):
        ids = rng.integers(-3, W + 4, size=(B, 4, topk), dtype=np.int32)
        ids[0, 0, :] = -1
        ids[0, 1, : min(topk, 3)] = 5                  # repeats
        ids[2, 2, :] = rng.permutation(np.arange(topk) % 3)
        dev = "cuda"
        pages, tokens = msa.msa_indexer_expand_pages(torch.from_numpy(ids).to(dev),
                                                     torch.from_numpy(bt).to(dev),
                                                     torch.from_numpy(lens).to(dev))
        want_p, want_t = oracle.expand_pages(ids, bt, lens)
        assert np.array_equal(pages.cpu().numpy(), want_p), topk
        assert np.array_equal(tokens.cpu().numpy(), want_t), topk


def test_expand_pages_of_oracle_selection(msa):
    inp = synth.config(4)
    ref_ids, _, _ = oracle.decode(inp)
    _, _, bt, lens = to_device(inp)
    pages, tokens = msa.msa_indexer_expand_pages(torch.from_numpy(ref_ids).to("cuda"), bt, lens)
    want_p, want_t = oracle.expand_pages(ref_ids, inp.block_table, inp.seq_lens)
    assert np.array_equal(pages.cpu().numpy(), want_p)
    assert np.array_equal(tokens.cpu().numpy(), want_t)


def test_expand_pages_strided_table(msa):
    # A table view with a row stride above its width: only the first W columns are rows.
    rng = np.random.default_rng(65)
    full = rng.integers(0, 1000, size=(3, 24), dtype=np.int32)
    lens = np.array([128 * 16, 128 * 5 + 1, 128 * 10], np.int32)
    ids = rng.integers(-1, 16, size=(3, 4, 16), dtype=np.int32)
    bt_dev = torch.from_numpy(full).to("cuda")[:, :16]
    assert bt_dev.stride(0) == 24
    from sparse_attention_block_amd import _lib
    out_p = torch.empty((3, 4, 128), dtype=torch.int32, device="cuda")
    out_t = torch.empty((3, 4), dtype=torch.int32, device="cuda")
    ids_dev = torch.from_numpy(ids).to("cuda")
    lens_dev = torch.from_numpy(lens).to("cuda")
    rc = _lib.load().msa_indexer_expand_pages(
        _lib._P(ids_dev.data_ptr()), _lib._P(bt_dev.data_ptr()), _lib._P(lens_dev.data_ptr()),
        3, 16, 24, 16, _lib._P(out_p.data_ptr()), _lib._P(out_t.data_ptr()),
        _lib._P(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    want_p, want_t = oracle.expand_pages(ids, np.ascontiguousarray(full[:, :16]), lens)
    assert np.array_equal(out_p.cpu().numpy(), want_p)
    assert np.array_equal(out_t.cpu().numpy(), want_t)


@pytest.mark.parametrize("Q", [1, 3, 4])
def test_expand_pages_multi_token(msa, Q):
    # The selections of a multi-token pass, expanded per (row, position) with the position's
    # causal length; each position's table equals the oracle's expansion with that length.
    inp = synth.multi_case(66, [128 * 30 + 2, 3, 0, 128 * 12, 129], 31, Q)
    q = torch.from_numpy(np.ascontiguousarray(inp.q).view(np.int16)).cuda().view(torch.bfloat16)
    k = torch.from_numpy(inp.k_cache.view(np.int16)).cuda().view(torch.bfloat16)
    bt = torch.from_numpy(inp.block_table).cuda()
    lens = torch.from_numpy(inp.seq_lens).cuda()
    ids, _ = msa.msa_indexer_decode_multi(q, k, bt, lens)
    pages, tokens = msa.msa_indexer_expand_pages_multi(ids, bt, lens)
    ids, pages, tokens = ids.cpu().numpy(), pages.cpu().numpy(), tokens.cpu().numpy()
    L = np.clip(inp.seq_lens.astype(np.int64), 0, inp.max_blocks * 128)
    for p in range(Q):
        lp = np.maximum(L - (Q - 1 - p), 0).astype(np.int32)
        want_p, want_t = oracle.expand_pages(np.ascontiguousarray(ids[:, p]), inp.block_table, lp)
        assert np.array_equal(pages[:, p], want_p), p
        assert np.array_equal(tokens[:, p], want_t), p
