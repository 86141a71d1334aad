"""The allocation-free decode (msa_indexer_decode_noalloc) against msa_indexer_decode.

Called through the C ABI (the ctypes binding), with preallocated outputs: two calls in a row
on the library's scratch array, the second with a smaller input (fewer rows, shorter rows,
another plan), each equal bit for bit to msa_indexer_decode on a workspace of its own, and to
the oracle's selection on the GPU's own block scores. Then a call past the scratch's limit is
refused on the host, and an out-of-range page sets the caller's error word.
"""
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


def _against_decode(msa, inp, num_splits=0):
    q, k, bt, lens = to_device(inp)
    B = inp.batch
    ids = torch.full((B, 4, 16), 7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, 4, 16), 7.0, dtype=torch.float32, device="cuda")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    msa.msa_indexer_decode_noalloc(q, k, bt, lens, out_ids=ids, out_scores=sc, error_flags=flags,
                                   num_splits=num_splits)
    ws = msa.new_workspace(B, inp.max_blocks, 16, num_splits)
    want_ids, want_sc = msa.msa_indexer_decode(q, k, bt, lens, workspace=ws, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(ids, want_ids) and torch.equal(sc, want_sc)
    assert int(flags.item()) == 0
    gpu_s = msa.msa_indexer_block_scores(q, k, bt, lens).cpu().numpy()
    check_selection_exact_given_scores(ids.cpu().numpy(), sc.cpu().numpy(), gpu_s, inp.seq_lens, 16, 1, 2)
    ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, inp.seq_lens)
    check_selection_vs_oracle(ids.cpu().numpy(), ref, inp.seq_lens, 16, 1, 2)


def test_noalloc_matches_decode_twice_then_smaller(msa):
    # First call: batch 12 x up to 1100 blocks (the device plan); second: batch 3 x up to 40
    # blocks (a host plan); a third, larger again, on what the first two left in the scratch.
    rng = np.random.default_rng(51)
    big = rng.integers(0, 128 * 1100 + 1, size=12).astype(np.int32)
    big[0] = 128 * 1100
    big[5] = 0
    _against_decode(msa, synth.paged_case(151, big, 1100))
    _against_decode(msa, synth.paged_case(152, [128 * 40 - 9, 300, 128 * 17], 40))
    _against_decode(msa, synth.paged_case(153, [128 * 300] * 9 + [5], 300), num_splits=19)
    _against_decode(msa, synth.config(5))


def test_noalloc_limits_and_error_word(msa):
    from sparse_attention_block_amd import _lib
    inp = synth.paged_case(154, [128 * 5, 77], 5)
    q, k, bt, lens = to_device(inp)
    big_q = torch.zeros((257, 4, 128), dtype=torch.bfloat16, device="cuda")
    big_bt = torch.zeros((257, 5), dtype=torch.int32, device="cuda")
    big_l = torch.zeros(257, dtype=torch.int32, device="cuda")
    with pytest.raises(_lib.MsaError) as e:  # batch above MSA_NOALLOC_MAX_BATCH
        msa.msa_indexer_decode_noalloc(big_q, k, big_bt, big_l)
    assert e.value.status == _lib.MSA_ERR_WORKSPACE_TOO_SMALL
    # keys beyond the scratch: 200 rows of a 16384-block table (128 KiB of keys per row)
    wq = torch.zeros((200, 4, 128), dtype=torch.bfloat16, device="cuda")
    wbt = torch.zeros((200, 16384), dtype=torch.int32, device="cuda")
    wl = torch.zeros(200, dtype=torch.int32, device="cuda")
    with pytest.raises(_lib.MsaError) as e:
        msa.msa_indexer_decode_noalloc(wq, k, wbt, wl)
    assert e.value.status == _lib.MSA_ERR_WORKSPACE_TOO_SMALL
    # an out-of-range page: scored -inf and flagged in the caller's error word
    bt_bad = bt.clone()
    bt_bad[0, 2] = k.shape[0] + 3
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids, sc = msa.msa_indexer_decode_noalloc(q, k, bt_bad, lens, error_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 1
    # row 0 has 5 blocks, all selected: pins 0, 3, 4 first, then block 1, then block 2 at -inf
    assert np.all(ids[0].cpu().numpy()[:, 3:5] == [1, 2])
    assert np.all(np.isneginf(sc[0].cpu().numpy()[:, 4]))
    ids2, _ = msa.msa_indexer_decode_noalloc(q, k, bt, lens)  # no error word: still exact
    want, _ = msa.msa_indexer_decode(q, k, bt, lens)
    assert torch.equal(ids2, want)
