"""One GPU standing in for P context-parallel ranks: each rank's share (round-robin blocks
j = local * P + rank, pins on the shard; vLLM PR #57832, Solution) is an ordinary decode
call, and the exact per-head merge of the P lists (pinned first, then score, then lower id)
must equal the decode of the whole row, ids and scores bit for bit, since a block in a
head's global top-k is in its own shard's top-k."""
import numpy as np
import pytest

from sparse_attention_block_amd import shard, synth

from gpu_util import to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_block_amd as m
    m.load()
    return m


def merge_lists(ids_list, sc_list, lens, W, topk, n_init, n_local):
    B = ids_list[0].shape[0]
    nb = (np.clip(lens.astype(np.int64), 0, W * 128) + 127) // 128
    out_ids = np.full((B, 4, topk), -1, dtype=np.int32)
    out_sc = np.full((B, 4, topk), -np.inf, dtype=np.float32)
    for b in range(B):
        for h in range(4):
            cand = [(int(i), float(s)) for ids, sc in zip(ids_list, sc_list)
                    for i, s in zip(ids[b, h], sc[b, h]) if i >= 0]
            pinned = lambda j: j < n_init or j >= nb[b] - n_local
            cand.sort(key=lambda c: (not pinned(c[0]), -c[1], c[0]))
            m = min(topk, int(nb[b]))
            for i, (j, s) in enumerate(cand[:m]):
                out_ids[b, h, i] = j
                out_sc[b, h, i] = s
    return out_ids, out_sc


@pytest.mark.parametrize("P", [2, 4])
@pytest.mark.parametrize("seed,B,L,W", [(501, 8, 32768 - 50, 256), (502, 4, 128 * 37 + 5, 40),
                                        (503, 32, 128 * 256 - 3, 256)])
def test_rank_shares_merge_to_the_full_decode(msa, P, seed, B, L, W):
    inp = synth.paged_case(seed, [L] * B, W, poison=False)
    q, k, bt, lens = to_device(inp)
    full_ids, full_sc = msa.msa_indexer_decode(q, k, bt, lens)
    ids_list, sc_list = [], []
    for r in range(P):
        bt_r, lens_r, ni, nl = shard.rank_share(inp.block_table, inp.seq_lens, P, r, 1, 2)
        ids, sc = msa.msa_indexer_decode(q, k, torch.from_numpy(bt_r).cuda(),
                                         torch.from_numpy(lens_r).cuda(), 16, ni, nl)
        ids_list.append(shard.global_ids(ids.cpu().numpy(), P, r))
        sc_list.append(sc.cpu().numpy())
    m_ids, m_sc = merge_lists(ids_list, sc_list, inp.seq_lens, W, 16, 1, 2)
    assert np.array_equal(m_ids, full_ids.cpu().numpy())
    assert np.array_equal(m_sc, full_sc.cpu().numpy())
