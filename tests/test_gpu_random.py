"""Randomized GPU parity over seeded shapes: batch, table width, row lengths (empty, partial
and full blocks, lengths past the table), topk and pins, split counts, engines, query
positions and cache types, each drawn from a fixed seed. Every case must select exactly what
the oracle selects on the GPU's own fp32 block scores (same precision on both sides), report
those scores bit for bit, and stay within the near-tie rule against the fp64 oracle.
MSA_RANDOM_SEEDS=lo:hi adds seeds lo..hi-1 to every generator (a wider sweep than the default)."""
import os

import numpy as np
import pytest

import oracle
from sparse_attention_block_amd import synth

from gpu_util import check_scores, check_selection_exact_given_scores, check_selection_vs_oracle, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_block_amd as m
    m.load()
    return m


def seeds(default):
    """The test's seeds, plus lo..hi-1 when MSA_RANDOM_SEEDS=lo:hi asks for a wider sweep."""
    extra = os.environ.get("MSA_RANDOM_SEEDS", "")
    if not extra:
        return list(default)
    lo, hi = (int(x) for x in extra.split(":"))
    return list(default) + list(range(lo, hi))


def draw_case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 41))
    W = int(rng.choice([1, 2, 3, 7, 16, 33, 64, 65, 130, 300]))
    kind = rng.random(B)
    lens = np.where(kind < 0.15, 0, np.where(kind < 0.3, 128 * W, rng.integers(1, 128 * W + 1, size=B)))
    topk = int(rng.choice([1, 2, 5, 16, 16, 16, 37, 64]))
    n_init = int(rng.integers(0, 3))
    n_local = int(rng.integers(0, 3))
    if n_init + n_local > topk:
        n_init, n_local = 0, min(n_local, topk)
    splits = int(rng.choice([0, 0, 1, 3, 9, 1000]))
    return B, W, lens.astype(np.int32), topk, n_init, n_local, splits


def feasible(splits, W):
    lo = max(1, -(-W // 64))
    return 0 if splits == 0 else min(max(splits, lo), 256)


@pytest.mark.parametrize("seed", seeds(range(500, 530)))
def test_random_single_token(msa, seed):
    B, W, lens, topk, n_init, n_local, splits = draw_case(seed)
    inp = synth.paged_case(seed, lens.tolist(), W, topk=topk, n_init=n_init, n_local=n_local)
    q, k, bt, lens_d = to_device(inp)
    if seed % 3 == 0:  # a length past the table is clamped to it
        lens_d[0] = 128 * W + 999
    L = lens_d.cpu().numpy()
    ns = feasible(splits, W)
    engine = 2 if seed % 4 == 1 else None
    ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, L)
    s = msa.msa_indexer_block_scores(q, k, bt, lens_d, engine=engine or 0).cpu().numpy()
    check_scores(s, ref)
    ids, sc = msa.msa_indexer_decode(q, k, bt, lens_d, topk, n_init, n_local, num_splits=ns, engine=engine)
    ids, sc = ids.cpu().numpy(), sc.cpu().numpy()
    check_selection_exact_given_scores(ids, sc, s, L, topk, n_init, n_local)
    check_selection_vs_oracle(ids, ref, L, topk, n_init, n_local)


@pytest.mark.parametrize("seed", seeds(range(700, 712)))
def test_random_long_rows_small_batch(msa, seed):
    # Small batches of long rows among short ones, where rows take up to 256 splits: the
    # pruned merge, the two-level count and single-split rows, under automatic and asked-for
    # split counts and several topk.
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 5))
    W = int(rng.choice([513, 700, 1024]))
    kind = rng.random(B)
    lens = np.where(kind < 0.2, rng.integers(0, 513, size=B),
                    np.where(kind < 0.6, 128 * W, rng.integers(1, 128 * W + 1, size=B))).astype(np.int32)
    topk = int(rng.choice([2, 3, 8, 16, 16]))
    n_init, n_local = (1, 1) if topk >= 2 else (0, 0)
    ns = int(rng.choice([0, 0, 129, 200, 256]))
    inp = synth.paged_case(seed, lens.tolist(), W, topk=topk, n_init=n_init, n_local=n_local)
    q, k, bt, lens_d = to_device(inp)
    ref = oracle.block_scores(inp.q, inp.k_cache, inp.block_table, inp.seq_lens)
    s = msa.msa_indexer_block_scores(q, k, bt, lens_d).cpu().numpy()
    check_scores(s, ref)
    ids, sc = msa.msa_indexer_decode(q, k, bt, lens_d, topk, n_init, n_local, num_splits=ns)
    ids, sc = ids.cpu().numpy(), sc.cpu().numpy()
    check_selection_exact_given_scores(ids, sc, s, inp.seq_lens, topk, n_init, n_local)
    check_selection_vs_oracle(ids, ref, inp.seq_lens, topk, n_init, n_local)


@pytest.mark.parametrize("seed", seeds(range(600, 615)))
def test_random_multi_and_fp8(msa, seed):
    B, W, lens, topk, n_init, n_local, splits = draw_case(seed)
    Q = int(np.random.default_rng(seed + 1).integers(1, 5))
    fp8 = seed % 2 == 0
    inp = synth.multi_case(seed, lens.tolist(), W, Q, topk=topk, n_init=n_init, n_local=n_local)
    if fp8:
        inp = synth.to_fp8(inp, k_scale=0.75, amp=3.0)
    tol = 1e-3 * (3.0 * 0.75 if fp8 else 1.0)
    qd = torch.from_numpy(np.ascontiguousarray(inp.q).view(np.int16)).cuda().view(torch.bfloat16)
    kd = (torch.from_numpy(inp.k_cache).cuda() if fp8 else
          torch.from_numpy(inp.k_cache.view(np.int16)).cuda().view(torch.bfloat16))
    bt = torch.from_numpy(inp.block_table).cuda()
    lens_d = torch.from_numpy(inp.seq_lens).cuda()
    ns = feasible(splits, W)
    _, _, ref = oracle.decode(inp)
    if fp8:
        s = msa.msa_indexer_block_scores_fp8(qd, kd, 0.75, bt, lens_d, num_splits=ns).cpu().numpy()
        ids, sc = msa.msa_indexer_decode_fp8(qd, kd, 0.75, bt, lens_d, topk, n_init, n_local, num_splits=ns)
    else:
        s = msa.msa_indexer_block_scores_multi(qd, kd, bt, lens_d, num_splits=ns).cpu().numpy()
        ids, sc = msa.msa_indexer_decode_multi(qd, kd, bt, lens_d, topk, n_init, n_local, num_splits=ns)
    check_scores(s, ref, tol)
    ids, sc = ids.cpu().numpy(), sc.cpu().numpy()
    Lc = np.clip(inp.seq_lens.astype(np.int64), 0, W * 128)
    for p in range(Q):
        lp = np.maximum(Lc - (Q - 1 - p), 0).astype(np.int32)
        check_selection_exact_given_scores(ids[:, p], sc[:, p], s[:, p], lp, topk, n_init, n_local)
        check_selection_vs_oracle(ids[:, p], ref[:, p], lp, topk, n_init, n_local, tol=tol)
