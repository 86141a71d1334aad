"""Helpers shared by the GPU tests: device upload and the parity checks."""
from __future__ import annotations

import numpy as np

import oracle
from sparse_attention_block_amd import synth

SCORE_TOL = 1e-3  # absolute, on fp32 block scores against the fp64 oracle


def to_device(inp: synth.Inputs, extra_cols: int = 0):
    """(q, k_cache, block_table, seq_lens) device tensors; extra_cols widens the table."""
    import torch
    dev = "cuda"
    q = torch.from_numpy(inp.q.view(np.int16)).to(dev).view(torch.bfloat16)
    k = torch.from_numpy(inp.k_cache.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = inp.block_table
    if extra_cols:
        bt = np.concatenate([bt, np.zeros((bt.shape[0], extra_cols), np.int32)], axis=1)
    bt = torch.from_numpy(np.ascontiguousarray(bt)).to(dev)
    lens = torch.from_numpy(np.ascontiguousarray(inp.seq_lens)).to(dev)
    return q, k, bt, lens


def nblocks(lens):
    return (np.clip(np.asarray(lens, dtype=np.int64), 0, None) + 127) // 128


def check_scores(gpu: np.ndarray, ref: np.ndarray, tol: float = SCORE_TOL):
    """fp32 GPU block scores vs fp64 oracle: same -inf pattern, |diff| <= tol elsewhere."""
    assert gpu.shape == ref.shape
    assert np.array_equal(np.isneginf(gpu), np.isneginf(ref)), "-inf pattern differs"
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(gpu[fin]))
    err = np.abs(gpu[fin].astype(np.float64) - ref[fin])
    assert err.size == 0 or err.max() <= tol, f"max |score diff| {err.max()}"
    return float(err.max()) if err.size else 0.0


def check_selection_exact_given_scores(ids, scores_out, gpu_scores, lens, topk, n_init, n_local):
    """The GPU's selection equals the oracle's selection run on the GPU's own fp32 block
    scores (the decision is taken in the kernel's precision on both sides), and the
    reported scores are those block scores bit for bit."""
    want_ids, want_sc = oracle.select(gpu_scores.astype(np.float64), lens, topk, n_init, n_local)
    assert np.array_equal(ids, want_ids), "selection differs from the oracle on the same scores"
    sel = want_ids >= 0
    assert np.array_equal(scores_out[sel].astype(np.float64), want_sc[sel])
    assert np.all(np.isneginf(scores_out[~sel]))


def check_selection_vs_oracle(ids, ref_scores, lens, topk, n_init, n_local, tol=SCORE_TOL):
    """Selection against the fp64 oracle scores, exact unless scores nearly tie:
    pins present, min(topk, nb) distinct valid ids, -1 padding, and no unselected
    unpinned block beats a selected one by more than tol. When the gap at the cut is
    above tol this forces the oracle's exact set."""
    B = ids.shape[0]
    nb = nblocks(np.minimum(lens, ref_scores.shape[2] * 128))
    exact_rows = 0
    for b in range(B):
        m = int(min(topk, nb[b]))
        pinned = {j for j in range(int(nb[b])) if j < n_init or j >= nb[b] - n_local}
        for h in range(4):
            sel = [int(x) for x in ids[b, h, :m]]
            assert len(set(sel)) == m and all(0 <= j < nb[b] for j in sel), (b, h, sel)
            assert np.all(ids[b, h, m:] == -1)
            assert pinned <= set(sel)
            chosen = [j for j in sel if j not in pinned]
            left = [j for j in range(int(nb[b])) if j not in set(sel)]
            if chosen and left:
                lo = ref_scores[b, h, chosen].min()
                hi = ref_scores[b, h, left].max()
                assert lo >= hi - tol, (b, h, lo, hi)
                exact_rows += int(lo > hi + tol)
    return exact_rows
