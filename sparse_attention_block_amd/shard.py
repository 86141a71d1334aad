"""One GPU's share of the context-parallel indexer pass (host-side layout only).

The pages shard the pass along the block axis: rank r of P scores the global blocks
j = local * P + r of every row, for all four heads, keeps its own per-head top-k with the
same pinned blocks, and the ranks' lists are then merged exactly per head (vLLM PR #57832,
Solution; SGLang PR #41488, Modifications: rank r reads blocks r, r+4, r+8, ...). A rank's
share is an ordinary call of the same kernel: its block table holds the row's entries at
j % P == r, its lengths count those blocks' tokens, and the pinned blocks that fall on the
rank are its first or last local blocks, so the kernel's scalar pin counts express them
as long as every row puts the same number of pins on the rank (rows of one block count, as
in the benchmark batch). This module only builds that share and maps its ids back; the
kernel is unchanged.
"""
from __future__ import annotations

import numpy as np

BLOCK = 128


def _nblocks(lens: np.ndarray, W: int) -> np.ndarray:
    L = np.clip(lens.astype(np.int64), 0, W * BLOCK)
    return (L + BLOCK - 1) // BLOCK


def rank_share(block_table: np.ndarray, seq_lens: np.ndarray, P: int, r: int,
               n_init: int, n_local: int):
    """(block_table_r [B][ceil(W/P)], seq_lens_r [B], n_init_r, n_local_r) of rank r of P.

    Raises ValueError when rows would need different pin counts on this rank."""
    if P < 1 or not 0 <= r < P:
        raise ValueError("need 0 <= r < P")
    bt = np.asarray(block_table, dtype=np.int32)
    B, W = bt.shape
    lens = np.asarray(seq_lens)
    L = np.clip(lens.astype(np.int64), 0, W * BLOCK)
    nb = _nblocks(lens, W)
    Wr = -(-W // P)
    cols = np.arange(Wr) * P + r
    ok = cols < W
    bt_r = np.zeros((B, Wr), dtype=np.int32)
    bt_r[:, ok] = bt[:, cols[ok]]
    n_r = np.maximum(0, -(-(nb - r) // P))                  # blocks j < nb with j % P == r
    owns_last = (nb > 0) & ((nb - 1) % P == r)
    tail = L - (nb - 1) * BLOCK                              # valid tokens of the row's last block
    lens_r = np.where(owns_last, (n_r - 1) * BLOCK + tail, n_r * BLOCK).astype(np.int32)
    # Pins on this rank: global blocks j < n_init, and j >= nb - n_local, with j % P == r.
    init_r = np.array([sum(1 for j in range(r, min(n_init, int(n)), P)) for n in nb])
    local_r = np.array([sum(1 for j in range(int(n) - 1, max(int(n) - n_local, 0) - 1, -1)
                            if j % P == r) for n in nb])
    live = n_r > 0
    if live.any():
        if len(set(init_r[live])) > 1 or len(set(local_r[live])) > 1:
            raise ValueError("rows need different pin counts on this rank")
        return bt_r, lens_r, int(init_r[live][0]), int(local_r[live][0])
    return bt_r, lens_r, 0, 0


def global_ids(local_ids: np.ndarray, P: int, r: int) -> np.ndarray:
    """Rank r's local block ids as global ids (local * P + r); -1 padding stays -1."""
    ids = np.asarray(local_ids)
    return np.where(ids >= 0, ids * P + r, -1).astype(np.int32)
