"""Seeded synthetic inputs for the MiniMax-M3 lightning-indexer decode pass.

This module only draws and lays out inputs. It holds none of the pass's
arithmetic (no dot products, maxima or selection), so the GPU path and the
CPU oracle can both consume exactly the same bf16 bits from it.

Layouts (row-major, as both sides read them):
  q            uint16 [B, 4, 128]        bf16 bit patterns, one decode token per row
               uint16 [B, Q, 4, 128]     or Q query positions per row (multi-token decode:
                                         the row's last Q context tokens are draft tokens)
  k_cache      uint16 [P, 128, 128]      bf16 bit patterns, page-major, token-major
               uint8  [P, 128, 128]      or FP8 E4M3 codes (OCP), keys = k_scale * value
  block_table  int32  [B, W]             logical block j of row b -> physical page
  seq_lens     int32  [B]                tokens in row b's context (0 .. W*128)

Workload shapes follow the pages: 4 index heads of dim 128 sharing one index-K
head, 128-token pages (SGLang PR #41488 "[AMD] Add opt-in MiniMax-M3 TP4 indexer
context partitioning", Modifications; TensorRT-LLM PR #17008, Performance/Kernel
table), a top-16 with pinned initial and recent blocks (vLLM PR #57832, Solution).

Random draws use NumPy PCG64. Big arrays are drawn in fixed chunks, each from
its own SeedSequence child, so the result does not depend on how the chunks
are scheduled.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEADS = 4
DIM = 128
BLOCK = 128  # tokens per logical block == tokens per page

_CHUNK_ELEMS = 1 << 22  # elements per independently seeded chunk


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    a = np.array(x, dtype=np.float32, order="C", copy=True)
    u = a.reshape(-1).view(np.uint32)
    lsb = u >> 16
    lsb &= 1
    u += lsb
    u += np.uint32(0x7FFF)
    u >>= 16
    return u.astype(np.uint16).reshape(a.shape)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _child(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream, chunk]))


def normal_bf16(seed: int, stream: int, shape) -> np.ndarray:
    """~N(0,1) bf16 bit patterns of `shape`, drawn chunk by chunk."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for c, lo in enumerate(range(0, n, _CHUNK_ELEMS)):
        hi = min(n, lo + _CHUNK_ELEMS)
        out[lo:hi] = bf16_bits(_child(seed, stream, c).standard_normal(hi - lo, dtype=np.float32))
    return out.reshape(shape)


@dataclass
class Inputs:
    """One decode-pass input set plus the selection parameters."""

    name: str
    q: np.ndarray
    k_cache: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    topk: int = 16
    n_init: int = 1
    n_local: int = 2
    meta: dict = field(default_factory=dict)
    k_scale: float = 1.0  # FP8 caches only

    @property
    def fp8(self) -> bool:
        return self.k_cache.dtype == np.uint8

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def qlen(self) -> int:
        """Query positions per row (1 for single-token decode)."""
        return 1 if self.q.ndim == 3 else int(self.q.shape[1])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def index_k_bytes(self) -> int:
        """Index-K bytes the pass must read: sum of seq_len * 128 dims * (2 B bf16, 1 B fp8)."""
        elem = 1 if self.fp8 else 2
        return int(np.asarray(self.seq_lens, dtype=np.int64).clip(min=0).sum()) * DIM * elem


def _nblocks(lens: np.ndarray) -> np.ndarray:
    return (np.asarray(lens, dtype=np.int64) + BLOCK - 1) // BLOCK


def poison_tokens(n: int, value: float = 64.0) -> np.ndarray:
    """Tokens that must never be read: +value / -value vectors, alternating.

    A pass that wrongly scores one of them gets |value * sum(q)|, far above
    any ~N(0,1) block score, whatever the sign of the query sum.
    """
    tok = np.empty((n, DIM), dtype=np.float32)
    tok[0::2] = value
    tok[1::2] = -value
    return bf16_bits(tok)


def paged_case(seed: int, seq_lens, max_blocks: int, *, permute: bool = True,
               poison: bool = True, extra_pages: int = 0, name: str | None = None,
               topk: int = 16, n_init: int = 1, n_local: int = 2) -> Inputs:
    """Random ~N(0,1) q / index-K with a paged block table.

    Every valid block gets its own page. With `permute` the pages are a random
    permutation; with `poison`, table entries past a row's last block point to
    a poison page and the invalid tail tokens of partial blocks are poison, so
    any read the pass should not make shows up in its scores.
    """
    lens = np.asarray(seq_lens, dtype=np.int32)
    B = int(lens.shape[0])
    W = int(max_blocks)
    nb = _nblocks(lens)
    assert np.all(lens >= 0) and np.all(nb <= W)
    n_valid = int(nb.sum())
    n_pages = n_valid + extra_pages + (1 if poison else 0)
    q = normal_bf16(seed, 0, (B, HEADS, DIM))
    k = normal_bf16(seed, 1, (n_pages, BLOCK, DIM))
    order = _child(seed, 2).permutation(n_pages) if permute else np.arange(n_pages)
    order = order.astype(np.int32)
    bt = np.zeros((B, W), dtype=np.int32)
    poison_page = int(order[-1]) if poison else 0
    pos = 0
    for b in range(B):
        n = int(nb[b])
        bt[b, :n] = order[pos:pos + n]
        pos += n
        bt[b, n:] = poison_page if poison else 0
    if poison:
        k[poison_page] = poison_tokens(BLOCK)
        for b in range(B):
            v = int(lens[b]) - (int(nb[b]) - 1) * BLOCK
            if nb[b] > 0 and v < BLOCK:
                k[bt[b, nb[b] - 1], v:] = poison_tokens(BLOCK - v)
    return Inputs(name or f"paged(seed={seed},B={B},W={W})", q, k, bt, lens,
                  topk=topk, n_init=n_init, n_local=n_local,
                  meta={"poison_page": poison_page if poison else None})


def multi_case(seed: int, seq_lens, max_blocks: int, qlen: int, **kw) -> Inputs:
    """paged_case with qlen query positions per row: q ~N(0,1) bf16 [B, qlen, 4, 128]."""
    inp = paged_case(seed, seq_lens, max_blocks, **kw)
    inp.q = normal_bf16(seed, 4, (inp.batch, qlen, HEADS, DIM))
    inp.name = kw.get("name") or f"multi(seed={seed},B={inp.batch},W={inp.max_blocks},Q={qlen})"
    return inp


def multi_planted(qlen: int = 4) -> Inputs:
    """Batch 16, 8576..8704 tokens (68-block table), qlen draft positions, exact integer scores.

    q[b,p,h,:] is +-1 and background index-K entries are uniform in {-1, 0, +1}, so every
    score is an exact integer. Planted, for each row:
      * for each (position p, head h), a run of 16 blocks at a seeded start whose token slot
        4p+h holds q[b,p,h,:] with all but its first T entries zeroed (score exactly T for
        (p, h); T in 100..115, ties included);
      * the draft tokens themselves: the token at absolute index L-qlen+i holds q[b,0,i%4,:]
        in full (score 128 for position 0, head i%4), so position 0 must see it only for
        i = 0 (causally, position p sees the first L-(qlen-1-p) tokens);
      * rows 3 and 11: q[b,qlen-1,h,:] in the invalid tail slots of the partial last block.
    Lengths put the boundary between positions' block counts in every place: some rows have
    position 0 one block short of the others.
    """
    B, W = 16, 68
    seed = 6
    lens = np.array([8700, 8704, 128 * 67 + 1, 128 * 67 + 2, 128 * 67 + 3, 128 * 67 + 4,
                     8699, 8577, 8578, 8579, 8600, 8650, 8701, 8702, 8703, 8576], dtype=np.int32)
    sgn = _child(seed, 0).standard_normal((B, qlen, HEADS, DIM))
    qf = np.where(sgn >= 0, 1.0, -1.0).astype(np.float32)
    nb = _nblocks(lens)
    n_pages = int(nb.sum()) + 1
    kf = _child(seed, 1).integers(-1, 2, size=(n_pages, BLOCK, DIM)).astype(np.float32)
    order = _child(seed, 2).permutation(n_pages).astype(np.int32)
    spare = int(order[-1])
    bt = np.full((B, W), spare, dtype=np.int32)
    pos = 0
    for b in range(B):
        bt[b, :nb[b]] = order[pos:pos + nb[b]]
        pos += int(nb[b])
    rng = _child(seed, 3)
    planted = {}
    for b in range(B):
        L = int(lens[b])
        for p in range(qlen):
            for h in range(HEADS):
                w0 = int(rng.integers(0, nb[b] - 2 - 16 + 1))
                kind = int(rng.integers(0, 3))
                if kind == 0:
                    targets = [100] * 16
                elif kind == 1:
                    targets = list(range(115, 99, -1))
                else:
                    targets = [100 + int(t) for t in rng.integers(0, 4, size=16)]
                for i, t in enumerate(targets):
                    tok = qf[b, p, h].copy()
                    tok[t:] = 0.0
                    kf[bt[b, w0 + i], 4 * p + h] = tok
                    planted[(b, p, h, w0 + i)] = t
        for i in range(qlen):
            a = L - qlen + i
            if a >= 0:
                kf[bt[b, a // BLOCK], a % BLOCK] = qf[b, 0, i % HEADS]
        if b in (3, 11):
            last = (L - 1) // BLOCK
            for t in range(L - last * BLOCK, BLOCK):
                kf[bt[b, last], t] = qf[b, qlen - 1, t % HEADS]
    return Inputs(f"multi planted B=16 Q={qlen}", bf16_bits(qf), bf16_bits(kf), bt, lens,
                  meta={"planted": planted})


def multi_query(qlen: int = 4) -> np.ndarray:
    """The queries of multi_config: ~N(0,1) bf16 [32, qlen, 4, 128]."""
    return normal_bf16(3, 5, (32, qlen, HEADS, DIM))


def multi_config(qlen: int = 4) -> Inputs:
    """The benchmark shape with qlen draft positions per row: batch 32 x 131072 tokens (1024
    blocks, 1 GiB of index-K, the same cache as config3), q ~N(0,1) [32, qlen, 4, 128]."""
    inp = config3()
    inp.q = multi_query(qlen)
    inp.name = f"B=32 x 131072, Q={qlen}"
    return inp


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """fp32 values -> OCP FP8 E4M3 codes (uint8), round to nearest even, saturated to +-448
    (so no NaN code is produced). Converted in chunks through torch's float8_e4m3fn."""
    import torch
    a = np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0).reshape(-1)
    out = np.empty(a.shape, dtype=np.uint8)
    for lo in range(0, a.size, _CHUNK_ELEMS):
        hi = min(a.size, lo + _CHUNK_ELEMS)
        out[lo:hi] = torch.from_numpy(a[lo:hi]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return out.reshape(np.shape(x))


def to_fp8(inp: Inputs, k_scale: float = 1.0, amp: float = 1.0) -> Inputs:
    """The same input with its bf16 index-K cache re-encoded as E4M3 codes of amp * value
    (amp = 1 keeps small integers exact: -1, 0, 1 and the +-64 poison are E4M3 values), and
    q shaped [B, Q, 4, 128]."""
    vals = bf16_to_f32(inp.k_cache) if amp == 1.0 else bf16_to_f32(inp.k_cache) * np.float32(amp)
    q = inp.q if inp.q.ndim == 4 else inp.q[:, None].copy()
    return Inputs(inp.name + f" fp8(scale={k_scale})", q, e4m3_codes(vals), inp.block_table,
                  inp.seq_lens, topk=inp.topk, n_init=inp.n_init, n_local=inp.n_local,
                  meta=dict(inp.meta), k_scale=float(k_scale))


def fp8_case(seed: int, seq_lens, max_blocks: int, qlen: int = 1, k_scale: float = 1.0,
             amp: float = 4.0, **kw) -> Inputs:
    """multi_case with the index-K cache as E4M3 codes of amp * N(0,1) (poison pages and
    tails stay +-64 * amp, inside the E4M3 range for amp <= 7)."""
    return to_fp8(multi_case(seed, seq_lens, max_blocks, qlen, **kw), k_scale, amp)


def fp8_config(qlen: int = 1, k_scale: float = 1.0) -> Inputs:
    """The benchmark shape with an FP8 cache: batch 32 x 131072 tokens (1024 blocks, 512 MiB of
    E4M3 codes of 4 * N(0,1)), shuffled pages, q ~N(0,1) bf16 [32, qlen, 4, 128]."""
    B, L, W = 32, 131072, 1024
    n = B * W * BLOCK * DIM
    codes = np.empty(n, dtype=np.uint8)
    for c, lo in enumerate(range(0, n, _CHUNK_ELEMS)):
        hi = min(n, lo + _CHUNK_ELEMS)
        codes[lo:hi] = e4m3_codes(4.0 * _child(7, 1, c).standard_normal(hi - lo, dtype=np.float32))
    q = normal_bf16(7, 0, (B, qlen, HEADS, DIM))
    bt = _child(7, 2).permutation(B * W).astype(np.int32).reshape(B, W)
    return Inputs(f"fp8 B=32 x 131072, Q={qlen}", q, codes.reshape(B * W, BLOCK, DIM), bt,
                  np.full(B, L, dtype=np.int32), k_scale=float(k_scale))


# ---------------------------------------------------------------------------
# The five workloads.


def config1() -> Inputs:
    """Batch 1, 8192 tokens (64 full blocks), identity block table."""
    B, L, W = 1, 8192, 64
    q = normal_bf16(1, 0, (B, HEADS, DIM))
    k = normal_bf16(1, 1, (W, BLOCK, DIM))
    bt = np.arange(W, dtype=np.int32).reshape(1, W)
    return Inputs("cfg1 B=1 x 8192", q, k, bt, np.full(B, L, dtype=np.int32))


def config2() -> Inputs:
    """Batch 8, 32768 tokens each (256 blocks), pages a random permutation."""
    B, L, W = 8, 32768, 256
    q = normal_bf16(2, 0, (B, HEADS, DIM))
    k = normal_bf16(2, 1, (B * W, BLOCK, DIM))
    bt = _child(2, 2).permutation(B * W).astype(np.int32).reshape(B, W)
    return Inputs("cfg2 B=8 x 32768", q, k, bt, np.full(B, L, dtype=np.int32))


def config3() -> Inputs:
    """Batch 32, 131072 tokens each (1024 blocks, 1 GiB of index-K), shuffled pages."""
    B, L, W = 32, 131072, 1024
    q = normal_bf16(3, 0, (B, HEADS, DIM))
    k = normal_bf16(3, 1, (B * W, BLOCK, DIM))
    bt = _child(3, 2).permutation(B * W).astype(np.int32).reshape(B, W)
    return Inputs("cfg3 B=32 x 131072", q, k, bt, np.full(B, L, dtype=np.int32))


def config4() -> Inputs:
    """Batch 16 of mixed lengths: one 131072-token row, one empty row, the rest U[1,1024].

    Lengths are drawn first (they size the page pool), then q, K and the page
    permutation. One poison page backs every table entry past a row's end, and
    the invalid tail tokens of partial blocks are poison.
    """
    B, W = 16, 1024
    rng = _child(4, 3)
    rows = rng.permutation(B)
    long_row, empty_row = int(rows[0]), int(rows[1])
    lens = rng.integers(1, 1025, size=B).astype(np.int32)
    lens[long_row] = 131072
    lens[empty_row] = 0
    inp = paged_case(4, lens, W, name="cfg4 B=16 mixed")
    inp.meta.update(long_row=long_row, empty_row=empty_row)
    return inp


# Planted runs for the adversarial workload. Each entry: per-head list of
# (first block, [target score per block of the run]); an empty list plants
# nothing for that head. Scores are exact integers, see config5().
def _cfg5_runs():
    t100 = [100] * 16
    runs = {
        0: [(16, t100)] * 4,                                   # split-aligned run, all tied
        1: [(5, [110, 120, 110, 110, 120, 110, 110, 120, 110, 110, 120, 110, 110, 120, 110, 120])] * 4,
        2: [(0, t100)] * 4,                                    # overlaps pinned initial block
        3: [(52, t100)] * 4,                                   # overlaps both pinned recent blocks
        4: [(32, list(range(115, 99, -1)))] * 4,               # distinct descending targets
        5: [(20, [100] * 10)] * 4,                             # 3 slots left to background ties
        6: [(40, t100), (44, t100), (48, t100), (36, t100)],   # heads disagree
        7: [(48, t100)] * 4,                                   # plus a planted masked tail
        8: [] ,                                                # background only: ties everywhere
        9: [(1, t100)] * 4,
        10: [(50, t100)] * 4,
        11: [(3, t100), (19, t100), (35, t100), (51, t100)],
        12: [(24, [100, 100, 100] + [127] * 13)] * 4,
        13: [(10, [105] * 20)] * 4,                            # more tied winners than slots
        14: [(8, [100, 101] * 8)] * 4,
        15: [(60, [100] * 8)] * 4,                             # reaches the pinned tail blocks
    }
    return {b: (r if r else [(0, [])] * 4) for b, r in runs.items()}


def config5() -> Inputs:
    """Batch 16 x 8700 tokens (68 blocks, last one has 124 valid), planted adversarial scores.

    Every score is an exact small integer, so any fp32 summation order gives
    the same value and the selected IDs must agree bit for bit:
      * q[b,h,:] is +-1 (signs of a seeded normal draw);
      * background index-K entries are uniform in {-1, 0, +1};
      * in each row a run of blocks gets, in token slot h, the vector q[b,h,:]
        with all but its first T entries zeroed, so that token scores exactly
        T >= 100 for head h, far above any background token;
      * row 7 also plants q[b,h,:] itself (score 128) in the invalid tail slots
        124+h of the partial last block, which the pass must ignore.
    Runs cover exact ties, runs aligned and unaligned to splits, runs that
    overlap the pinned initial / recent blocks and heads that disagree.
    """
    B, L, W = 16, 8700, 68
    seed = 5
    sgn = _child(seed, 0).standard_normal((B, HEADS, DIM))
    qf = np.where(sgn >= 0, 1.0, -1.0).astype(np.float32)
    q = bf16_bits(qf)
    n_pages = B * W
    kf = _child(seed, 1).integers(-1, 2, size=(n_pages, BLOCK, DIM)).astype(np.float32)
    bt = _child(seed, 2).permutation(n_pages).astype(np.int32).reshape(B, W)
    planted = {}
    for b, per_head in _cfg5_runs().items():
        for h, (w0, targets) in enumerate(per_head):
            for i, t in enumerate(targets):
                j = w0 + i
                tok = qf[b, h].copy()
                tok[t:] = 0.0
                kf[bt[b, j], h] = tok
                planted[(b, h, j)] = t
    masked_row = 7
    last = (L - 1) // BLOCK
    v = L - last * BLOCK
    for h in range(HEADS):
        kf[bt[masked_row, last], v + h] = qf[masked_row, h]
    k = bf16_bits(kf)
    return Inputs("cfg5 B=16 x 8700 planted", q, k, bt, np.full(B, L, dtype=np.int32),
                  meta={"planted": planted, "masked_row": masked_row})


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def config(i: int) -> Inputs:
    return CONFIGS[i]()
