"""CPU oracle for the MiniMax-M3 lightning-indexer decode pass (fp64, plain C).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers. Nothing on the product path
imports this package. The computation itself is in msa_oracle.c, whose header
states the definition it follows and the passages it comes from.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import build, library_path

HEADS = 4


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """Bindings to one build of msa_oracle.c (the default build, or a test's variant)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.msa_oracle_block_scores.argtypes = [P, P, P, P, i32, i32, i32, i64, P]
        lib.msa_oracle_block_scores.restype = ctypes.c_int
        lib.msa_oracle_select.argtypes = [P, P, i32, i32, i32, i32, i32, P, P]
        lib.msa_oracle_select.restype = ctypes.c_int
        lib.msa_oracle_expand_pages.argtypes = [P, P, P, i32, i32, i32, i32, P, P]
        lib.msa_oracle_expand_pages.restype = ctypes.c_int
        lib.msa_oracle_decode_multi.argtypes = [P, P, P, P, i32, i32, i32, i64, i32, i32, i32, i32,
                                                 P, P, P]
        lib.msa_oracle_decode_multi.restype = ctypes.c_int
        f64 = ctypes.c_double
        lib.msa_oracle_block_scores_fp8.argtypes = [P, P, f64, P, P, i32, i32, i32, i64, P]
        lib.msa_oracle_block_scores_fp8.restype = ctypes.c_int
        lib.msa_oracle_decode_multi_fp8.argtypes = [P, P, f64, P, P, i32, i32, i32, i64, i32, i32,
                                                    i32, i32, P, P, P]
        lib.msa_oracle_decode_multi_fp8.restype = ctypes.c_int
        lib.msa_oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.msa_oracle_set_num_threads.restype = None
        lib.msa_oracle_num_threads.argtypes = []
        lib.msa_oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.msa_oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.msa_oracle_set_num_threads(int(n))

    def block_scores(self, q, k_cache, block_table, seq_lens) -> np.ndarray:
        """fp64 block scores [B, 4, W]; -inf at and past each row's end."""
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k_cache = np.ascontiguousarray(k_cache, dtype=np.uint16)
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        B, W = block_table.shape
        assert q.shape == (B, HEADS, 128) and k_cache.shape[1:] == (128, 128)
        assert seq_lens.shape == (B,)
        out = np.empty((B, HEADS, W), dtype=np.float64)
        rc = self.lib.msa_oracle_block_scores(_ptr(q), _ptr(k_cache), _ptr(block_table),
                                              _ptr(seq_lens), B, W, W, k_cache.shape[0], _ptr(out))
        if rc != 0:
            raise ValueError(f"oracle block_scores failed with code {rc}")
        return out

    def select(self, scores, seq_lens, topk: int, n_init: int, n_local: int):
        """Pinned top-k per (row, head): (ids int32 [B,4,topk], scores fp64 [B,4,topk])."""
        scores = np.ascontiguousarray(scores, dtype=np.float64)
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        B, H, W = scores.shape
        assert H == HEADS and seq_lens.shape == (B,)
        ids = np.empty((B, HEADS, topk), dtype=np.int32)
        out = np.empty((B, HEADS, topk), dtype=np.float64)
        rc = self.lib.msa_oracle_select(_ptr(scores), _ptr(seq_lens), B, W, topk, n_init, n_local,
                                        _ptr(ids), _ptr(out))
        if rc != 0:
            raise ValueError(f"oracle select failed with code {rc}")
        return ids, out

    def expand_pages(self, ids, block_table, seq_lens):
        """16-token page tables of selections ids [B,4,topk]: (pages [B,4,8*topk], tokens [B,4])."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        B, H, topk = ids.shape
        W = block_table.shape[1]
        pages = np.empty((B, HEADS, 8 * topk), dtype=np.int32)
        tokens = np.empty((B, HEADS), dtype=np.int32)
        rc = self.lib.msa_oracle_expand_pages(_ptr(ids), _ptr(block_table), _ptr(seq_lens), B, W, W,
                                              topk, _ptr(pages), _ptr(tokens))
        if rc != 0:
            raise ValueError(f"oracle expand_pages failed with code {rc}")
        return pages, tokens

    def decode_multi(self, q, k_cache, block_table, seq_lens, topk: int, n_init: int, n_local: int):
        """Multi-token decode, q [B, Q, 4, 128]: (ids int32 [B,Q,4,topk], selected scores fp64
        [B,Q,4,topk], block scores fp64 [B,Q,4,W])."""
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k_cache = np.ascontiguousarray(k_cache, dtype=np.uint16)
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        B, W = block_table.shape
        assert q.ndim == 4 and q.shape[0] == B and q.shape[2:] == (HEADS, 128)
        Q = q.shape[1]
        blocks = np.empty((B, Q, HEADS, W), dtype=np.float64)
        ids = np.empty((B, Q, HEADS, topk), dtype=np.int32)
        sc = np.empty((B, Q, HEADS, topk), dtype=np.float64)
        rc = self.lib.msa_oracle_decode_multi(_ptr(q), _ptr(k_cache), _ptr(block_table),
                                              _ptr(seq_lens), B, W, W, k_cache.shape[0], Q, topk,
                                              n_init, n_local, _ptr(blocks), _ptr(ids), _ptr(sc))
        if rc != 0:
            raise ValueError(f"oracle decode_multi failed with code {rc}")
        return ids, sc, blocks

    def block_scores_fp8(self, q, k_codes, k_scale: float, block_table, seq_lens) -> np.ndarray:
        """fp64 block scores [B, 4, W] over an FP8 E4M3 cache (uint8 codes) with scale k_scale."""
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k_codes = np.ascontiguousarray(k_codes, dtype=np.uint8)
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        B, W = block_table.shape
        assert q.shape == (B, HEADS, 128) and k_codes.shape[1:] == (128, 128)
        out = np.empty((B, HEADS, W), dtype=np.float64)
        rc = self.lib.msa_oracle_block_scores_fp8(_ptr(q), _ptr(k_codes), float(k_scale),
                                                  _ptr(block_table), _ptr(seq_lens), B, W, W,
                                                  k_codes.shape[0], _ptr(out))
        if rc != 0:
            raise ValueError(f"oracle block_scores_fp8 failed with code {rc}")
        return out

    def decode_multi_fp8(self, q, k_codes, k_scale: float, block_table, seq_lens, topk: int,
                         n_init: int, n_local: int):
        """decode_multi over an FP8 E4M3 cache (uint8 codes) with scale k_scale."""
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k_codes = np.ascontiguousarray(k_codes, dtype=np.uint8)
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        B, W = block_table.shape
        assert q.ndim == 4 and q.shape[0] == B and q.shape[2:] == (HEADS, 128)
        Q = q.shape[1]
        blocks = np.empty((B, Q, HEADS, W), dtype=np.float64)
        ids = np.empty((B, Q, HEADS, topk), dtype=np.int32)
        sc = np.empty((B, Q, HEADS, topk), dtype=np.float64)
        rc = self.lib.msa_oracle_decode_multi_fp8(_ptr(q), _ptr(k_codes), float(k_scale),
                                                  _ptr(block_table), _ptr(seq_lens), B, W, W,
                                                  k_codes.shape[0], Q, topk, n_init, n_local,
                                                  _ptr(blocks), _ptr(ids), _ptr(sc))
        if rc != 0:
            raise ValueError(f"oracle decode_multi_fp8 failed with code {rc}")
        return ids, sc, blocks

    def decode(self, inp):
        """Whole pass on a synth.Inputs: (ids, selected scores, block scores). Inputs with
        several query positions (q [B, Q, 4, 128]) go through decode_multi; an FP8 cache
        (uint8 codes, inp.k_scale) through decode_multi_fp8, with [B, Q, ...] results."""
        if inp.k_cache.dtype == np.uint8:
            q = inp.q if inp.q.ndim == 4 else inp.q[:, None]
            return self.decode_multi_fp8(q, inp.k_cache, inp.k_scale, inp.block_table,
                                         inp.seq_lens, inp.topk, inp.n_init, inp.n_local)
        if inp.q.ndim == 4:
            return self.decode_multi(inp.q, inp.k_cache, inp.block_table, inp.seq_lens, inp.topk,
                                     inp.n_init, inp.n_local)
        s = self.block_scores(inp.q, inp.k_cache, inp.block_table, inp.seq_lens)
        ids, sc = self.select(s, inp.seq_lens, inp.topk, inp.n_init, inp.n_local)
        return ids, sc, s


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        path = library_path()
        if not os.path.exists(path):
            build()
        _default = Oracle(path)
    return _default


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)


def block_scores(q, k_cache, block_table, seq_lens) -> np.ndarray:
    return default().block_scores(q, k_cache, block_table, seq_lens)


def select(scores, seq_lens, topk: int, n_init: int, n_local: int):
    return default().select(scores, seq_lens, topk, n_init, n_local)


def decode(inp):
    return default().decode(inp)


def expand_pages(ids, block_table, seq_lens):
    return default().expand_pages(ids, block_table, seq_lens)


def decode_multi(q, k_cache, block_table, seq_lens, topk: int, n_init: int, n_local: int):
    return default().decode_multi(q, k_cache, block_table, seq_lens, topk, n_init, n_local)
