"""ctypes binding of libmsa_indexer.so (include/msa_indexer.h).

Argument marshalling only: every step of the pass runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream. There is no fallback: if the
library is missing, or a tensor is not a suitable device tensor, the call raises.
"""
from __future__ import annotations

import ctypes
import functools
import os
import re

from .build import HERE, INCLUDE, library_path

MSA_OK = 0
MSA_ERR_INVALID_ARG = -1
MSA_ERR_WORKSPACE_TOO_SMALL = -2
MSA_ERR_UNSUPPORTED = -3
MSA_ERR_HIP = -4

ENGINE_DEFAULT = 0
ENGINE_VALU = 1
ENGINE_MFMA = 2

DEVERR_PAGE_OUT_OF_RANGE = 1

HEADS = 4
DIM = 128
BLOCK = 128
MAX_TOPK = 64

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F32 = ctypes.c_float

_SIGNATURES = {
    "msa_status_string": ([_I32], ctypes.c_char_p),
    "msa_indexer_num_splits": ([_I32, _I32, _I32, _I32], _I32),
    "msa_indexer_workspace_bytes": ([_I32, _I32, _I32, _I32], _SZ),
    "msa_indexer_plan": ([_I32, _I32, _I32, _I32, _P, _P, _P, _P], _I32),
    "msa_indexer_decode": ([_P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _I32, _P, _P, _P,
                            _SZ, _I32, _P], _I32),
    "msa_indexer_decode_noalloc": ([_P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _I32, _P, _P,
                                    _P, _I32, _P], _I32),
    "msa_indexer_decode_engine": ([_P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _I32, _P, _P,
                                   _P, _SZ, _I32, _I32, _P], _I32),
    "msa_indexer_decode_pages": ([_P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _I32, _P, _P,
                                  _P, _P, _P, _SZ, _I32, _I32, _P], _I32),
    "msa_indexer_expand_pages": ([_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P], _I32),
    "msa_indexer_expand_pages_multi": ([_P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P], _I32),
    "msa_indexer_workspace_bytes_multi": ([_I32, _I32, _I32, _I32, _I32], _SZ),
    "msa_indexer_decode_multi": ([_P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _I32, _I32, _P,
                                  _P, _P, _SZ, _I32, _P], _I32),
    "msa_indexer_block_scores_multi": ([_P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _P, _I32, _P],
                                       _I32),
    "msa_indexer_decode_fp8": ([_P, _P, _F32, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _I32, _I32,
                                _P, _P, _P, _SZ, _I32, _P], _I32),
    "msa_indexer_block_scores_fp8": ([_P, _P, _F32, _P, _P, _I32, _I32, _I32, _I64, _I32, _P, _I32,
                                      _P], _I32),
    "msa_indexer_split_topk": ([_P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _I32, _P, _SZ,
                                _I32, _I32, _P], _I32),
    "msa_indexer_merge": ([_P, _I32, _I32, _I32, _P, _P, _P, _SZ, _I32, _P], _I32),
    "msa_indexer_block_scores": ([_P, _P, _P, _P, _I32, _I32, _I32, _I64, _P, _I32, _I32, _P],
                                 _I32),
    "msa_indexer_read_error": ([_P, _P, _P], _I32),
}

_lib = None


class MsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status} ({status_string(status)})")
        self.status = status


def header_functions() -> list[str]:
    """Names of the functions include/msa_indexer.h declares."""
    text = open(os.path.join(INCLUDE, "msa_indexer.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(msa_\w+)\s*\(", text)


def load(path: str | None = None):
    """Loads the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with sparse_attention_block_amd.build.build() "
                           "(or __graft_entry__.build()); there is no non-HIP fallback")
    # The library needs libamdhip64.so.7. PyTorch ships its own HIP runtime under that soname
    # but links it by another name, so loading the library first would bring in the system's
    # runtime and then PyTorch its copy: two runtimes in one process, and the library's
    # launches on PyTorch's streams and memory fail. With PyTorch loaded first, the library
    # binds to the runtime already in the process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path == library_path():
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().msa_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != MSA_OK:
        raise MsaError(fn, status)


def num_splits(batch: int, max_blocks: int, topk: int, splits: int = 0) -> int:
    s = load().msa_indexer_num_splits(batch, max_blocks, topk, splits)
    _check("msa_indexer_num_splits", min(s, 0))
    return s


def plan(batch: int, max_blocks: int, topk: int, splits: int = 0) -> dict:
    """The library's plan (msa_indexer_plan): splits per row, blocks per split, candidates
    kept per split and head, fused merge. blocks_per_split = 0 marks the device plan, whose
    split width is chosen per call from seq_lens; splits is then the list capacity per row
    (the workspace holds splits * topk keys per row and head)."""
    out = [ctypes.c_int32() for _ in range(4)]
    rc = load().msa_indexer_plan(batch, max_blocks, topk, splits, *[ctypes.byref(o) for o in out])
    _check("msa_indexer_plan", rc)
    return {"splits": out[0].value, "blocks_per_split": out[1].value,
            "candidates_per_split": out[2].value, "fused": bool(out[3].value)}


def workspace_bytes(batch: int, max_blocks: int, topk: int, splits: int = 0) -> int:
    return int(load().msa_indexer_workspace_bytes(batch, max_blocks, topk, splits))


# ---------------------------------------------------------------------------
# Tensor marshalling.

def _torch():
    import torch
    return torch


def _dev(t, name, dtype, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return _P(t.data_ptr())


def _on_tensor_device(fn):
    """Runs a call with the device of its tensors current, so that its default stream and
    the stream the kernels go to are that device's. Tensors on several devices, or a stream
    of another device, are refused (a kernel would be handed another device's memory)."""
    @functools.wraps(fn)
    def call(*args, **kwargs):
        torch = _torch()
        devs = {a.device for a in (*args, *kwargs.values()) if isinstance(a, torch.Tensor) and a.is_cuda}
        if not devs:
            return fn(*args, **kwargs)  # host tensors: the marshalling refuses them
        if len(devs) > 1:
            raise ValueError(f"{fn.__name__}: tensors on several devices: {sorted(map(str, devs))}")
        dev = devs.pop()
        stream = kwargs.get("stream")
        if stream is not None and stream.device != dev:
            raise ValueError(f"{fn.__name__}: stream of {stream.device}, tensors on {dev}")
        with torch.cuda.device(dev):
            return fn(*args, **kwargs)
    return call


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return _P(s.cuda_stream)


def _inputs(q, k_cache, block_table, seq_lens):
    torch = _torch()
    B = q.shape[0]
    if q.dim() != 3 or tuple(q.shape[1:]) != (HEADS, DIM):
        raise ValueError("q: expected [batch, 4, 128]")
    if k_cache.dim() != 3 or tuple(k_cache.shape[1:]) != (BLOCK, DIM):
        raise ValueError("k_cache: expected [pages, 128, 128]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table: expected [batch, max_blocks]")
    ptrs = (_dev(q, "q", torch.bfloat16), _dev(k_cache, "k_cache", torch.bfloat16),
            _dev(block_table, "block_table", torch.int32),
            _dev(seq_lens, "seq_lens", torch.int32, (B,)))
    return ptrs, B, block_table.shape[1], block_table.stride(0), k_cache.shape[0]


WS_HEADER_BYTES = 256   # MSA_WORKSPACE_HEADER_BYTES
WS_ROW_BYTES = 4352     # MSA_WORKSPACE_ROW_BYTES: the counter lines of one row

_WS_CACHE = {}


def _default_workspace(nbytes: int, batch: int, device, stream):
    """The workspace of a call that passes none: one zeroed buffer per (device, stream),
    reused by every such call on that stream. The library keeps each row's counter lines at
    a fixed offset and a call's keys at the end of the buffer, so a buffer serves any call
    whose batch's counter lines plus key region fit it; it is replaced by a larger zeroed one
    when a call needs more (the largest batch seen times the counter lines per row, plus the
    largest key region seen). Calls on one stream run in order, so they never use it at the
    same time, and the old buffer goes back to torch's allocator on that stream. Under graph
    capture a fresh buffer is made instead (it then belongs to the graph's memory)."""
    torch = _torch()
    if nbytes == 0:
        raise ValueError("invalid arguments for a workspace")
    if torch.cuda.is_current_stream_capturing():
        return torch.zeros(nbytes, dtype=torch.uint8, device=device)
    s = torch.cuda.current_stream(device) if stream is None else stream
    key = (device.index, s.cuda_stream)
    rows, keys = batch, nbytes - WS_HEADER_BYTES - WS_ROW_BYTES * batch
    ent = _WS_CACHE.get(key)
    if ent is not None and ent[1] >= rows and ent[2] >= keys:
        return ent[0]
    if ent is not None:
        rows, keys = max(rows, ent[1]), max(keys, ent[2])
    ws = torch.zeros(WS_HEADER_BYTES + WS_ROW_BYTES * rows + keys, dtype=torch.uint8, device=device)
    _WS_CACHE[key] = (ws, rows, keys)
    return ws


def new_workspace(batch: int, max_blocks: int, topk: int, splits: int = 0, device="cuda"):
    """A zeroed workspace tensor (uint8) of the size the library asks for."""
    torch = _torch()
    n = workspace_bytes(batch, max_blocks, topk, splits)
    if n == 0:
        raise ValueError("invalid arguments for a workspace")
    return torch.zeros(n, dtype=torch.uint8, device=device)


@_on_tensor_device
def msa_indexer_decode(q, k_cache, block_table, seq_lens, topk=16, n_init=1, n_local=2,
                       out_ids=None, out_scores=None, workspace=None, num_splits=0, stream=None,
                       engine=None):
    """The decode pass. Returns (out_ids int32 [B,4,topk], out_scores fp32 [B,4,topk]).
    With `engine` set, calls msa_indexer_decode_engine instead."""
    torch = _torch()
    (pq, pk, pbt, pl), B, W, stride, pages = _inputs(q, k_cache, block_table, seq_lens)
    if out_ids is None:
        out_ids = torch.empty((B, HEADS, topk), dtype=torch.int32, device=q.device)
    if out_scores is None:
        out_scores = torch.empty((B, HEADS, topk), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _default_workspace(workspace_bytes(B, W, topk, num_splits), B, q.device, stream)
    args = [pq, pk, pbt, pl, B, W, stride, pages, topk, n_init, n_local,
            _dev(out_ids, "out_ids", torch.int32, (B, HEADS, topk)),
            _dev(out_scores, "out_scores", torch.float32, (B, HEADS, topk)),
            _dev(workspace, "workspace", torch.uint8), workspace.numel(), num_splits]
    if engine is None:
        rc = load().msa_indexer_decode(*args, _stream(stream))
        _check("msa_indexer_decode", rc)
    else:
        rc = load().msa_indexer_decode_engine(*args, engine, _stream(stream))
        _check("msa_indexer_decode_engine", rc)
    return out_ids, out_scores


def _bound(name: str, args: list):
    """A zero-argument call of C entry point `name` with arguments marshalled once: the tensors'
    addresses and the stream are fixed, so each call costs one ctypes call and no Python-side
    checks (for timing loops that must keep the launch queue full)."""
    fn = getattr(load(), name)
    args = tuple(args)

    def call():
        rc = fn(*args)
        if rc != MSA_OK:
            raise MsaError(name, rc)
    return call


@_on_tensor_device
def bind_decode(q, k_cache, block_table, seq_lens, topk, n_init, n_local, out_ids, out_scores,
                workspace, num_splits=0, stream=None):
    """msa_indexer_decode on these tensors, marshalled once: returns a zero-argument callable
    that enqueues the call on `stream` (default: the current stream now)."""
    torch = _torch()
    (pq, pk, pbt, pl), B, W, stride, pages = _inputs(q, k_cache, block_table, seq_lens)
    return _bound("msa_indexer_decode", [
        pq, pk, pbt, pl, B, W, stride, pages, topk, n_init, n_local,
        _dev(out_ids, "out_ids", torch.int32, (B, HEADS, topk)),
        _dev(out_scores, "out_scores", torch.float32, (B, HEADS, topk)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), num_splits, _stream(stream)])


@_on_tensor_device
def bind_decode_multi(q, k_cache, block_table, seq_lens, topk, n_init, n_local, out_ids, out_scores,
                      workspace, num_splits=0, stream=None, k_scale=None):
    """msa_indexer_decode_multi (or, with k_scale, msa_indexer_decode_fp8 over a uint8 E4M3 cache)
    on these tensors, marshalled once: a zero-argument callable."""
    torch = _torch()
    fp8 = k_scale is not None
    (pq, pk, pbt, pl), B, Q, W, stride, pages = _inputs_multi(q, k_cache, block_table, seq_lens,
                                                              torch.uint8 if fp8 else None)
    head = [pq, pk, _F32(float(k_scale))] if fp8 else [pq, pk]
    return _bound("msa_indexer_decode_fp8" if fp8 else "msa_indexer_decode_multi", head + [
        pbt, pl, B, W, stride, pages, Q, topk, n_init, n_local,
        _dev(out_ids, "out_ids", torch.int32, (B, Q, HEADS, topk)),
        _dev(out_scores, "out_scores", torch.float32, (B, Q, HEADS, topk)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), num_splits, _stream(stream)])


@_on_tensor_device
def msa_indexer_decode_noalloc(q, k_cache, block_table, seq_lens, topk=16, n_init=1, n_local=2,
                               out_ids=None, out_scores=None, error_flags=None, num_splits=0,
                               stream=None):
    """The decode pass on the library's own scratch array instead of a workspace (the library
    allocates nothing; pass out_ids / out_scores to allocate nothing here either).
    error_flags: optional int32 [1] device tensor the device error bits are OR-ed into.
    Returns (out_ids, out_scores)."""
    torch = _torch()
    (pq, pk, pbt, pl), B, W, stride, pages = _inputs(q, k_cache, block_table, seq_lens)
    if out_ids is None:
        out_ids = torch.empty((B, HEADS, topk), dtype=torch.int32, device=q.device)
    if out_scores is None:
        out_scores = torch.empty((B, HEADS, topk), dtype=torch.float32, device=q.device)
    flags = _P(None) if error_flags is None else _dev(error_flags, "error_flags", torch.int32, (1,))
    rc = load().msa_indexer_decode_noalloc(
        pq, pk, pbt, pl, B, W, stride, pages, topk, n_init, n_local,
        _dev(out_ids, "out_ids", torch.int32, (B, HEADS, topk)),
        _dev(out_scores, "out_scores", torch.float32, (B, HEADS, topk)), flags, num_splits,
        _stream(stream))
    _check("msa_indexer_decode_noalloc", rc)
    return out_ids, out_scores


@_on_tensor_device
def msa_indexer_decode_pages(q, k_cache, block_table, seq_lens, topk=16, n_init=1, n_local=2,
                             out_ids=None, out_scores=None, out_pages=None, out_tokens=None,
                             workspace=None, num_splits=0, engine=ENGINE_DEFAULT, stream=None):
    """The decode pass plus its 16-token page table. Returns (out_ids, out_scores,
    out_pages int32 [B,4,8*topk], out_tokens int32 [B,4])."""
    torch = _torch()
    (pq, pk, pbt, pl), B, W, stride, pages = _inputs(q, k_cache, block_table, seq_lens)
    dev = q.device
    out_ids = torch.empty((B, HEADS, topk), dtype=torch.int32, device=dev) if out_ids is None else out_ids
    if out_scores is None:
        out_scores = torch.empty((B, HEADS, topk), dtype=torch.float32, device=dev)
    if out_pages is None:
        out_pages = torch.empty((B, HEADS, 8 * topk), dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, HEADS), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = _default_workspace(workspace_bytes(B, W, topk, num_splits), B, dev, stream)
    rc = load().msa_indexer_decode_pages(
        pq, pk, pbt, pl, B, W, stride, pages, topk, n_init, n_local,
        _dev(out_ids, "out_ids", torch.int32, (B, HEADS, topk)),
        _dev(out_scores, "out_scores", torch.float32, (B, HEADS, topk)),
        _dev(out_pages, "out_pages", torch.int32, (B, HEADS, 8 * topk)),
        _dev(out_tokens, "out_tokens", torch.int32, (B, HEADS)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), num_splits, engine,
        _stream(stream))
    _check("msa_indexer_decode_pages", rc)
    return out_ids, out_scores, out_pages, out_tokens


@_on_tensor_device
def msa_indexer_expand_pages(ids, block_table, seq_lens, out_pages=None, out_tokens=None,
                             stream=None):
    """16-token page table of given selections ids int32 [B,4,topk]: (out_pages, out_tokens)."""
    torch = _torch()
    if ids.dim() != 3 or ids.shape[1] != HEADS:
        raise ValueError("ids: expected [batch, 4, topk]")
    B, topk = ids.shape[0], ids.shape[2]
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table: expected [batch, max_blocks]")
    if out_pages is None:
        out_pages = torch.empty((B, HEADS, 8 * topk), dtype=torch.int32, device=ids.device)
    if out_tokens is None:
        out_tokens = torch.empty((B, HEADS), dtype=torch.int32, device=ids.device)
    rc = load().msa_indexer_expand_pages(
        _dev(ids, "ids", torch.int32), _dev(block_table, "block_table", torch.int32),
        _dev(seq_lens, "seq_lens", torch.int32, (B,)), B, block_table.shape[1],
        block_table.stride(0), topk, _dev(out_pages, "out_pages", torch.int32, (B, HEADS, 8 * topk)),
        _dev(out_tokens, "out_tokens", torch.int32, (B, HEADS)), _stream(stream))
    _check("msa_indexer_expand_pages", rc)
    return out_pages, out_tokens


def workspace_bytes_multi(batch: int, max_blocks: int, qlen: int, topk: int, splits: int = 0) -> int:
    return int(load().msa_indexer_workspace_bytes_multi(batch, max_blocks, qlen, topk, splits))


def _inputs_multi(q, k_cache, block_table, seq_lens, kv_dtype=None):
    torch = _torch()
    if q.dim() != 4 or tuple(q.shape[2:]) != (HEADS, DIM):
        raise ValueError("q: expected [batch, qlen, 4, 128]")
    B, Q = q.shape[0], q.shape[1]
    if k_cache.dim() != 3 or tuple(k_cache.shape[1:]) != (BLOCK, DIM):
        raise ValueError("k_cache: expected [pages, 128, 128]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table: expected [batch, max_blocks]")
    ptrs = (_dev(q, "q", torch.bfloat16), _dev(k_cache, "k_cache", kv_dtype or torch.bfloat16),
            _dev(block_table, "block_table", torch.int32),
            _dev(seq_lens, "seq_lens", torch.int32, (B,)))
    return ptrs, B, Q, block_table.shape[1], block_table.stride(0), k_cache.shape[0]


@_on_tensor_device
def msa_indexer_decode_multi(q, k_cache, block_table, seq_lens, topk=16, n_init=1, n_local=2,
                             out_ids=None, out_scores=None, workspace=None, num_splits=0,
                             stream=None):
    """Multi-token decode, q [B, Q, 4, 128]: (out_ids int32 [B,Q,4,topk], out_scores fp32)."""
    torch = _torch()
    (pq, pk, pbt, pl), B, Q, W, stride, pages = _inputs_multi(q, k_cache, block_table, seq_lens)
    dev = q.device
    if out_ids is None:
        out_ids = torch.empty((B, Q, HEADS, topk), dtype=torch.int32, device=dev)
    if out_scores is None:
        out_scores = torch.empty((B, Q, HEADS, topk), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _default_workspace(workspace_bytes_multi(B, W, Q, topk, num_splits), B, dev, stream)
    rc = load().msa_indexer_decode_multi(
        pq, pk, pbt, pl, B, W, stride, pages, Q, topk, n_init, n_local,
        _dev(out_ids, "out_ids", torch.int32, (B, Q, HEADS, topk)),
        _dev(out_scores, "out_scores", torch.float32, (B, Q, HEADS, topk)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), num_splits, _stream(stream))
    _check("msa_indexer_decode_multi", rc)
    return out_ids, out_scores


@_on_tensor_device
def msa_indexer_block_scores_multi(q, k_cache, block_table, seq_lens, num_splits=0, out=None,
                                   stream=None):
    """fp32 block scores [B, Q, 4, W] of the multi-token pass; -inf where a position sees no block."""
    torch = _torch()
    (pq, pk, pbt, pl), B, Q, W, stride, pages = _inputs_multi(q, k_cache, block_table, seq_lens)
    if out is None:
        out = torch.empty((B, Q, HEADS, W), dtype=torch.float32, device=q.device)
    rc = load().msa_indexer_block_scores_multi(pq, pk, pbt, pl, B, W, stride, pages, Q,
                                               _dev(out, "out", torch.float32, (B, Q, HEADS, W)),
                                               num_splits, _stream(stream))
    _check("msa_indexer_block_scores_multi", rc)
    return out


@_on_tensor_device
def msa_indexer_decode_fp8(q, k_cache, k_scale, block_table, seq_lens, topk=16, n_init=1,
                           n_local=2, out_ids=None, out_scores=None, workspace=None, num_splits=0,
                           stream=None):
    """Decode over an FP8 E4M3 cache (uint8 codes [pages, 128, 128], scale k_scale), q
    [B, Q, 4, 128]: (out_ids int32 [B,Q,4,topk], out_scores fp32 [B,Q,4,topk])."""
    torch = _torch()
    (pq, pk, pbt, pl), B, Q, W, stride, pages = _inputs_multi(q, k_cache, block_table, seq_lens,
                                                              torch.uint8)
    dev = q.device
    if out_ids is None:
        out_ids = torch.empty((B, Q, HEADS, topk), dtype=torch.int32, device=dev)
    if out_scores is None:
        out_scores = torch.empty((B, Q, HEADS, topk), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _default_workspace(workspace_bytes_multi(B, W, Q, topk, num_splits), B, dev, stream)
    rc = load().msa_indexer_decode_fp8(
        pq, pk, float(k_scale), pbt, pl, B, W, stride, pages, Q, topk, n_init, n_local,
        _dev(out_ids, "out_ids", torch.int32, (B, Q, HEADS, topk)),
        _dev(out_scores, "out_scores", torch.float32, (B, Q, HEADS, topk)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), num_splits, _stream(stream))
    _check("msa_indexer_decode_fp8", rc)
    return out_ids, out_scores


@_on_tensor_device
def msa_indexer_block_scores_fp8(q, k_cache, k_scale, block_table, seq_lens, num_splits=0,
                                 out=None, stream=None):
    """fp32 block scores [B, Q, 4, W] over an FP8 E4M3 cache."""
    torch = _torch()
    (pq, pk, pbt, pl), B, Q, W, stride, pages = _inputs_multi(q, k_cache, block_table, seq_lens,
                                                              torch.uint8)
    if out is None:
        out = torch.empty((B, Q, HEADS, W), dtype=torch.float32, device=q.device)
    rc = load().msa_indexer_block_scores_fp8(pq, pk, float(k_scale), pbt, pl, B, W, stride, pages, Q,
                                             _dev(out, "out", torch.float32, (B, Q, HEADS, W)),
                                             num_splits, _stream(stream))
    _check("msa_indexer_block_scores_fp8", rc)
    return out


@_on_tensor_device
def msa_indexer_expand_pages_multi(ids, block_table, seq_lens, out_pages=None, out_tokens=None,
                                   stream=None):
    """16-token page tables of multi-token selections ids int32 [B,Q,4,topk]:
    (out_pages [B,Q,4,8*topk], out_tokens [B,Q,4])."""
    torch = _torch()
    if ids.dim() != 4 or ids.shape[2] != HEADS:
        raise ValueError("ids: expected [batch, qlen, 4, topk]")
    B, Q, topk = ids.shape[0], ids.shape[1], ids.shape[3]
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table: expected [batch, max_blocks]")
    if out_pages is None:
        out_pages = torch.empty((B, Q, HEADS, 8 * topk), dtype=torch.int32, device=ids.device)
    if out_tokens is None:
        out_tokens = torch.empty((B, Q, HEADS), dtype=torch.int32, device=ids.device)
    rc = load().msa_indexer_expand_pages_multi(
        _dev(ids, "ids", torch.int32), _dev(block_table, "block_table", torch.int32),
        _dev(seq_lens, "seq_lens", torch.int32, (B,)), B, block_table.shape[1],
        block_table.stride(0), Q, topk,
        _dev(out_pages, "out_pages", torch.int32, (B, Q, HEADS, 8 * topk)),
        _dev(out_tokens, "out_tokens", torch.int32, (B, Q, HEADS)), _stream(stream))
    _check("msa_indexer_expand_pages_multi", rc)
    return out_pages, out_tokens


@_on_tensor_device
def msa_indexer_split_topk(q, k_cache, block_table, seq_lens, workspace, topk=16, n_init=1,
                           n_local=2, num_splits=0, engine=ENGINE_DEFAULT, stream=None):
    """Stage 1 alone: per-split top-k candidate keys into `workspace`."""
    torch = _torch()
    (pq, pk, pbt, pl), B, W, stride, pages = _inputs(q, k_cache, block_table, seq_lens)
    rc = load().msa_indexer_split_topk(pq, pk, pbt, pl, B, W, stride, pages, topk, n_init, n_local,
                                       _dev(workspace, "workspace", torch.uint8), workspace.numel(),
                                       num_splits, engine, _stream(stream))
    _check("msa_indexer_split_topk", rc)


@_on_tensor_device
def msa_indexer_merge(seq_lens, max_blocks, workspace, out_ids, out_scores, topk=16,
                      num_splits=0, stream=None):
    """Stage 2 alone: exact merge of the split candidates into out_ids / out_scores."""
    torch = _torch()
    B = seq_lens.shape[0]
    rc = load().msa_indexer_merge(_dev(seq_lens, "seq_lens", torch.int32, (B,)), B, max_blocks, topk,
                                  _dev(out_ids, "out_ids", torch.int32, (B, HEADS, topk)),
                                  _dev(out_scores, "out_scores", torch.float32, (B, HEADS, topk)),
                                  _dev(workspace, "workspace", torch.uint8), workspace.numel(),
                                  num_splits, _stream(stream))
    _check("msa_indexer_merge", rc)


@_on_tensor_device
def msa_indexer_block_scores(q, k_cache, block_table, seq_lens, num_splits=0,
                             engine=ENGINE_DEFAULT, out=None, stream=None):
    """fp32 block scores [B, 4, W]; -inf past each row's end."""
    torch = _torch()
    (pq, pk, pbt, pl), B, W, stride, pages = _inputs(q, k_cache, block_table, seq_lens)
    if out is None:
        out = torch.empty((B, HEADS, W), dtype=torch.float32, device=q.device)
    rc = load().msa_indexer_block_scores(pq, pk, pbt, pl, B, W, stride, pages,
                                         _dev(out, "out", torch.float32, (B, HEADS, W)),
                                         num_splits, engine, _stream(stream))
    _check("msa_indexer_block_scores", rc)
    return out


@_on_tensor_device
def msa_indexer_read_error(workspace, stream=None) -> int:
    """Device error bits of `workspace` (synchronizes the stream, then clears them)."""
    torch = _torch()
    flags = ctypes.c_uint32(0)
    rc = load().msa_indexer_read_error(_dev(workspace, "workspace", torch.uint8),
                                       ctypes.byref(flags), _stream(stream))
    _check("msa_indexer_read_error", rc)
    return int(flags.value)
