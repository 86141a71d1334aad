"""The C ABI without a GPU: the library loads, exports what the header declares, and
rejects bad arguments on the host before any HIP call (vLLM PR #57832, Test Result:
unsupported configurations fail at startup instead of running)."""
import ctypes
import os
import subprocess

import pytest

from sparse_attention_block_amd import _lib
from sparse_attention_block_amd.build import library_path

OK, INVALID, WS_SMALL, UNSUPPORTED = 0, -1, -2, -3

# Aligned, never-dereferenced stand-ins for device pointers: every call below must be
# refused by the host-side checks, so nothing ever reaches the device.
FAKE = 1 << 20
CTR = 17 * 256  # counter bytes per row: the row counter and 16 group counters, a 256-byte line each


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(library_path()):
        from sparse_attention_block_amd.build import build
        build()
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    declared = _lib.header_functions()
    assert len(declared) >= 8
    out = subprocess.run(["nm", "-D", "--defined-only", library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    for code in (OK, INVALID, WS_SMALL, UNSUPPORTED, -4):
        assert lib.msa_status_string(code)
    assert lib.msa_status_string(123) == b"unknown status"


def test_split_plan(lib):
    ns = lib.msa_indexer_num_splits
    # Automatic plan with W <= 4096 and topk <= 16: chosen on the device; the host reports the
    # most splits a row can get (64, or ceil(W/4) for narrow tables).
    assert ns(32, 1024, 16, 0) == 64
    assert ns(16, 4096, 16, 0) == 64
    assert ns(8, 1024, 16, 0) == 64
    # small tables (batch * W < 8192 blocks) keep the host plan; the smallest (batch * W <= 512
    # blocks) split into single blocks (up to 256 blocks) or pairs, for the spread layout
    assert ns(1, 64, 16, 0) == 64
    assert ns(4, 64, 16, 0) == 64
    assert ns(2, 200, 16, 0) == 100
    assert ns(3, 200, 16, 0) == 50
    # where 4-block splits would put a few CUs at two workgroups, rows of 4..64 take 256 / batch
    # even splits of at most 5 blocks (widths C - 1 and C), one workgroup per CU
    assert ns(16, 68, 16, 0) == 16
    assert ns(4, 300, 16, 0) == 64
    assert ns(32, 68, 16, 0) == 17      # 8 even splits would be 9 blocks wide: kept
    assert ns(16, 64, 16, 0) == 16      # 256 workgroups already
    assert ns(7, 1024, 16, 0) == 128
    # Wider tables or larger topk: the host plan, about batch*W/1024 blocks per split.
    assert ns(32, 1024, 17, 0) == 32
    assert ns(1, 8192, 16, 0) == 256
    # Requested counts are honoured up to empty trailing splits.
    assert ns(16, 68, 16, 4) == 4
    assert ns(16, 68, 16, 60) == 34
    assert ns(1, 1024, 16, 1024) == 256            # at most 256 splits per row
    assert ns(1, 1024, 64, 0) == 256               # 4-block splits keep 4 keys: S * Lk <= 4096
    assert ns(1, 0, 16, 0) == 1
    assert ns(1, 16385, 16, 0) == UNSUPPORTED
    assert ns(1, 8192, 64, 0) == UNSUPPORTED       # 128 blocks per split needed
    assert ns(-1, 8, 16, 0) == INVALID
    assert ns(1, 8, 0, 0) == INVALID and ns(1, 8, 65, 0) == INVALID
    assert ns(1, 8, 16, -1) == INVALID


def test_workspace_size(lib):
    ws = lib.msa_indexer_workspace_bytes
    # error word (256 B), 17 256-byte counter lines per row (CTR), then the keys: per row, the
    # most any plan of this (W, topk, num_splits) may write at any batch size. Automatic split
    # counts: the device plan (S = min(64, ceil(W/4)) lists of topk keys per row and head, which
    # any of its split widths fits) or a host plan of 4 .. 64 blocks per split.
    assert ws(32, 1024, 16, 0) == 256 + 32 * CTR + 32 * 64 * 4 * 16 * 8
    assert ws(32, 1024, 16, 32) == 256 + 32 * CTR + 32 * 32 * 4 * 16 * 8
    # batch 16 x 68 blocks runs the host plan, but a larger batch of the same width would
    # take the device plan (17 lists of 16 keys per head), so the rows are sized for it
    assert ws(16, 68, 16, 0) == 256 + 16 * CTR + 16 * 17 * 4 * 16 * 8
    assert ws(16, 68, 16, 17) == 256 + 16 * CTR + 16 * 17 * 4 * 4 * 8   # 4-block splits keep 4 keys
    # past the device plan's widths (W > 4096): the host plan of the smallest split width
    assert ws(1, 8192, 16, 0) == 256 + CTR + 256 * 4 * 16 * 8
    assert ws(0, 1024, 16, 0) == 256
    assert ws(1, 8, 0, 0) == 0


@pytest.mark.parametrize("W,topk,splits", [(1024, 16, 0), (68, 16, 0), (200, 16, 7), (4097, 16, 0),
                                           (300, 64, 0), (5, 3, 0), (16384, 16, 0), (0, 16, 0)])
def test_workspace_keys_grow_linearly_with_batch(lib, W, topk, splits):
    # The key region is batch times a per-row bound that does not depend on the batch (rounded
    # up to 256 bytes), single-token and multi-token alike: a buffer sized for the largest batch
    # of a shape then holds every smaller batch's keys clear of the larger batch's counter lines.
    for qlen in (0, 1, 4):
        if qlen == 0:
            size = lambda b: lib.msa_indexer_workspace_bytes(b, W, topk, splits)
        else:
            size = lambda b, q=qlen: lib.msa_indexer_workspace_bytes_multi(b, W, q, topk, splits)
        per_row = (size(256) - 256 - 256 * CTR) // 256
        assert per_row > 0
        for b in (1, 2, 3, 4, 7, 8, 31, 64, 100):
            keys = size(b) - 256 - b * CTR
            assert keys == -(-b * per_row // 256) * 256, (qlen, b)


def test_plan_fuses_the_merge_when_it_fits(lib):
    from sparse_attention_block_amd import plan
    # device plan: blocks per split chosen per call (reported as 0)
    assert plan(32, 1024, 16) == {"splits": 64, "blocks_per_split": 0,
                                  "candidates_per_split": 16, "fused": True}
    assert plan(32, 1024, 16, 32) == {"splits": 32, "blocks_per_split": 32,
                                      "candidates_per_split": 16, "fused": True}
    assert plan(1, 64, 16)["fused"] and plan(16, 68, 16)["fused"] and plan(8, 256, 16)["fused"]
    assert plan(16, 1024, 16)["fused"]
    # Host plans past 64 splits fuse while the lists fit the merge network (S * Lk2 <= 1024).
    assert plan(1, 1024, 16) == {"splits": 256, "blocks_per_split": 4,
                                 "candidates_per_split": 4, "fused": True}
    assert plan(1, 1024, 16, 129)["fused"] and plan(6, 1024, 16)["fused"]
    assert not plan(1, 2048, 16)["fused"]  # 256 splits x 8 candidates: 2048 keys per head
    assert not plan(1, 1024, 17)["fused"]  # topk past the network, more than 64 splits
    big = plan(1, 16384, 16)          # 256 splits x 16 candidates: merged by a second kernel
    assert big["splits"] == 256 and not big["fused"]


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, bt=FAKE, lens=FAKE, batch=2, W=8, stride=8, pages=16, topk=16,
             n_init=1, n_local=2, ids=FAKE, scores=FAKE, ws=FAKE, ws_bytes=1 << 20, splits=0,
             stream=None)
    a.update(kw)
    return lib.msa_indexer_decode(a["q"], a["k"], a["bt"], a["lens"], a["batch"], a["W"],
                                  a["stride"], a["pages"], a["topk"], a["n_init"], a["n_local"],
                                  a["ids"], a["scores"], a["ws"], a["ws_bytes"], a["splits"],
                                  a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID),
    (dict(k=None), INVALID),
    (dict(bt=None), INVALID),
    (dict(lens=None), INVALID),
    (dict(ids=None), INVALID),
    (dict(scores=None), INVALID),
    (dict(ws=None), INVALID),
    (dict(q=FAKE + 8), INVALID),            # 16-byte alignment of q
    (dict(k=FAKE + 2), INVALID),            # 16-byte alignment of the cache
    (dict(ws=FAKE + 64), INVALID),          # 256-byte alignment of the workspace
    (dict(ids=FAKE + 2), INVALID),
    (dict(batch=-1), INVALID),
    (dict(W=-1), INVALID),
    (dict(stride=7), INVALID),              # stride below the table width
    (dict(pages=-1), INVALID),
    (dict(topk=0), INVALID),
    (dict(topk=65), INVALID),
    (dict(n_init=-1), INVALID),
    (dict(n_local=-1), INVALID),
    (dict(n_init=10, n_local=7), INVALID),  # pins exceed topk
    (dict(splits=-3), INVALID),
    (dict(W=16385, stride=16385), UNSUPPORTED),
    (dict(ws_bytes=255), WS_SMALL),
])
def test_decode_rejects_on_host(lib, kw, code):
    assert _decode(lib, **kw) == code


def test_batch_zero_is_a_no_op(lib):
    assert _decode(lib, batch=0, q=None, k=None, bt=None, lens=None, ids=None, scores=None,
                   ws=None, ws_bytes=0) == OK


def _decode_noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE, bt=FAKE, lens=FAKE, batch=2, W=8, stride=8, pages=16, topk=16,
             n_init=1, n_local=2, ids=FAKE, scores=FAKE, flags=None, splits=0, stream=None)
    a.update(kw)
    return lib.msa_indexer_decode_noalloc(a["q"], a["k"], a["bt"], a["lens"], a["batch"], a["W"],
                                          a["stride"], a["pages"], a["topk"], a["n_init"],
                                          a["n_local"], a["ids"], a["scores"], a["flags"],
                                          a["splits"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID),
    (dict(lens=None), INVALID),
    (dict(ids=None), INVALID),
    (dict(scores=FAKE + 2), INVALID),
    (dict(flags=FAKE + 2), INVALID),        # the optional error word must be 4-byte aligned
    (dict(topk=65), INVALID),
    (dict(n_init=10, n_local=7), INVALID),
    (dict(W=16385, stride=16385), UNSUPPORTED),
    # the scratch array's limits: 256 rows, and the keys after their counter lines
    (dict(batch=257), WS_SMALL),
    (dict(batch=200, W=16384, stride=16384), WS_SMALL),  # 128 KiB of keys per row
])
def test_decode_noalloc_rejects_on_host(lib, kw, code):
    # The allocation-free decode checks every argument, and its scratch limits, before it
    # touches the device (its scratch set-up included).
    assert _decode_noalloc(lib, **kw) == code


def test_decode_noalloc_batch_zero_is_a_no_op(lib):
    assert _decode_noalloc(lib, batch=0, q=None, k=None, bt=None, lens=None, ids=None,
                           scores=None) == OK


def test_stage_entry_points_reject_on_host(lib):
    st = lib.msa_indexer_split_topk(FAKE, FAKE, FAKE, FAKE, 2, 8, 8, 16, 16, 1, 2, FAKE, 1 << 20,
                                    0, 7, None)
    assert st == INVALID                     # unknown engine
    st = lib.msa_indexer_split_topk(FAKE, FAKE, FAKE, FAKE, 2, 8, 8, 16, 16, 1, 2, FAKE, 100, 0, 1,
                                    None)
    assert st == WS_SMALL
    mg = lib.msa_indexer_merge(FAKE, 2, 8, 16, None, FAKE, FAKE, 1 << 20, 0, None)
    assert mg == INVALID
    mg = lib.msa_indexer_merge(FAKE, 2, 8, 16, FAKE, FAKE, FAKE, 8, 0, None)
    assert mg == WS_SMALL
    bs = lib.msa_indexer_block_scores(FAKE, FAKE, FAKE, FAKE, 2, 8, 8, 16, None, 0, 0, None)
    assert bs == INVALID
    bs = lib.msa_indexer_block_scores(FAKE, FAKE, FAKE, FAKE, 2, 8, 8, 16, FAKE, 0, 3, None)
    assert bs == INVALID
    assert lib.msa_indexer_read_error(None, ctypes.byref(ctypes.c_uint32()), None) == INVALID


def _decode_pages(lib, **kw):
    a = dict(q=FAKE, k=FAKE, bt=FAKE, lens=FAKE, batch=2, W=8, stride=8, pages=16, topk=16,
             n_init=1, n_local=2, ids=FAKE, scores=FAKE, pt=FAKE, tok=FAKE, ws=FAKE,
             ws_bytes=1 << 20, splits=0, engine=0, stream=None)
    a.update(kw)
    return lib.msa_indexer_decode_pages(a["q"], a["k"], a["bt"], a["lens"], a["batch"], a["W"],
                                        a["stride"], a["pages"], a["topk"], a["n_init"],
                                        a["n_local"], a["ids"], a["scores"], a["pt"], a["tok"],
                                        a["ws"], a["ws_bytes"], a["splits"], a["engine"],
                                        a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(pt=None), INVALID),
    (dict(tok=None), INVALID),
    (dict(pt=FAKE + 4), INVALID),                # 16-byte alignment of the page table
    (dict(tok=FAKE + 2), INVALID),
    (dict(pages=(1 << 28) + 1), UNSUPPORTED),    # 8 * page would not fit int32
    (dict(engine=3), INVALID),
    (dict(ids=None), INVALID),
    (dict(topk=65), INVALID),
    (dict(ws_bytes=255), WS_SMALL),
])
def test_decode_pages_rejects_on_host(lib, kw, code):
    assert _decode_pages(lib, **kw) == code


def test_decode_pages_batch_zero_is_a_no_op(lib):
    assert _decode_pages(lib, batch=0, q=None, k=None, bt=None, lens=None, ids=None, scores=None,
                         pt=None, tok=None, ws=None, ws_bytes=0) == OK


def _expand(lib, **kw):
    a = dict(ids=FAKE, bt=FAKE, lens=FAKE, batch=2, W=8, stride=8, topk=16, pt=FAKE, tok=FAKE,
             stream=None)
    a.update(kw)
    return lib.msa_indexer_expand_pages(a["ids"], a["bt"], a["lens"], a["batch"], a["W"],
                                        a["stride"], a["topk"], a["pt"], a["tok"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(ids=None), INVALID),
    (dict(bt=None), INVALID),
    (dict(lens=None), INVALID),
    (dict(pt=None), INVALID),
    (dict(tok=None), INVALID),
    (dict(ids=FAKE + 2), INVALID),
    (dict(pt=FAKE + 8), INVALID),
    (dict(batch=-1), INVALID),
    (dict(W=-1), INVALID),
    (dict(stride=7), INVALID),
    (dict(topk=0), INVALID),
    (dict(topk=65), INVALID),
    (dict(W=16385, stride=16385), UNSUPPORTED),
])
def test_expand_pages_rejects_on_host(lib, kw, code):
    assert _expand(lib, **kw) == code


def test_expand_pages_multi_rejects_on_host(lib):
    ex = lib.msa_indexer_expand_pages_multi
    assert ex(FAKE, FAKE, FAKE, 2, 8, 8, 0, 16, FAKE, FAKE, None) == INVALID    # qlen 0
    assert ex(FAKE, FAKE, FAKE, 2, 8, 8, 5, 16, FAKE, FAKE, None) == INVALID    # qlen 5
    assert ex(FAKE, FAKE, FAKE, 2, 8, 8, 4, 65, FAKE, FAKE, None) == INVALID    # topk
    assert ex(FAKE, FAKE, FAKE, 2, 8, 8, 4, 16, FAKE + 4, FAKE, None) == INVALID
    assert ex(None, None, None, 0, 8, 8, 4, 16, None, None, None) == OK


def test_expand_pages_batch_zero_is_a_no_op(lib):
    assert _expand(lib, batch=0, ids=None, bt=None, lens=None, pt=None, tok=None) == OK


def _decode_multi(lib, **kw):
    a = dict(q=FAKE, k=FAKE, bt=FAKE, lens=FAKE, batch=2, W=8, stride=8, pages=16, qlen=4,
             topk=16, n_init=1, n_local=2, ids=FAKE, scores=FAKE, ws=FAKE, ws_bytes=1 << 20,
             splits=0, stream=None)
    a.update(kw)
    return lib.msa_indexer_decode_multi(a["q"], a["k"], a["bt"], a["lens"], a["batch"], a["W"],
                                        a["stride"], a["pages"], a["qlen"], a["topk"], a["n_init"],
                                        a["n_local"], a["ids"], a["scores"], a["ws"], a["ws_bytes"],
                                        a["splits"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(qlen=0), INVALID),
    (dict(qlen=5), INVALID),
    (dict(q=None), INVALID),
    (dict(q=FAKE + 8), INVALID),
    (dict(ids=None), INVALID),
    (dict(scores=FAKE + 1), INVALID),
    (dict(ws=None), INVALID),
    (dict(ws=FAKE + 128), INVALID),
    (dict(stride=7), INVALID),
    (dict(topk=65), INVALID),
    (dict(n_init=9, n_local=8), INVALID),
    (dict(W=16385, stride=16385), UNSUPPORTED),
    (dict(ws_bytes=256 + 2 * CTR + 2 * 2 * 16 * 4 * 8 - 1), WS_SMALL),
])
def test_decode_multi_rejects_on_host(lib, kw, code):
    assert _decode_multi(lib, **kw) == code


def test_decode_multi_workspace_and_no_op(lib):
    ws = lib.msa_indexer_workspace_bytes_multi
    # header, counter lines, then keys [batch][S][qlen*4][Lk]: an 8-block table runs 2 splits of
    # 4 blocks (Lk 4) at batch 2, but the rows are sized for the device plan a larger batch of
    # the same width takes (2 lists of topk keys per task)
    assert ws(2, 8, 4, 16, 0) == 256 + 2 * CTR + 2 * 2 * 16 * 16 * 8
    assert ws(2, 8, 4, 16, 2) == 256 + 2 * CTR + 2 * 2 * 16 * 4 * 8
    # with num_splits = 0 the device plan (S = 64 list slots of topk keys per row and head)
    assert ws(32, 1024, 4, 16, 0) == 256 + 32 * CTR + 32 * 64 * 16 * 16 * 8
    assert ws(32, 1024, 1, 16, 0) == 256 + 32 * CTR + 32 * 64 * 4 * 16 * 8
    assert ws(32, 1024, 4, 16, 32) == 256 + 32 * CTR + 32 * 32 * 16 * 16 * 8
    assert ws(2, 8, 0, 16, 0) == 0 and ws(2, 8, 5, 16, 0) == 0
    assert _decode_multi(lib, ws_bytes=ws(2, 8, 4, 16, 0) - 1) == WS_SMALL
    assert _decode_multi(lib, batch=0, q=None, k=None, bt=None, lens=None, ids=None, scores=None,
                         ws=None, ws_bytes=0) == OK
    bs = lib.msa_indexer_block_scores_multi
    assert bs(FAKE, FAKE, FAKE, FAKE, 2, 8, 8, 16, 4, None, 0, None) == INVALID
    assert bs(FAKE, FAKE, FAKE, FAKE, 2, 8, 8, 16, 5, FAKE, 0, None) == INVALID
    assert bs(None, None, None, None, 0, 8, 8, 16, 4, None, 0, None) == OK


def _decode_fp8(lib, **kw):
    a = dict(q=FAKE, k=FAKE, scale=1.0, bt=FAKE, lens=FAKE, batch=2, W=8, stride=8, pages=16, qlen=1,
             topk=16, n_init=1, n_local=2, ids=FAKE, scores=FAKE, ws=FAKE, ws_bytes=1 << 20,
             splits=0, stream=None)
    a.update(kw)
    return lib.msa_indexer_decode_fp8(a["q"], a["k"], a["scale"], a["bt"], a["lens"], a["batch"],
                                      a["W"], a["stride"], a["pages"], a["qlen"], a["topk"],
                                      a["n_init"], a["n_local"], a["ids"], a["scores"], a["ws"],
                                      a["ws_bytes"], a["splits"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(scale=0.0), INVALID),
    (dict(scale=-1.0), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(qlen=0), INVALID),
    (dict(qlen=5), INVALID),
    (dict(k=None), INVALID),
    (dict(k=FAKE + 8), INVALID),
    (dict(ids=None), INVALID),
    (dict(topk=0), INVALID),
    (dict(ws_bytes=100), WS_SMALL),
])
def test_decode_fp8_rejects_on_host(lib, kw, code):
    assert _decode_fp8(lib, **kw) == code


def test_decode_fp8_no_op_and_scores_rejections(lib):
    assert _decode_fp8(lib, batch=0, q=None, k=None, bt=None, lens=None, ids=None, scores=None,
                       ws=None, ws_bytes=0) == OK
    bs = lib.msa_indexer_block_scores_fp8
    assert bs(FAKE, FAKE, 0.0, FAKE, FAKE, 2, 8, 8, 16, 1, FAKE, 0, None) == INVALID
    assert bs(FAKE, FAKE, 1.0, FAKE, FAKE, 2, 8, 8, 16, 1, None, 0, None) == INVALID
    assert bs(None, None, 1.0, None, None, 0, 8, 8, 16, 1, None, 0, None) == OK


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    from sparse_attention_block_amd import msa_indexer_decode
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16)
    k = torch.zeros((1, 128, 128), dtype=torch.bfloat16)
    bt = torch.zeros((1, 1), dtype=torch.int32)
    lens = torch.zeros((1,), dtype=torch.int32)
    with pytest.raises((ValueError, RuntimeError, AssertionError)):
        msa_indexer_decode(q, k, bt, lens, workspace=torch.zeros(1024, dtype=torch.uint8))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="no non-HIP fallback"):
        _lib.load(str(tmp_path / "absent.so"))


def test_binding_shares_pytorchs_hip_runtime():
    # Loaded through the binding before anything imports PyTorch, the library must still end
    # up on the one HIP runtime PyTorch uses: a second copy of the runtime in the process makes
    # every launch on PyTorch's streams and memory fail.
    pytest.importorskip("torch")
    script = (
        "import re, sys\n"
        f"sys.path.insert(0, {os.path.dirname(os.path.dirname(os.path.abspath(__file__)))!r})\n"
        "from sparse_attention_block_amd import _lib\n"
        "_lib.load()\n"
        "import torch\n"
        "maps = open('/proc/self/maps').read()\n"
        "print(len(set(re.findall(r'\\S*/libamdhip64\\.so\\S*', maps))))\n"
    )
    out = subprocess.run(["python3", "-c", script], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"
