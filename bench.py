#!/usr/bin/env python3
"""Decode-step benchmark of the MiniMax-M3 lightning-indexer pass on one MI355X.

One step = one msa_indexer_decode call (a single kernel launch: split scoring, per-split
top-16, and the exact merge by each row's last split) over batch 32 x 131072-token rows (1024 blocks of 128
tokens each, 1 GiB of bf16 index-K behind a shuffled block table), 4 index heads x 128,
top-16 with 1 initial and 2 recent blocks pinned. Inputs are seeded synthetic data,
resident in HBM before timing starts.

Prints one JSON line: the metric is index-K GB/s (bytes = sum seq_len * 128 * 2 per step)
with us/step beside it, a roofline object for the dominant kernel (the fused decode kernel,
timed with HIP events on the launch stream), and the CPU oracle's rate on the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/decode step + index-K GB/s (% of 8 TB/s) at batch 32 × 128K ctx"
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "sparse_attention_block_amd", "csrc", "msa_indexer.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_split_kernel_b32_128k.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def code_hash(text: str) -> str:
    """sha256 (first 16 hex) of HIP/C++ source with its comments and whitespace removed, so
    that an edit of comments alone does not count as a change of the kernel."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def kernel_source_hash() -> str:
    return code_hash(open(KERNEL_SOURCE).read())


def measured_traffic(engine: int):
    """HBM bytes per stage-1 launch from the committed rocprofv3 counter runs, if they were
    taken on the current kernel source; otherwise None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash() or rec.get("engine") != engine:
        return None
    return rec.get("hbm_bytes_per_launch")


def graph_us_per_call(torch, fn, calls: int = 8, replays: int = 100, rounds: int = 7) -> float:
    """The pages' protocol: `calls` back-to-back calls captured in one HIP graph, replayed
    `replays` times per round, median over `rounds` of the per-call time (us)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    per_call = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        per_call.append(e0.elapsed_time(e1) * 1e3 / (replays * calls))
    return statistics.median(per_call)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_passes(inp, budget_s: float, min_repeats: int):
    import oracle
    times = []
    t_start = time.perf_counter()
    while len(times) < min_repeats or time.perf_counter() - t_start < budget_s:
        t0 = time.perf_counter()
        oracle.decode(inp)
        times.append(time.perf_counter() - t0)
    return len(times), statistics.median(times)


def cpu_baseline(inp, budget_s: float = 10.0, min_repeats: int = 3):
    """The oracle as it is, on this host's cores: whole passes over the workload, repeated
    until about budget_s seconds of wall time (at least min_repeats), median pass time; then
    the same on one thread."""
    import oracle
    threads = oracle.num_threads()
    repeats, t = _oracle_passes(inp, budget_s, min_repeats)
    oracle.set_num_threads(1)
    repeats1, t1 = _oracle_passes(inp, budget_s, min_repeats)
    oracle.set_num_threads(threads)
    return {
        "value": round(inp.index_k_bytes / t / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the whole workload (all {inp.batch} rows x {inp.max_blocks} blocks"
                  f"{' x %d positions' % inp.qlen if inp.qlen > 1 else ''}), median of {repeats} "
                  f"passes of scores + selection, fp64, {t * 1e3:.1f} ms/pass",
        "ms_per_step": round(t * 1e3, 3),
        "single_thread": {"value": round(inp.index_k_bytes / t1 / 1e9, 3), "unit": "GB/s",
                          "ms_per_step": round(t1 * 1e3, 3), "passes": repeats1},
        "cpu_model": cpu_model(),
    }


def time_page_table(msa, torch, args, q, k, bt, lens, ids, ws, stream, topk, n_init, n_local,
                    engine, B):
    """The 16-token page table on the same workload: the decode step that also writes it
    (msa_indexer_decode_pages, one launch), and the table alone from given selections
    (msa_indexer_expand_pages). Both are timed like the main step."""
    dev = q.device
    sc = torch.empty((B, 4, topk), dtype=torch.float32, device=dev)
    pages = torch.empty((B, 4, 8 * topk), dtype=torch.int32, device=dev)
    tokens = torch.empty((B, 4), dtype=torch.int32, device=dev)

    def dp():
        msa.msa_indexer_decode_pages(q, k, bt, lens, topk, n_init, n_local, out_ids=ids,
                                     out_scores=sc, out_pages=pages, out_tokens=tokens,
                                     workspace=ws, engine=engine or 0)

    def ex():
        msa.msa_indexer_expand_pages(ids, bt, lens, out_pages=pages, out_tokens=tokens)

    res = {}
    for name, fn in (("decode_pages", dp), ("expand_pages", ex)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        wall_us = (time.perf_counter() - t0) * 1e6 / args.steps
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        res[name] = {"us_per_call": round(wall_us, 2),
                     "kernel_us": round(statistics.mean(e0.elapsed_time(e1) for e0, e1 in ev) * 1e3, 2)}
    # The table alone moves ids (read), table entries (gathered), pages and counts (written).
    res["expand_pages"]["bytes_per_call"] = B * 4 * (topk * 4 + topk * 4 + topk * 32 + 4)
    log(f"page table: {res}")
    return res


def bench_configs(msa, synth, np, torch) -> int:
    """The four smaller workloads, one JSON line each: the decode call under the graph
    protocol on warm inputs, and cycling through enough copies of the inputs (at least 8,
    more than 512 MB together) that no call finds its cache lines left by the previous one."""
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    for i in (1, 2, 4, 5):
        inp = synth.config(i)
        B, W = inp.batch, inp.max_blocks
        copies = max(8, -(-(512 << 20) // (inp.k_cache.nbytes + 1)) + 1)
        k_host = torch.from_numpy(inp.k_cache.view(np.int16))
        ks = [k_host.to(dev).view(torch.bfloat16) for _ in range(copies)]
        q = torch.from_numpy(inp.q.view(np.int16)).to(dev).view(torch.bfloat16)
        bt = torch.from_numpy(inp.block_table).to(dev)
        lens = torch.from_numpy(inp.seq_lens).to(dev)
        ws = msa.new_workspace(B, W, inp.topk, 0, dev)
        ids = torch.empty((B, 4, inp.topk), dtype=torch.int32, device=dev)
        sc = torch.empty((B, 4, inp.topk), dtype=torch.float32, device=dev)

        def call(k):
            msa.msa_indexer_decode(q, k, bt, lens, inp.topk, inp.n_init, inp.n_local, out_ids=ids,
                                   out_scores=sc, workspace=ws)

        warm = graph_us_per_call(torch, lambda: call(ks[0]))

        def rotating():
            for k in ks:
                call(k)
        rot = graph_us_per_call(torch, rotating, calls=1, replays=max(1, 800 // copies)) / copies
        nbytes = inp.index_k_bytes
        print(json.dumps({"config": i, "workload": inp.name, "index_k_bytes": nbytes,
                          "warm_us": round(warm, 2), "rotating_us": round(rot, 2),
                          "rotating_GBs": round(nbytes / (rot * 1e-6) / 1e9, 1),
                          "copies": copies, "plan": msa.plan(B, W, inp.topk)}), flush=True)
        del ks
        torch.cuda.empty_cache()
    return 0


def bench_sweep(msa, np, torch) -> int:
    """The batch x context grid the SGLang PR #41488 Speed Tests table measures (batch 1, 8,
    16, 32 at 8K, 32K and 128K tokens, and batches of 16 and 32 with one 128K row and the rest
    1K), for the bf16 and the FP8 E4M3 cache, one JSON line per shape: the decode call (one
    position) under the graph protocol. The pages' numbers are for four GPUs with
    communication, so they are context, not a comparison. Each shape draws its pages
    without repetition from one random pool (a 1 GiB bf16 cache and a 512 MiB FP8 one,
    ~N(0,1) values), so every call reads distinct pages."""
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    pool_pages = 32768
    k_bf16 = torch.randn((pool_pages, 128, 128), generator=gen, device=dev).to(torch.bfloat16)
    k_fp8 = torch.randn((pool_pages, 128, 128), generator=gen, device=dev).clamp_(-448, 448)
    k_fp8 = k_fp8.to(torch.float8_e4m3fn).view(torch.uint8)
    rng = np.random.default_rng(9)
    shapes = [(b, ctx) for ctx in (8192, 32768, 131072) for b in (1, 8, 16, 32)]
    shapes += [("mixed", 16), ("mixed", 32)]
    for shape in shapes:
        if shape[0] == "mixed":
            B = shape[1]
            lens_np = np.full(B, 1024, dtype=np.int32)
            lens_np[0] = 131072
            name = f"batch {B}: one 131072-token row, the rest 1024"
        else:
            B, ctx = shape
            lens_np = np.full(B, ctx, dtype=np.int32)
            name = f"batch {B} x {ctx}"
        W = int(-(-int(lens_np.max()) // 128))
        nb = -(-lens_np // 128)
        pages = rng.permutation(pool_pages)[:int(nb.sum())].astype(np.int32)
        bt_np = np.zeros((B, W), dtype=np.int32)
        off = 0
        for b in range(B):
            bt_np[b, :nb[b]] = pages[off:off + nb[b]]
            off += nb[b]
        bt = torch.from_numpy(bt_np).to(dev)
        lens = torch.from_numpy(lens_np).to(dev)
        q = torch.randn((B, 4, 128), generator=gen, device=dev).to(torch.bfloat16)
        q1 = q[:, None].contiguous()
        ids = torch.empty((B, 4, 16), dtype=torch.int32, device=dev)
        sc = torch.empty((B, 4, 16), dtype=torch.float32, device=dev)
        ws = msa.new_workspace(B, W, 16, 0, dev)
        ws8 = torch.zeros(msa.workspace_bytes_multi(B, W, 1, 16), dtype=torch.uint8, device=dev)
        tokens = int(lens_np.sum())
        us = graph_us_per_call(torch, lambda: msa.msa_indexer_decode(q, k_bf16, bt, lens, out_ids=ids,
                                                                     out_scores=sc, workspace=ws))
        ids8 = ids.view(B, 1, 4, 16)
        sc8 = sc.view(B, 1, 4, 16)
        us8 = graph_us_per_call(torch, lambda: msa.msa_indexer_decode_fp8(q1, k_fp8, 1.0, bt, lens,
                                                                          out_ids=ids8, out_scores=sc8,
                                                                          workspace=ws8))
        print(json.dumps({"workload": name, "batch": B, "tokens": tokens,
                          "bf16_us": round(us, 2), "bf16_GBs": round(tokens * 256 / (us * 1e-6) / 1e9, 1),
                          "fp8_us": round(us8, 2), "fp8_GBs": round(tokens * 128 / (us8 * 1e-6) / 1e9, 1),
                          "protocol": "8 calls per HIP graph, 100 replays per round, median of 7 rounds"}),
              flush=True)
    return 0


def bench_shard(args, msa, synth, np, torch) -> int:
    """One GPU's share of the benchmark workload under P-way context parallelism (round-robin
    blocks j = local * P + rank, vLLM PR #57832, Solution): for each rank, the decode call on
    its share of the batch 32 x 128K cache (bf16, or FP8 with --fp8, the cache the pages'
    four-GPU figures use) under the graph protocol, one JSON line per rank.
    The cache stays whole and resident (each rank holds it replicated); a rank reads 1/P of
    it. The gathers of q and of the per-rank lists are not part of this single-GPU build."""
    from sparse_attention_block_amd import shard
    P = args.shard
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    kind = "FP8 E4M3" if args.fp8 else "bf16"
    log(f"generating the batch 32 x 131072 workload ({kind} index-K) for {P} ranks")
    inp = synth.fp8_config(1) if args.fp8 else synth.config3()
    q = torch.from_numpy(np.ascontiguousarray(inp.q).view(np.int16)).to(dev).view(torch.bfloat16)
    if args.fp8:
        k = torch.from_numpy(inp.k_cache).to(dev)
    else:
        k = torch.from_numpy(inp.k_cache.view(np.int16)).to(dev).view(torch.bfloat16)
    B = inp.batch
    elem = 1 if args.fp8 else 2
    for r in range(P):
        bt_np, lens_np, ni, nl = shard.rank_share(inp.block_table, inp.seq_lens, P, r,
                                                  inp.n_init, inp.n_local)
        W = bt_np.shape[1]
        bt = torch.from_numpy(bt_np).to(dev)
        lens = torch.from_numpy(lens_np).to(dev)
        if args.fp8:
            ws = torch.zeros(msa.workspace_bytes_multi(B, W, 1, inp.topk), dtype=torch.uint8, device=dev)
            ids = torch.empty((B, 1, 4, inp.topk), dtype=torch.int32, device=dev)
            sc = torch.empty((B, 1, 4, inp.topk), dtype=torch.float32, device=dev)
            fn = lambda: msa.msa_indexer_decode_fp8(q, k, inp.k_scale, bt, lens, inp.topk, ni, nl,
                                                    out_ids=ids, out_scores=sc, workspace=ws)
        else:
            ws = msa.new_workspace(B, W, inp.topk, 0, dev)
            ids = torch.empty((B, 4, inp.topk), dtype=torch.int32, device=dev)
            sc = torch.empty((B, 4, inp.topk), dtype=torch.float32, device=dev)
            fn = lambda: msa.msa_indexer_decode(q, k, bt, lens, inp.topk, ni, nl, out_ids=ids,
                                                out_scores=sc, workspace=ws)
        us = graph_us_per_call(torch, fn)
        nbytes = int(lens_np.astype(np.int64).sum()) * 128 * elem
        gbs = nbytes / (us * 1e-6) / 1e9
        print(json.dumps({"workload": f"rank {r} of {P}: batch 32 x {int(lens_np[0])} tokens "
                                      f"(every {P}th block of the 131072-token rows, {kind} index-K)",
                          "rank": r, "ranks": P, "n_init": ni, "n_local": nl,
                          "index_k_bytes": nbytes, "us_per_call": round(us, 2),
                          "GBs": round(gbs, 1), "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
                          "plan": msa.plan(B, W, inp.topk),
                          "protocol": "8 calls per HIP graph, 100 replays per round, median of 7 rounds"}),
              flush=True)
    return 0


def bench_multi(args, msa, synth, np, torch) -> int:
    """Multi-token decode step (qlen draft positions per row) over the benchmark's cache."""
    Q = args.qlen
    kind = "FP8 E4M3" if args.fp8 else "bf16"
    log(f"generating the batch 32 x 131072 workload ({kind} cache) with {Q} query positions per row")
    inp = synth.fp8_config(Q) if args.fp8 else synth.multi_config(Q)
    B, W, topk, n_init, n_local = inp.batch, inp.max_blocks, inp.topk, inp.n_init, inp.n_local
    nbytes = inp.index_k_bytes
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q = torch.from_numpy(inp.q.view(np.int16)).to(dev).view(torch.bfloat16)
    if args.fp8:
        k = torch.from_numpy(inp.k_cache).to(dev)
    else:
        k = torch.from_numpy(inp.k_cache.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(inp.block_table).to(dev)
    lens = torch.from_numpy(inp.seq_lens).to(dev)
    plan = msa.plan(B, W, topk, args.splits)
    ws = torch.zeros(msa.workspace_bytes_multi(B, W, Q, topk, args.splits), dtype=torch.uint8,
                     device=dev)
    ids = torch.empty((B, Q, 4, topk), dtype=torch.int32, device=dev)
    sc = torch.empty((B, Q, 4, topk), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"inputs resident in HBM; plan {plan}")

    def step():
        if args.fp8:
            msa.msa_indexer_decode_fp8(q, k, inp.k_scale, bt, lens, topk, n_init, n_local,
                                       out_ids=ids, out_scores=sc, workspace=ws,
                                       num_splits=args.splits)
        else:
            msa.msa_indexer_decode_multi(q, k, bt, lens, topk, n_init, n_local, out_ids=ids,
                                         out_scores=sc, workspace=ws, num_splits=args.splits)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    k_ms = statistics.mean(e0.elapsed_time(e1) for e0, e1 in ev)
    if msa.msa_indexer_read_error(ws) != 0:
        log("device error flag set")
        return 1
    graph_us = graph_us_per_call(torch, step)
    ms_per_step = elapsed * 1e3 / args.steps
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    k_gbs = nbytes / (k_ms * 1e-3) / 1e9
    out = {
        "metric": (f"µs/verify step ({Q} draft positions per row)" if Q > 1 else "µs/decode step")
                  + f" + index-K GB/s (% of 8 TB/s) at batch 32 × 128K ctx, {kind} index cache",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x bf16" if args.fp8 else "bf16",
        "data": ("synthetic (seeded N(0,1) bf16 q, E4M3 codes of 4 N(0,1) index-K, shuffled page "
                 "table)") if args.fp8 else
                "synthetic (seeded N(0,1) bf16 q and index-K, shuffled page table)",
        "config": {
            "workload": f"batch 32 x 131072-token rows ({kind} index-K), {Q} query position(s) each (causal), 1024 "
                        "blocks of 128 tokens, 4 index heads x 128, top-16, 1 initial + 2 recent "
                        "blocks pinned",
            "batch": B, "qlen": Q, "seq_len": int(inp.seq_lens[0]), "topk": topk,
            "num_splits": plan["splits"] if plan["blocks_per_split"] else "chosen per call on the device",
            "blocks_per_split": plan["blocks_per_split"] or "chosen per call on the device",
            "index_k_bytes": nbytes,
            "step_call": "msa_indexer_decode_fp8" if args.fp8 else "msa_indexer_decode_multi",
        },
        "roofline": {
            "kernel": "verify_kernel + verify_merge_kernel (the whole step, timed together)",
            "bound": "hbm",
            "achieved": round(k_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(k_gbs / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel_us": round(k_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": nbytes,
        },
        "graph": {"us_per_step": round(graph_us, 2),
                  "GBs": round(nbytes / (graph_us * 1e-6) / 1e9, 2),
                  "protocol": "8 calls per HIP graph, 100 replays per round, median of 7 rounds"},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the same workload")
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--engine", type=int, default=0, help="0 default, 1 VALU dot2, 2 MFMA")
    ap.add_argument("--splits", type=int, default=0, help="0 = automatic split count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step", choices=("decode", "decode_pages"), default="decode",
                    help="the call timed as one step (decode_pages also writes the 16-token page table)")
    ap.add_argument("--qlen", type=int, default=1,
                    help="query positions per row; above 1 the step is a multi-token (draft verify) "
                         "decode of the same cache, msa_indexer_decode_multi")
    ap.add_argument("--fp8", action="store_true",
                    help="an FP8 E4M3 index-K cache (msa_indexer_decode_fp8, 512 MiB at this shape)")
    ap.add_argument("--configs", action="store_true",
                    help="time the four smaller workloads (graph protocol, warm and with rotating "
                         "input copies) instead of the benchmark step")
    ap.add_argument("--sweep", action="store_true",
                    help="time the decode call (bf16 and FP8 caches) over a batch x context grid "
                         "instead of the benchmark step")
    ap.add_argument("--shard", type=int, default=0, metavar="P",
                    help="time each rank's share of the benchmark workload under P-way context "
                         "parallelism (round-robin blocks), on this one GPU")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip timing the page-table entry points")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (for scaling HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        # A plain device-to-device copy of exactly 1 GiB, to calibrate FETCH_SIZE/WRITE_SIZE.
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.warmup + args.steps} x 1 GiB")
        return 0

    import sparse_attention_block_amd as msa
    from sparse_attention_block_amd import synth

    lib = msa.load()  # raises if the HIP library is not built
    if args.configs:
        return bench_configs(msa, synth, np, torch)
    if args.sweep:
        return bench_sweep(msa, np, torch)
    if args.shard:
        return bench_shard(args, msa, synth, np, torch)
    if args.qlen != 1 or args.fp8:
        return bench_multi(args, msa, synth, np, torch)
    log("generating the batch 32 x 131072 workload (1 GiB of bf16 index-K)")
    t0 = time.time()
    inp = synth.config3()
    log(f"generated in {time.time() - t0:.1f} s")
    B, W, topk, n_init, n_local = inp.batch, inp.max_blocks, inp.topk, inp.n_init, inp.n_local
    nbytes = inp.index_k_bytes

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q = torch.from_numpy(inp.q.view(np.int16)).to(dev).view(torch.bfloat16)
    k = torch.from_numpy(inp.k_cache.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(inp.block_table).to(dev)
    lens = torch.from_numpy(inp.seq_lens).to(dev)
    plan = msa.plan(B, W, topk, args.splits)
    splits = plan["splits"]
    ws = msa.new_workspace(B, W, topk, args.splits, dev)
    ids = torch.empty((B, 4, topk), dtype=torch.int32, device=dev)
    sc = torch.empty((B, 4, topk), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"inputs resident in HBM; plan {plan}, engine {args.engine}")

    stream = torch.cuda.current_stream()
    engine_arg = args.engine if args.engine else None

    pt = torch.empty((B, 4, 8 * topk), dtype=torch.int32, device=dev)
    ptok = torch.empty((B, 4), dtype=torch.int32, device=dev)

    def step(ev0=None, ev1=None):
        # A fused plan is one kernel launch per step (the last split of each row merges
        # it); otherwise stage 1 is timed alone and stage 2 follows it.
        if ev0 is not None:
            ev0.record(stream)
        if plan["fused"] and args.step == "decode_pages":
            msa.msa_indexer_decode_pages(q, k, bt, lens, topk, n_init, n_local, out_ids=ids,
                                         out_scores=sc, out_pages=pt, out_tokens=ptok,
                                         workspace=ws, num_splits=args.splits,
                                         engine=args.engine)
        elif plan["fused"]:
            msa.msa_indexer_decode(q, k, bt, lens, topk, n_init, n_local, out_ids=ids, out_scores=sc,
                                   workspace=ws, num_splits=args.splits, engine=engine_arg)
        else:
            msa.msa_indexer_split_topk(q, k, bt, lens, ws, topk, n_init, n_local,
                                       num_splits=args.splits, engine=args.engine)
        if ev1 is not None:
            ev1.record(stream)
        if not plan["fused"]:
            msa.msa_indexer_merge(lens, W, ws, ids, sc, topk, num_splits=args.splits)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # Timed region: K back-to-back steps, bracketed by synchronizations, with nothing else
    # in the stream (event markers between launches would add a few us of queue gap each).
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    log(f"timed {args.steps} steps in {elapsed:.3f} s")

    # Kernel timing: the same K steps again, each launch of the dominant kernel bracketed
    # by HIP events on the stream it is launched on.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for e0, e1 in ev:
        step(e0, e1)
    torch.cuda.synchronize()
    kernel_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    if msa.msa_indexer_read_error(ws) != 0:
        log("device error flag set")
        return 1

    graph_us = graph_us_per_call(torch, step)
    log(f"graph protocol: {graph_us:.2f} us per call")

    extra = {}
    if plan["fused"] and not args.no_extra:
        extra = time_page_table(msa, torch, args, q, k, bt, lens, ids, ws, stream, topk, n_init,
                                n_local, engine_arg, B)

    ms_per_step = elapsed * 1e3 / args.steps
    us_per_step = ms_per_step * 1e3
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    k_ms = statistics.mean(kernel_ms)
    k_gbs = nbytes / (k_ms * 1e-3) / 1e9
    engine = args.engine if args.engine else 1
    traffic = measured_traffic(engine)

    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(us_per_step, 2),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q and index-K, shuffled page table)",
        "config": {
            "workload": "batch 32 x 131072-token rows, 1024 blocks of 128 tokens, 4 index heads x 128, "
                        "top-16, 1 initial + 2 recent blocks pinned",
            "batch": B, "seq_len": int(inp.seq_lens[0]), "index_heads": 4, "head_dim": 128,
            "block_tokens": 128, "topk": topk, "n_init": n_init, "n_local": n_local,
            "num_splits": splits if plan["blocks_per_split"] else "chosen per call on the device",
            "blocks_per_split": plan["blocks_per_split"] or "chosen per call on the device",
            "fused_merge": plan["fused"], "engine": engine, "index_k_bytes": nbytes,
            "step_call": "msa_indexer_decode_pages" if args.step == "decode_pages" and plan["fused"]
                         else "msa_indexer_decode",
        },
        "roofline": {
            "kernel": ("split_kernel, fused: block scores + per-split top-16 + merge by each row's "
                       "last split (the whole step)") if plan["fused"] else
                      "split_kernel (stage 1: block scores + per-split top-16)",
            "bound": "hbm",
            "achieved": round(k_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(k_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel_us": round(k_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": nbytes,
        },
    }
    out["graph"] = {"us_per_step": round(graph_us, 2),
                    "GBs": round(nbytes / (graph_us * 1e-6) / 1e9, 2),
                    "protocol": "8 calls per HIP graph, 100 replays per round, median of 7 rounds"}
    if extra:
        out["page_table"] = extra
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the same workload")
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
