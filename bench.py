#!/usr/bin/env python3
"""Benchmark of the int8-KV decode hot path on one MI355X.

One step = one decode step of a Qwen3-VL-2B-shaped model at 8K context
(28 layers x 16 query / 8 kv heads, head dim 128, batch 1, paged int8 cache
with 16-token blocks): for every layer, the write path quantizes the current
token's K and V (float32) into its cache slot, then decode attention reads
the layer's 8192 cached tokens.  Inputs are seeded synthetic tensors already
resident in HBM; the 28 layer caches (484 MB) exceed the 256 MB Infinity
Cache, so the layers are streamed from HBM.

Output: one JSON line with the effective HBM bandwidth of the whole step
(algorithmic bytes: int8 K+V codes and float32 steps read by decode, plus the
write path's input read and code/step writes), microseconds per step, a
roofline entry for one decode call (chunk + merge kernel) timed with HIP
events over the timed region on the launch stream, and the CPU oracle timed
on a bounded sample on the host.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
# bytes of other reads between two touches of the same cache data in the timed
# decode workloads: twice the 256 MB Infinity Cache
MALL_FLUSH_BYTES = 512 << 20
TOK_HEAD_BYTES = 2 * 128 + 2 * 4   # K+V codes + K/V float32 steps per (token, kv-head)


# HBM bytes per decode call from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# passes over this benchmark (KiB per dispatch), scaled by what the same
# counters read for a plain 256 MiB device copy (--calibrate-copy 256):
# FETCH_SIZE 131085.3 KiB -> 2.000 bytes per counted byte, WRITE_SIZE
# 262144 KiB -> 1.000.  Valid only for the kernel sources they were taken on.
PMC = {"sources_sha256_16": "9da138b901489462",
       "fetch_kib": {"chunk": 8619.30, "merge": 164.56}, "write_kib": {"chunk": 290.06, "merge": 8.00},
       "fetch_scale": 268435456 / (131085.31 * 1024), "write_scale": 268435456 / (262144.0 * 1024)}


def kernel_sources_digest() -> str:
    import hashlib
    import glob
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "decode_attention_int8_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes one decode call moves (chunk + merge kernels), or None when
    the kernel sources changed since the counters were taken."""
    if kernel_sources_digest() != PMC["sources_sha256_16"]:
        return None
    rd = sum(PMC["fetch_kib"].values()) * 1024 * PMC["fetch_scale"]
    wr = sum(PMC["write_kib"].values()) * 1024 * PMC["write_scale"]
    return int(round(rd + wr))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--layers", type=int, default=28)
    p.add_argument("--ctx", type=int, default=8192)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-configuration summary (batch-32 layer, 64K write and decode, int4 128K)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="CPU time of each oracle sample (one core, then all cores)")
    p.add_argument("--workloads", action="store_true",
                   help="instead of the step benchmark, time every other workload of the hot path (one JSON line each)")
    p.add_argument("--only", default="", metavar="NAMES",
                   help="with --workloads: only the comma-separated workloads (and the set-up they share)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (for scaling memory counters) and exit")
    return p.parse_args()


def calibrate_copy(mib: int):
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give
    the scale between those counters and bytes moved."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}), flush=True)


class Layer:
    """One layer's paged int8 cache and per-step inputs.  All layers share the
    sequence's block table and length (as an engine does: one table per
    sequence, one pool per layer)."""

    def __init__(self, K, W, torch, layer, L, nq, nkv, bs, bt_np, nb, bt, lens):
        shp = (nb, bs, nkv, 128)
        self.k = torch.zeros(shp, dtype=torch.int8, device="cuda")
        self.v = torch.zeros(shp, dtype=torch.int8, device="cuda")
        self.ks = torch.zeros(shp[:3], dtype=torch.float32, device="cuda")
        self.vs = torch.zeros(shp[:3], dtype=torch.float32, device="cuda")
        kf = W.torch_normal((L, nkv, 128), "cuda", (2, layer, 0))
        vf = W.torch_normal((L, nkv, 128), "cuda", (2, layer, 1))
        slots = W.slots_for_positions(bt_np, [0] * L, np.arange(L), bs)
        K.kvq8_quantize_append(self.k, self.v, self.ks, self.vs, kf, vf, torch.from_numpy(slots).cuda())
        self.k_new = kf[L - 1:L].clone()            # the current token's K / V (re-written each step)
        self.v_new = vf[L - 1:L].clone()
        del kf, vf
        self.q = W.torch_normal((1, nq, 128), "cuda", (2, layer, 2))
        self.bt = bt
        self.lens = lens
        self.out = torch.empty((1, nq, 128), dtype=torch.float32, device="cuda")


def _oracle_layer(nq, nkv, bs, L, seed):
    """The CPU workload of one layer: a paged int8 cache of L tokens written
    by the oracle, the current token's rows, and one query row per head."""
    import workloads as W
    from oracle import kvq8 as O8
    r = W.rng(2, 1000, seed)
    bt, nb = W.paged_block_tables(r, [L], bs)
    k = W.normal_f32(r, (L, nkv, 128))
    v = W.normal_f32(r, (L, nkv, 128))
    kp = np.zeros((nb, bs, nkv, 128), np.int8)
    vp = np.zeros_like(kp)
    ks = np.zeros((nb, bs, nkv), np.float32)
    vs = np.zeros_like(ks)
    slots = W.slots_for_positions(bt, [0] * L, np.arange(L), bs)
    O8.quantize_append(kp, vp, ks, vs, k, v, slots)
    q = W.normal_f32(r, (1, nq, 128))
    return dict(bt=bt, kp=kp, vp=vp, ks=ks, vs=vs, k_new=k[-1:], v_new=v[-1:], slot=slots[-1:], q=q)


def _oracle_units_worker(job):
    """One host worker: (kv-head) units of the layer -- write the current
    token's rows of that head, then decode its query heads over L tokens --
    with the oracle unchanged, until `seconds` have passed.  BLAS is pinned to
    one thread.  Returns the number of units done and the seconds taken."""
    nq, nkv, bs, L, seconds, wid = job
    from threadpoolctl import threadpool_limits

    from oracle import kvq8 as O8
    d = _oracle_layer(nq, nkv, bs, L, wid)
    g = nq // nkv
    sm = float(np.float32(1) / np.sqrt(np.float32(128)))
    # each unit is one kv-head's slice of the pools: the oracle sees a one-head cache
    heads = []
    for kh in range(nkv):
        sl = slice(kh, kh + 1)
        heads.append(tuple(np.ascontiguousarray(x[:, :, sl]) for x in (d["kp"], d["vp"], d["ks"], d["vs"]))
                     + (np.ascontiguousarray(d["k_new"][:, sl]), np.ascontiguousarray(d["v_new"][:, sl]),
                        np.ascontiguousarray(d["q"][:, kh * g:(kh + 1) * g])))
    units = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            kp, vp, ks, vs, kn, vn, qh = heads[(units + wid) % nkv]
            O8.quantize_append(kp, vp, ks, vs, kn, vn, d["slot"])
            O8.decode_attention_q8(qh, kp, ks, vp, vs, d["bt"], [L], bs, sm)
            units += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return units, el


def host_workers() -> int:
    """Host cores this process may use, at most 16 (the share of a shared
    host's cores that goes with one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(args, nq, nkv, bs, L, bytes_per_layer):
    """The oracle, untouched, on a bounded sample of the same workload, timed
    twice: whole layers (write the current token, then decode over L tokens)
    on one core, then the layer's independent (kv-head) units spread over
    every usable host core, one worker process each.  Runs before anything
    touches the GPU, so the workers fork from a process with no GPU state."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    from oracle import kvq8 as O8

    sm = float(np.float32(1) / np.sqrt(np.float32(128)))
    d = _oracle_layer(nq, nkv, bs, L, 0)
    layers = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            O8.quantize_append(d["kp"], d["vp"], d["ks"], d["vs"], d["k_new"], d["v_new"], d["slot"])
            O8.decode_attention_q8(d["q"], d["kp"], d["ks"], d["vp"], d["vs"], d["bt"], [L], bs, sm)
            layers += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
    one = bytes_per_layer * layers / el / 1e9

    P = host_workers()
    unit_bytes = bytes_per_layer / nkv
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(P) as pool:
        res = pool.map(_oracle_units_worker, [(nq, nkv, bs, L, args.cpu_seconds, w) for w in range(P)])
    wall = time.perf_counter() - t0
    units = sum(u for u, _ in res)
    span = max(e for _, e in res)
    allc = unit_bytes * units / span / 1e9
    return {"value": round(allc, 4), "unit": "GB/s", "cores": P, "kind": "oracle",
            "single_core": {"value": round(one, 4), "unit": "GB/s", "cores": 1},
            "sample": f"same workload as the GPU step (write 1 token + decode over {L} tokens, {nq}/{nkv} heads), "
                      f"numpy oracle with BLAS on one thread per process: {layers} whole layers on 1 core in "
                      f"{el:.1f} s (ms/layer {1e3 * el / layers:.1f}); {units} (kv-head) units on {P} worker "
                      f"processes, {span:.1f} s each ({wall:.1f} s wall with start-up)"}


def time_calls(torch, fn, iters, warmup=10, graph=False):
    """Average microseconds per call of fn() on the current stream, HIP events
    around `iters` back-to-back calls (captured as one graph when `graph`).
    The mode is recorded for `report`."""
    time_calls.last_mode = "graph replay" if graph else "eager, back to back"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(iters):
                fn()
        g.replay()
        torch.cuda.synchronize()
        run = g.replay
    else:
        def run():
            for _ in range(iters):
                fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run()
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / iters


REPORTS = []


def report(name, desc, nbytes, us, **extra):
    gbs = nbytes / (us * 1e-6) / 1e9
    line = {"workload": name, "desc": desc, "algorithmic_bytes": int(nbytes), "us_per_call": round(us, 2),
            "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "timing": getattr(time_calls, "last_mode", None)}
    line.update(extra)
    REPORTS.append(line)
    if not report.quiet:
        print(json.dumps(line), flush=True)


report.quiet = False


def run_workloads(only=None):
    """Every workload of the hot path besides the step benchmark, timed on one
    GPU: the pages' unit experiment, the batch-32 long-context layer, the 64K
    write path and the decode over it, the int4 128K mixed decode, and the
    int8 -> int4 re-quantization of aging time blocks.  Inputs follow the
    recipes of `workloads` (generated on the GPU, quantized through the
    library's write paths).  Calls of under about 50 us are timed as one graph
    replay of back-to-back calls (eager calls would measure the host's launch
    path); longer ones as back-to-back eager calls, which run them faster on
    this GPU than a graph replay does.  Each line names its timing mode."""
    import torch

    import decode_attention_int8_amd as K
    import workloads as W
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    sm = 1.0 / math.sqrt(128)

    def want(*names):
        return not only or any(n in only for n in names)

    def q8_pool(nb, bs, nkv):
        shp = (nb, bs, nkv, 128)
        return [torch.zeros(shp, dtype=torch.int8, device="cuda"), torch.zeros(shp, dtype=torch.int8, device="cuda"),
                torch.zeros(shp[:3], dtype=torch.float32, device="cuda"),
                torch.zeros(shp[:3], dtype=torch.float32, device="cuda")]

    def mall_copies(nbytes):
        """Cache copies to cycle through so that a call's data was last touched
        at least 512 MB of other reads earlier, past the 256 MB Infinity Cache
        (a working set of that size or more needs no second copy)."""
        return 1 if nbytes >= MALL_FLUSH_BYTES else 1 + math.ceil(MALL_FLUSH_BYTES / nbytes)

    def cycled(call, pools, iters):
        """fn() calling `call(pool)` for the pools in turn, and an iteration
        count that is a multiple of their number (at least `iters`)."""
        state = [0]

        def fn():
            call(pools[state[0] % len(pools)])
            state[0] += 1
        return fn, len(pools) * math.ceil(iters / len(pools))

    def q4_pool(nb, bs, nkv):
        shp = (nb, nkv, bs)                        # head-major inside a block
        return [torch.zeros(shp + (64,), dtype=torch.uint8, device="cuda"),
                torch.zeros(shp + (64,), dtype=torch.uint8, device="cuda")] + \
               [torch.zeros(shp + (2,), dtype=torch.float16, device="cuda") for _ in range(4)]

    def q2_pool(nb, bs, nkv):
        shp = (nb, nkv, bs)                        # head-major inside a block
        return [torch.zeros(shp + (32,), dtype=torch.uint8, device="cuda"),
                torch.zeros(shp + (32,), dtype=torch.uint8, device="cuda")] + \
               [torch.zeros(shp + (2,), dtype=torch.float16, device="cuda") for _ in range(4)]

    if want("unit_256"):
        # unit experiment: 1 / 1 heads, 256 tokens (launch-bound)
        q, k, v = W.unit_experiment(0)
        bt, nb = W.paged_block_tables(None, [256], 16)
        p = q8_pool(nb, 16, 1)
        K.kvq8_quantize_append(*p, dev(k[:, None]), dev(v[:, None]), dev(np.arange(256, dtype=np.int32)))
        out = torch.empty((1, 1, 128), device="cuda")
        qd, btd, ld = dev(q[None, None]), dev(bt), dev(np.array([256], np.int32))
        ws = K.alloc_workspace(K.kvq8_decode_workspace_size(1, 1, 1, 256), "cuda")
        us = time_calls(torch, lambda: K.kvq8_decode_attn(out, qd, *p, btd, ld, 256, sm, 0, ws), 200, graph=True)
        report("unit_256", "decode, 1 query / 1 kv head, 256 tokens (graph replay)", 256 * 264, us)
        del p

    if want("qwen8b_b32"):
        # batch-32 Qwen-8B-shaped layer: lengths U[1024, 32768], K, V = 0.5 Student-t(3)
        cfg = W.QWEN8B_B32
        lens = W.qwen8b_lengths(0)
        B, nq, nkv, bs = cfg["batch"], cfg["nq"], cfg["nkv"], cfg["kv_bs"]
        bt, nb = W.paged_block_tables(W.rng(3, 0, 1), lens, bs)
        p = q8_pool(nb, bs, nkv)
        for b in range(B):
            kk = W.torch_student_t3((int(lens[b]), nkv, 128), "cuda", (3, 0, b, 0))
            vv = W.torch_student_t3((int(lens[b]), nkv, 128), "cuda", (3, 0, b, 1))
            K.kvq8_quantize_append(*p, kk, vv, dev(W.slots_for_positions(bt, [b] * int(lens[b]), np.arange(lens[b]), bs)))
            del kk, vv
        qd = W.torch_normal((B, nq, 128), "cuda", (3, 0, 99))
        out = torch.empty((B, nq, 128), device="cuda")
        btd, ld, L = dev(bt), dev(lens), int(lens.max())
        ch = K.kvq8_decode_chunk_tokens(B, nkv, L)
        ws = K.alloc_workspace(K.kvq8_decode_workspace_size(B, nq, nkv, L), "cuda")
        # the layer's rate settles over its first few hundred calls (up to ~7%
        # slower before): time 400 calls after 300
        us = time_calls(torch, lambda: K.kvq8_decode_attn(out, qd, *p, btd, ld, L, sm, 0, ws), 400, warmup=300)
        report("qwen8b_b32", f"decode layer, batch 32 x 32 / 8 heads, lengths U[1024, 32768] (sum {int(lens.sum())})",
               int(lens.sum()) * nkv * 264, us, chunk_tokens=ch)
        del p

    if want("append_64k", "decode_64k"):
        # 64K tokens written from bf16 (1% x20 outliers), then a GQA-4 decode over them
        cfg = W.APPEND_64K
        n, nq, nkv, bs = cfg["n_tok"], cfg["nq"], cfg["nkv"], cfg["kv_bs"]
        bt, nb = W.paged_block_tables(W.rng(4, 0, 1), [n], bs)
        p = q8_pool(nb, bs, nkv)
        kk = W.torch_outlier_normal_bf16((n, nkv, 128), "cuda", (4, 0, 0))
        vv = W.torch_outlier_normal_bf16((n, nkv, 128), "cuda", (4, 0, 1))
        slots = dev(W.slots_for_positions(bt, [0] * n, np.arange(n), bs))
        us = time_calls(torch, lambda: K.kvq8_quantize_append(*p, kk, vv, slots), 50, warmup=30)
        report("append_64k", "write path, 65536 tokens x 8 kv heads from bf16", n * nkv * (2 * 128 * 2 + 2 * 132), us)
        qd = W.torch_normal((1, nq, 128), "cuda", (4, 0, 2))
        out = torch.empty((1, nq, 128), device="cuda")
        btd, ld = dev(bt), dev(np.array([n], np.int32))
        ch = K.kvq8_decode_chunk_tokens(1, nkv, n)
        ws = K.alloc_workspace(K.kvq8_decode_workspace_size(1, nq, nkv, n), "cuda")
        del kk, vv
        nbytes = n * nkv * 264
        pools = [p] + [[t.clone() for t in p] for _ in range(mall_copies(nbytes) - 1)]
        fn, iters = cycled(lambda pp: K.kvq8_decode_attn(out, qd, *pp, btd, ld, n, sm, 0, ws), pools, 50)
        us = time_calls(torch, fn, iters, graph=True)
        report("decode_64k", f"decode, 1 sequence x 32 / 8 heads over the 65536 written tokens ({len(pools)} copies "
               "of the cache cycled)", nbytes, us, chunk_tokens=ch)
        del pools
        del p

    if want("q4_append_64k", "q2_append_64k"):
        # the group write paths on the 64K bf16 rows of the int8 write workload
        cfg = W.APPEND_64K
        n, nkv, bs = cfg["n_tok"], cfg["nkv"], cfg["kv_bs"]
        bt, nb = W.paged_block_tables(W.rng(4, 0, 1), [n], bs)
        kk = W.torch_outlier_normal_bf16((n, nkv, 128), "cuda", (4, 0, 0))
        vv = W.torch_outlier_normal_bf16((n, nkv, 128), "cuda", (4, 0, 1))
        slots = dev(W.slots_for_positions(bt, [0] * n, np.arange(n), bs))
        if want("q4_append_64k"):
            p4 = q4_pool(nb, bs, nkv)
            us = time_calls(torch, lambda: K.kvq4_quantize_append(*p4, kk, vv, slots), 50, warmup=30)
            # per (token, kv-head): K and V rows read (bf16), codes + binary16 scale / zero of both groups written
            report("q4_append_64k", "int4 write path, 65536 tokens x 8 kv heads from bf16",
                   n * nkv * (2 * 128 * 2 + 2 * (64 + 8)), us)
            del p4
        if want("q2_append_64k"):
            p2 = q2_pool(nb, bs, nkv)
            us = time_calls(torch, lambda: K.kvq2_quantize_append(*p2, kk, vv, slots), 50, warmup=30)
            report("q2_append_64k", "2-bit write path, 65536 tokens x 8 kv heads from bf16",
                   n * nkv * (2 * 128 * 2 + 2 * (32 + 8)), us)
            del p2
        del kk, vv

    if want("q4_128k", "requant_block", "requant_window"):
        # int4 group cache, 128K tokens (last 2048 int8), batch 4 x 32 / 4 heads
        cfg = W.Q4_128K
        B, nq, nkv, L, win, bs = cfg["batch"], cfg["nq"], cfg["nkv"], cfg["L"], cfg["window"], cfg["kv_bs"]
        n4, n8 = L - win, win
        bt4, nb4 = W.paged_block_tables(W.rng(5, 0, 1), [n4] * B, bs)
        bt8, nb8 = W.paged_block_tables(W.rng(5, 0, 2), [n8] * B, bs)
        p4, p8 = q4_pool(nb4, bs, nkv), q8_pool(nb8, bs, nkv)
        sig = W.rng(5, 0, 3).uniform(0.2, 5.0, size=(B, nkv, 2))
        for b in range(B):
            sk = torch.tensor(sig[b, :, 0], dtype=torch.float32, device="cuda")[None, :, None]
            sv = torch.tensor(sig[b, :, 1], dtype=torch.float32, device="cuda")[None, :, None]
            kk = W.torch_normal((L, nkv, 128), "cuda", (5, 0, b, 0)) * sk
            vv = W.torch_normal((L, nkv, 128), "cuda", (5, 0, b, 1)) * sv
            K.kvq4_quantize_append(*p4, kk[:n4], vv[:n4], dev(W.slots_for_positions(bt4, [b] * n4, np.arange(n4), bs)))
            K.kvq8_quantize_append(*p8, kk[n4:], vv[n4:], dev(W.slots_for_positions(bt8, [b] * n8, np.arange(n8), bs)))
            del kk, vv
        qd = W.torch_normal((B, nq, 128), "cuda", (5, 0, 99))
        out = torch.empty((B, nq, 128), device="cuda")
        bt4d, l4 = dev(bt4), dev(np.full(B, n4, np.int32))
        bt8d, l8 = dev(bt8), dev(np.full(B, n8, np.int32))
        ch = K.kvq4_decode_chunk_tokens(B, nkv, n4, n8)
        ws = K.alloc_workspace(K.kvq4_decode_workspace_size(B, nq, nkv, n4, n8), "cuda")
        nbytes = B * nkv * (n4 * 144 + n8 * 264)
        pools = [(p4, p8)] + [([t.clone() for t in p4], [t.clone() for t in p8])
                              for _ in range(mall_copies(nbytes) - 1)]
        fn, iters = cycled(lambda pp: K.kvq4_decode_attn(out, qd, pp[0], bt4d, l4, n4, pp[1], bt8d, l8, n8, sm, 0, ws),
                           pools, 48)
        us = time_calls(torch, fn, iters, warmup=24)
        report("q4_128k", f"mixed decode, batch 4 x 32 / 4 heads, 129024 int4 + 2048 int8 tokens ({len(pools)} "
               "copies of the cache cycled)", nbytes, us, chunk_tokens=ch)
        del pools

        # re-quantization of the window's oldest 512-token time block of every
        # sequence into the int4 pool (into the int4 pool's first 512 slots per
        # sequence: the timing, not the cache's meaning, is what is measured here)
        T = 512
        src = dev(np.concatenate([W.slots_for_positions(bt8, [b] * T, np.arange(T), bs) for b in range(B)]))
        dst = dev(np.concatenate([W.slots_for_positions(bt4, [b] * T, np.arange(T), bs) for b in range(B)]))
        us = time_calls(torch, lambda: K.kvq4_requantize_q8(p4, p8, src, dst), 50, graph=True)
        report("requant_block", "int8 -> int4 re-quantization of one 512-token time block x 4 sequences x 4 kv heads "
               "(graph replay)", B * T * nkv * (264 + 144), us)
        n_all = B * n8
        src = dev(np.concatenate([W.slots_for_positions(bt8, [b] * n8, np.arange(n8), bs) for b in range(B)]))
        dst = dev(np.concatenate([W.slots_for_positions(bt4, [b] * n8, np.arange(n8), bs) for b in range(B)]))
        us = time_calls(torch, lambda: K.kvq4_requantize_q8(p4, p8, src, dst), 50, graph=True)
        report("requant_window", "int8 -> int4 re-quantization of the whole 2048-token window x 4 sequences",
               n_all * nkv * (264 + 144), us)
        del p4, p8

    if want("q2_128k", "requant2_block"):
        # three bands, 128K tokens: 114688 2-bit + 14336 int4 + 2048 int8, batch 4 x 32 / 4 heads
        cfg = W.Q2_128K
        B, nq, nkv, L, bs = cfg["batch"], cfg["nq"], cfg["nkv"], cfg["L"], cfg["kv_bs"]
        n8 = cfg["window"]
        n4 = cfg["edge4"] - n8
        n2 = L - n4 - n8
        bt2, nb2 = W.paged_block_tables(W.rng(9, 0, 1), [n2] * B, bs)
        bt4, nb4 = W.paged_block_tables(W.rng(9, 0, 2), [n4] * B, bs)
        bt8, nb8 = W.paged_block_tables(W.rng(9, 0, 3), [n8] * B, bs)
        p2, p4, p8 = q2_pool(nb2, bs, nkv), q4_pool(nb4, bs, nkv), q8_pool(nb8, bs, nkv)
        sig = W.rng(9, 0, 4).uniform(0.2, 5.0, size=(B, nkv, 2))
        for b in range(B):
            sk = torch.tensor(sig[b, :, 0], dtype=torch.float32, device="cuda")[None, :, None]
            sv = torch.tensor(sig[b, :, 1], dtype=torch.float32, device="cuda")[None, :, None]
            kk = W.torch_normal((L, nkv, 128), "cuda", (9, 0, b, 0)) * sk
            vv = W.torch_normal((L, nkv, 128), "cuda", (9, 0, b, 1)) * sv
            K.kvq2_quantize_append(*p2, kk[:n2], vv[:n2], dev(W.slots_for_positions(bt2, [b] * n2, np.arange(n2), bs)))
            K.kvq4_quantize_append(*p4, kk[n2:n2 + n4], vv[n2:n2 + n4],
                                   dev(W.slots_for_positions(bt4, [b] * n4, np.arange(n4), bs)))
            K.kvq8_quantize_append(*p8, kk[n2 + n4:], vv[n2 + n4:],
                                   dev(W.slots_for_positions(bt8, [b] * n8, np.arange(n8), bs)))
            del kk, vv
        qd = W.torch_normal((B, nq, 128), "cuda", (9, 0, 99))
        out = torch.empty((B, nq, 128), device="cuda")
        bt2d, l2 = dev(bt2), dev(np.full(B, n2, np.int32))
        bt4d, l4 = dev(bt4), dev(np.full(B, n4, np.int32))
        bt8d, l8 = dev(bt8), dev(np.full(B, n8, np.int32))
        ch = K.kvq2_decode_chunk_tokens(B, nkv, n2, n4, n8)
        ws = K.alloc_workspace(K.kvq2_decode_workspace_size(B, nq, nkv, n2, n4, n8), "cuda")
        nbytes = B * nkv * (n2 * 80 + n4 * 144 + n8 * 264)
        pools = [(p2, p4, p8)] + [tuple([t.clone() for t in pp] for pp in (p2, p4, p8))
                                  for _ in range(mall_copies(nbytes) - 1)]
        fn, iters = cycled(lambda pp: K.kvq2_decode_attn(out, qd, pp[0], bt2d, l2, n2, pp[1], bt4d, l4, n4, pp[2],
                                                         bt8d, l8, n8, sm, 0, ws), pools, 48)
        us = time_calls(torch, fn, iters, warmup=24)
        report("q2_128k", f"banded decode, batch 4 x 32 / 4 heads, {n2} 2-bit + {n4} int4 + {n8} int8 tokens "
               f"({len(pools)} copies of the cache cycled)", nbytes, us, chunk_tokens=ch)
        del pools

        # re-quantization of the int4 band's oldest 512-token time block of
        # every sequence into the 2-bit pool (timing only, as for requant_block)
        T = 512
        src = dev(np.concatenate([W.slots_for_positions(bt4, [b] * T, np.arange(T), bs) for b in range(B)]))
        dst = dev(np.concatenate([W.slots_for_positions(bt2, [b] * T, np.arange(T), bs) for b in range(B)]))
        us = time_calls(torch, lambda: K.kvq2_requantize_q4(p2, p4, src, dst), 50, graph=True)
        report("requant2_block", "int4 -> 2-bit re-quantization of one 512-token time block x 4 sequences x 4 kv "
               "heads (graph replay)", B * T * nkv * (144 + 80), us)
        del p2, p4, p8

    # Q4_0 mode (80 B per row: 160 B per (token, kv-head) for K and V)
    def q40_pool(nb, bs, nkv):
        shp = (nb, nkv, bs)                        # head-major inside a block
        return [torch.zeros(shp + (64,), dtype=torch.uint8, device="cuda"),
                torch.zeros(shp + (64,), dtype=torch.uint8, device="cuda"),
                torch.zeros(shp + (4,), dtype=torch.float32, device="cuda"),
                torch.zeros(shp + (4,), dtype=torch.float32, device="cuda")]

    if want("q40_8k"):
        # the 8K batch-1 layer shape, 28 layers cycled in one graph (as the step)
        cfg = W.QWEN2B_8K
        nl, nq, nkv, bs, L = cfg["layers"], cfg["nq"], cfg["nkv"], cfg["kv_bs"], cfg["L"]
        bt, nb = W.paged_block_tables(W.rng(6, 0, 1), [L], bs)
        btd, ld = dev(bt), dev(np.array([L], np.int32))
        slots = dev(W.slots_for_positions(bt, [0] * L, np.arange(L), bs))
        layers = []
        for layer in range(nl):
            p = q40_pool(nb, bs, nkv)
            kk = W.torch_normal((L, nkv, 128), "cuda", (6, layer, 0))
            vv = W.torch_normal((L, nkv, 128), "cuda", (6, layer, 1))
            K.kvq4_0_quantize_append(*p, kk, vv, slots)
            layers.append((p, W.torch_normal((1, nq, 128), "cuda", (6, layer, 2)), torch.empty((1, nq, 128), device="cuda")))
            del kk, vv
        ws = K.alloc_workspace(K.kvq4_0_decode_workspace_size(1, nq, nkv, L), "cuda")

        def q40_step():
            for p, qd, out in layers:
                K.kvq4_0_decode_attn(out, qd, *p, btd, ld, L, sm, 0, ws)
        us = time_calls(torch, q40_step, 5, graph=True) / nl
        report("q40_8k", "Q4_0 decode, 28 layers x (1 x 16 / 8 heads, 8192 tokens), per layer call (graph replay)",
               L * nkv * 160, us, chunk_tokens=K.kvq4_0_decode_chunk_tokens(1, nkv, L))
        del layers

    if want("q40_qwen8b_b32"):
        # the batch-32 long-context layer in Q4_0
        cfg = W.QWEN8B_B32
        lens = W.qwen8b_lengths(0)
        B, nq, nkv, bs = cfg["batch"], cfg["nq"], cfg["nkv"], cfg["kv_bs"]
        bt, nb = W.paged_block_tables(W.rng(3, 0, 1), lens, bs)
        p = q40_pool(nb, bs, nkv)
        for b in range(B):
            kk = W.torch_student_t3((int(lens[b]), nkv, 128), "cuda", (3, 0, b, 0))
            vv = W.torch_student_t3((int(lens[b]), nkv, 128), "cuda", (3, 0, b, 1))
            K.kvq4_0_quantize_append(*p, kk, vv,
                                     dev(W.slots_for_positions(bt, [b] * int(lens[b]), np.arange(lens[b]), bs)))
            del kk, vv
        qd = W.torch_normal((B, nq, 128), "cuda", (3, 0, 99))
        out = torch.empty((B, nq, 128), device="cuda")
        btd, ld, L = dev(bt), dev(lens), int(lens.max())
        ws = K.alloc_workspace(K.kvq4_0_decode_workspace_size(B, nq, nkv, L), "cuda")
        us = time_calls(torch, lambda: K.kvq4_0_decode_attn(out, qd, *p, btd, ld, L, sm, 0, ws), 50, warmup=30)
        report("q40_qwen8b_b32", f"Q4_0 decode layer, batch 32 x 32 / 8 heads, lengths U[1024, 32768] "
               f"(sum {int(lens.sum())})", int(lens.sum()) * nkv * 160, us,
               chunk_tokens=K.kvq4_0_decode_chunk_tokens(B, nkv, L))
        del p

    if want("q40_append_64k", "q40_decode_64k"):
        # 64K tokens written from bf16 into the Q4_0 pool, then a GQA-4 decode
        cfg = W.APPEND_64K
        n, nq, nkv, bs = cfg["n_tok"], cfg["nq"], cfg["nkv"], cfg["kv_bs"]
        bt, nb = W.paged_block_tables(W.rng(4, 0, 1), [n], bs)
        p = q40_pool(nb, bs, nkv)
        kk = W.torch_outlier_normal_bf16((n, nkv, 128), "cuda", (4, 0, 0))
        vv = W.torch_outlier_normal_bf16((n, nkv, 128), "cuda", (4, 0, 1))
        slots = dev(W.slots_for_positions(bt, [0] * n, np.arange(n), bs))
        us = time_calls(torch, lambda: K.kvq4_0_quantize_append(*p, kk, vv, slots), 50, warmup=30)
        report("q40_append_64k", "Q4_0 write path, 65536 tokens x 8 kv heads from bf16",
               n * nkv * (2 * 128 * 2 + 2 * 80), us)
        qd = W.torch_normal((1, nq, 128), "cuda", (4, 0, 2))
        out = torch.empty((1, nq, 128), device="cuda")
        btd, ld = dev(bt), dev(np.array([n], np.int32))
        ws = K.alloc_workspace(K.kvq4_0_decode_workspace_size(1, nq, nkv, n), "cuda")
        del kk, vv
        nbytes = n * nkv * 160
        pools = [p] + [[t.clone() for t in p] for _ in range(mall_copies(nbytes) - 1)]
        fn, iters = cycled(lambda pp: K.kvq4_0_decode_attn(out, qd, *pp, btd, ld, n, sm, 0, ws), pools, 50)
        us = time_calls(torch, fn, iters, graph=True)
        report("q40_decode_64k", f"Q4_0 decode, 1 sequence x 32 / 8 heads over the 65536 written tokens ({len(pools)} "
               "copies of the cache cycled)", nbytes, us, chunk_tokens=K.kvq4_0_decode_chunk_tokens(1, nkv, n))
        del pools


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.workloads:
        run_workloads([n for n in args.only.split(",") if n])
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library has no multi-GPU path)",
              file=sys.stderr)
        sys.exit(2)
    import workloads as W

    cfg = W.QWEN2B_8K
    nq, nkv, bs, L, n_layers = cfg["nq"], cfg["nkv"], cfg["kv_bs"], args.ctx, args.layers
    decode_bytes_layer = L * nkv * TOK_HEAD_BYTES
    write_bytes_layer = nkv * 2 * 128 * 4 + nkv * 2 * (128 + 4)
    # the CPU baseline first: its worker processes fork before any GPU state exists
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, nq, nkv, bs, L,
                                                         decode_bytes_layer + write_bytes_layer)

    import torch

    import decode_attention_int8_amd as K
    sm = 1.0 / math.sqrt(128)
    bt_np, nb = W.paged_block_tables(W.rng(2, 0, 3), [L], bs)
    bt = torch.from_numpy(bt_np).cuda()
    lens = torch.tensor([L], dtype=torch.int32, device="cuda")
    layers = [Layer(K, W, torch, i, L, nq, nkv, bs, bt_np, nb, bt, lens) for i in range(n_layers)]
    chunk = K.kvq8_decode_chunk_tokens(1, nkv, L)
    ws = K.alloc_workspace(K.kvq8_decode_workspace_size(1, nq, nkv, L, 0), "cuda")

    def step():
        # one decode step: per layer, write the newest token and attend (one call)
        for ly in layers:
            K.kvq8_append_decode_attn(ly.out, ly.q, ly.k_new, ly.v_new, ly.k, ly.v, ly.ks, ly.vs, ly.bt, ly.lens, L,
                                      sm, 0, ws)

    # warm up eagerly on a side stream, then capture the whole step in a graph
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(3, args.warmup)):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()

    # timed region: K whole steps (graph replays)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for _ in range(args.steps):
        graph.replay()
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    step_bytes = n_layers * (decode_bytes_layer + write_bytes_layer)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # the timed region is n_layers back-to-back calls per step on one stream
    call_us = 1e3 * ms_per_step / n_layers
    achieved = decode_bytes_layer / (call_us * 1e-6) / 1e9

    res = {
        "metric": "q8-KV decode attention: effective HBM GB/s (% of peak) and us/step at 8K ctx",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 KV codes, fp32 steps and accumulation",
        "data": "synthetic (seeded N(0,1) K/V/q; one block table in shuffled order shared by the layers' pools)",
        "config": {"workload": f"qwen2b-shaped decode: {n_layers} layers x {nq}q/{nkv}kv heads, hd 128, batch 1, "
                               f"ctx {L}, kv_bs {bs}, per layer: write the newest token + decode (one fused "
                               f"call), step replayed as a HIP graph",
                   "global_batch": 1, "seq_len": L, "chunk_tokens": chunk, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "one kvq8_append_decode_attn call: kvq_decode_mfma_kernel<0, false, false> + kvq_merge1_kernel<2>",
                     "bytes_per_launch": decode_bytes_layer, "avg_call_us": round(call_us, 3),
                     "note": "latency-bound: batch 1 moves 17.3 MB per layer call through two dependent "
                             "launches (chunk kernel, then merge), about 2.2 us of transfer at peak; the "
                             "long-context configurations below are the bandwidth-bound ones"},
    }
    if not args.no_configs:
        # the other configurations' fractions of peak, next to the headline
        # (the batch-1 8K call above is latency-bound by construction)
        del layers, graph
        torch.cuda.synchronize()
        report.quiet = True
        run_workloads(["qwen8b_b32", "append_64k", "decode_64k", "q4_128k"])
        res["configs"] = [{k: r[k] for k in ("workload", "us_per_call", "GB/s", "frac_of_hbm_peak", "timing")}
                          for r in REPORTS if r["workload"] in ("qwen8b_b32", "append_64k", "decode_64k", "q4_128k")]
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
