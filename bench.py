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
TOK_HEAD_BYTES = 2 * 128 + 2 * 4   # K+V codes + K/V float32 steps per (token, kv-head)


# HBM bytes per decode call from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# passes over this benchmark (KiB per dispatch), scaled by what the same
# counters read for a plain 256 MiB device copy (--calibrate-copy 256):
# FETCH_SIZE 131085.3 KiB -> 2.000 bytes per counted byte, WRITE_SIZE
# 262144 KiB -> 1.000.  Valid only for the kernel sources they were taken on.
PMC = {"sources_sha256_16": "598909cae9f0473b",
       "fetch_kib": {"chunk": 8583.39, "merge": 174.54}, "write_kib": {"chunk": 290.06, "merge": 8.0},
       "fetch_scale": 268435456 / (131085.25 * 1024), "write_scale": 268435456 / (262144.0 * 1024)}


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
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
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


def cpu_baseline(args, nq, nkv, bs, L, bytes_per_layer):
    """The oracle, untouched, on a bounded sample of the same workload: whole
    layers (write the current token, then decode over L tokens) until about
    args.cpu_seconds of host time.  BLAS is pinned to one thread."""
    from threadpoolctl import threadpool_limits

    import workloads as W
    from oracle import kvq8 as O8

    sm = float(np.float32(1) / np.sqrt(np.float32(128)))
    r = W.rng(2, 1000)
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
    layers = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            O8.quantize_append(kp, vp, ks, vs, k[-1:], v[-1:], slots[-1:])
            O8.decode_attention_q8(q, kp, ks, vp, vs, bt, [L], bs, sm)
            layers += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
    return {"value": round(bytes_per_layer * layers / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{layers} layers of the same workload (write 1 token + decode over {L} tokens, {nq}/{nkv} "
                      f"heads), {el:.1f} s single-threaded numpy; ms/layer {1e3 * el / layers:.1f}"}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build has no multi-GPU path)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_attention_int8_amd as K
    import workloads as W

    cfg = W.QWEN2B_8K
    nq, nkv, bs, L, n_layers = cfg["nq"], cfg["nkv"], cfg["kv_bs"], args.ctx, args.layers
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

    decode_bytes_layer = L * nkv * TOK_HEAD_BYTES
    write_bytes_layer = nkv * 2 * 128 * 4 + nkv * 2 * (128 + 4)
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
                     "kernel": "one kvq8_append_decode_attn call: kvq_decode_mfma_kernel<0,false> + kvq_merge_kernel",
                     "bytes_per_launch": decode_bytes_layer, "avg_call_us": round(call_us, 3)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args, nq, nkv, bs, L, decode_bytes_layer + write_bytes_layer)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
