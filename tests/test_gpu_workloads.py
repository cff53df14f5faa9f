"""GPU parity at the full sizes of the five workloads, with the default
launch configuration (the one the benchmark times).

  unit      1 / 1 heads, L = 256, N(0, 1)                     (test_gpu_kvq8)
  qwen2b    28 layers x 16 / 8 heads, L = 8192, batch 1        layers 0 and 27, separate
                                                               calls and the fused step
                                                               (eager and graph replays)
  qwen8b    36 layers x 32 / 8 heads, batch 32, L in [1K, 32K],
            K/V 0.5 * Student-t(3)                             layer 0, all 32 sequences
  append64k 65536 bf16 tokens (1% outliers x20) x 8 heads, then
            one GQA-4 decode over the 65536 tokens             everything
  q4_128k   int4 groups + int8 window, 32 / 4 heads, batch 4,
            L = 131072                                         sequences 0 and 3
  q2_128k   the same shape in three bands: 2-bit up to 16384
            tokens from the newest, int4 up to 2048, int8 window   sequences 0 and 3
  Q4_0      the qwen8b batch-32 layer and the 64K append + decode
            through the Q4_0 mode                              everything

Write-path codes and steps are compared bit for bit with the oracle's own
quantization of the same generated inputs; the decode reference is the
oracle run on the oracle's codes.
"""
import numpy as np
import pytest

import workloads as W
from oracle import kvq2 as O2
from oracle import kvq4 as O4
from oracle import kvq4_0 as O40
from oracle import kvq8 as O8
from tests.helpers import SM, assert_attn_close, dev, host, pool_pages_order, q4_key_pages_order, slot_major

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import decode_attention_int8_amd as K
    return K


def _q8_pools(torch, nb, bs, nkv):
    shp = (nb, bs, nkv, 128)
    return (torch.zeros(shp, dtype=torch.int8, device="cuda"), torch.zeros(shp, dtype=torch.int8, device="cuda"),
            torch.zeros(shp[:3], dtype=torch.float32, device="cuda"),
            torch.zeros(shp[:3], dtype=torch.float32, device="cuda"))


def _host_pools(nb, bs, nkv):
    shp = (nb, bs, nkv, 128)
    return [np.zeros(shp, np.int8), np.zeros(shp, np.int8), np.zeros(shp[:3], np.float32),
            np.zeros(shp[:3], np.float32)]


def _same(a, b):
    return np.array_equal(a.view(np.uint8) if a.dtype != np.int8 else a, b.view(np.uint8) if b.dtype != np.int8 else b)


@pytest.mark.parametrize("layer", [0, 27])
def test_qwen2b_8k_layer(K, layer):
    import torch
    cfg = W.QWEN2B_8K
    L, nq, nkv, bs = cfg["L"], cfg["nq"], cfg["nkv"], cfg["kv_bs"]
    bt, nb = W.paged_block_tables(W.rng(2, layer, 3), [L], bs)
    k = W.torch_normal((L, nkv, 128), "cuda", (2, layer, 0))
    v = W.torch_normal((L, nkv, 128), "cuda", (2, layer, 1))
    q = W.torch_normal((1, nq, 128), "cuda", (2, layer, 2))
    slots = W.slots_for_positions(bt, [0] * L, np.arange(L), bs)
    gk, gv, gks, gvs = _q8_pools(torch, nb, bs, nkv)
    K.kvq8_quantize_append(gk, gv, gks, gvs, k, v, dev(slots))
    out = torch.empty((1, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq8_decode_attn(out, q, gk, gv, gks, gvs, dev(bt), dev(np.array([L], np.int32)), L, SM)
    torch.cuda.synchronize()
    hk, hv, hks, hvs = _host_pools(nb, bs, nkv)
    O8.quantize_append(hk, hv, hks, hvs, host(k), host(v), slots)
    assert _same(pool_pages_order(host(gk)), hk) and _same(pool_pages_order(host(gv)), hv)
    assert _same(host(gks), hks) and _same(host(gvs), hvs)
    ref = O8.decode_attention_q8(host(q), hk, hks, hv, hvs, bt, [L], bs, SM)
    assert_attn_close(host(out), ref, f"qwen2b layer {layer}")


@pytest.mark.parametrize("layer", [0, 27])
def test_qwen2b_8k_fused_step_and_graph_replays(K, layer):
    """The benchmark's step as it runs: the layer's cache holds all L tokens,
    the slot of position L-1 holds a stale row, and one fused call writes the
    newest token there and attends over the L tokens.  Eagerly first, checked
    against the oracle (cache bytes and outputs); then captured in a graph and
    replayed three times, with the stale row re-written eagerly and the stream
    synchronized between replays, every replay equal to the eager call bit for
    bit."""
    import torch
    cfg = W.QWEN2B_8K
    L, nq, nkv, bs = cfg["L"], cfg["nq"], cfg["nkv"], cfg["kv_bs"]
    bt, nb = W.paged_block_tables(W.rng(2, layer, 3), [L], bs)
    k = W.torch_normal((L, nkv, 128), "cuda", (2, layer, 0))
    v = W.torch_normal((L, nkv, 128), "cuda", (2, layer, 1))
    q = W.torch_normal((1, nq, 128), "cuda", (2, layer, 2))
    stale = W.torch_normal((1, nkv, 128), "cuda", (2, layer, 9)) * 3.0
    slots = W.slots_for_positions(bt, [0] * L, np.arange(L), bs)
    gk, gv, gks, gvs = _q8_pools(torch, nb, bs, nkv)
    K.kvq8_quantize_append(gk, gv, gks, gvs, k, v, dev(slots))
    last = dev(slots[L - 1:])
    k_new, v_new = k[L - 1:L].clone(), v[L - 1:L].clone()
    btd, ld = dev(bt), dev(np.array([L], np.int32))
    ws = K.alloc_workspace(K.kvq8_decode_workspace_size(1, nq, nkv, L), "cuda")

    def step(out):
        K.kvq8_append_decode_attn(out, q, k_new, v_new, gk, gv, gks, gvs, btd, ld, L, SM, 0, ws)

    K.kvq8_quantize_append(gk, gv, gks, gvs, stale, stale, last)
    out_eager = torch.empty((1, nq, 128), dtype=torch.float32, device="cuda")
    step(out_eager)
    torch.cuda.synchronize()
    hk, hv, hks, hvs = _host_pools(nb, bs, nkv)
    O8.quantize_append(hk, hv, hks, hvs, host(k), host(v), slots)
    assert _same(pool_pages_order(host(gk)), hk) and _same(pool_pages_order(host(gv)), hv)
    assert _same(host(gks), hks) and _same(host(gvs), hvs)
    ref = O8.decode_attention_q8(host(q), hk, hks, hv, hvs, bt, [L], bs, SM)
    assert_attn_close(host(out_eager), ref, f"qwen2b fused step layer {layer}")

    out = torch.empty_like(out_eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    for rep in range(3):
        K.kvq8_quantize_append(gk, gv, gks, gvs, stale, stale, last)      # eager work between replays
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), host(out_eager)), f"replay {rep}"
        assert _same(pool_pages_order(host(gk)), hk) and _same(host(gks), hks), f"replay {rep} cache"


def test_qwen8b_batch32_layer0(K):
    import torch
    cfg = W.QWEN8B_B32
    nq, nkv, bs, B = cfg["nq"], cfg["nkv"], cfg["kv_bs"], cfg["batch"]
    lens = W.qwen8b_lengths(0)
    bt, nb = W.paged_block_tables(W.rng(3, 0, 1), lens, bs)
    gk, gv, gks, gvs = _q8_pools(torch, nb, bs, nkv)
    hk, hv, hks, hvs = _host_pools(nb, bs, nkv)
    for b in range(B):
        Lb = int(lens[b])
        k = W.torch_student_t3((Lb, nkv, 128), "cuda", (3, 0, b, 0), 0.5)
        v = W.torch_student_t3((Lb, nkv, 128), "cuda", (3, 0, b, 1), 0.5)
        slots = W.slots_for_positions(bt, [b] * Lb, np.arange(Lb), bs)
        K.kvq8_quantize_append(gk, gv, gks, gvs, k, v, dev(slots))
        O8.quantize_append(hk, hv, hks, hvs, host(k), host(v), slots)
        del k, v
    q = W.torch_normal((B, nq, 128), "cuda", (3, 0, 99))
    out = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq8_decode_attn(out, q, gk, gv, gks, gvs, dev(bt), dev(lens), int(lens.max()), SM)
    torch.cuda.synchronize()
    assert _same(pool_pages_order(host(gk)), hk) and _same(pool_pages_order(host(gv)), hv)
    assert _same(host(gks), hks) and _same(host(gvs), hvs)
    ref = O8.decode_attention_q8(host(q), hk, hks, hv, hvs, bt, lens, bs, SM)
    assert_attn_close(host(out), ref, "qwen8b batch 32")


def test_append64k_then_decode(K):
    import torch
    cfg = W.APPEND_64K
    n, nq, nkv, bs = cfg["n_tok"], cfg["nq"], cfg["nkv"], cfg["kv_bs"]
    bt, nb = W.paged_block_tables(W.rng(4, 0, 2), [n], bs)
    k = W.torch_outlier_normal_bf16((n, nkv, 128), "cuda", (4, 0, 0))
    v = W.torch_outlier_normal_bf16((n, nkv, 128), "cuda", (4, 0, 1))
    slots = W.slots_for_positions(bt, [0] * n, np.arange(n), bs)
    gk, gv, gks, gvs = _q8_pools(torch, nb, bs, nkv)
    K.kvq8_quantize_append(gk, gv, gks, gvs, k, v, dev(slots))
    q = W.torch_normal((1, nq, 128), "cuda", (4, 0, 3))
    out = torch.empty((1, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq8_decode_attn(out, q, gk, gv, gks, gvs, dev(bt), dev(np.array([n], np.int32)), n, SM)
    torch.cuda.synchronize()
    hk, hv, hks, hvs = _host_pools(nb, bs, nkv)
    O8.quantize_append(hk, hv, hks, hvs, host(k.float()), host(v.float()), slots)
    assert _same(pool_pages_order(host(gk)), hk) and _same(pool_pages_order(host(gv)), hv)
    assert _same(host(gks), hks) and _same(host(gvs), hvs)
    ref = O8.decode_attention_q8(host(q), hk, hks, hv, hvs, bt, [n], bs, SM)
    assert_attn_close(host(out), ref, "append64k decode")


def test_q4_128k(K):
    import torch
    cfg = W.Q4_128K
    B, nq, nkv, L, win, bs = cfg["batch"], cfg["nq"], cfg["nkv"], cfg["L"], cfg["window"], cfg["kv_bs"]
    n4, n8 = L - win, win
    bt4, nb4 = W.paged_block_tables(W.rng(5, 0, 1), [n4] * B, bs)
    bt8, nb8 = W.paged_block_tables(W.rng(5, 0, 2), [n8] * B, bs)
    shp4, gshp4 = (nb4, bs, nkv), (nb4, nkv, bs)         # oracle slot-major, device head-major
    g4 = [torch.zeros(gshp4 + (64,), dtype=torch.uint8, device="cuda"),
          torch.zeros(gshp4 + (64,), dtype=torch.uint8, device="cuda")] + \
         [torch.zeros(gshp4 + (2,), dtype=torch.float16, device="cuda") for _ in range(4)]
    g8 = _q8_pools(torch, nb8, bs, nkv)
    sig = W.rng(5, 0, 3).uniform(0.2, 5.0, size=(B, nkv, 2))
    checked = (0, 3)
    host_cache = {}
    for b in range(B):
        sk = torch.tensor(sig[b, :, 0], dtype=torch.float32, device="cuda")[None, :, None]
        sv = torch.tensor(sig[b, :, 1], dtype=torch.float32, device="cuda")[None, :, None]
        k = W.torch_normal((L, nkv, 128), "cuda", (5, 0, b, 0)) * sk
        v = W.torch_normal((L, nkv, 128), "cuda", (5, 0, b, 1)) * sv
        s4 = W.slots_for_positions(bt4, [b] * n4, np.arange(n4), bs)
        s8 = W.slots_for_positions(bt8, [b] * n8, np.arange(n8), bs)
        K.kvq4_quantize_append(g4[0], g4[1], g4[2], g4[3], g4[4], g4[5], k[:n4], v[:n4], dev(s4))
        K.kvq8_quantize_append(g8[0], g8[1], g8[2], g8[3], k[n4:], v[n4:], dev(s8))
        if b in checked:
            host_cache[b] = (host(k), host(v), s4, s8)
        del k, v
    q = W.torch_normal((B, nq, 128), "cuda", (5, 0, 99))
    out = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq4_decode_attn(out, q, g4, dev(bt4), dev(np.full(B, n4, np.int32)), n4, g8, dev(bt8),
                       dev(np.full(B, n8, np.int32)), n8, SM)
    torch.cuda.synchronize()
    got = host(out)
    gh4 = [slot_major(host(x)) for x in g4]             # the oracle's slot-major order
    gh4[0] = q4_key_pages_order(gh4[0])                 # int4 key rows in the pages' order
    gh8 = [host(x) for x in g8]
    gh8[:2] = [pool_pages_order(x) for x in gh8[:2]]      # codes in the pages' order, as the oracle keeps them
    for b in checked:
        k, v, s4, s8 = host_cache[b]
        p4 = [np.zeros(shp4 + (64,), np.uint8), np.zeros(shp4 + (64,), np.uint8)] + \
             [np.zeros(shp4 + (2,), np.float16) for _ in range(4)]
        O4.quantize_append_q4(p4[0], p4[1], p4[2], p4[3], p4[4], p4[5], k[:n4], v[:n4], s4)
        p8 = _host_pools(nb8, bs, nkv)
        O8.quantize_append(p8[0], p8[1], p8[2], p8[3], k[n4:], v[n4:], s8)
        rows4 = bt4[b][bt4[b] >= 0]
        rows8 = bt8[b][bt8[b] >= 0]
        for x, y in zip(gh4, p4):
            assert _same(x[rows4], y[rows4]), f"int4 pool differs (seq {b})"
        for x, y in zip(gh8, p8):
            assert _same(x[rows8], y[rows8]), f"int8 window differs (seq {b})"
        ref = O4.decode_attention_mixed(host(q)[b:b + 1], (p4[0], p4[2], p4[3], p4[1], p4[4], p4[5]),
                                        bt4[b:b + 1], [n4], (p8[0], p8[2], p8[1], p8[3]), bt8[b:b + 1], [n8],
                                        bs, SM)
        assert_attn_close(got[b:b + 1], ref, f"q4_128k seq {b}")


def test_q2_128k(K):
    import torch
    cfg = W.Q2_128K
    B, nq, nkv, L, bs = cfg["batch"], cfg["nq"], cfg["nkv"], cfg["L"], cfg["kv_bs"]
    n8 = cfg["window"]
    n4 = cfg["edge4"] - n8
    n2 = L - n4 - n8
    assert (n2, n4, n8) == O2.band_lengths(L)
    bt2, nb2 = W.paged_block_tables(W.rng(9, 0, 1), [n2] * B, bs)
    bt4, nb4 = W.paged_block_tables(W.rng(9, 0, 2), [n4] * B, bs)
    bt8, nb8 = W.paged_block_tables(W.rng(9, 0, 3), [n8] * B, bs)

    def group_pool(nb, row, host_side):
        if host_side:                                   # the oracle's slot-major order
            shp = (nb, bs, nkv)
            return [np.zeros(shp + (row,), np.uint8), np.zeros(shp + (row,), np.uint8)] + \
                   [np.zeros(shp + (2,), np.float16) for _ in range(4)]
        shp = (nb, nkv, bs)                             # the device's head-major order
        return [torch.zeros(shp + (row,), dtype=torch.uint8, device="cuda"),
                torch.zeros(shp + (row,), dtype=torch.uint8, device="cuda")] + \
               [torch.zeros(shp + (2,), dtype=torch.float16, device="cuda") for _ in range(4)]
    g2, g4 = group_pool(nb2, 32, False), group_pool(nb4, 64, False)
    g8 = _q8_pools(torch, nb8, bs, nkv)
    sig = W.rng(9, 0, 4).uniform(0.2, 5.0, size=(B, nkv, 2))
    checked = (0, 3)
    host_cache = {}
    for b in range(B):
        sk = torch.tensor(sig[b, :, 0], dtype=torch.float32, device="cuda")[None, :, None]
        sv = torch.tensor(sig[b, :, 1], dtype=torch.float32, device="cuda")[None, :, None]
        k = W.torch_normal((L, nkv, 128), "cuda", (9, 0, b, 0)) * sk
        v = W.torch_normal((L, nkv, 128), "cuda", (9, 0, b, 1)) * sv
        s2 = W.slots_for_positions(bt2, [b] * n2, np.arange(n2), bs)
        s4 = W.slots_for_positions(bt4, [b] * n4, np.arange(n4), bs)
        s8 = W.slots_for_positions(bt8, [b] * n8, np.arange(n8), bs)
        K.kvq2_quantize_append(*g2, k[:n2], v[:n2], dev(s2))
        K.kvq4_quantize_append(*g4, k[n2:n2 + n4], v[n2:n2 + n4], dev(s4))
        K.kvq8_quantize_append(*g8, k[n2 + n4:], v[n2 + n4:], dev(s8))
        if b in checked:
            host_cache[b] = (host(k), host(v), s2, s4, s8)
        del k, v
    q = W.torch_normal((B, nq, 128), "cuda", (9, 0, 99))
    out = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq2_decode_attn(out, q, g2, dev(bt2), dev(np.full(B, n2, np.int32)), n2, g4, dev(bt4),
                       dev(np.full(B, n4, np.int32)), n4, g8, dev(bt8), dev(np.full(B, n8, np.int32)), n8, SM)
    torch.cuda.synchronize()
    got = host(out)
    gh2, gh4 = [slot_major(host(x)) for x in g2], [slot_major(host(x)) for x in g4]
    gh8 = [host(x) for x in g8]
    gh4[0] = q4_key_pages_order(gh4[0])                 # int4 key rows in the pages' order
    gh8[:2] = [pool_pages_order(x) for x in gh8[:2]]      # codes in the pages' order, as the oracle keeps them
    for b in checked:
        k, v, s2, s4, s8 = host_cache[b]
        p2, p4 = group_pool(nb2, 32, True), group_pool(nb4, 64, True)
        O2.quantize_append_q2(p2[0], p2[1], p2[2], p2[3], p2[4], p2[5], k[:n2], v[:n2], s2)
        O4.quantize_append_q4(p4[0], p4[1], p4[2], p4[3], p4[4], p4[5], k[n2:n2 + n4], v[n2:n2 + n4], s4)
        p8 = _host_pools(nb8, bs, nkv)
        O8.quantize_append(p8[0], p8[1], p8[2], p8[3], k[n2 + n4:], v[n2 + n4:], s8)
        for gh, ph, bt, name in ((gh2, p2, bt2, "2-bit"), (gh4, p4, bt4, "int4"), (gh8, p8, bt8, "int8")):
            rows = bt[b][bt[b] >= 0]
            for x, y in zip(gh, ph):
                assert _same(x[rows], y[rows]), f"{name} pool differs (seq {b})"
        ref = O2.decode_attention_banded(
            host(q)[b:b + 1], (p2[0], p2[2], p2[3], p2[1], p2[4], p2[5]), bt2[b:b + 1], [n2],
            (p4[0], p4[2], p4[3], p4[1], p4[4], p4[5]), bt4[b:b + 1], [n4], (p8[0], p8[2], p8[1], p8[3]),
            bt8[b:b + 1], [n8], bs, SM)
        assert_attn_close(got[b:b + 1], ref, f"q2_128k seq {b}")


def _q40_pools(torch, nb, bs, nkv):
    shp = (nb, nkv, bs)                                 # the device's head-major order
    return (torch.zeros(shp + (64,), dtype=torch.uint8, device="cuda"),
            torch.zeros(shp + (64,), dtype=torch.uint8, device="cuda"),
            torch.zeros(shp + (4,), dtype=torch.float32, device="cuda"),
            torch.zeros(shp + (4,), dtype=torch.float32, device="cuda"))


def _q40_host(nb, bs, nkv):
    shp = (nb, bs, nkv)
    return [np.zeros(shp + (64,), np.uint8), np.zeros(shp + (64,), np.uint8), np.zeros(shp + (4,), np.float32),
            np.zeros(shp + (4,), np.float32)]


def test_q40_qwen8b_batch32_layer0(K):
    import torch
    cfg = W.QWEN8B_B32
    nq, nkv, bs, B = cfg["nq"], cfg["nkv"], cfg["kv_bs"], cfg["batch"]
    lens = W.qwen8b_lengths(0)
    bt, nb = W.paged_block_tables(W.rng(3, 0, 1), lens, bs)
    gk, gv, gks, gvs = _q40_pools(torch, nb, bs, nkv)
    hk, hv, hks, hvs = _q40_host(nb, bs, nkv)
    for b in range(B):
        Lb = int(lens[b])
        k = W.torch_student_t3((Lb, nkv, 128), "cuda", (3, 0, b, 0), 0.5)
        v = W.torch_student_t3((Lb, nkv, 128), "cuda", (3, 0, b, 1), 0.5)
        slots = W.slots_for_positions(bt, [b] * Lb, np.arange(Lb), bs)
        K.kvq4_0_quantize_append(gk, gv, gks, gvs, k, v, dev(slots))
        O40.quantize_append_q4_0(hk, hv, hks, hvs, host(k), host(v), slots)
        del k, v
    q = W.torch_normal((B, nq, 128), "cuda", (3, 0, 99))
    out = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq4_0_decode_attn(out, q, gk, gv, gks, gvs, dev(bt), dev(lens), int(lens.max()), SM)
    torch.cuda.synchronize()
    assert np.array_equal(slot_major(host(gk)), hk) and np.array_equal(slot_major(host(gv)), hv)
    assert _same(slot_major(host(gks)), hks) and _same(slot_major(host(gvs)), hvs)
    ref = O40.decode_attention_q4_0(host(q), hk, hks, hv, hvs, bt, lens, bs, SM)
    assert_attn_close(host(out), ref, "Q4_0 qwen8b batch 32")


def test_q40_append64k_then_decode(K):
    import torch
    cfg = W.APPEND_64K
    n, nq, nkv, bs = cfg["n_tok"], cfg["nq"], cfg["nkv"], cfg["kv_bs"]
    bt, nb = W.paged_block_tables(W.rng(4, 0, 2), [n], bs)
    k = W.torch_outlier_normal_bf16((n, nkv, 128), "cuda", (4, 0, 0))
    v = W.torch_outlier_normal_bf16((n, nkv, 128), "cuda", (4, 0, 1))
    slots = W.slots_for_positions(bt, [0] * n, np.arange(n), bs)
    gk, gv, gks, gvs = _q40_pools(torch, nb, bs, nkv)
    K.kvq4_0_quantize_append(gk, gv, gks, gvs, k, v, dev(slots))
    q = W.torch_normal((1, nq, 128), "cuda", (4, 0, 3))
    out = torch.empty((1, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq4_0_decode_attn(out, q, gk, gv, gks, gvs, dev(bt), dev(np.array([n], np.int32)), n, SM)
    torch.cuda.synchronize()
    hk, hv, hks, hvs = _q40_host(nb, bs, nkv)
    O40.quantize_append_q4_0(hk, hv, hks, hvs, host(k.float()), host(v.float()), slots)
    assert np.array_equal(slot_major(host(gk)), hk) and np.array_equal(slot_major(host(gv)), hv)
    assert _same(slot_major(host(gks)), hks) and _same(slot_major(host(gvs)), hvs)
    ref = O40.decode_attention_q4_0(host(q), hk, hks, hv, hvs, bt, [n], bs, SM)
    assert_attn_close(host(out), ref, "Q4_0 append64k decode")
