"""HIP graph capture and replay of every decode, re-quantization and
write entry point (the int8 fused step has its own replay test with the qwen2b
workload).  Each call is checked eagerly against the oracle, then captured
once and replayed three times.  Between replays the program does eager work
of its own: it poisons the output, overwrites the destination rows and
synchronizes.  Every replay must equal the eager call bit for bit."""
import numpy as np
import pytest

import workloads as W
from oracle import kvq2 as O2
from oracle import kvq4 as O4
from oracle import kvq4_0 as O40
from oracle import kvq8 as O8
from tests.helpers import SM, Q8Cache, assert_attn_close, dev, fill_sequences, host, pool_library_order
from tests.test_gpu_kvq2 import Q2Pool, _banded
from tests.test_gpu_kvq4 import Q4Pool
from tests.test_gpu_kvq4_0 import Q40Cache

pytestmark = pytest.mark.gpu

NQ, NKV, BS = 8, 2, 16


@pytest.fixture(scope="module")
def K():
    import decode_attention_int8_amd as K
    return K


def _replays(call, reset, check):
    """Warm up on a side stream (as capture requires), capture `call`, then
    three rounds of: eager `reset`, sync, replay, sync, `check`."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(rep)


def _decode_replays(K, call, out, what):
    """Eager result of `call(out)`, then replays of it into the same output."""
    import torch
    call()
    torch.cuda.synchronize()
    eager = host(out).copy()

    def check(rep):
        assert np.array_equal(host(out), eager), f"{what}: replay {rep} differs from the eager call"

    _replays(call, lambda: out.fill_(float("nan")), check)
    return eager


@pytest.mark.parametrize("chunk", [0, 256])
def test_int8_decode_replays(K, chunk):
    import torch
    r = W.rng(950, chunk)
    lens = np.array([700, 1300, 33, 0], np.int32)
    B, Lm = len(lens), int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, BS, spare_blocks=1)
    c = Q8Cache(nb, BS, NKV)
    fill_sequences(c, bt, lens, W.normal_f32(r, (B, Lm, NKV, 128)), W.normal_f32(r, (B, Lm, NKV, 128)))
    q = dev(W.normal_f32(r, (B, NQ, 128)))
    btd, ld = dev(bt), dev(lens)
    ws = K.alloc_workspace(K.kvq8_decode_workspace_size(B, NQ, NKV, Lm, chunk), "cuda")
    out = torch.empty((B, NQ, 128), dtype=torch.float32, device="cuda")
    got = _decode_replays(K, lambda: K.kvq8_decode_attn(out, q, c.gk, c.gv, c.gks, c.gvs, btd, ld, Lm, SM,
                                                        chunk, ws), out, "int8")
    ref = O8.decode_attention_q8(host(q), c.kp, c.ks, c.vp, c.vs, bt, lens, BS, SM)
    assert_attn_close(got, ref, f"int8 chunk={chunk}")


@pytest.mark.parametrize("B", [1, 3])
def test_q40_decode_replays(K, B):
    import torch
    r = W.rng(951, B)
    lens = np.array([1000, 37, 513][:B], np.int32)
    Lm = int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, BS, spare_blocks=1)
    c = Q40Cache(nb, BS, NKV)
    for b in range(B):
        sl = W.slots_for_positions(bt, [b] * int(lens[b]), np.arange(lens[b]), BS)
        c.append(W.normal_f32(r, (int(lens[b]), NKV, 128)), W.normal_f32(r, (int(lens[b]), NKV, 128)), sl)
    q = dev(W.normal_f32(r, (B, NQ, 128)))
    btd, ld = dev(bt), dev(lens)
    ws = K.alloc_workspace(K.kvq4_0_decode_workspace_size(B, NQ, NKV, Lm), "cuda")
    out = torch.empty((B, NQ, 128), dtype=torch.float32, device="cuda")
    got = _decode_replays(K, lambda: K.kvq4_0_decode_attn(out, q, c.gk, c.gv, c.gks, c.gvs, btd, ld, Lm, SM,
                                                          0, ws), out, "Q4_0")
    ref = O40.decode_attention_q4_0(host(q), c.kp, c.ks, c.vp, c.vs, bt, lens, BS, SM)
    assert_attn_close(got, ref, f"Q4_0 B={B}")


def test_group_band_decode_replays(K):
    """The int4 + int8 decode and the three-band decode over the same pools."""
    import torch
    r = W.rng(952)
    lens2 = np.array([900, 0, 300], np.int32)
    lens4 = np.array([256, 100, 17], np.int32)
    lens8 = np.array([64, 200, 5], np.int32)
    B = len(lens2)
    (p2, bt2), (p4, bt4), (c8, bt8) = _banded(K, r, lens2, lens4, lens8, NQ, NKV, BS)
    q = dev(W.normal_f32(r, (B, NQ, 128), 2.0))
    m2, m4, m8 = int(lens2.max()), int(lens4.max()), int(lens8.max())
    d2, d4, d8 = (dev(bt2), dev(lens2)), (dev(bt4), dev(lens4)), (dev(bt8), dev(lens8))
    pool8 = (c8.gk, c8.gv, c8.gks, c8.gvs)
    host8 = (c8.kp, c8.ks, c8.vp, c8.vs)

    ws4 = K.alloc_workspace(K.kvq4_decode_workspace_size(B, NQ, NKV, m4, m8), "cuda")
    out4 = torch.empty((B, NQ, 128), dtype=torch.float32, device="cuda")
    got4 = _decode_replays(K, lambda: K.kvq4_decode_attn(out4, q, p4.g, *d4, m4, pool8, *d8, m8, SM, 0, ws4),
                           out4, "int4 + int8")
    ref4 = O4.decode_attention_mixed(host(q), p4.oracle_pools(), bt4, lens4, host8, bt8, lens8, BS, SM)
    assert_attn_close(got4, ref4, "int4 + int8")

    ws2 = K.alloc_workspace(K.kvq2_decode_workspace_size(B, NQ, NKV, m2, m4, m8), "cuda")
    out2 = torch.empty((B, NQ, 128), dtype=torch.float32, device="cuda")
    got2 = _decode_replays(K, lambda: K.kvq2_decode_attn(out2, q, p2.g, *d2, m2, p4.g, *d4, m4, pool8, *d8, m8,
                                                         SM, 0, ws2), out2, "three bands")
    ref2 = O2.decode_attention_banded(host(q), p2.oracle_pools(), bt2, lens2, p4.oracle_pools(), bt4, lens4,
                                      host8, bt8, lens8, BS, SM)
    assert_attn_close(got2, ref2, "three bands")


def _requant_replays(call, dst_pool, expect, what):
    """`call` writes `dst_pool` (device tensors); between replays the pool is
    zeroed eagerly.  Eager and replayed contents must equal `expect` (host
    arrays in the same order) bit for bit."""
    import torch

    def same(rep):
        for i, (x, y) in enumerate(zip(dst_pool, expect)):
            assert np.array_equal(host(x).view(np.uint8), y.view(np.uint8)), f"{what}: {rep} array {i} differs"

    call()
    torch.cuda.synchronize()
    same("eager")
    _replays(call, lambda: [t.zero_() for t in dst_pool], lambda rep: same(f"replay {rep}"))


def test_requantize_replays(K):
    """int8 -> int4 and int4 -> 2-bit re-quantization of 300 rows, including
    skipped pairs (negative source, destination past the pool)."""
    r = W.rng(953)
    n, nb8, nb4, nb2 = 300, 24, 24, 24
    c8 = Q8Cache(nb8, BS, NKV)
    x = W.per_unit_sigma_normal(r, (n, NKV, 128), 1, 0.2, 5.0)
    c8.append(x, W.student_t3_f32(r, x.shape, 0.5), r.permutation(nb8 * BS)[:n].astype(np.int32))
    src8 = r.permutation(nb8 * BS)[:n].astype(np.int32)
    dst4 = r.permutation(nb4 * BS)[:n].astype(np.int32)
    src8[0], dst4[1] = -1, nb4 * BS
    p4 = Q4Pool(nb4, BS, NKV)
    O4.requantize_q8_to_q4((c8.kp, c8.ks, c8.vp, c8.vs), p4.oracle_pools(), src8, dst4)
    s8, d4 = dev(src8), dev(dst4)
    _requant_replays(lambda: K.kvq4_requantize_q8(p4.g, (c8.gk, c8.gv, c8.gks, c8.gvs), s8, d4), p4.g,
                     p4.device_expect(), "int8 -> int4")

    src4 = r.permutation(nb4 * BS)[:n].astype(np.int32)
    dst2 = r.permutation(nb2 * BS)[:n].astype(np.int32)
    src4[2], dst2[3] = -1, nb2 * BS
    p2 = Q2Pool(nb2, BS, NKV)
    O2.requantize_q4_to_q2(p4.oracle_pools(), p2.oracle_pools(), src4, dst2)
    s4, d2 = dev(src4), dev(dst2)
    _requant_replays(lambda: K.kvq2_requantize_q4(p2.g, p4.g, s4, d2), p2.g, p2.device_expect(), "int4 -> 2-bit")


@pytest.mark.parametrize("mode", ["int8", "int4", "2-bit", "Q4_0"])
def test_write_path_replays(K, mode):
    """The quantize-append of 300 bf16 rows into a paged pool, with the pool
    zeroed eagerly between replays; the eager write equals the oracle's."""
    import torch
    r = W.rng(954, ["int8", "int4", "2-bit", "Q4_0"].index(mode))
    n, nb = 300, 24
    x = W.per_unit_sigma_normal(r, (n, NKV, 128), 1, 0.2, 5.0)
    y = W.student_t3_f32(r, x.shape, 0.5)
    kb = torch.from_numpy(x).to("cuda", torch.bfloat16)
    vb = torch.from_numpy(y).to("cuda", torch.bfloat16)
    xe, ye = host(kb.float()), host(vb.float())      # the exact values the kernel reads
    slots = r.permutation(nb * BS)[:n].astype(np.int32)
    sd = dev(slots)
    if mode == "int8":
        c = Q8Cache(nb, BS, NKV)
        O8.quantize_append(c.kp, c.vp, c.ks, c.vs, xe, ye, slots)
        pool = [c.gk, c.gv, c.gks, c.gvs]
        expect = [pool_library_order(c.kp), pool_library_order(c.vp), c.ks, c.vs]   # the device's storage order
        call = lambda: K.kvq8_quantize_append(*pool, kb, vb, sd)
    elif mode == "Q4_0":
        c = Q40Cache(nb, BS, NKV)
        O40.quantize_append_q4_0(c.kp, c.vp, c.ks, c.vs, xe, ye, slots)
        pool = [c.gk, c.gv, c.gks, c.gvs]
        expect = c.device_expect()
        call = lambda: K.kvq4_0_quantize_append(*pool, kb, vb, sd)
    elif mode == "int4":
        p = Q4Pool(nb, BS, NKV)
        O4.quantize_append_q4(*p.h, xe, ye, slots)
        pool, expect = p.g, p.device_expect()
        call = lambda: K.kvq4_quantize_append(*pool, kb, vb, sd)
    else:
        p = Q2Pool(nb, BS, NKV)
        O2.quantize_append_q2(*p.h, xe, ye, slots)
        pool, expect = p.g, p.device_expect()
        call = lambda: K.kvq2_quantize_append(*pool, kb, vb, sd)
    _requant_replays(call, pool, expect, f"{mode} write")
