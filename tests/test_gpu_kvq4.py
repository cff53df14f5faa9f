"""GPU parity of the int4 group variant against the CPU oracle: write path
bit-exact (packed codes, binary16 scales and zero points), mixed int4 / int8
decode within 1e-4 + 1e-4 |oracle|."""
import numpy as np
import pytest

import workloads as W
from oracle import kvq4 as O4
from oracle import kvq8 as O8
from tests.helpers import (SM, Q8Cache, assert_attn_close, dev, head_major, host, q4_key_library_order,
                           q4_key_pages_order, slot_major)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import decode_attention_int8_amd as K
    return K


class Q4Pool:
    """An int4 pool held both on the host (oracle: slot-major, key rows in the
    pages' order) and on the GPU (head-major, the library's key order)."""

    def __init__(self, nb, bs, nkv):
        import torch
        shp, gshp = (nb, bs, nkv), (nb, nkv, bs)
        self.bs = bs
        self.h = [np.zeros(shp + (64,), np.uint8), np.zeros(shp + (64,), np.uint8)] + \
                 [np.zeros(shp + (2,), np.float16) for _ in range(4)]
        self.g = [torch.zeros(gshp + (64,), dtype=torch.uint8, device="cuda"),
                  torch.zeros(gshp + (64,), dtype=torch.uint8, device="cuda")] + \
                 [torch.zeros(gshp + (2,), dtype=torch.float16, device="cuda") for _ in range(4)]

    def append(self, K, k, v, slots, gk=None, gv=None):
        h = self.h
        O4.quantize_append_q4(h[0], h[1], h[2], h[3], h[4], h[5], k, v, slots)
        K.kvq4_quantize_append(*self.g, dev(k) if gk is None else gk, dev(v) if gv is None else gv,
                               dev(np.asarray(slots, np.int32)))

    def oracle_pools(self):
        h = self.h
        return (h[0], h[2], h[3], h[1], h[4], h[5])

    def device_expect(self):
        """The oracle's pool in the device's order."""
        return [head_major(q4_key_library_order(self.h[0]))] + [head_major(x) for x in self.h[1:]]

    def assert_same(self):
        # compared in the oracle's order: slot-major, key rows in the pages' order
        got = [q4_key_pages_order(slot_major(host(self.g[0])))] + [slot_major(host(x)) for x in self.g[1:]]
        for x, y in zip(got, self.h):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_q4_write_bit_exact(K, dtype):
    import torch
    r = W.rng(400, ["f32", "bf16", "f16"].index(dtype))
    n, nkv, bs, nb = 333, 4, 16, 32
    x = W.per_unit_sigma_normal(r, (n, nkv, 128), 2, 0.2, 5.0)
    y = W.student_t3_f32(r, (n, nkv, 128), 0.5)
    x[0, 0, :64] = 1.25                       # constant group -> scale 1
    x[1, 1] = np.abs(x[1, 1]) + 3             # groups above zero: zero point clamps
    x[2, 2] = -np.abs(x[2, 2]) - 3            # groups below zero
    x[3, 3, :] = 1e-9                         # tiny spread: scale floor
    x[3, 3, 5] = 2e-9
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    gx, gy = dev(x).to(tdt), dev(y).to(tdt)
    slots = r.permutation(nb * bs)[:n].astype(np.int32)
    slots[7] = -1
    p = Q4Pool(nb, bs, nkv)
    p.append(K, gx.float().cpu().numpy(), gy.float().cpu().numpy(), slots, gx, gy)
    torch.cuda.synchronize()
    p.assert_same()


@pytest.mark.parametrize("g", [1, 4, 8])
def test_q4_mixed_decode(K, g):
    r = W.rng(410, g)
    nkv, bs = 2, 16
    nq = g * nkv
    lens4 = np.array([0, 1, 300, 1500, 64], np.int32)
    lens8 = np.array([5, 0, 64, 257, 0], np.int32)
    B = len(lens4)
    bt4, nb4 = W.paged_block_tables(r, lens4, bs, spare_blocks=1)
    bt8, nb8 = W.paged_block_tables(r, lens8, bs, spare_blocks=1)
    p4 = Q4Pool(nb4, bs, nkv)
    c8 = Q8Cache(nb8, bs, nkv)
    for b in range(B):
        if lens4[b]:
            k = W.per_unit_sigma_normal(r, (int(lens4[b]), nkv, 128), 0, 0.5, 2.0)
            sl = W.slots_for_positions(bt4, [b] * lens4[b], np.arange(lens4[b]), bs)
            p4.append(K, k, W.normal_f32(r, k.shape), sl)
        if lens8[b]:
            k = W.normal_f32(r, (int(lens8[b]), nkv, 128))
            sl = W.slots_for_positions(bt8, [b] * lens8[b], np.arange(lens8[b]), bs)
            c8.append(k, W.normal_f32(r, k.shape), sl)
    import torch
    q = W.normal_f32(r, (B, nq, 128), 2.0)
    out = torch.full((B, nq, 128), float("nan"), dtype=torch.float32, device="cuda")
    K.kvq4_decode_attn(out, dev(q), p4.g, dev(bt4), dev(lens4), int(lens4.max()),
                       (c8.gk, c8.gv, c8.gks, c8.gvs), dev(bt8), dev(lens8), int(lens8.max()), SM)
    torch.cuda.synchronize()
    p4.assert_same()
    ref = O4.decode_attention_mixed(q, p4.oracle_pools(), bt4, lens4, (c8.kp, c8.ks, c8.vp, c8.vs), bt8, lens8,
                                    bs, SM)
    assert_attn_close(host(out), ref, f"int4 mixed g={g}")


@pytest.mark.parametrize("chunk", [512, 768, 1280, 2048])
def test_q4_mixed_decode_chunk_sizes(K, chunk):
    """Chunks of 2-8 tiles per wave with ragged lengths: every wave count of
    tiles from 1 to 8 occurs (the walks run two tiles per trip, then one or
    two more)."""
    r = W.rng(411, chunk)
    nkv, bs, g = 2, 16, 4
    nq = g * nkv
    lens4 = np.array([3001, 1, 700, 2300, 1279], np.int32)
    lens8 = np.array([100, 64, 0, 257, 1], np.int32)
    B = len(lens4)
    bt4, nb4 = W.paged_block_tables(r, lens4, bs)
    bt8, nb8 = W.paged_block_tables(r, lens8, bs, spare_blocks=1)
    p4 = Q4Pool(nb4, bs, nkv)
    c8 = Q8Cache(nb8, bs, nkv)
    for b in range(B):
        k = W.per_unit_sigma_normal(r, (int(lens4[b]), nkv, 128), 0, 0.5, 2.0)
        p4.append(K, k, W.normal_f32(r, k.shape), W.slots_for_positions(bt4, [b] * lens4[b], np.arange(lens4[b]), bs))
        if lens8[b]:
            k = W.normal_f32(r, (int(lens8[b]), nkv, 128))
            c8.append(k, W.normal_f32(r, k.shape), W.slots_for_positions(bt8, [b] * lens8[b], np.arange(lens8[b]), bs))
    import torch
    q = W.normal_f32(r, (B, nq, 128), 2.0)
    out = torch.full((B, nq, 128), float("nan"), dtype=torch.float32, device="cuda")
    K.kvq4_decode_attn(out, dev(q), p4.g, dev(bt4), dev(lens4), int(lens4.max()),
                       (c8.gk, c8.gv, c8.gks, c8.gvs), dev(bt8), dev(lens8), int(lens8.max()), SM, chunk=chunk)
    torch.cuda.synchronize()
    ref = O4.decode_attention_mixed(q, p4.oracle_pools(), bt4, lens4, (c8.kp, c8.ks, c8.vp, c8.vs), bt8, lens8,
                                    bs, SM)
    assert_attn_close(host(out), ref, f"int4 mixed chunk {chunk}")


def test_q4_only_int8_window_equals_int8_path(K):
    import torch
    r = W.rng(420)
    nq, nkv, bs = 8, 2, 16
    lens = np.array([700, 33], np.int32)
    bt, nb = W.paged_block_tables(r, lens, bs)
    c8 = Q8Cache(nb, bs, nkv)
    for b in range(2):
        k = W.normal_f32(r, (int(lens[b]), nkv, 128))
        c8.append(k, k * np.float32(0.5), W.slots_for_positions(bt, [b] * lens[b], np.arange(lens[b]), bs))
    p4 = Q4Pool(4, bs, nkv)
    q = W.normal_f32(r, (2, nq, 128))
    o4 = torch.empty((2, nq, 128), dtype=torch.float32, device="cuda")
    o8 = torch.empty_like(o4)
    zero = np.zeros(2, np.int32)
    K.kvq4_decode_attn(o4, dev(q), p4.g, dev(np.zeros((2, 1), np.int32)), dev(zero), 0,
                       (c8.gk, c8.gv, c8.gks, c8.gvs), dev(bt), dev(lens), 700, SM)
    K.kvq8_decode_attn(o8, dev(q), c8.gk, c8.gv, c8.gks, c8.gvs, dev(bt), dev(lens), 700, SM)
    torch.cuda.synchronize()
    ref = O8.decode_attention_q8(q, c8.kp, c8.ks, c8.vp, c8.vs, bt, lens, bs, SM)
    assert_attn_close(host(o4), ref, "int4 entry, int8 only")
    assert_attn_close(host(o8), ref, "int8 entry")


# ----------------------------------------------------------------------------
# re-quantization of aging int8 tokens into the int4 pool ([P4] Sec. 3.3)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("bs", [8, 16])
def test_requantize_bit_exact(K, bs):
    """int8 -> int4 migration equals the oracle bit for bit (codes, binary16
    scales and zero points), including skipped pairs and groups whose zero
    point clamps."""
    import torch
    r = W.rng(420, bs)
    nkv, nb8, nb4, n = 4, 24, 20, 150
    c8 = Q8Cache(nb8, bs, nkv)
    x = W.per_unit_sigma_normal(r, (nb8 * bs, nkv, 128), 2, 0.2, 5.0)
    y = W.student_t3_f32(r, (nb8 * bs, nkv, 128), 0.5)
    x[3, 1] = np.abs(x[3, 1]) + 2               # all above zero
    x[4, 2, :] = 0.75                           # constant row
    c8.append(x, y, np.arange(nb8 * bs, dtype=np.int32))
    p4 = Q4Pool(nb4, bs, nkv)
    src = r.permutation(nb8 * bs)[:n].astype(np.int32)
    dst = r.permutation(nb4 * bs)[:n].astype(np.int32)
    src[5], dst[9], src[11] = -1, nb4 * bs, nb8 * bs + 3   # skipped pairs
    O4.requantize_q8_to_q4((c8.kp, c8.ks, c8.vp, c8.vs), p4.oracle_pools(), src, dst)
    K.kvq4_requantize_q8(p4.g, (c8.gk, c8.gv, c8.gks, c8.gvs), dev(src), dev(dst))
    torch.cuda.synchronize()
    c8.assert_device_matches_host()
    p4.assert_same()


def test_requantize_time_block_then_decode(K):
    """The lifecycle of the 128K workload in miniature: a sequence keeps its
    newest tokens in the int8 window; the oldest 512-token time block moves to
    the int4 pool (bit-exact against the oracle), the block tables are
    switched, and the mixed decode over both pools matches the oracle."""
    import torch
    r = W.rng(421)
    nq, nkv, bs, B = 16, 4, 16, 2
    L4, L8, T = 1024, 1024, 512                     # int4 history, int8 window, time block
    bt4, nb4 = W.paged_block_tables(r, [L4 + T] * B, bs)
    bt8, nb8 = W.paged_block_tables(r, [L8] * B, bs)
    p4 = Q4Pool(nb4, bs, nkv)
    c8 = Q8Cache(nb8, bs, nkv)
    for b in range(B):
        s4 = W.slots_for_positions(bt4, [b] * L4, np.arange(L4), bs)
        p4.append(K, W.normal_f32(r, (L4, nkv, 128)), W.normal_f32(r, (L4, nkv, 128)), s4)
        s8 = W.slots_for_positions(bt8, [b] * L8, np.arange(L8), bs)
        c8.append(W.normal_f32(r, (L8, nkv, 128), 0.7), W.normal_f32(r, (L8, nkv, 128), 1.3), s8)
    # move window positions [0, T) of each sequence to int4 positions [L4, L4 + T)
    src = np.concatenate([W.slots_for_positions(bt8, [b] * T, np.arange(T), bs) for b in range(B)]).astype(np.int32)
    dst = np.concatenate([W.slots_for_positions(bt4, [b] * T, L4 + np.arange(T), bs)
                          for b in range(B)]).astype(np.int32)
    O4.requantize_q8_to_q4((c8.kp, c8.ks, c8.vp, c8.vs), p4.oracle_pools(), src, dst)
    K.kvq4_requantize_q8(p4.g, (c8.gk, c8.gv, c8.gks, c8.gvs), dev(src), dev(dst))
    torch.cuda.synchronize()
    p4.assert_same()
    # the window now starts T tokens later: shift its table by T / bs blocks
    bt8n = np.full_like(bt8, -1)
    bt8n[:, :(L8 - T) // bs] = bt8[:, T // bs:L8 // bs]
    lens4 = np.full(B, L4 + T, np.int32)
    lens8 = np.full(B, L8 - T, np.int32)
    q = W.normal_f32(r, (B, nq, 128))
    ref = O4.decode_attention_mixed(q, p4.oracle_pools(), bt4, lens4, (c8.kp, c8.ks, c8.vp, c8.vs), bt8n, lens8,
                                    bs, SM)
    out = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq4_decode_attn(out, dev(q), tuple(p4.g), dev(bt4), dev(lens4), L4 + T, (c8.gk, c8.gv, c8.gks, c8.gvs),
                       dev(bt8n), dev(lens8), L8 - T, SM)
    assert_attn_close(host(out), ref, "after migration")


def test_requantize_large_bit_exact(K):
    """A move above 65536 rows (the kernel's four-rows-per-group form), with a
    ragged tail of rows and skipped pairs."""
    import torch
    r = W.rng(422)
    nkv, bs, n = 4, 16, 8195                        # 65560 rows: not a multiple of the 64-row workgroup
    nb8, nb4 = 540, 560
    c8 = Q8Cache(nb8, bs, nkv)
    x = W.per_unit_sigma_normal(r, (nb8 * bs, nkv, 128), 2, 0.2, 5.0)
    y = W.normal_f32(r, (nb8 * bs, nkv, 128), 0.3)
    c8.append(x, y, np.arange(nb8 * bs, dtype=np.int32))
    p4 = Q4Pool(nb4, bs, nkv)
    src = r.permutation(nb8 * bs)[:n].astype(np.int32)
    dst = r.permutation(nb4 * bs)[:n].astype(np.int32)
    src[17], dst[4000], src[n - 1] = -5, -1, nb8 * bs
    O4.requantize_q8_to_q4((c8.kp, c8.ks, c8.vp, c8.vs), p4.oracle_pools(), src, dst)
    K.kvq4_requantize_q8(p4.g, (c8.gk, c8.gv, c8.gks, c8.gvs), dev(src), dev(dst))
    torch.cuda.synchronize()
    p4.assert_same()
