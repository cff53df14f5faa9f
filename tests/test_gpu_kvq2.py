"""GPU parity of the 2-bit band against the CPU oracle: write path and int4 ->
2-bit re-quantization bit-exact (packed codes, binary16 scales and zero
points), banded decode (2-bit + int4 + int8) within 1e-4 + 1e-4 |oracle|."""
import numpy as np
import pytest

import workloads as W
from oracle import kvq2 as O2
from tests.helpers import SM, Q8Cache, assert_attn_close, dev, head_major, host, slot_major
from tests.test_gpu_kvq4 import Q4Pool

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import decode_attention_int8_amd as K
    return K


class Q2Pool:
    """A 2-bit pool held both on the host (oracle) and on the GPU; device
    order (k, v, k_scale, k_zero, v_scale, v_zero)."""

    def __init__(self, nb, bs, nkv):
        import torch
        shp, gshp = (nb, bs, nkv), (nb, nkv, bs)     # oracle slot-major, device head-major
        self.bs = bs
        self.h = [np.zeros(shp + (32,), np.uint8), np.zeros(shp + (32,), np.uint8)] + \
                 [np.zeros(shp + (2,), np.float16) for _ in range(4)]
        self.g = [torch.zeros(gshp + (32,), dtype=torch.uint8, device="cuda"),
                  torch.zeros(gshp + (32,), dtype=torch.uint8, device="cuda")] + \
                 [torch.zeros(gshp + (2,), dtype=torch.float16, device="cuda") for _ in range(4)]

    def append(self, K, k, v, slots, gk=None, gv=None):
        h = self.h
        O2.quantize_append_q2(h[0], h[1], h[2], h[3], h[4], h[5], k, v, slots)
        K.kvq2_quantize_append(*self.g, dev(k) if gk is None else gk, dev(v) if gv is None else gv,
                               dev(np.asarray(slots, np.int32)))

    def oracle_pools(self):
        h = self.h
        return (h[0], h[2], h[3], h[1], h[4], h[5])

    def device_expect(self):
        """The oracle's pool in the device's order."""
        return [head_major(x) for x in self.h]

    def assert_same(self, what=""):
        for i, (x, y) in enumerate(zip(self.g, self.h)):
            assert np.array_equal(slot_major(host(x)).view(np.uint8), y.view(np.uint8)), f"{what} array {i} differs"


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_q2_write_bit_exact(K, dtype):
    import torch
    r = W.rng(800, ["f32", "bf16", "f16"].index(dtype))
    n, nkv, bs, nb = 333, 4, 16, 32
    x = W.per_unit_sigma_normal(r, (n, nkv, 128), 2, 0.2, 5.0)
    y = W.student_t3_f32(r, (n, nkv, 128), 0.5)
    x[0, 0, :64] = 1.25                       # constant group -> scale 1
    x[1, 1] = np.abs(x[1, 1]) + 3             # groups above zero: zero point clamps at 0
    x[2, 2] = -np.abs(x[2, 2]) - 3            # groups below zero: clamps at 3
    x[3, 3, :] = 1e-9                         # tiny spread: scale floor
    x[3, 3, 5] = 2e-9
    x[4, 0] = np.repeat(np.arange(4, dtype=np.float32), 32) * np.float32(0.5)   # exact grid
    x[5, 1, :64] = np.float32(0.75) * (np.arange(64) % 7 - 3).astype(np.float32)  # ties at x / s + z
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    gx, gy = dev(x).to(tdt), dev(y).to(tdt)
    slots = r.permutation(nb * bs)[:n].astype(np.int32)
    slots[7] = -1
    slots[8] = nb * bs + 3
    p = Q2Pool(nb, bs, nkv)
    p.append(K, gx.float().cpu().numpy(), gy.float().cpu().numpy(), slots, gx, gy)
    torch.cuda.synchronize()
    p.assert_same("write")


@pytest.mark.parametrize("nkv", [1, 3, 5])
def test_q2_write_head_counts_and_overwrite(K, nkv):
    import torch
    r = W.rng(801, nkv)
    n, bs = 1001, 8
    nb = (n + 40) // bs + 2
    p = Q2Pool(nb, bs, nkv)
    x = W.normal_f32(r, (n, nkv, 128))
    slots = r.permutation(nb * bs)[:n].astype(np.int32)
    p.append(K, x, x[::-1].copy(), slots)
    b = W.normal_f32(r, (3, nkv, 128), 9.0)
    p.append(K, b[:2], b[:2], slots[[5, 7]])  # rewrite two slots
    p.append(K, b[2:], b[2:], slots[[5]])     # and one again: the later call wins
    K.kvq2_quantize_append(*p.g, dev(b[:0]), dev(b[:0]), dev(np.zeros(0, np.int32)))
    torch.cuda.synchronize()
    p.assert_same("write")


@pytest.mark.parametrize("n", [5, 3000])
def test_requantize_q4_to_q2_bit_exact(K, n):
    """Both kernel shapes (1 and 4 rows per 16-lane group): int4 rows written
    by the int4 write path move to other 2-bit slots; skipped pairs leave
    their destinations alone."""
    import torch
    r = W.rng(802, n)
    nkv, bs = 4, 16
    nb4 = n // bs + 4
    nb2 = n // bs + 6
    p4 = Q4Pool(nb4, bs, nkv)
    x = W.per_unit_sigma_normal(r, (n, nkv, 128), 1, 0.2, 5.0)
    p4.append(K, x, W.student_t3_f32(r, x.shape, 0.5), r.permutation(nb4 * bs)[:n].astype(np.int32))
    p2 = Q2Pool(nb2, bs, nkv)
    src = r.permutation(nb4 * bs)[:n].astype(np.int32)
    dst = r.permutation(nb2 * bs)[:n].astype(np.int32)
    src[0] = -1
    if n > 3:
        dst[2] = nb2 * bs
        src[3] = nb4 * bs + 1
    O2.requantize_q4_to_q2(p4.oracle_pools(), p2.oracle_pools(), src, dst)
    K.kvq2_requantize_q4(p2.g, p4.g, dev(src), dev(dst))
    torch.cuda.synchronize()
    p4.assert_same()
    p2.assert_same("requant")


def _banded(K, r, lens2, lens4, lens8, nq, nkv, bs, spare=1):
    B = len(lens2)
    bt2, nb2 = W.paged_block_tables(r, lens2, bs, spare_blocks=spare)
    bt4, nb4 = W.paged_block_tables(r, lens4, bs, spare_blocks=spare)
    bt8, nb8 = W.paged_block_tables(r, lens8, bs, spare_blocks=spare)
    p2, p4, c8 = Q2Pool(nb2, bs, nkv), Q4Pool(nb4, bs, nkv), Q8Cache(nb8, bs, nkv)
    for b in range(B):
        for L, bt, fill in ((lens2[b], bt2, lambda k, v, s: p2.append(K, k, v, s)),
                            (lens4[b], bt4, lambda k, v, s: p4.append(K, k, v, s)),
                            (lens8[b], bt8, lambda k, v, s: c8.append(k, v, s))):
            if L:
                k = W.per_unit_sigma_normal(r, (int(L), nkv, 128), 0, 0.5, 2.0)
                fill(k, W.normal_f32(r, k.shape), W.slots_for_positions(bt, [b] * L, np.arange(L), bs))
    return (p2, bt2), (p4, bt4), (c8, bt8)


def _decode_and_check(K, q, bands, lens, what, chunk=0, bad=None):
    import torch
    (p2, bt2), (p4, bt4), (c8, bt8) = bands
    lens2, lens4, lens8 = lens
    gbt2 = bt2 if bad is None else bad
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    K.kvq2_decode_attn(out, dev(q), p2.g, dev(gbt2), dev(lens2), int(max(lens2.max(), 0)), p4.g, dev(bt4),
                       dev(lens4), int(max(lens4.max(), 0)), (c8.gk, c8.gv, c8.gks, c8.gvs), dev(bt8), dev(lens8),
                       int(max(lens8.max(), 0)), SM, chunk=chunk)
    torch.cuda.synchronize()
    ref = O2.decode_attention_banded(q, p2.oracle_pools(), bt2, lens2, p4.oracle_pools(), bt4, lens4,
                                     (c8.kp, c8.ks, c8.vp, c8.vs), bt8, lens8, p2.bs, SM)
    return host(out), ref


@pytest.mark.parametrize("g", [1, 2, 4, 8])
@pytest.mark.parametrize("bs", [8, 16, 64])
def test_banded_decode_ragged(K, g, bs):
    r = W.rng(810, g, bs)
    nkv = 2 if g < 8 else 1
    nq = g * nkv
    lens2 = np.array([0, 1, 700, 1500, 64, 0, 257], np.int32)
    lens4 = np.array([5, 0, 300, 64, 0, 0, 1000], np.int32)
    lens8 = np.array([5, 0, 64, 257, 1, 0, 0], np.int32)
    bands = _banded(K, r, lens2, lens4, lens8, nq, nkv, bs)
    bands[0][0].assert_same("2-bit fill")
    q = W.normal_f32(r, (len(lens2), nq, 128), 2.0)
    got, ref = _decode_and_check(K, q, bands, (lens2, lens4, lens8), f"g={g} bs={bs}")
    assert_attn_close(got, ref, f"banded g={g} bs={bs}")
    assert np.all(got[5] == 0.0)                          # empty context in every band


@pytest.mark.parametrize("chunk", [256, 512, 768, 2048])
def test_banded_decode_chunk_sizes(K, chunk):
    r = W.rng(811, chunk)
    nkv, bs, g = 2, 16, 4
    lens2 = np.array([3001, 1, 700, 2300], np.int32)
    lens4 = np.array([1279, 64, 0, 2048], np.int32)
    lens8 = np.array([100, 64, 5, 257], np.int32)
    bands = _banded(K, r, lens2, lens4, lens8, g * nkv, nkv, bs)
    q = W.normal_f32(r, (4, g * nkv, 128), 3.0)
    got, ref = _decode_and_check(K, q, bands, (lens2, lens4, lens8), f"chunk {chunk}", chunk=chunk)
    assert_attn_close(got, ref, f"banded chunk {chunk}")


def test_banded_decode_two_bit_only_and_skipped_blocks(K):
    """Only the 2-bit band holds tokens in some sequences; a block id outside
    the 2-bit pool skips its tokens (the oracle drops the same block)."""
    r = W.rng(812)
    nkv, bs, g = 2, 16, 2
    lens2 = np.array([500, 96], np.int32)
    lens4 = np.array([0, 0], np.int32)
    lens8 = np.array([0, 17], np.int32)
    bands = _banded(K, r, lens2, lens4, lens8, g * nkv, nkv, bs)
    (p2, bt2) = bands[0]
    q = W.normal_f32(r, (2, g * nkv, 128))
    got, ref = _decode_and_check(K, q, bands, (lens2, lens4, lens8), "2-bit only")
    assert_attn_close(got, ref, "2-bit only")
    bad = bt2.copy()
    bad[0, 3] = p2.g[0].shape[0] + 7                      # outside the pool: tokens 48..63 skipped
    got_bad, _ = _decode_and_check(K, q, bands, (lens2, lens4, lens8), "bad block", bad=bad)
    keep = np.r_[0:48, 64:500]
    from oracle import kvq8 as O8
    qi, qsc = O8.quantize_q_blocks(q[0])
    q_hat = O8.dequantize_q_blocks(qi, qsc)
    h2 = p2.oracle_pools()
    for h in range(g * nkv):
        G = lambda pool: O8.gather_rows(pool, bt2[0], 500, bs, h // g)  # noqa: E731
        Kd = O2.dequantize_groups_q2(O2.unpack_k2(G(h2[0])), G(h2[1]), G(h2[2]))[keep]
        Vd = O2.dequantize_groups_q2(O2.unpack_v2(G(h2[3])), G(h2[4]), G(h2[5]))[keep]
        assert_attn_close(got_bad[0, h], O8.softmax_attention_f64(q_hat[h], Kd, Vd, SM), f"bad block head {h}")
    assert_attn_close(got_bad[1], ref[1], "other sequence unchanged")


def test_aging_round_trip_decode(K):
    """The band lifecycle: int4 tokens re-quantized into the 2-bit pool and
    attended there give the oracle's banded decode of the re-quantized rows."""
    import torch
    r = W.rng(813)
    nkv, bs, g, n = 2, 16, 4, 640
    bt4, nb4 = W.paged_block_tables(r, [n], bs)
    p4 = Q4Pool(nb4, bs, nkv)
    x = W.per_unit_sigma_normal(r, (n, nkv, 128), 1, 0.2, 5.0)
    s4 = W.slots_for_positions(bt4, [0] * n, np.arange(n), bs)
    p4.append(K, x, W.normal_f32(r, x.shape), s4)
    bt2, nb2 = W.paged_block_tables(r, [n], bs)
    p2 = Q2Pool(nb2, bs, nkv)
    s2 = W.slots_for_positions(bt2, [0] * n, np.arange(n), bs)
    O2.requantize_q4_to_q2(p4.oracle_pools(), p2.oracle_pools(), s4, s2)
    K.kvq2_requantize_q4(p2.g, p4.g, dev(s4.astype(np.int32)), dev(s2.astype(np.int32)))
    torch.cuda.synchronize()
    p2.assert_same("aged")
    c8 = Q8Cache(1, bs, nkv)
    zero = np.zeros(1, np.int32)
    bands = ((p2, bt2), (p4, bt4), (c8, np.zeros((1, 1), np.int32)))
    q = W.normal_f32(r, (1, g * nkv, 128))
    got, ref = _decode_and_check(K, q, bands, (np.array([n], np.int32), zero, zero), "aged")
    assert_attn_close(got, ref, "aged 2-bit decode")


@pytest.mark.parametrize("case", range(6))
def test_banded_decode_random_shapes(K, case):
    """Seeded random shapes: batch 1-6, kv heads 1-4, GQA 1-8, block sizes
    8-128, band lengths 0-1500 each (whole sequences empty too), default or
    explicit chunk sizes."""
    r = W.rng(814, case)
    B = int(r.integers(1, 7))
    nkv = int(r.integers(1, 5))
    g = int(r.integers(1, 9))
    bs = int(2 ** r.integers(3, 8))
    lens = [np.where(r.random(B) < 0.2, 0, r.integers(1, 1500, size=B)).astype(np.int32) for _ in range(3)]
    chunk = int(r.choice([0, 256, 512, 1024]))
    bands = _banded(K, r, lens[0], lens[1], lens[2], g * nkv, nkv, bs)
    q = W.normal_f32(r, (B, g * nkv, 128), float(r.uniform(0.5, 3.0)))
    what = f"case {case}: B={B} nkv={nkv} g={g} bs={bs} chunk={chunk} lens={[l.tolist() for l in lens]}"
    got, ref = _decode_and_check(K, q, bands, tuple(lens), what, chunk=chunk)
    assert_attn_close(got, ref, what)
