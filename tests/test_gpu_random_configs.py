"""Seeded random configurations of every decode against the CPU oracle,
through the C ABI: kv-head counts 1-8 (not only powers of two), query groups
1-8, block sizes 8-256, batches of 1-5 sequences with ragged lengths
(empty ones included), the default and explicit chunk lengths, and, for the
int8 cache, the fused write-then-attend call; and every write path and
re-quantization over random pools and slot lists.  Each case draws its shape
from its own seed, so a failure names a reproducible configuration.
Outputs within 1e-4 + 1e-4 |oracle|; the pools written by the library
equal the oracle's bit for bit."""
import numpy as np
import pytest

import workloads as W
from oracle import kvq2 as O2
from oracle import kvq4 as O4
from oracle import kvq4_0 as O40
from oracle import kvq8 as O8
from tests.helpers import SM, Q8Cache, assert_attn_close, dev, fill_sequences, host
from tests.test_gpu_kvq2 import Q2Pool, _banded, _decode_and_check
from tests.test_gpu_kvq4 import Q4Pool
from tests.test_gpu_kvq4_0 import Q40Cache

pytestmark = pytest.mark.gpu

SEEDS = range(16)


@pytest.fixture(scope="module")
def K():
    import decode_attention_int8_amd as K
    return K


def _shape(seed, max_len):
    """(nkv, g, bs, lens, chunk) of one case: chunk 0 is the library's choice."""
    r = W.rng(990, seed)
    nkv = int(r.integers(1, 9))
    g = int(r.choice([1, 2, 3, 4, 5, 8]))
    bs = int(r.choice([8, 16, 32, 64, 256]))
    B = int(r.integers(1, 6))
    lens = r.integers(0, max_len + 1, size=B).astype(np.int32)
    i = int(r.integers(0, B))
    lens[i] = int(r.integers(max_len // 2, max_len + 1))     # one long sequence
    if B >= 3:
        lens[(i + 1) % B] = 0                                  # and an empty one
    chunk = int(r.choice([0, 0, 256, 512, 1024]))
    return r, nkv, g, bs, lens, chunk


@pytest.mark.parametrize("seed", SEEDS)
def test_int8_decode_and_fused_step(K, seed):
    import torch
    r, nkv, g, bs, lens, chunk = _shape(seed, 1800)
    nq, B, Lm = g * nkv, len(lens), int(lens.max())
    what = f"seed {seed}: nkv={nkv} g={g} bs={bs} lens={lens.tolist()} chunk={chunk}"
    bt, nb = W.paged_block_tables(r, lens, bs, spare_blocks=1)
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    v = W.student_t3_f32(r, (B, Lm, nkv, 128), 0.5)
    c = Q8Cache(nb, bs, nkv)
    prev = np.maximum(lens - 1, 0)
    fill_sequences(c, bt, prev, k, v)
    q = W.normal_f32(r, (B, nq, 128), 2.0)
    # fused: each non-empty sequence's token at lens - 1 is written, then attended
    kn = dev(np.stack([k[b, max(int(lens[b]) - 1, 0)] for b in range(B)]))
    vn = dev(np.stack([v[b, max(int(lens[b]) - 1, 0)] for b in range(B)]))
    out = torch.full((B, nq, 128), float("nan"), dtype=torch.float32, device="cuda")
    K.kvq8_append_decode_attn(out, dev(q), kn, vn, c.gk, c.gv, c.gks, c.gvs, dev(bt), dev(lens), Lm, SM,
                              chunk=chunk)
    torch.cuda.synchronize()
    sl = np.array([bt[b, (lens[b] - 1) // bs] * bs + (lens[b] - 1) % bs if lens[b] > 0 else -1 for b in range(B)],
                  np.int32)
    O8.quantize_append(c.kp, c.vp, c.ks, c.vs, host(kn), host(vn), sl)
    c.assert_device_matches_host()
    ref = O8.decode_attention_q8(q, c.kp, c.ks, c.vp, c.vs, bt, lens, bs, SM)
    assert_attn_close(host(out), ref, "fused " + what)
    assert np.all(host(out)[lens == 0] == 0.0), what
    # the plain decode over the same cache
    out2 = torch.full((B, nq, 128), float("nan"), dtype=torch.float32, device="cuda")
    K.kvq8_decode_attn(out2, dev(q), c.gk, c.gv, c.gks, c.gvs, dev(bt), dev(lens), Lm, SM, chunk=chunk)
    torch.cuda.synchronize()
    assert np.array_equal(host(out2), host(out)), "decode after the fused write differs: " + what


@pytest.mark.parametrize("seed", SEEDS)
def test_int4_mixed_decode(K, seed):
    import torch
    r, nkv, g, bs, lens4, chunk = _shape(seed + 100, 1500)
    lens8 = r.integers(0, 300, size=len(lens4)).astype(np.int32)
    nq = g * nkv
    what = f"seed {seed}: nkv={nkv} g={g} bs={bs} lens4={lens4.tolist()} lens8={lens8.tolist()} chunk={chunk}"
    bt4, nb4 = W.paged_block_tables(r, lens4, bs, spare_blocks=1)
    bt8, nb8 = W.paged_block_tables(r, lens8, bs, spare_blocks=1)
    p4, c8 = Q4Pool(nb4, bs, nkv), Q8Cache(nb8, bs, nkv)
    for b in range(len(lens4)):
        for L, bt, fill in ((lens4[b], bt4, lambda kk, vv, s: p4.append(K, kk, vv, s)),
                            (lens8[b], bt8, c8.append)):
            if L:
                kk = W.per_unit_sigma_normal(r, (int(L), nkv, 128), 0, 0.2, 5.0)
                fill(kk, W.normal_f32(r, kk.shape), W.slots_for_positions(bt, [b] * L, np.arange(L), bs))
    p4.assert_same()
    q = W.normal_f32(r, (len(lens4), nq, 128), 2.0)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    K.kvq4_decode_attn(out, dev(q), p4.g, dev(bt4), dev(lens4), int(lens4.max()),
                       (c8.gk, c8.gv, c8.gks, c8.gvs), dev(bt8), dev(lens8), int(max(lens8.max(), 0)), SM,
                       chunk=chunk)
    torch.cuda.synchronize()
    ref = O4.decode_attention_mixed(q, p4.oracle_pools(), bt4, lens4, (c8.kp, c8.ks, c8.vp, c8.vs), bt8, lens8,
                                    bs, SM)
    assert_attn_close(host(out), ref, what)


@pytest.mark.parametrize("seed", SEEDS)
def test_three_band_decode(K, seed):
    r, nkv, g, bs, lens2, chunk = _shape(seed + 200, 1500)
    B = len(lens2)
    lens4 = r.integers(0, 500, size=B).astype(np.int32)
    lens8 = r.integers(0, 200, size=B).astype(np.int32)
    nq = g * nkv
    what = (f"seed {seed}: nkv={nkv} g={g} bs={bs} lens={lens2.tolist()}/{lens4.tolist()}/{lens8.tolist()} "
            f"chunk={chunk}")
    bands = _banded(K, r, lens2, lens4, lens8, nq, nkv, bs)
    bands[0][0].assert_same("2-bit fill")
    q = W.normal_f32(r, (B, nq, 128), 2.0)
    got, ref = _decode_and_check(K, q, bands, (lens2, lens4, lens8), what, chunk=chunk)
    assert_attn_close(got, ref, what)


@pytest.mark.parametrize("seed", SEEDS)
def test_q40_decode(K, seed):
    import torch
    r, nkv, g, bs, lens, chunk = _shape(seed + 300, 1800)
    nq = g * nkv
    what = f"seed {seed}: nkv={nkv} g={g} bs={bs} lens={lens.tolist()} chunk={chunk}"
    bt, nb = W.paged_block_tables(r, lens, bs, spare_blocks=1)
    c = Q40Cache(nb, bs, nkv)
    for b, L in enumerate(lens):
        if L:
            kk = W.per_unit_sigma_normal(r, (int(L), nkv, 128), 0, 0.5, 2.0)
            c.append(kk, W.normal_f32(r, kk.shape), W.slots_for_positions(bt, [b] * L, np.arange(L), bs))
    c.assert_device_matches_host()
    q = W.normal_f32(r, (len(lens), nq, 128), 2.0)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    K.kvq4_0_decode_attn(out, dev(q), c.gk, c.gv, c.gks, c.gvs, dev(bt), dev(lens), int(lens.max()), SM,
                         chunk=chunk)
    torch.cuda.synchronize()
    ref = O40.decode_attention_q4_0(q, c.kp, c.ks, c.vp, c.vs, bt, lens, bs, SM)
    assert_attn_close(host(out), ref, what)


# ----------------------------------------------------------------------------
# write paths and re-quantizations: random pools, row counts and slot lists
# (a permutation of the pool's slots with some rows sent to a negative slot
# and some past the pool, both skipped); pools bit for bit against the oracle
# ----------------------------------------------------------------------------

def _write_shape(seed):
    r = W.rng(991, seed)
    nkv = int(r.integers(1, 13))
    bs = int(r.choice([8, 16, 32, 64, 256]))
    n = int(r.choice([1, 7, 64, 65, 300, 1000, 2500]))
    nb = n // bs + int(r.integers(1, 4))
    return r, nkv, bs, n, nb


def _slots(r, n, n_slots):
    sl = r.permutation(n_slots)[:n].astype(np.int32)
    k = max(n // 10, 1) if n > 1 else 0
    sl[r.choice(n, size=k, replace=False)] = -1 - r.integers(0, 5, size=k)
    if n > 2:
        sl[int(r.integers(0, n))] = n_slots + int(r.integers(0, 7))
    return sl


def _rows(r, n, nkv):
    x = W.per_unit_sigma_normal(r, (n, nkv, 128), 1, 0.2, 5.0)
    y = W.student_t3_f32(r, (n, nkv, 128), 0.5)
    return x, y


@pytest.mark.parametrize("seed", SEEDS)
def test_write_paths(K, seed):
    import torch
    r, nkv, bs, n, nb = _write_shape(seed)
    what = f"seed {seed}: nkv={nkv} bs={bs} n={n} blocks={nb}"
    c8, p4, p2, c40 = Q8Cache(nb, bs, nkv), Q4Pool(nb, bs, nkv), Q2Pool(nb, bs, nkv), Q40Cache(nb, bs, nkv)
    x, y = _rows(r, n, nkv)
    c8.append(x, y, _slots(r, n, nb * bs))
    p4.append(K, x, y, _slots(r, n, nb * bs))
    p2.append(K, x, y, _slots(r, n, nb * bs))
    c40.append(x, y, _slots(r, n, nb * bs))
    torch.cuda.synchronize()
    c8.assert_device_matches_host()
    p4.assert_same()
    p2.assert_same(what)
    c40.assert_device_matches_host()


@pytest.mark.parametrize("seed", SEEDS)
def test_requantizations(K, seed):
    import torch
    r, nkv, bs, n, nb = _write_shape(seed + 100)
    c8, p4, p2 = Q8Cache(nb, bs, nkv), Q4Pool(nb + 1, bs, nkv), Q2Pool(nb + 2, bs, nkv)
    x, y = _rows(r, nb * bs, nkv)
    c8.append(x, y, np.arange(nb * bs, dtype=np.int32))
    # int8 -> int4, then int4 -> 2-bit, over random slot pairs with skips
    src, dst = _slots(r, n, nb * bs), _slots(r, n, (nb + 1) * bs)
    O4.requantize_q8_to_q4((c8.kp, c8.ks, c8.vp, c8.vs), p4.oracle_pools(), src, dst)
    K.kvq4_requantize_q8(p4.g, (c8.gk, c8.gv, c8.gks, c8.gvs), dev(src), dev(dst))
    src2, dst2 = _slots(r, n, (nb + 1) * bs), _slots(r, n, (nb + 2) * bs)
    O2.requantize_q4_to_q2(p4.oracle_pools(), p2.oracle_pools(), src2, dst2)
    K.kvq2_requantize_q4(p2.g, p4.g, dev(src2), dev(dst2))
    torch.cuda.synchronize()
    c8.assert_device_matches_host()
    p4.assert_same()
    p2.assert_same(f"seed {seed}: nkv={nkv} bs={bs} n={n}")
