"""Large cache blocks (kv_bs 256 and 1024, the largest the library accepts)
through every write path and decode: a 64-token tile then lies inside one
block, and sequences end inside, at and just past block boundaries.  Also a
single sequence shorter than the length bound (the one-region merge masks
chunks that were never written).  Codes bit for bit, outputs within
1e-4 + 1e-4 |oracle|."""
import numpy as np
import pytest

import workloads as W
from oracle import kvq2 as O2
from oracle import kvq4 as O4
from oracle import kvq4_0 as O40
from oracle import kvq8 as O8
from tests.helpers import SM, Q8Cache, assert_attn_close, dev, fill_sequences, host
from tests.test_gpu_kvq2 import Q2Pool
from tests.test_gpu_kvq4 import Q4Pool
from tests.test_gpu_kvq4_0 import Q40Cache

pytestmark = pytest.mark.gpu

BLOCKS = [256, 1024]


@pytest.fixture(scope="module")
def K():
    import decode_attention_int8_amd as K
    return K


def _lens(bs):
    return np.array([1, bs - 1, bs, bs + 1, 2 * bs + 77, 0], np.int32)


@pytest.mark.parametrize("bs", BLOCKS)
def test_int8_large_blocks(K, bs):
    import torch
    r = W.rng(900, bs)
    nq, nkv = 8, 2
    lens = _lens(bs)
    B, Lm = len(lens), int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, bs, spare_blocks=1)
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    v = W.student_t3_f32(r, (B, Lm, nkv, 128), 0.5)
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, lens, k, v)
    torch.cuda.synchronize()
    c.assert_device_matches_host()
    q = W.normal_f32(r, (B, nq, 128), 2.0)
    out = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq8_decode_attn(out, dev(q), c.gk, c.gv, c.gks, c.gvs, dev(bt), dev(lens), Lm, SM)
    torch.cuda.synchronize()
    ref = O8.decode_attention_q8(q, c.kp, c.ks, c.vp, c.vs, bt, lens, bs, SM)
    assert_attn_close(host(out), ref, f"int8 bs={bs}")


@pytest.mark.parametrize("bs", BLOCKS)
def test_q40_large_blocks(K, bs):
    import torch
    r = W.rng(901, bs)
    nq, nkv = 8, 2
    lens = _lens(bs)
    B, Lm = len(lens), int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, bs, spare_blocks=1)
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    v = W.normal_f32(r, (B, Lm, nkv, 128))
    c = Q40Cache(nb, bs, nkv)
    for b in range(B):
        if lens[b]:
            sl = W.slots_for_positions(bt, [b] * lens[b], np.arange(lens[b]), bs)
            c.append(np.ascontiguousarray(k[b, :lens[b]]), np.ascontiguousarray(v[b, :lens[b]]), sl)
    torch.cuda.synchronize()
    c.assert_device_matches_host()
    q = W.normal_f32(r, (B, nq, 128), 2.0)
    out = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq4_0_decode_attn(out, dev(q), c.gk, c.gv, c.gks, c.gvs, dev(bt), dev(lens), Lm, SM)
    torch.cuda.synchronize()
    ref = O40.decode_attention_q4_0(q, c.kp, c.ks, c.vp, c.vs, bt, lens, bs, SM)
    assert_attn_close(host(out), ref, f"Q4_0 bs={bs}")


@pytest.mark.parametrize("bs", BLOCKS)
def test_group_bands_large_blocks(K, bs):
    """int4 + int8 (kvq4_decode_attn) and 2-bit + int4 + int8
    (kvq2_decode_attn) over the same large-block pools."""
    import torch
    r = W.rng(902, bs)
    nq, nkv = 8, 2
    lens2 = _lens(bs)
    lens4 = np.roll(lens2, 1)
    lens8 = np.roll(lens2, 2)
    B = len(lens2)
    bt2, nb2 = W.paged_block_tables(r, lens2, bs, spare_blocks=1)
    bt4, nb4 = W.paged_block_tables(r, lens4, bs, spare_blocks=1)
    bt8, nb8 = W.paged_block_tables(r, lens8, bs, spare_blocks=1)
    p2, p4, c8 = Q2Pool(nb2, bs, nkv), Q4Pool(nb4, bs, nkv), Q8Cache(nb8, bs, nkv)
    for b in range(B):
        for L, bt, fill in ((lens2[b], bt2, lambda x, y, s: p2.append(K, x, y, s)),
                            (lens4[b], bt4, lambda x, y, s: p4.append(K, x, y, s)),
                            (lens8[b], bt8, lambda x, y, s: c8.append(x, y, s))):
            if L:
                x = W.per_unit_sigma_normal(r, (int(L), nkv, 128), 0, 0.5, 2.0)
                fill(x, W.normal_f32(r, x.shape), W.slots_for_positions(bt, [b] * L, np.arange(L), bs))
    torch.cuda.synchronize()
    p2.assert_same("2-bit fill")
    p4.assert_same()
    c8.assert_device_matches_host()
    q = W.normal_f32(r, (B, nq, 128), 2.0)
    pool8 = (c8.gk, c8.gv, c8.gks, c8.gvs)
    m2, m4, m8 = int(lens2.max()), int(lens4.max()), int(lens8.max())
    out = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq4_decode_attn(out, dev(q), p4.g, dev(bt4), dev(lens4), m4, pool8, dev(bt8), dev(lens8), m8, SM)
    torch.cuda.synchronize()
    ref = O4.decode_attention_mixed(q, p4.oracle_pools(), bt4, lens4, (c8.kp, c8.ks, c8.vp, c8.vs), bt8, lens8,
                                    bs, SM)
    assert_attn_close(host(out), ref, f"int4 + int8 bs={bs}")
    out2 = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq2_decode_attn(out2, dev(q), p2.g, dev(bt2), dev(lens2), m2, p4.g, dev(bt4), dev(lens4), m4, pool8,
                       dev(bt8), dev(lens8), m8, SM)
    torch.cuda.synchronize()
    ref2 = O2.decode_attention_banded(q, p2.oracle_pools(), bt2, lens2, p4.oracle_pools(), bt4, lens4,
                                      (c8.kp, c8.ks, c8.vp, c8.vs), bt8, lens8, bs, SM)
    assert_attn_close(host(out2), ref2, f"three bands bs={bs}")


@pytest.mark.parametrize("L", [300, 0, -3, 5000])
def test_batch1_lengths_below_the_bound(K, L):
    """One sequence whose length is below max_ctx_len (chunks past it are
    never written and must be masked by the merge), empty, negative, and at
    the bound: int8 and Q4_0 decodes against the oracle."""
    import torch
    r = W.rng(903, L + 10)
    nq, nkv, bs, bound = 8, 2, 16, 5000
    n = max(L, 0)
    bt, nb = W.paged_block_tables(r, [bound], bs)
    k = W.normal_f32(r, (1, bound, nkv, 128))
    v = W.normal_f32(r, (1, bound, nkv, 128))
    lens = np.array([L], np.int32)
    c8 = Q8Cache(nb, bs, nkv)
    c40 = Q40Cache(nb, bs, nkv)
    if n:
        sl = W.slots_for_positions(bt, [0] * n, np.arange(n), bs)
        c8.append(np.ascontiguousarray(k[0, :n]), np.ascontiguousarray(v[0, :n]), sl)
        c40.append(np.ascontiguousarray(k[0, :n]), np.ascontiguousarray(v[0, :n]), sl)
    q = W.normal_f32(r, (1, nq, 128))
    out = torch.full((1, nq, 128), float("nan"), dtype=torch.float32, device="cuda")
    K.kvq8_decode_attn(out, dev(q), c8.gk, c8.gv, c8.gks, c8.gvs, dev(bt), dev(lens), bound, SM)
    out40 = torch.full((1, nq, 128), float("nan"), dtype=torch.float32, device="cuda")
    K.kvq4_0_decode_attn(out40, dev(q), c40.gk, c40.gv, c40.gks, c40.gvs, dev(bt), dev(lens), bound, SM)
    torch.cuda.synchronize()
    ref = O8.decode_attention_q8(q, c8.kp, c8.ks, c8.vp, c8.vs, bt, [n], bs, SM)
    ref40 = O40.decode_attention_q4_0(q, c40.kp, c40.ks, c40.vp, c40.vs, bt, [n], bs, SM)
    assert_attn_close(host(out), ref, f"int8 L={L}")
    assert_attn_close(host(out40), ref40, f"Q4_0 L={L}")
    if n == 0:
        assert np.all(host(out) == 0.0) and np.all(host(out40) == 0.0)
