"""GPU parity of the int8 path against the CPU oracle, through the C ABI.

Bit-exact: K/V codes and steps of the write path, query codes and block
scales, int32 block partials.  Float outputs: |gpu - oracle| <= 1e-4 +
1e-4 |oracle| elementwise.  Sizes span several tiles and chunks with ragged
tails; the full-size workloads are in test_gpu_workloads.py.
"""
import numpy as np
import pytest

import workloads as W
from oracle import kvq8 as O8
from tests.helpers import SM, Q8Cache, assert_attn_close, dev, fill_sequences, host, pool_columns

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


@pytest.fixture(scope="module")
def K():
    import decode_attention_int8_amd as K
    return K


# ----------------------------------------------------------------------------
# write path
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_quantize_append_bit_exact(K, dtype):
    torch = _torch()
    r = W.rng(300, ["f32", "bf16", "f16"].index(dtype))
    n, nkv, bs, nb = 777, 4, 16, 64
    x = np.concatenate([W.normal_f32(r, (n // 2, nkv, 128)),
                        W.student_t3_f32(r, (n - n // 2, nkv, 128), 0.5)]).astype(np.float32)
    y = W.outlier_normal_bf16(r, (n, nkv, 128))
    x[3, 1] = 0.0                                   # guarded zero row
    x[5, 0, :] = 2.5                                # equal row
    x[6, 2, :3] = [127.0, 0.5, -0.5]                # ties
    x[6, 2, 3:] = 0.0
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    gx, gy = dev(x).to(tdt), dev(y).to(tdt)
    xh = gx.float().cpu().numpy()                   # exact values the kernel sees
    yh = gy.float().cpu().numpy()
    slots = r.permutation(nb * bs)[:n].astype(np.int32)
    slots[10] = -1                                  # padding token: skipped
    slots[11] = nb * bs + 5                         # out of the pool: skipped
    c = Q8Cache(nb, bs, nkv)
    c.append(xh, yh, slots, gx, gy)
    torch.cuda.synchronize()
    c.assert_device_matches_host()


def test_quantize_append_overwrite_and_empty(K):
    torch = _torch()
    r = W.rng(301)
    c = Q8Cache(8, 16, 2)
    a = W.normal_f32(r, (5, 2, 128))
    c.append(a, a, np.array([0, 1, 2, 3, 4], np.int32))
    b = W.normal_f32(r, (2, 2, 128), 7.0)
    c.append(b, b, np.array([4, 2], np.int32))        # rewrite two slots
    K.kvq8_quantize_append(c.gk, c.gv, c.gks, c.gvs, dev(b[:0]), dev(b[:0]), dev(np.zeros(0, np.int32)))
    torch.cuda.synchronize()
    c.assert_device_matches_host()


# ----------------------------------------------------------------------------
# query quantization and integer partials (debug exports of the decode code)
# ----------------------------------------------------------------------------

def test_quantize_q_bit_exact(K):
    torch = _torch()
    r = W.rng(310)
    q = np.concatenate([W.normal_f32(r, (200, 128)), W.normal_f32(r, (50, 128), 300.0),
                        W.normal_f32(r, (50, 128), 1e-4)])
    q[0, 32:64] = 0.0
    q[1, :] = 0.0
    q[2, :32] = np.linspace(-1, 1, 32, dtype=np.float32)
    gq = dev(q)
    qi = torch.empty((len(q), 128), dtype=torch.int8, device="cuda")
    qs = torch.empty((len(q), 4), dtype=torch.float32, device="cuda")
    K.kvq8_quantize_q(qi, qs, gq)
    want_i, want_s = O8.quantize_q_blocks(q)
    assert np.array_equal(host(qi), want_i)
    assert np.array_equal(host(qs).view(np.uint32), want_s.view(np.uint32))


@pytest.mark.parametrize("nq,nkv,bs", [(1, 1, 16), (8, 2, 8), (12, 4, 64), (16, 2, 16)])
def test_qk_partials_bit_exact(K, nq, nkv, bs):
    torch = _torch()
    r = W.rng(320, nq, nkv, bs)
    lens = np.array([1, 70, 200, 0, 129], np.int32)
    B, Lm = len(lens), int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, bs, spare_blocks=3)
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, lens, k, k)
    q = W.normal_f32(r, (B, nq, 128))
    part = torch.full((B, nq, Lm, 4), -7, dtype=torch.int32, device="cuda")
    K.kvq8_qk_partials(part, dev(q), c.gk, dev(bt), dev(lens), Lm)
    got = host(part)
    qi, _ = O8.quantize_q_blocks(q)
    g = nq // nkv
    for b in range(B):
        for h in range(nq):
            rows = O8.gather_rows(c.kp, bt[b], lens[b], bs, h // g)
            want = O8.qk_block_partials(qi[b, h], rows)
            assert np.array_equal(got[b, h, :lens[b]], want), (b, h)
            assert np.all(got[b, h, lens[b]:] == -7)


# ----------------------------------------------------------------------------
# decode attention
# ----------------------------------------------------------------------------

def _decode(K, c, q, bt, lens, max_ctx, chunk=0):
    torch = _torch()
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    K.kvq8_decode_attn(out, dev(q), c.gk, c.gv, c.gks, c.gvs, dev(bt), dev(lens), max_ctx, SM, chunk=chunk)
    torch.cuda.synchronize()
    return host(out)


def test_unit_experiment_shape(K):
    # the pages' unit experiment: 1 head, L = 256, N(0, 1) K/V and query
    for seed in range(3):
        q, k, v = W.unit_experiment(seed)
        bt, nb = W.paged_block_tables(None, [256], 16)
        c = Q8Cache(nb, 16, 1)
        fill_sequences(c, bt, [256], k[None, :, None], v[None, :, None])
        got = _decode(K, c, q[None, None], bt, np.array([256], np.int32), 256)
        ref = O8.decode_attention_q8(q[None, None], c.kp, c.ks, c.vp, c.vs, bt, [256], 16, SM)
        assert_attn_close(got, ref, f"unit seed {seed}")


@pytest.mark.parametrize("g", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("bs", [8, 16, 128])
def test_decode_ragged_batch(K, g, bs):
    r = W.rng(330, g, bs)
    nkv = 2 if g < 8 else 1
    nq = g * nkv
    lens = np.array([1, 63, 64, 65, 300, 1025, 0, 2049], np.int32)
    B, Lm = len(lens), int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, bs, spare_blocks=2)
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    v = W.student_t3_f32(r, (B, Lm, nkv, 128), 0.5)
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, lens, k, v)
    q = W.normal_f32(r, (B, nq, 128), 2.0)
    got = _decode(K, c, q, bt, lens, Lm)
    ref = O8.decode_attention_q8(q, c.kp, c.ks, c.vp, c.vs, bt, lens, bs, SM)
    assert_attn_close(got, ref, f"g={g} bs={bs}")
    assert np.all(got[6] == 0.0)                          # empty context


@pytest.mark.parametrize("chunk", [256, 512, 2048, 16384])
def test_decode_chunk_sizes_agree(K, chunk):
    r = W.rng(331, chunk)
    nq, nkv, bs = 8, 2, 16
    lens = np.array([5000, 257, 4096], np.int32)
    B, Lm = len(lens), int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, bs)
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    v = W.normal_f32(r, (B, Lm, nkv, 128))
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, lens, k, v)
    q = W.normal_f32(r, (B, nq, 128), 3.0)
    got = _decode(K, c, q, bt, lens, Lm, chunk=chunk)
    ref = O8.decode_attention_q8(q, c.kp, c.ks, c.vp, c.vs, bt, lens, bs, SM)
    assert_attn_close(got, ref, f"chunk {chunk}")


def test_decode_many_chunks(K):
    """157 chunks of 256 tokens per sequence: the merge splits a head's chunks
    over 8 parts of two batches each."""
    r = W.rng(335)
    nq, nkv, bs = 4, 1, 16
    lens = np.array([40000, 9000], np.int32)
    B, Lm = len(lens), int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, bs)
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    v = W.student_t3_f32(r, (B, Lm, nkv, 128), 0.5)
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, lens, k, v)
    q = W.normal_f32(r, (B, nq, 128), 3.0)
    got = _decode(K, c, q, bt, lens, Lm, chunk=256)
    ref = O8.decode_attention_q8(q, c.kp, c.ks, c.vp, c.vs, bt, lens, bs, SM)
    assert_attn_close(got, ref, "157 chunks")


def test_decode_single_token_and_peaked_softmax(K):
    r = W.rng(332)
    nq, nkv, bs = 4, 1, 16
    lens = np.array([1, 500], np.int32)
    bt, nb = W.paged_block_tables(r, lens, bs)
    k = W.normal_f32(r, (2, 500, nkv, 128))
    v = W.normal_f32(r, (2, 500, nkv, 128))
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, lens, k, v)
    q = W.normal_f32(r, (2, nq, 128))
    q[1, 0] = k[1, 321, 0] * 30.0                   # one dominant token
    got = _decode(K, c, q, bt, lens, 500)
    ref = O8.decode_attention_q8(q, c.kp, c.ks, c.vp, c.vs, bt, lens, bs, SM)
    assert_attn_close(got, ref, "single / peaked")
    # L = 1: exactly the dequantized value row (weight 1)
    np.testing.assert_allclose(got[0], np.repeat(c.vp[bt[0, 0], 0, 0][None].astype(np.float64) * c.vs[bt[0, 0], 0, 0],
                                                 nq, 0), rtol=1e-6, atol=1e-7)


def test_decode_clamps_lengths_and_skips_bad_blocks(K):
    r = W.rng(333)
    nq, nkv, bs = 4, 2, 16
    lens = np.array([100, 100, 100], np.int32)
    bt, nb = W.paged_block_tables(r, lens, bs)
    k = W.normal_f32(r, (3, 100, nkv, 128))
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, lens, k, k)
    q = W.normal_f32(r, (3, nq, 128))
    glens = np.array([100, 100 + 1000, -5], np.int32)      # beyond max_ctx / negative
    bt_bad = bt.copy()
    bt_bad[0, 2] = nb + 100                               # block id outside the pool
    got = _decode(K, c, q, bt_bad, glens, 100)
    keep = np.r_[0:32, 48:100]                            # tokens of block index 2 are skipped
    ref0 = np.stack([O8.softmax_attention_f64(
        O8.dequantize_q_blocks(*O8.quantize_q_blocks(q[0, h][None]))[0],
        O8.dequantize_rows_q8(O8.gather_rows(c.kp, bt[0], 100, bs, h // 2), O8.gather_rows(c.ks, bt[0], 100, bs, h // 2))[keep],
        O8.dequantize_rows_q8(O8.gather_rows(c.vp, bt[0], 100, bs, h // 2), O8.gather_rows(c.vs, bt[0], 100, bs, h // 2))[keep],
        SM) for h in range(nq)])
    assert_attn_close(got[0], ref0, "bad block skipped")
    ref1 = O8.decode_attention_q8(q[1:2], c.kp, c.ks, c.vp, c.vs, bt[1:2], [100], bs, SM)
    assert_attn_close(got[1:2], ref1, "length clamped to max_ctx")
    assert np.all(got[2] == 0.0)


def test_decode_repeatable_and_stream_ordered(K):
    torch = _torch()
    r = W.rng(334)
    nq, nkv, bs = 8, 4, 16
    lens = np.array([3000, 1500], np.int32)
    bt, nb = W.paged_block_tables(r, lens, bs)
    k = W.normal_f32(r, (2, 3000, nkv, 128))
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, lens, k, k)
    q = W.normal_f32(r, (2, nq, 128))
    s = torch.cuda.Stream()
    outs = []
    with torch.cuda.stream(s):
        gq, gbt, gl = dev(q), dev(bt), dev(lens)
        for _ in range(3):
            o = torch.empty((2, nq, 128), dtype=torch.float32, device="cuda")
            K.kvq8_decode_attn(o, gq, c.gk, c.gv, c.gks, c.gvs, gbt, gl, 3000, SM)
            outs.append(o)
    s.synchronize()
    a = [host(o) for o in outs]
    assert np.array_equal(a[0], a[1]) and np.array_equal(a[1], a[2])


# ----------------------------------------------------------------------------
# fused write path + decode (one pass per layer step)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("g,dtype", [(2, "f32"), (4, "bf16"), (1, "f16"), (8, "f32"), (3, "bf16")])
def test_append_decode_equals_append_then_decode(K, g, dtype):
    torch = _torch()
    r = W.rng(340, g, ["f32", "bf16", "f16"].index(dtype))
    nkv, bs = 2, 16
    nq = g * nkv
    lens = np.array([1, 64, 65, 300, 0, 2049, 1000, 257], np.int32)   # new token at lens - 1
    B, Lm = len(lens), int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, bs, spare_blocks=2)
    bt[6, 62] = nb + 7                        # newest token of sequence 6 sits in an invalid block
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    v = W.student_t3_f32(r, (B, Lm, nkv, 128), 0.5)
    prev = np.maximum(lens - 1, 0)
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, prev, k, v)           # history without the newest token
    stale = W.normal_f32(r, (B, nkv, 128), 3.0)  # old contents of the newest slots
    have = lens > 0
    sl = np.array([bt[b, (lens[b] - 1) // bs] * bs + (lens[b] - 1) % bs if have[b] else -1 for b in range(B)],
                  np.int32)
    sl[6] = -1
    c.append(stale, stale, sl)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    kn = dev(np.stack([k[b, max(lens[b] - 1, 0)] for b in range(B)])).to(tdt)
    vn = dev(np.stack([v[b, max(lens[b] - 1, 0)] for b in range(B)])).to(tdt)
    q = W.normal_f32(r, (B, nq, 128), 2.0)
    # separate: write path, then decode, on a copy of the cache
    gk2, gv2, gks2, gvs2 = c.gk.clone(), c.gv.clone(), c.gks.clone(), c.gvs.clone()
    K.kvq8_quantize_append(gk2, gv2, gks2, gvs2, kn, vn, dev(sl))
    out_sep = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq8_decode_attn(out_sep, dev(q), gk2, gv2, gks2, gvs2, dev(bt), dev(lens), Lm, SM)
    # fused
    out = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq8_append_decode_attn(out, dev(q), kn, vn, c.gk, c.gv, c.gks, c.gvs, dev(bt), dev(lens), Lm, SM)
    torch.cuda.synchronize()
    assert np.array_equal(host(c.gk), host(gk2)) and np.array_equal(host(c.gv), host(gv2))
    assert np.array_equal(host(c.gks).view(np.uint32), host(gks2).view(np.uint32))
    assert np.array_equal(host(c.gvs).view(np.uint32), host(gvs2).view(np.uint32))
    assert np.array_equal(host(out), host(out_sep))
    # and against the oracle: write the new tokens there too
    O8.quantize_append(c.kp, c.vp, c.ks, c.vs, kn.float().cpu().numpy(), vn.float().cpu().numpy(), sl)
    keep = np.ones(B, bool)
    keep[6] = False              # block 62 of sequence 6 is outside the pool: its tokens are skipped
    ref = O8.decode_attention_q8(q[keep], c.kp, c.ks, c.vp, c.vs, bt[keep], lens[keep], bs, SM)
    assert_attn_close(host(out)[keep], ref, f"fused g={g} {dtype}")
    assert np.all(host(out)[4] == 0.0)


@pytest.mark.parametrize("max_ctx,lens", [
    (120, [60, 121, 500, 120]),          # max_ctx_len binds (a table row holds 128 tokens)
    (200, [60, 129, 500, 128]),          # the table row binds
])
def test_append_decode_lengths_above_the_bound(K, max_ctx, lens):
    """A sequence whose length exceeds max_ctx_len, or what its block-table
    row can hold, is attended over the clamped length and its new token is
    not written: every cached token stays as it was, and the output equals
    the oracle over the clamped context."""
    torch = _torch()
    r = W.rng(345, max_ctx)
    nkv, nq, bs, mb = 2, 4, 16, 8
    lens = np.array(lens, np.int32)
    B = len(lens)
    clamp = np.minimum(lens, min(max_ctx, mb * bs)).astype(np.int32)
    nb = B * mb + 2
    bt = r.permutation(nb)[:B * mb].reshape(B, mb).astype(np.int32)
    k = W.normal_f32(r, (B, mb * bs, nkv, 128))
    v = W.normal_f32(r, (B, mb * bs, nkv, 128))
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, np.full(B, mb * bs, np.int32), k, v)      # every slot of every row holds a token
    before = [host(t).copy() for t in (c.gk, c.gv, c.gks, c.gvs)]
    kn = W.normal_f32(r, (B, nkv, 128), 5.0)
    vn = W.normal_f32(r, (B, nkv, 128), 5.0)
    q = W.normal_f32(r, (B, nq, 128))
    out = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq8_append_decode_attn(out, dev(q), dev(kn), dev(vn), c.gk, c.gv, c.gks, c.gvs, dev(bt), dev(lens),
                              max_ctx, SM)
    torch.cuda.synchronize()
    # only the in-bound sequences' newest slots were written, exactly as the write path does
    sl = np.array([bt[b, (lens[b] - 1) // bs] * bs + (lens[b] - 1) % bs if lens[b] == clamp[b] else -1
                   for b in range(B)], np.int32)
    assert list(sl >= 0) == [True, False, False, True]
    O8.quantize_append(c.kp, c.vp, c.ks, c.vs, kn, vn, sl)
    c.assert_device_matches_host()
    flat_before = [x.reshape(nb * bs, -1) for x in before]
    flat_after = [host(t).reshape(nb * bs, -1) for t in (c.gk, c.gv, c.gks, c.gvs)]
    untouched = np.setdiff1d(np.arange(nb * bs), sl[sl >= 0])
    for x0, x1 in zip(flat_before, flat_after):
        assert np.array_equal(x0[untouched], x1[untouched])
    ref = O8.decode_attention_q8(q, c.kp, c.ks, c.vp, c.vs, bt, clamp, bs, SM)
    assert_attn_close(host(out), ref, "lengths above the bound")


def test_default_score_scale_is_one_over_sqrt_hd(K):
    """No score scale given: the library's default equals an explicit
    1 / sqrt(128) bit for bit (int8 and Q4_0 decodes)."""
    torch = _torch()
    r = W.rng(346)
    nkv, nq, bs = 2, 8, 16
    lens = np.array([300, 17, 1024], np.int32)
    B, Lm = len(lens), int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, bs)
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, lens, k, k)
    q = dev(W.normal_f32(r, (B, nq, 128), 3.0))
    outs = []
    for sm in (None, 0.0, -2.0, SM):
        o = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
        K.kvq8_decode_attn(o, q, c.gk, c.gv, c.gks, c.gvs, dev(bt), dev(lens), Lm, sm)
        outs.append(host(o))
    torch.cuda.synchronize()
    for o in outs[:3]:
        assert np.array_equal(o.view(np.uint32), outs[3].view(np.uint32))
    # Q4_0 cache from the same keys
    k4 = torch.zeros((nb, nkv, bs, 64), dtype=torch.uint8, device="cuda")     # head-major inside a block
    v4 = torch.zeros_like(k4)
    ks4 = torch.zeros((nb, nkv, bs, 4), dtype=torch.float32, device="cuda")
    vs4 = torch.zeros_like(ks4)
    for b in range(B):
        sl = W.slots_for_positions(bt, [b] * int(lens[b]), np.arange(lens[b]), bs)
        K.kvq4_0_quantize_append(k4, v4, ks4, vs4, dev(k[b, :lens[b]]), dev(k[b, :lens[b]]), dev(sl))
    o1 = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(o1)
    K.kvq4_0_decode_attn(o1, q, k4, v4, ks4, vs4, dev(bt), dev(lens), Lm)
    K.kvq4_0_decode_attn(o2, q, k4, v4, ks4, vs4, dev(bt), dev(lens), Lm, SM)
    torch.cuda.synchronize()
    assert np.array_equal(host(o1).view(np.uint32), host(o2).view(np.uint32))


@pytest.mark.parametrize("nkv,bs", [(1, 16), (2, 8), (3, 16), (4, 16), (6, 8), (8, 16), (8, 8), (12, 16), (16, 16)])
def test_int8_pool_storage_order(K, nkv, bs):
    """Where the write path puts a head's codes: head kh of slot s at column
    (kh & ~(P - 1)) | ((kh + s) & (P - 1)) of the slot's row, P the largest
    power of two dividing nkv (at most 8).  Each (token, head) row is a
    constant that names it, so its codes say where it went."""
    torch = _torch()
    nb = 3
    n = nb * bs
    x = np.zeros((n, nkv, 128), np.float32)
    for t in range(n):
        for h in range(nkv):
            x[t, h] = 1.0 + (t % 8) * 16 + h        # code 127 everywhere, the step names (t, h)
    c = Q8Cache(nb, bs, nkv)
    slots = np.arange(n, dtype=np.int32)[::-1].copy()  # token t -> slot n - 1 - t
    c.append(x, x, slots)
    torch.cuda.synchronize()
    c.assert_device_matches_host()
    raw = host(c.gk).reshape(n, nkv * 128)
    assert np.all(raw == 127)
    # steps are not rotated; the codes follow the rule (spelled out for nkv = 8 and 12)
    cols = pool_columns(n, nkv)
    if nkv == 8:
        assert cols[0].tolist() == list(range(8)) and cols[1].tolist() == [1, 2, 3, 4, 5, 6, 7, 0]
        assert cols[9].tolist() == [1, 2, 3, 4, 5, 6, 7, 0]
    if nkv == 12:
        assert cols[1].tolist() == [1, 2, 3, 0, 5, 6, 7, 4, 9, 10, 11, 8]
    if nkv in (1, 3):
        assert np.all(cols == np.arange(nkv)[None, :])
    # a row whose codes differ per head: head h holds code h + 1 in element 0
    y = np.zeros((n, nkv, 128), np.float32)
    y[:, :, 1] = 127.0
    for h in range(nkv):
        y[:, h, 0] = h + 1
    c2 = Q8Cache(nb, bs, nkv)
    c2.append(y, y, slots)
    torch.cuda.synchronize()
    raw = host(c2.gk).reshape(n, nkv, 128)
    for s in range(n):
        assert raw[s, cols[s], 0].tolist() == [h + 1 for h in range(nkv)], (s, raw[s, :, 0])
    c2.assert_device_matches_host()


@pytest.mark.parametrize("B,chunk", [(2, 256), (17, 512), (64, 256), (65, 256)])
def test_decode_batches_dense_work_order(K, B, chunk):
    """Batches of 2 .. 64 sequences number their (sequence, chunk) pairs
    densely (full chunks first, partial ones longest first); 65 takes the
    strided order.  Lengths include 0, 1, exact chunk multiples, negative
    values and values above the bound; every pair must be computed once."""
    r = W.rng(347, B, chunk)
    nkv, nq, bs = 2, 4, 16
    max_ctx = 3 * chunk + 100
    lens = r.integers(0, max_ctx + 1, size=B).astype(np.int32)
    lens[0] = 0
    lens[1] = 1
    if B > 2:
        lens[2] = chunk
        lens[-1] = -3
    if B > 5:
        lens[3] = 2 * chunk
        lens[4] = max_ctx + 500          # clamped to max_ctx
    cap = np.clip(lens, 0, max_ctx)
    bt, nb = W.paged_block_tables(r, np.maximum(lens, 0), bs, spare_blocks=1)
    Lm = int(np.maximum(lens, 0).max())
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    v = W.normal_f32(r, (B, Lm, nkv, 128))
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, np.maximum(lens, 0), k, v)
    q = W.normal_f32(r, (B, nq, 128))
    got = _decode(K, c, q, bt, lens, max_ctx, chunk=chunk)
    ref = O8.decode_attention_q8(q, c.kp, c.ks, c.vp, c.vs, bt, cap, bs, SM)
    assert_attn_close(got, ref, f"B={B} chunk={chunk}")
    assert np.all(got[cap == 0] == 0.0)
