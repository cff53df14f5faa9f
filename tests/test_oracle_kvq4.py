"""Pins of the int4 group oracle ([P4] Sec. 3.2, 3.3, 5.2) against exact
rational brute force, round-trip bounds and reductions to the int8 path or to
library attention."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import kvq4, kvq8
from tests.exact import f16, f32, fr, round_half_even
import workloads as W

SM = float(np.float32(1.0) / np.sqrt(np.float32(128.0)))


def _brute_group(vals):
    xs = [fr(v) for v in vals]
    mx, mn = max(xs), min(xs)
    s32 = Fraction(1) if mx == mn else f32(f32(mx - mn) / 15)
    s32 = max(s32, f32(Fraction(1, 10 ** 7)))
    s = f16(s32)
    z = min(15, max(0, round_half_even(f32(-mn / s)))) + 0   # integer: no signed zero
    codes = [min(15, max(0, round_half_even(f32(f32(x / s) + z)))) for x in xs]
    return codes, s, z


@pytest.mark.parametrize("seed", range(4))
def test_group_quantization_bruteforce(seed):
    r = W.rng(200, seed)
    x = np.concatenate([W.normal_f32(r, (2, 128)), W.normal_f32(r, (1, 128), 4.0),
                        W.normal_f32(r, (1, 128), 0.01), np.abs(W.normal_f32(r, (1, 128))),
                        # groups lying wholly above or below zero: the zero-point clamp binds
                        W.normal_f32(r, (1, 128), 0.1) + np.float32(3), W.normal_f32(r, (1, 128), 0.1) - np.float32(3)])
    c, s, z = kvq4.quantize_groups_q4(x)
    assert c.dtype == np.uint8 and s.dtype == np.float16 and z.dtype == np.float16
    for i in range(len(x)):
        for g in range(2):
            bc, bs, bz = _brute_group(x[i, 64 * g:64 * g + 64])
            assert fr(s[i, g]) == bs and fr(z[i, g]) == bz
            assert c[i, 64 * g:64 * g + 64].tolist() == bc


def test_codes_range_and_half_step_round_trip():
    r = W.rng(201)
    x = W.per_unit_sigma_normal(r, (400, 128), 1, 0.2, 5.0)
    c, s, z = kvq4.quantize_groups_q4(x)
    assert c.max() <= 15
    assert np.all((z >= 0) & (z <= 15)) and np.all(z == np.round(z))
    xr = kvq4.dequantize_groups_q4(c, s, z)
    step = np.repeat(s.astype(np.float64), 64, axis=-1)
    # [P4] Sec. 3.2: asymmetric rounding error stays within half a step (plus
    # the float16 rounding of the scale, which moves the grid ends slightly)
    lo = np.repeat(x.reshape(400, 2, 64).min(-1), 64, axis=-1)
    inside = np.abs(x - lo) <= 14.5 * step
    assert np.all(np.abs(x - xr)[inside] <= step[inside] * 0.5 * (1 + 1e-3) + 1e-7)
    assert np.all(np.abs(x - xr) <= step * 1.5)


def test_constant_groups_use_unit_scale():
    # [P4] Sec. 3.2: a group with max == min gets scale 1.0, so integer
    # constants in [-15, 15] come back exactly and others within half a unit
    x = np.zeros((3, 128), np.float32)
    x[0, :64], x[0, 64:] = -3.0, 0.0
    x[1, :64], x[1, 64:] = 5.0, -15.0
    x[2, :] = 0.25
    c, s, z = kvq4.quantize_groups_q4(x)
    assert np.all(s == np.float16(1.0))
    xr = kvq4.dequantize_groups_q4(c, s, z)
    np.testing.assert_array_equal(xr[:2], x[:2].astype(np.float64))
    assert np.all(xr[2] == 0.0)


def test_zero_point_zero_is_positive_zero():
    # a group whose minimum is slightly above zero has zero point 0; its
    # binary16 bits are those of +0.0 (the integer 0 has one encoding here)
    x = np.full((1, 128), 1e-9, np.float32)
    x[0, 5] = 2e-9
    x[0, 64:] = np.linspace(0.001, 1.0, 64, dtype=np.float32)
    _, _, z = kvq4.quantize_groups_q4(x)
    assert z.view(np.uint16).tolist() == [[0, 0]]


def test_pack_high_nibble_first_and_round_trip():
    assert kvq4.pack_nibbles(np.array([1, 2, 15, 0], np.uint8)).tolist() == [0x12, 0xF0]
    r = W.rng(202)
    c = r.integers(0, 16, size=(7, 128)).astype(np.uint8)
    p = kvq4.pack_nibbles(c)
    assert p.shape == (7, 64)
    assert np.array_equal(kvq4.unpack_nibbles(p), c)
    pv = kvq4.pack_v4(c)
    assert pv.shape == (7, 64) and np.array_equal(kvq4.unpack_v4(pv), c)
    # value rows: the same bytes (pairs, even element high), in another order
    assert sorted(pv[0].tolist()) == sorted(p[0].tolist())


def test_value_row_pair_placement():
    """Pair (e, e + 1), e = 64g + 4m + 2k, lands in byte 4m + 2g + k with the
    even element in the high nibble: word m holds d = 4m .. 4m + 3 of both
    groups."""
    for e in range(0, 128, 2):
        c = np.zeros(128, np.uint8)
        c[e], c[e + 1] = 9, 4
        g, m, k = e // 64, (e % 64) // 4, (e % 4) // 2
        pv = kvq4.pack_v4(c)
        assert np.flatnonzero(pv).tolist() == [4 * m + 2 * g + k] and pv[4 * m + 2 * g + k] == 0x94


def _pools(r, B, n4, n8, nkv, kv_bs, k4=None, v4=None, k8=None, v8=None):
    bt4, nb4 = W.paged_block_tables(r, [n4] * B, kv_bs)
    bt8, nb8 = W.paged_block_tables(r, [n8] * B, kv_bs)
    P4 = [np.zeros((nb4, kv_bs, nkv, 64), np.uint8), np.zeros((nb4, kv_bs, nkv, 2), np.float16),
          np.zeros((nb4, kv_bs, nkv, 2), np.float16), np.zeros((nb4, kv_bs, nkv, 64), np.uint8),
          np.zeros((nb4, kv_bs, nkv, 2), np.float16), np.zeros((nb4, kv_bs, nkv, 2), np.float16)]
    P8 = [np.zeros((nb8, kv_bs, nkv, 128), np.int8), np.zeros((nb8, kv_bs, nkv), np.float32),
          np.zeros((nb8, kv_bs, nkv, 128), np.int8), np.zeros((nb8, kv_bs, nkv), np.float32)]
    for b in range(B):
        if n4:
            sl = W.slots_for_positions(bt4, [b] * n4, np.arange(n4), kv_bs)
            kvq4.quantize_append_q4(P4[0], P4[3], P4[1], P4[2], P4[4], P4[5], k4[b], v4[b], sl)
        if n8:
            sl = W.slots_for_positions(bt8, [b] * n8, np.arange(n8), kv_bs)
            kvq8.quantize_append(P8[0], P8[2], P8[1], P8[3], k8[b], v8[b], sl)
    return (P4[0], P4[1], P4[2], P4[3], P4[4], P4[5]), bt4, (P8[0], P8[1], P8[2], P8[3]), bt8


def test_all_int8_equals_int8_path():
    r = W.rng(210)
    B, n8, nq, nkv, bs = 2, 40, 8, 2, 16
    k8 = W.normal_f32(r, (B, n8, nkv, 128))
    v8 = W.normal_f32(r, (B, n8, nkv, 128))
    q = W.normal_f32(r, (B, nq, 128))
    p4, bt4, p8, bt8 = _pools(r, B, 0, n8, nkv, bs, k8=k8, v8=v8)
    out = kvq4.decode_attention_mixed(q, p4, bt4, [0] * B, p8, bt8, [n8] * B, bs, SM)
    ref = kvq8.decode_attention_q8(q, p8[0], p8[1], p8[2], p8[3], bt8, [n8] * B, bs, SM)
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-15)


def test_grid_exact_int4_matches_library_attention():
    # values (c - z) * s with power-of-two s, integer z in [0, 15], and every
    # group touching both code 0 and code 15: the quantizer returns them
    # exactly, so the mixed decode must equal plain attention.
    r = W.rng(211)
    B, n4, n8, nq, nkv, bs = 2, 50, 20, 8, 2, 16

    def grid(shape):
        c = r.integers(0, 16, size=shape + (2, 64))
        c[..., 0], c[..., 1] = 0, 15
        z = r.integers(0, 16, size=shape + (2, 1))
        s = 2.0 ** r.integers(-6, -2, size=shape + (2, 1))
        return ((c - z) * s).reshape(shape + (128,)).astype(np.float32)
    k4, v4 = grid((B, n4, nkv)), grid((B, n4, nkv))
    k8c = r.integers(-126, 127, size=(B, n8, nkv, 128))
    k8c[..., 5] = 127
    k8 = (k8c * 2.0 ** -7).astype(np.float32)
    v8 = (np.roll(k8c, 3, axis=-1) * 2.0 ** -6).astype(np.float32)
    qc = r.integers(-126, 127, size=(B, nq, 4, 32))
    qc[..., 0] = -127
    q = (qc * 2.0 ** -5).reshape(B, nq, 128).astype(np.float32)
    p4, bt4, p8, bt8 = _pools(r, B, n4, n8, nkv, bs, k4, v4, k8, v8)
    out = kvq4.decode_attention_mixed(q, p4, bt4, [n4] * B, p8, bt8, [n8] * B, bs, SM)
    K = np.concatenate([k4, k8], 1).astype(np.float64)
    V = np.concatenate([v4, v8], 1).astype(np.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[:, :, None], torch.from_numpy(K).permute(0, 2, 1, 3),
        torch.from_numpy(V).permute(0, 2, 1, 3), scale=SM, enable_gqa=True)[:, :, 0].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-7)


def test_page_order_and_empty_context():
    # attention does not depend on token order: permuting whole pages of a
    # full sequence leaves the output unchanged; an empty context is zero
    r = W.rng(212)
    nkv, bs, n = 1, 16, 48
    k4 = W.normal_f32(r, (1, n, nkv, 128))
    v4 = W.normal_f32(r, (1, n, nkv, 128))
    p4, bt4, p8, bt8 = _pools(r, 1, n, 0, nkv, bs, k4, v4)
    q = W.normal_f32(r, (1, 2, 128))
    a = kvq4.decode_attention_mixed(q, p4, bt4, [n], p8, bt8, [0], bs, SM)
    bt4p = bt4[:, [2, 0, 1]]
    b = kvq4.decode_attention_mixed(q, p4, bt4p, [n], p8, bt8, [0], bs, SM)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    z = kvq4.decode_attention_mixed(q, p4, bt4, [0], p8, bt8, [0], bs, SM)
    assert np.all(z == 0)


# ----------------------------------------------------------------------------
# re-quantization of aging int8 tokens into the int4 pool ([P4] Sec. 3.3)
# ----------------------------------------------------------------------------

def _rq_pools(nb8, nb4, bs, nkv):
    q8 = (np.zeros((nb8, bs, nkv, 128), np.int8), np.zeros((nb8, bs, nkv), np.float32),
          np.zeros((nb8, bs, nkv, 128), np.int8), np.zeros((nb8, bs, nkv), np.float32))
    q4 = (np.zeros((nb4, bs, nkv, 64), np.uint8), np.zeros((nb4, bs, nkv, 2), np.float16),
          np.zeros((nb4, bs, nkv, 2), np.float16), np.zeros((nb4, bs, nkv, 64), np.uint8),
          np.zeros((nb4, bs, nkv, 2), np.float16), np.zeros((nb4, bs, nkv, 2), np.float16))
    return q8, q4


@pytest.mark.parametrize("j", [6, 8, 11])
def test_requantize_reproduces_an_int4_grid(j):
    """int8 values that lie on an int4 grid (step 2^-j, int4 scale 8 * 2^-j,
    codes spanning 0..15) come back as exactly that grid's codes, scale and
    zero point: closed form of the group rule, independent of the quantizer."""
    r = W.rng(210, j)
    bs, nkv, n = 16, 2, 40
    q8, q4 = _rq_pools(4, 5, bs, nkv)
    kc8, ks8, vc8, vs8 = q8
    want = {}
    for pool in (kc8, vc8):
        c = r.integers(0, 16, size=pool.shape[:3] + (2, 64))
        c[..., 0], c[..., 1] = 0, 15                  # the group spans all 16 codes
        z = r.integers(0, 16, size=pool.shape[:3] + (2,))
        pool[:] = (8 * (c - z[..., None])).reshape(pool.shape).astype(np.int8)
        want[id(pool)] = (c, z)
    ks8[:] = vs8[:] = np.float32(2.0 ** -j)
    src = r.permutation(4 * bs)[:n]
    dst = r.permutation(5 * bs)[:n]
    kvq4.requantize_q8_to_q4(q8, q4, src, dst)
    k4, k4s, k4z, v4, v4s, v4z = q4
    for pool8, (packed, sc, zp), unpack in ((kc8, (k4, k4s, k4z), kvq4.unpack_nibbles),
                                            (vc8, (v4, v4s, v4z), kvq4.unpack_v4)):
        c, z = want[id(pool8)]
        c = c.reshape((-1,) + c.shape[2:])[src]          # [n][nkv][group][64]
        z = z.reshape((-1,) + z.shape[2:])[src]          # [n][nkv][group]
        got = unpack(packed.reshape((-1,) + packed.shape[2:])[dst]).reshape(c.shape)
        assert np.array_equal(got, c)
        assert np.all(sc.reshape(-1, nkv, 2)[dst] == np.float16(8 * 2.0 ** -j))
        assert np.array_equal(zp.reshape(-1, nkv, 2)[dst].astype(np.int64), z)


def test_requantize_error_within_half_an_int4_step():
    """Every element's int4 value lies within half an int4 step of the int8
    value it came from (groups that straddle zero, so the zero point never
    clamps)."""
    r = W.rng(211)
    bs, nkv, n = 8, 4, 64
    q8, q4 = _rq_pools(16, 8, bs, nkv)
    kc8, ks8, vc8, vs8 = q8
    for pool, st in ((kc8, ks8), (vc8, vs8)):
        pool[:] = r.integers(-127, 128, size=pool.shape).astype(np.int8)
        pool[..., 0], pool[..., 64] = -100, -100
        pool[..., 1], pool[..., 65] = 100, 100
        st[:] = np.exp(r.uniform(-6, 2, size=st.shape)).astype(np.float32)
    src = r.permutation(16 * bs)[:n]
    dst = r.permutation(8 * bs)[:n]
    kvq4.requantize_q8_to_q4(q8, q4, src, dst)
    k4, k4s, k4z, v4, v4s, v4z = q4
    for (pool, st), (packed, sc, zp), unpack in (((kc8, ks8), (k4, k4s, k4z), kvq4.unpack_nibbles),
                                                 ((vc8, vs8), (v4, v4s, v4z), kvq4.unpack_v4)):
        x8 = pool.reshape(-1, nkv, 128)[src].astype(np.float64) * st.reshape(-1, nkv)[src][..., None]
        c = unpack(packed.reshape(-1, nkv, 64)[dst]).astype(np.float64)
        s = np.repeat(sc.reshape(-1, nkv, 2)[dst].astype(np.float64), 64, axis=-1)
        z = np.repeat(zp.reshape(-1, nkv, 2)[dst].astype(np.float64), 64, axis=-1)
        err = np.abs((c - z) * s - x8)
        # half a step, plus the f16 rounding of the step over up to 15 steps
        assert np.all(err <= s * (0.5 + 15 * 2.0 ** -11) + 1e-12)


def test_requantize_constant_groups_and_skipped_pairs():
    """An all-zero group takes the unit scale and zero point 0 (codes 0); pairs
    whose source or destination lies outside its pool change nothing."""
    bs, nkv = 8, 1
    q8, q4 = _rq_pools(2, 2, bs, nkv)
    kc8, ks8, vc8, vs8 = q8
    kc8[:] = 5
    kc8[:, :, :, 64:] = 0
    vc8[:] = 0
    ks8[:] = vs8[:] = np.float32(0.25)
    for a in q4:
        a.fill(0x55 if a.dtype == np.uint8 else np.float16(7.0))
    kvq4.requantize_q8_to_q4(q8, q4, [3, -1, 99, 4], [0, 1, 2, 17])
    k4, k4s, k4z, v4, v4s, v4z = q4
    flat = lambda a: a.reshape((-1,) + a.shape[2:])
    # pair (3 -> 0): K group 0 constant 1.25 -> unit scale, zero clamp(rint(-1.25)) = 0, code rint(1.25) = 1
    assert flat(k4s)[0, 0, 1] == np.float16(1.0) and flat(k4z)[0, 0, 1] == 0
    assert np.all(kvq4.unpack_nibbles(flat(k4)[0, 0])[64:] == 0)
    assert np.all(kvq4.unpack_nibbles(flat(k4)[0, 0])[:64] == 1)
    assert np.all(flat(v4s)[0] == np.float16(1.0)) and np.all(flat(v4z)[0] == 0)
    # pairs with -1, 99 (source) or 17 (destination) are skipped
    for a in q4:
        fa = flat(a)
        assert np.all(fa[1:] == (0x55 if a.dtype == np.uint8 else np.float16(7.0)))
