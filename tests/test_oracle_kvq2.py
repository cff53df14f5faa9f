"""Pins of the 2-bit band oracle ([P4] Sec. 3.2 quantizer at bits = 2,
Sec. 3.3 band schedule and re-quantization) against exact rational brute
force, closed forms on grid-exact data, round-trip bounds and reductions to
the int4 oracle or to library attention."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import kvq2, kvq4, kvq8
from tests.exact import f16, f32, fr, round_half_even
import workloads as W

SM = float(np.float32(1.0) / np.sqrt(np.float32(128.0)))


def _brute_group(vals):
    """The page's group rule with bits = 2, in exact rationals with explicit
    binary32 / binary16 rounding."""
    xs = [fr(v) for v in vals]
    mx, mn = max(xs), min(xs)
    s32 = Fraction(1) if mx == mn else f32(f32(mx - mn) / 3)
    s32 = max(s32, f32(Fraction(1, 10 ** 7)))
    s = f16(s32)
    z = min(3, max(0, round_half_even(f32(-mn / s)))) + 0
    codes = [min(3, max(0, round_half_even(f32(f32(x / s) + z)))) for x in xs]
    return codes, s, z


@pytest.mark.parametrize("seed", range(4))
def test_group_quantization_bruteforce(seed):
    r = W.rng(700, seed)
    x = np.concatenate([W.normal_f32(r, (2, 128)), W.normal_f32(r, (1, 128), 4.0),
                        W.normal_f32(r, (1, 128), 0.01), np.abs(W.normal_f32(r, (1, 128))),
                        W.normal_f32(r, (1, 128), 0.1) + np.float32(3), W.normal_f32(r, (1, 128), 0.1) - np.float32(3)])
    c, s, z = kvq2.quantize_groups_q2(x)
    assert c.dtype == np.uint8 and s.dtype == np.float16 and z.dtype == np.float16
    for i in range(len(x)):
        for g in range(2):
            bc, bs, bz = _brute_group(x[i, 64 * g:64 * g + 64])
            assert fr(s[i, g]) == bs and fr(z[i, g]) == bz
            assert c[i, 64 * g:64 * g + 64].tolist() == bc


def test_four_levels_and_half_step_round_trip():
    r = W.rng(701)
    x = W.per_unit_sigma_normal(r, (400, 128), 1, 0.2, 5.0)
    c, s, z = kvq2.quantize_groups_q2(x)
    assert c.max() <= 3 and set(np.unique(c).tolist()) == {0, 1, 2, 3}
    assert np.all((z >= 0) & (z <= 3)) and np.all(z == np.round(z))
    xr = kvq2.dequantize_groups_q2(c, s, z)
    step = np.repeat(s.astype(np.float64), 64, axis=-1)
    lo = np.repeat(x.reshape(400, 2, 64).min(-1), 64, axis=-1)
    inside = np.abs(x - lo) <= 2.5 * step
    assert np.all(np.abs(x - xr)[inside] <= step[inside] * 0.5 * (1 + 1e-3) + 1e-7)
    assert np.all(np.abs(x - xr) <= step * 1.5)
    # three steps span the group: the scale is a third of its range
    rng = np.ptp(x.reshape(400, 2, 64), axis=-1)
    np.testing.assert_allclose(s.astype(np.float64) * 3, rng, rtol=2 ** -10)


def test_grid_values_come_back_exactly():
    """Values (c - z) s with a power-of-two s, integer z in [0, 3] and both
    ends of the code range present are reproduced exactly (closed form)."""
    r = W.rng(702)
    c = r.integers(0, 4, size=(50, 2, 64))
    c[..., 0], c[..., 1] = 0, 3
    z = r.integers(0, 4, size=(50, 2, 1))
    s = 2.0 ** r.integers(-8, 3, size=(50, 2, 1))
    x = ((c - z) * s).reshape(50, 128).astype(np.float32)
    qc, qs, qz = kvq2.quantize_groups_q2(x)
    assert np.array_equal(qc.reshape(50, 2, 64), c)
    assert np.array_equal(qs.astype(np.float64), s[..., 0])
    assert np.array_equal(qz.astype(np.int64), z[..., 0])


def test_constant_groups_use_unit_scale():
    x = np.zeros((2, 128), np.float32)
    x[0, :64], x[0, 64:] = -3.0, 2.0
    x[1, :] = 0.25
    c, s, z = kvq2.quantize_groups_q2(x)
    assert np.all(s == np.float16(1.0))
    xr = kvq2.dequantize_groups_q2(c, s, z)
    # -3: zero point 3, code 0; +2: zero point 0 (clamped), code 2
    np.testing.assert_array_equal(xr[0], x[0].astype(np.float64))
    assert np.all(xr[1] == 0.0)


def test_pack_round_trip_and_sizes():
    r = W.rng(703)
    c = r.integers(0, 4, size=(9, 128)).astype(np.uint8)
    pk, pv = kvq2.pack_k2(c), kvq2.pack_v2(c)
    assert pk.shape == (9, 32) and pv.shape == (9, 32)
    assert np.array_equal(kvq2.unpack_k2(pk), c) and np.array_equal(kvq2.unpack_v2(pv), c)
    # K and V: 32 code bytes + 2 x (scale, zero) binary16 each, against 264 B
    # for int8 and 144 B for int4
    assert kvq2.kv_bytes_per_token_head() == 80


@pytest.mark.parametrize("d", [0, 1, 5, 16, 37, 63, 64, 100, 127])
def test_single_code_placement(d):
    """Key: d = 64h + 16g + 4k + j in byte 4(2g + h) + j at bit 2k.  Value:
    d = 64(s / 4) + 4m + s % 4 in byte 2m + s / 4 at bit 2 (s % 4)."""
    c = np.zeros(128, np.uint8)
    c[d] = 3
    h, g, i = d // 64, (d % 64) // 16, d % 16
    k, j = i // 4, i % 4
    pk = kvq2.pack_k2(c)
    assert np.flatnonzero(pk).tolist() == [4 * (2 * g + h) + j] and pk[4 * (2 * g + h) + j] == 3 << (2 * k)
    grp, m, rr = d // 64, (d % 64) // 4, d % 4
    pv = kvq2.pack_v2(c)
    assert np.flatnonzero(pv).tolist() == [2 * m + grp] and pv[2 * m + grp] == 3 << (2 * rr)


def test_band_lengths_follow_the_page_schedule():
    # [P4] Sec. 3.3 example edges 2048 and 16384; newest tokens keep 8 bits
    assert kvq2.band_lengths(0) == (0, 0, 0)
    assert kvq2.band_lengths(1) == (0, 0, 1)
    assert kvq2.band_lengths(2048) == (0, 0, 2048)
    assert kvq2.band_lengths(2049) == (0, 1, 2048)
    assert kvq2.band_lengths(16384) == (0, 14336, 2048)
    assert kvq2.band_lengths(16385) == (1, 14336, 2048)
    assert kvq2.band_lengths(131072) == (114688, 14336, 2048)
    for L in (7, 3000, 20000, 99999):
        assert sum(kvq2.band_lengths(L)) == L


# ----------------------------------------------------------------------------
# re-quantization int4 -> 2-bit
# ----------------------------------------------------------------------------

def _pools4(nb, bs, nkv):
    return (np.zeros((nb, bs, nkv, 64), np.uint8), np.zeros((nb, bs, nkv, 2), np.float16),
            np.zeros((nb, bs, nkv, 2), np.float16), np.zeros((nb, bs, nkv, 64), np.uint8),
            np.zeros((nb, bs, nkv, 2), np.float16), np.zeros((nb, bs, nkv, 2), np.float16))


def _pools2(nb, bs, nkv):
    return (np.zeros((nb, bs, nkv, 32), np.uint8), np.zeros((nb, bs, nkv, 2), np.float16),
            np.zeros((nb, bs, nkv, 2), np.float16), np.zeros((nb, bs, nkv, 32), np.uint8),
            np.zeros((nb, bs, nkv, 2), np.float16), np.zeros((nb, bs, nkv, 2), np.float16))


def test_requantize_reproduces_a_two_bit_grid():
    """int4 rows whose values lie on a 2-bit grid -- int4 codes 5 c2 with
    zero point 5 z2 and scale a = 2^-6, i.e. (c2 - z2) 5a -- come back as
    exactly c2, z2 and the 2-bit scale 5a (closed form of the group rule)."""
    r = W.rng(710)
    bs, nkv, n = 16, 2, 40
    a = 2.0 ** -6
    q4, q2 = _pools4(4, bs, nkv), _pools2(5, bs, nkv)
    k4, k4s, k4z, v4, v4s, v4z = q4
    want = []
    for packed, sc, zp, pack in ((k4, k4s, k4z, kvq4.pack_nibbles), (v4, v4s, v4z, kvq4.pack_v4)):
        c2 = r.integers(0, 4, size=packed.shape[:3] + (2, 64))
        c2[..., 0], c2[..., 1] = 0, 3                  # the group spans all four codes
        z2 = r.integers(0, 4, size=packed.shape[:3] + (2,))
        packed[:] = pack((5 * c2).reshape(packed.shape[:3] + (128,)).astype(np.uint8))
        sc[:] = np.float16(a)
        zp[:] = (5 * z2).astype(np.float16)
        want.append((c2, z2))
    src = r.permutation(4 * bs)[:n]
    dst = r.permutation(5 * bs)[:n]
    kvq2.requantize_q4_to_q2(q4, q2, src, dst)
    k2, k2s, k2z, v2, v2s, v2z = q2
    for (c2, z2), (packed, sc, zp), unpack in zip(want, ((k2, k2s, k2z), (v2, v2s, v2z)),
                                                  (kvq2.unpack_k2, kvq2.unpack_v2)):
        c2 = c2.reshape((-1,) + c2.shape[2:])[src]
        z2 = z2.reshape((-1,) + z2.shape[2:])[src]
        got = unpack(packed.reshape((-1,) + packed.shape[2:])[dst]).reshape(c2.shape)
        assert np.array_equal(got, c2)
        assert np.array_equal(zp.reshape(-1, nkv, 2)[dst].astype(np.int64), z2)
        assert np.all(sc.reshape(-1, nkv, 2)[dst] == np.float16(5 * a))


def test_requantize_error_within_half_a_two_bit_step():
    r = W.rng(711)
    bs, nkv, n = 8, 4, 64
    q4, q2 = _pools4(16, bs, nkv), _pools2(8, bs, nkv)
    src_rows = W.normal_f32(r, (16 * bs, nkv, 128))
    src_rows[..., 0], src_rows[..., 64] = -3.0, -3.0       # groups straddle zero: no zero clamp
    src_rows[..., 1], src_rows[..., 65] = 3.0, 3.0
    kvq4.quantize_append_q4(q4[0], q4[3], q4[1], q4[2], q4[4], q4[5], src_rows, src_rows[::-1].copy(),
                            np.arange(16 * bs))
    src = r.permutation(16 * bs)[:n]
    dst = r.permutation(8 * bs)[:n]
    kvq2.requantize_q4_to_q2(q4, q2, src, dst)
    k4, k4s, k4z, v4, v4s, v4z = q4
    for (p4, s4, z4, unp4), (p2, s2, z2, unp2) in (((k4, k4s, k4z, kvq4.unpack_nibbles), (q2[0], q2[1], q2[2], kvq2.unpack_k2)),
                                                   ((v4, v4s, v4z, kvq4.unpack_v4), (q2[3], q2[4], q2[5], kvq2.unpack_v2))):
        x4 = kvq4.dequantize_groups_q4(unp4(p4.reshape(-1, nkv, 64)[src]), s4.reshape(-1, nkv, 2)[src],
                                       z4.reshape(-1, nkv, 2)[src])
        x2 = kvq2.dequantize_groups_q2(unp2(p2.reshape(-1, nkv, 32)[dst]), s2.reshape(-1, nkv, 2)[dst],
                                       z2.reshape(-1, nkv, 2)[dst])
        s = np.repeat(s2.reshape(-1, nkv, 2)[dst].astype(np.float64), 64, axis=-1)
        assert np.all(np.abs(x2 - x4) <= s * (0.5 + 3 * 2.0 ** -11) + 1e-12)


def test_requantize_skips_pairs_outside_the_pools():
    q4, q2 = _pools4(2, 8, 1), _pools2(2, 8, 1)
    for a in q2:
        a.fill(0x55 if a.dtype == np.uint8 else np.float16(7.0))
    kvq2.requantize_q4_to_q2(q4, q2, [-1, 99, 3], [0, 1, 16])
    for a in q2:
        assert np.all(a == (0x55 if a.dtype == np.uint8 else np.float16(7.0)))


# ----------------------------------------------------------------------------
# decode over the three bands
# ----------------------------------------------------------------------------

def _fill(r, B, n2, n4, n8, nkv, bs, x2=None, x4=None, x8=None):
    bt2, nb2 = W.paged_block_tables(r, [n2] * B, bs)
    bt4, nb4 = W.paged_block_tables(r, [n4] * B, bs)
    bt8, nb8 = W.paged_block_tables(r, [n8] * B, bs)
    P2, P4 = _pools2(nb2, bs, nkv), _pools4(nb4, bs, nkv)
    P8 = (np.zeros((nb8, bs, nkv, 128), np.int8), np.zeros((nb8, bs, nkv), np.float32),
          np.zeros((nb8, bs, nkv, 128), np.int8), np.zeros((nb8, bs, nkv), np.float32))
    for b in range(B):
        if n2:
            sl = W.slots_for_positions(bt2, [b] * n2, np.arange(n2), bs)
            kvq2.quantize_append_q2(P2[0], P2[3], P2[1], P2[2], P2[4], P2[5], x2[0][b], x2[1][b], sl)
        if n4:
            sl = W.slots_for_positions(bt4, [b] * n4, np.arange(n4), bs)
            kvq4.quantize_append_q4(P4[0], P4[3], P4[1], P4[2], P4[4], P4[5], x4[0][b], x4[1][b], sl)
        if n8:
            sl = W.slots_for_positions(bt8, [b] * n8, np.arange(n8), bs)
            kvq8.quantize_append(P8[0], P8[2], P8[1], P8[3], x8[0][b], x8[1][b], sl)
    return P2, bt2, P4, bt4, P8, bt8


def test_no_two_bit_tokens_equals_int4_mixed_decode():
    r = W.rng(720)
    B, n4, n8, nq, nkv, bs = 2, 30, 20, 8, 2, 16
    x4 = (W.normal_f32(r, (B, n4, nkv, 128)), W.normal_f32(r, (B, n4, nkv, 128)))
    x8 = (W.normal_f32(r, (B, n8, nkv, 128)), W.normal_f32(r, (B, n8, nkv, 128)))
    P2, bt2, P4, bt4, P8, bt8 = _fill(r, B, 0, n4, n8, nkv, bs, x4=x4, x8=x8)
    q = W.normal_f32(r, (B, nq, 128))
    out = kvq2.decode_attention_banded(q, P2, bt2, [0] * B, P4, bt4, [n4] * B, P8, bt8, [n8] * B, bs, SM)
    ref = kvq4.decode_attention_mixed(q, P4, bt4, [n4] * B, (P8[0], P8[1], P8[2], P8[3]), bt8, [n8] * B, bs, SM)
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-15)


def test_grid_exact_bands_match_library_attention():
    """2-bit and int4 values on their grids and int8 values on the int8 grid
    are reproduced exactly by their quantizers, so the banded decode equals
    plain attention over the concatenated values (library SDPA, float64)."""
    r = W.rng(721)
    B, n2, n4, n8, nq, nkv, bs = 2, 40, 30, 20, 8, 2, 16

    def grid(shape, top):
        c = r.integers(0, top + 1, size=shape + (2, 64))
        c[..., 0], c[..., 1] = 0, top
        z = r.integers(0, top + 1, size=shape + (2, 1))
        s = 2.0 ** r.integers(-5, -1, size=shape + (2, 1))
        return ((c - z) * s).reshape(shape + (128,)).astype(np.float32)
    x2 = (grid((B, n2, nkv), 3), grid((B, n2, nkv), 3))
    x4 = (grid((B, n4, nkv), 15), grid((B, n4, nkv), 15))
    k8c = r.integers(-126, 127, size=(B, n8, nkv, 128))
    k8c[..., 5] = 127
    x8 = ((k8c * 2.0 ** -7).astype(np.float32), (np.roll(k8c, 3, axis=-1) * 2.0 ** -6).astype(np.float32))
    qc = r.integers(-126, 127, size=(B, nq, 4, 32))
    qc[..., 0] = -127
    q = (qc * 2.0 ** -5).reshape(B, nq, 128).astype(np.float32)
    P2, bt2, P4, bt4, P8, bt8 = _fill(r, B, n2, n4, n8, nkv, bs, x2, x4, x8)
    out = kvq2.decode_attention_banded(q, P2, bt2, [n2] * B, P4, bt4, [n4] * B, P8, bt8, [n8] * B, bs, SM)
    K = np.concatenate([x2[0], x4[0], x8[0]], 1).astype(np.float64)
    V = np.concatenate([x2[1], x4[1], x8[1]], 1).astype(np.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[:, :, None], torch.from_numpy(K).permute(0, 2, 1, 3),
        torch.from_numpy(V).permute(0, 2, 1, 3), scale=SM, enable_gqa=True)[:, :, 0].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-7)


def test_page_order_and_empty_contexts():
    r = W.rng(722)
    nkv, bs, n = 1, 16, 48
    x2 = (W.normal_f32(r, (1, n, nkv, 128)), W.normal_f32(r, (1, n, nkv, 128)))
    P2, bt2, P4, bt4, P8, bt8 = _fill(r, 1, n, 0, 0, nkv, bs, x2=x2)
    q = W.normal_f32(r, (1, 2, 128))
    a = kvq2.decode_attention_banded(q, P2, bt2, [n], P4, bt4, [0], P8, bt8, [0], bs, SM)
    b = kvq2.decode_attention_banded(q, P2, bt2[:, [2, 0, 1]], [n], P4, bt4, [0], P8, bt8, [0], bs, SM)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    z = kvq2.decode_attention_banded(q, P2, bt2, [0], P4, bt4, [0], P8, bt8, [0], bs, SM)
    assert np.all(z == 0)
