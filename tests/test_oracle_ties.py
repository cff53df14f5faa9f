"""Exact-tie pins of the oracle's rounding rules.

Every quantizer rounds a quotient to an integer, and the rules differ only
where the quotient is exactly a half-integer:

  * query blocks ([P3] "Day 9-2" Sec. 2 seg. 1, read as the Q8_0 rule):
    round half away from zero, like C roundf;
  * K/V rows ([P1] "Day 9-3" Sec. 2): round half away from zero;
  * int4 and 2-bit groups ([P4] "UltraQuant" Sec. 3.2, written with
    torch.round): round half to even, for the zero point and for the codes.

The inputs below are chosen so that the quotients land exactly on
half-integers (the multipliers and scales are powers of two, so every
product and quotient is exact in float32), and the expected codes are
written out by hand from the rule, not computed by it.  A slip from one rule
to the other changes at least one listed code.

The write path's slot rule (a slot outside the pool writes nothing) is pinned
at the end, against the row quantizer.
"""
from fractions import Fraction

import numpy as np

from oracle import kvq2, kvq4, kvq8
from tests.exact import f32

F32 = np.float32


def _row(blocks):
    """A 128-value row from four 32-value blocks given as leading values
    (the rest of each block is zero)."""
    row = np.zeros(128, F32)
    for b, vals in enumerate(blocks):
        row[32 * b:32 * b + len(vals)] = np.asarray(vals, F32)
    return row


# ----------------------------------------------------------------------------
# query blocks: ties away from zero
# ----------------------------------------------------------------------------

def test_query_block_ties_round_away_from_zero():
    # block 0: max |q| = 127, so 127 / qm = 1 exactly and the code is roundf(q)
    # block 1: max |q| = 254, multiplier 0.5 exactly
    # block 2: max |q| = 63.5, multiplier 2 exactly
    # block 3: the extreme is negative (-127), multiplier 1
    q = _row([
        [127.0, 2.5, -2.5, 0.5, -0.5, 4.5, -4.5, 126.5, -126.5, 1.5, -1.5, 0.0, 6.5, -6.5],
        [254.0, 5.0, -5.0, 1.0, -1.0, 9.0, -9.0, 253.0, -253.0, 3.0, -3.0],
        [63.5, 1.25, -1.25, 0.25, -0.25, 2.25, -2.25, 63.25, -63.25, 0.75, -0.75],
        [-127.0, 3.5, 5.5, 6.5, -8.5, 10.5, -0.5, 0.5],
    ])
    qi, qsc = kvq8.quantize_q_blocks(q[None])
    want = [
        [127, 3, -3, 1, -1, 5, -5, 127, -127, 2, -2, 0, 7, -7],
        [127, 3, -3, 1, -1, 5, -5, 127, -127, 2, -2],
        [127, 3, -3, 1, -1, 5, -5, 127, -127, 2, -2],
        [-127, 4, 6, 7, -9, 11, -1, 1],
    ]
    for b, w in enumerate(want):
        got = qi[0, 32 * b:32 * b + 32].tolist()
        assert got[:len(w)] == w, (b, got[:len(w)])
        assert got[len(w):] == [0] * (32 - len(w))
    # block scale: qm * (1/127) with both factors float32
    inv127 = f32(Fraction(1, 127))
    for b, qm in enumerate([127, 254, Fraction(127, 2), 127]):
        assert Fraction(float(qsc[0, b])) == f32(qm * inv127)


def test_query_ties_through_the_integer_dots():
    """The tie codes feed the block dot products unchanged: against a key row
    with a single code of 1 at element i, dot_b is the query's code i."""
    q = _row([[127.0, 2.5, -2.5], [254.0, 1.0], [63.5, -0.25], [-127.0, 6.5]])
    qi, _ = kvq8.quantize_q_blocks(q[None])
    expect = {1: 3, 2: -3, 33: 1, 65: -1, 97: 7}
    for i, code in expect.items():
        k = np.zeros((1, 128), np.int8)
        k[0, i] = 1
        dots = kvq8.qk_block_partials(qi[0], k)[0]
        assert dots.tolist() == [code if b == i // 32 else 0 for b in range(4)]


# ----------------------------------------------------------------------------
# K/V rows: ties away from zero
# ----------------------------------------------------------------------------

def test_kv_row_ties_round_away_from_zero():
    # amax = 127 * 2^-3, so the step is 2^-3 exactly and x / step = 8 x
    step = 0.125
    x = np.zeros(128, F32)
    vals = [127.0, 0.5, -0.5, 2.5, -2.5, 125.5, -125.5, 7.5, 1.5]
    x[:len(vals)] = np.asarray(vals, F32) * F32(step)
    c, d = kvq8.quantize_rows_q8(x[None])
    assert float(d[0]) == step
    assert c[0, :len(vals)].tolist() == [127, 1, -1, 3, -3, 126, -126, 8, 2]


# ----------------------------------------------------------------------------
# int4 groups: ties to even (zero point and codes)
# ----------------------------------------------------------------------------

def test_int4_group_code_ties_round_half_to_even():
    # group 0: min 0, max 15 / 8, so scale = 1/8 exactly and zero = 0;
    # x = (k + 1/2) / 8 gives x / s = k + 1/2
    s0 = F32(0.125)
    half = (np.arange(14, dtype=F32) + F32(0.5)) * s0
    g0 = np.concatenate([[F32(0.0), F32(15.0) * s0], half, np.zeros(64 - 16, F32)])
    # group 1: min = -2.5 s, max = 12.5 s with s = 1/4: the zero point -min / s
    # is 2.5 and rounds to 2; then x / s + 2 for the listed x
    s1 = F32(0.25)
    g1_vals = np.asarray([-2.5, 12.5, 0.5, 1.5, 0.0, 2.5, -1.5, -0.5, 10.5, 11.5], F32) * s1
    g1 = np.concatenate([g1_vals, np.zeros(64 - len(g1_vals), F32)])
    c, s, z = kvq4.quantize_groups_q4(np.concatenate([g0, g1])[None])
    assert float(s[0, 0]) == 0.125 and float(z[0, 0]) == 0.0
    assert float(s[0, 1]) == 0.25 and float(z[0, 1]) == 2.0
    assert c[0, :16].tolist() == [0, 15, 0, 2, 2, 4, 4, 6, 6, 8, 8, 10, 10, 12, 12, 14]
    # -0.5 -> 0 (clamped -0), 14.5 -> 14, 2.5 -> 2, 3.5 -> 4, 2, 4.5 -> 4,
    # 0.5 -> 0, 1.5 -> 2, 12.5 -> 12, 13.5 -> 14
    assert c[0, 64:64 + len(g1_vals)].tolist() == [0, 14, 2, 4, 2, 4, 0, 2, 12, 14]
    assert set(c[0, 64 + len(g1_vals):].tolist()) == {2}     # x = 0 -> code = zero


def test_int4_requantized_ties_follow_the_group_rule():
    """Aging an int8 token into the int4 pool: values code * step that land on
    int4 half-steps take the same tie rule (the values are exact in
    float32), in the key and the value layout."""
    bs, nkv = 8, 1
    codes8 = np.zeros(128, np.int8)
    # step 2^-5; group 0: min 0, max 60 / 32 = 15 / 8, so s = 1/8, zero 0,
    # and 2 / 32, 6 / 32 are 0.5 s and 1.5 s
    codes8[:4] = [0, 60, 2, 6]
    # group 1: min -10 / 32 = -2.5 s, max 50 / 32 = 12.5 s: zero 2.5 -> 2;
    # 2 / 32 and 10 / 32 are 0.5 s and 2.5 s
    codes8[64:68] = [-10, 50, 2, 10]
    kc8 = np.zeros((1, bs, nkv, 128), np.int8)
    kc8[0, 3, 0] = codes8
    vc8 = kc8.copy()
    st8 = np.full((1, bs, nkv), 0.03125, F32)
    k4 = np.zeros((1, bs, nkv, 64), np.uint8)
    v4 = np.zeros_like(k4)
    k4s, k4z, v4s, v4z = (np.zeros((1, bs, nkv, 2), np.float16) for _ in range(4))
    kvq4.requantize_q8_to_q4((kc8, st8, vc8, st8.copy()), (k4, k4s, k4z, v4, v4s, v4z),
                             np.array([3], np.int32), np.array([5], np.int32))
    for codes, sc, zp in ((kvq4.unpack_nibbles(k4[0, 5, 0]), k4s, k4z),
                          (kvq4.unpack_v4(v4[0, 5, 0]), v4s, v4z)):
        assert sc[0, 5, 0].tolist() == [0.125, 0.125] and zp[0, 5, 0].tolist() == [0.0, 2.0]
        assert codes[:4].tolist() == [0, 15, 0, 2]
        # -2.5 + 2 = -0.5 -> 0; 14.5 -> 14; 2.5 -> 2; 4.5 -> 4
        assert codes[64:68].tolist() == [0, 14, 2, 4]


# ----------------------------------------------------------------------------
# 2-bit groups: ties to even (zero point and codes)
# ----------------------------------------------------------------------------

def test_int2_group_ties_round_half_to_even():
    # group 0: min 0, max 3 s with s = 1/4: zero 0; x / s = 0.5, 1.5, 2.5
    s = F32(0.25)
    g0 = np.concatenate([np.asarray([0.0, 3.0, 0.5, 1.5, 2.5, 1.0], F32) * s, np.zeros(58, F32)])
    # group 1: min = -2.5 s, max = 0.5 s: -min / s = 2.5 -> zero 2;
    # x / s + 2 = -0.5, 2.5, 0.5, 1.5, 2 for the listed x
    g1_vals = np.asarray([-2.5, 0.5, -1.5, -0.5, 0.0], F32) * s
    g1 = np.concatenate([g1_vals, np.zeros(64 - len(g1_vals), F32)])
    c, sc, z = kvq2.quantize_groups_q2(np.concatenate([g0, g1])[None])
    assert float(sc[0, 0]) == 0.25 and float(z[0, 0]) == 0.0
    assert float(sc[0, 1]) == 0.25 and float(z[0, 1]) == 2.0
    assert c[0, :6].tolist() == [0, 3, 0, 2, 2, 1]
    assert c[0, 64:69].tolist() == [0, 2, 0, 2, 2]


def test_int2_zero_point_tie_at_one_half():
    # min = -0.5 s, max = 2.5 s: -min / s = 0.5 rounds to the even 0, so the
    # codes are round(x / s): -0.5 -> 0, 2.5 -> 2, 1.5 -> 2, 0.5 -> 0
    s = F32(0.5)
    g = np.asarray([-0.5, 2.5, 1.5, 0.5, 2.0], F32) * s
    row = np.concatenate([g, np.zeros(64 - len(g), F32), np.zeros(64, F32)])
    c, sc, z = kvq2.quantize_groups_q2(row[None])
    assert float(sc[0, 0]) == 0.5 and float(z[0, 0]) == 0.0
    assert c[0, :5].tolist() == [0, 2, 2, 0, 2]


# ----------------------------------------------------------------------------
# the write path's slot rule
# ----------------------------------------------------------------------------

def test_quantize_append_skips_slots_outside_the_pool():
    """Negative slots (padding) and slots at or past n_blocks * kv_bs leave
    the pools untouched; every other token's codes and step equal the row
    quantizer's, at its slot."""
    rng = np.random.default_rng(42)
    nb, bs, nkv = 3, 8, 2
    kp = np.full((nb, bs, nkv, 128), 99, np.int8)
    vp = np.full((nb, bs, nkv, 128), -99, np.int8)
    ks = np.full((nb, bs, nkv), 7.0, F32)
    vs = np.full((nb, bs, nkv), -7.0, F32)
    n = 7
    kn = rng.standard_normal((n, nkv, 128)).astype(F32)
    vn = rng.standard_normal((n, nkv, 128)).astype(F32)
    slots = np.array([5, -1, nb * bs, 23, -7, 0, nb * bs + 40], np.int32)
    kvq8.quantize_append(kp, vp, ks, vs, kn, vn, slots)
    kc, kd = kvq8.quantize_rows_q8(kn)
    vc, vd = kvq8.quantize_rows_q8(vn)
    written = {5: 0, 23: 3, 0: 5}
    for slot in range(nb * bs):
        blk, off = divmod(slot, bs)
        if slot in written:
            i = written[slot]
            assert np.array_equal(kp[blk, off], kc[i]) and np.array_equal(vp[blk, off], vc[i])
            assert np.array_equal(ks[blk, off], kd[i]) and np.array_equal(vs[blk, off], vd[i])
        else:
            assert np.all(kp[blk, off] == 99) and np.all(vp[blk, off] == -99)
            assert np.all(ks[blk, off] == 7.0) and np.all(vs[blk, off] == -7.0)
