"""Pins of the Q4_0 oracle ([P2] Sec. 1 and 3: a Q4_0 payload cache about
1.65x denser than q8 whose decode dot reads the nibbles directly) against
brute force over the code grid, exact bounds, closed forms and the page's
density figure."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import kvq4_0 as Q, kvq8
from tests.exact import fr
import workloads as W

SM = float(np.float32(1.0) / np.sqrt(np.float32(128.0)))
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _blocks(seed):
    r = W.rng(400, seed)
    return np.concatenate([
        W.normal_f32(r, (6, 128)), W.normal_f32(r, (2, 128), 7.0), W.normal_f32(r, (2, 128), 1e-3),
        np.abs(W.normal_f32(r, (1, 128))), -np.abs(W.normal_f32(r, (1, 128))),
        W.student_t3_f32(r, (4, 128)), W.outlier_normal_bf16(r, (4, 128)).astype(np.float32)])


@pytest.mark.parametrize("seed", range(3))
def test_codes_are_the_nearest_grid_point(seed):
    """Brute force over all 16 codes with exact rationals: the stored code is
    a nearest grid point, the higher code on an exact tie.  Where x / step
    lies within float32 rounding of a midpoint either neighbour is allowed
    (the code is decided in float32)."""
    x = _blocks(seed)
    c, s = Q.quantize_blocks_q4_0(x)
    assert c.dtype == np.uint8 and s.dtype == np.float32 and c.max() <= 15
    for i in range(len(x)):
        for b in range(4):
            d = fr(s[i, b])
            assert d != 0
            for e in range(32):
                xv = fr(x[i, 32 * b + e])
                dist = [abs(xv - (k - 8) * d) for k in range(16)]
                best = min(dist)
                nearest = [k for k in range(16) if dist[k] == best]
                code = int(c[i, 32 * b + e])
                if code == max(nearest):
                    continue
                # float32 rounding of x / step (and of + 8.5) near a midpoint
                y = xv / d + Fraction(17, 2)
                assert abs(y - round(y)) < Fraction(1, 2 ** 18), (i, b, e, code, nearest)
                assert abs(code - max(nearest)) == 1


def test_extreme_is_exact_and_error_bounds():
    x = np.concatenate([_blocks(s) for s in range(3)])
    c, s = Q.quantize_blocks_q4_0(x)
    xr = Q.dequantize_blocks_q4_0(c, s)
    m = Q.block_extreme(x)
    for b in range(4):
        blk = x[:, 32 * b:32 * b + 32]
        # the extreme value lands on code 0 and is reproduced exactly
        j = np.argmax(np.where(blk == m[:, b:b + 1], 1, 0), axis=1)
        rows = np.arange(len(x))
        assert np.all(c[rows, 32 * b + j] == 0)
        assert np.all(xr[rows, 32 * b + j] == m[:, b].astype(np.float64))
        step = np.abs(s[:, b:b + 1]).astype(np.float64)
        err = np.abs(blk.astype(np.float64) - xr[:, 32 * b:32 * b + 32])
        ratio = blk.astype(np.float64) / s[:, b:b + 1].astype(np.float64)
        inner = ratio <= 7.5
        # half a step on the grid (float32 decides codes: tiny slack), at most
        # one step above 7.5 steps where the top code clamps
        assert np.all(err[inner] <= step.repeat(32, 1)[inner] * (0.5 + 2 ** -18))
        assert np.all(err <= step * (1 + 2 ** -18))
        assert np.all(c[:, 32 * b:32 * b + 32][~inner] == 15)


@pytest.mark.parametrize("k", [-20, -3, 1, 9])
def test_power_of_two_scaling_moves_only_the_step(k):
    x = _blocks(5)
    c1, s1 = Q.quantize_blocks_q4_0(x)
    c2, s2 = Q.quantize_blocks_q4_0((x * np.float32(2.0 ** k)).astype(np.float32))
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2, (s1 * np.float32(2.0 ** k)).astype(np.float32))


def test_zero_block_and_sign_of_step():
    x = np.zeros((1, 128), np.float32)
    x[0, 32:64] = np.float32(-0.0)
    x[0, 64:96] = np.linspace(-1, 3, 32, dtype=np.float32)      # positive extreme 3
    x[0, 96:] = np.linspace(-4, 1, 32, dtype=np.float32)        # negative extreme -4
    c, s = Q.quantize_blocks_q4_0(x)
    assert np.all(c[0, :64] == 8)
    assert s[0, 0] == 0 and not np.signbit(s[0, 0]) and s[0, 1] == 0 and not np.signbit(s[0, 1])
    assert s[0, 2] == np.float32(3.0) / np.float32(-8.0) and s[0, 3] == np.float32(0.5)
    assert c[0, 64 + 31] == 0 and c[0, 96] == 0


def test_tie_between_signs_takes_the_negative_extreme_and_half_up():
    x = np.zeros((1, 128), np.float32)
    x[0, :32] = 0.25
    x[0, 3], x[0, 17] = 8.0, -8.0          # tie: extreme -8, step +1
    x[0, 4], x[0, 5] = 0.5, -0.5           # exact midpoints: half up on x / step
    x[0, 6], x[0, 7] = 7.5, 7.4375
    c, s = Q.quantize_blocks_q4_0(x)
    assert s[0, 0] == 1.0
    assert c[0, 17] == 0 and c[0, 3] == 15                 # +8 clamps to +7
    assert c[0, 4] == 9 and c[0, 5] == 8                   # 0.5 -> 1, -0.5 -> 0
    assert c[0, 6] == 15 and c[0, 7] == 15                 # 7.5 -> 8 clamps; 7.4375 -> 7
    assert c[0, 0] == 8                                    # 0.25 -> 0
    # a positive extreme: step negative, half up on x / step means toward -inf in x
    y = np.zeros((1, 128), np.float32)
    y[0, 0], y[0, 1], y[0, 2] = 8.0, 0.5, -0.5
    c, s = Q.quantize_blocks_q4_0(y)
    assert s[0, 0] == -1.0 and c[0, 0] == 0 and c[0, 1] == 8 and c[0, 2] == 9


def test_layouts_place_single_elements_and_round_trip():
    for e in range(128):
        codes = np.zeros(128, np.uint8)
        codes[e] = 5
        pk, pv = Q.pack_k(codes), Q.pack_v(codes)
        # key: element j low nibble of byte j, element 64 + j high nibble
        jb, sh = (e, 0) if e < 64 else (e - 64, 4)
        assert np.flatnonzero(pk).tolist() == [jb] and pk[jb] == 5 << sh
        # value: byte 4m + k holds 32k + 2m (low) and 32k + 2m + 1 (high)
        k, r = divmod(e, 32)
        m, odd = divmod(r, 2)
        assert np.flatnonzero(pv).tolist() == [4 * m + k] and pv[4 * m + k] == 5 << (4 * odd)
    r = W.rng(401)
    codes = r.integers(0, 16, (7, 3, 128)).astype(np.uint8)
    assert np.array_equal(Q.unpack_k(Q.pack_k(codes)), codes)
    assert np.array_equal(Q.unpack_v(Q.pack_v(codes)), codes)


def test_density_matches_the_page():
    """[P2] Sec. 1 / Sec. 3: the q4 KV mode is about 1.65x denser than q8."""
    with open(os.path.join(GOLDEN, "p2_kv_q4_density.json")) as f:
        gold = json.load(f)
    q8 = kvq8.kv_bytes_per_token_layer(gold["nkv"], gold["hd"], "q8")
    q4 = Q.kv_bytes_per_token_head() * gold["nkv"]
    assert q4 == 1280
    assert round(q8 / q4, 2) == gold["denser_than_q8"]


def test_scores_without_dequantization():
    r = W.rng(402)
    q = W.normal_f32(r, (5, 128))
    kx = _blocks(6)
    kc, ks = Q.quantize_blocks_q4_0(kx)
    qi, qsc = kvq8.quantize_q_blocks(q)
    k_hat = Q.dequantize_blocks_q4_0(kc, ks)
    q_hat = kvq8.dequantize_q_blocks(qi, qsc)
    for h in range(len(q)):
        P, R = Q.qk_block_terms(qi[h], kc)
        # integer sums by brute force with Python integers
        for t in (0, 3, len(kc) - 1):
            for b in range(4):
                assert P[t, b] == sum(int(qi[h, 32 * b + i]) * int(kc[t, 32 * b + i]) for i in range(32))
                assert R[b] == sum(int(qi[h, 32 * b + i]) for i in range(32))
        s = Q.qk_scores_no_dequant(qi[h], qsc[h], kc, ks)
        np.testing.assert_allclose(s, k_hat @ q_hat[h], rtol=1e-12, atol=1e-12)


def _pool(x_k, x_v, bs, seed=0):
    """Contiguous cache of one sequence (len(x_k) tokens, nkv heads) through the
    oracle's write path; returns pools and a shuffled block table."""
    L, nkv, _ = x_k.shape
    nblk = (L + bs - 1) // bs + 2
    kp = np.zeros((nblk, bs, nkv, 64), np.uint8)
    vp = np.zeros_like(kp)
    ksp = np.zeros((nblk, bs, nkv, 4), np.float32)
    vsp = np.zeros_like(ksp)
    bt = W.rng(403, seed).permutation(nblk)[: (L + bs - 1) // bs].astype(np.int32)
    t = np.arange(L)
    slots = bt[t // bs] * bs + t % bs
    Q.quantize_append_q4_0(kp, vp, ksp, vsp, x_k, x_v, slots)
    return kp, vp, ksp, vsp, bt


def test_decode_closed_forms():
    r = W.rng(404)
    nkv, g, bs = 2, 3, 4
    q = W.normal_f32(r, (1, nkv * g, 128))
    # L = 1: every head of a group returns its kv-head's dequantized value row
    xk = W.normal_f32(r, (1, nkv, 128))
    xv = W.normal_f32(r, (1, nkv, 128))
    kp, vp, ksp, vsp, bt = _pool(xk, xv, bs)
    out = Q.decode_attention_q4_0(q, kp, ksp, vp, vsp, bt[None], np.array([1]), bs, SM)
    vc, vs = Q.quantize_blocks_q4_0(xv[0])
    v_hat = Q.dequantize_blocks_q4_0(vc, vs)
    for h in range(nkv * g):
        assert np.array_equal(out[0, h], v_hat[h // g])
    # equal keys, or a zero query: the plain mean of the value rows
    L = 9
    xk = np.repeat(W.normal_f32(r, (1, nkv, 128)), L, axis=0)
    xv = W.normal_f32(r, (L, nkv, 128))
    kp, vp, ksp, vsp, bt = _pool(xk, xv, bs, seed=1)
    vc, vs = Q.quantize_blocks_q4_0(xv)
    mean = Q.dequantize_blocks_q4_0(vc, vs).mean(axis=0)
    for qq in (q, np.zeros_like(q)):
        out = Q.decode_attention_q4_0(qq, kp, ksp, vp, vsp, bt[None], np.array([L]), bs, SM)
        for h in range(nkv * g):
            np.testing.assert_allclose(out[0, h], mean[h // g], rtol=1e-12, atol=1e-12)
    # two tokens: weights 1 / (1 + e^(s1 - s0)) and its complement
    xk = W.normal_f32(r, (2, nkv, 128))
    xv = W.normal_f32(r, (2, nkv, 128))
    kp, vp, ksp, vsp, bt = _pool(xk, xv, bs, seed=2)
    out = Q.decode_attention_q4_0(q, kp, ksp, vp, vsp, bt[None], np.array([2]), bs, SM)
    kc, ks = Q.quantize_blocks_q4_0(xk)
    vc, vs = Q.quantize_blocks_q4_0(xv)
    qi, qsc = kvq8.quantize_q_blocks(q[0])
    for h in range(nkv * g):
        kh = h // g
        s0, s1 = (SM * Q.qk_scores_no_dequant(qi[h], qsc[h], kc[:, kh], ks[:, kh]))
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        want = w0 * Q.dequantize_blocks_q4_0(vc[0, kh], vs[0, kh]) + \
            (1 - w0) * Q.dequantize_blocks_q4_0(vc[1, kh], vs[1, kh])
        np.testing.assert_allclose(out[0, h], want, rtol=1e-12, atol=1e-12)


def test_decode_paging_invariance_and_empty_sequence():
    r = W.rng(405)
    L, nkv, bs = 37, 2, 8
    q = W.normal_f32(r, (2, 4, 128))
    xk = W.student_t3_f32(r, (L, nkv, 128))
    xv = W.student_t3_f32(r, (L, nkv, 128))
    outs = []
    for seed in (0, 1):
        kp, vp, ksp, vsp, bt = _pool(xk, xv, bs, seed=seed)
        tables = np.stack([bt, bt])
        outs.append(Q.decode_attention_q4_0(q, kp, ksp, vp, vsp, tables, np.array([L, 0]), bs, SM))
    assert np.array_equal(outs[0], outs[1])
    assert np.all(outs[0][1] == 0)
