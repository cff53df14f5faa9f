"""Pins of the int8 oracle against facts fixed by the pages and by mathematics.

Each test names the passage or the mathematical fact it relies on.  None of
them re-types the oracle's own formula: they use exact rational brute force,
closed forms, invariants, a library attention routine on inputs where
quantization is exact, and the figures printed on the pages.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import kvq8
from tests.exact import f32, fr, round_half_away
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SM = float(np.float32(1.0) / np.sqrt(np.float32(128.0)))


# ----------------------------------------------------------------------------
# K/V row quantization ([P1] Sec. 2; [P2] Sec. 2)
# ----------------------------------------------------------------------------

def _brute_row_q8(row):
    """Exact-rational evaluation of: amax -> d = fl32(amax/127) ->
    code = roundf(fl32(x/d)) clamped to +-127."""
    xs = [fr(v) for v in row]
    amax = max(abs(v) for v in xs)
    if amax < fr(np.float32(1e-6)):
        amax = Fraction1
    d = f32(amax / 127)
    codes = [max(-127, min(127, round_half_away(f32(v / d)))) for v in xs]
    return codes, d


from fractions import Fraction  # noqa: E402
Fraction1 = Fraction(1)


@pytest.mark.parametrize("seed", range(6))
def test_quantize_rows_bruteforce(seed):
    r = W.rng(100, seed)
    rows = np.concatenate([W.normal_f32(r, (3, 128)), W.student_t3_f32(r, (3, 128), 0.5),
                           W.normal_f32(r, (2, 128), 1e-3)])
    codes, d = kvq8.quantize_rows_q8(rows)
    for i, row in enumerate(rows):
        bc, bd = _brute_row_q8(row)
        assert fr(d[i]) == bd
        assert codes[i].tolist() == bc


def test_argmax_gets_full_code_and_half_step_bound():
    r = W.rng(101)
    x = np.concatenate([W.normal_f32(r, (500, 128)), W.student_t3_f32(r, (500, 128), 0.5)])
    c, d = kvq8.quantize_rows_q8(x)
    i = np.abs(x).argmax(-1)
    top = c[np.arange(len(x)), i].astype(int)
    assert np.all(np.abs(top) == 127)
    assert np.all(np.sign(top) == np.sign(x[np.arange(len(x)), i]))
    err = np.abs(x.astype(np.float64) - c.astype(np.float64) * d[:, None].astype(np.float64))
    # [P1] Sec. 3: every dequantized value is within half a step
    assert np.all(err <= d[:, None].astype(np.float64) * 0.5 * (1 + 2.0 ** -20))
    assert c.min() >= -127


def test_ties_round_away_from_zero():
    # amax = 127 gives step exactly 1, so x / d = x and the halves are exact ties
    row = np.zeros(128, np.float32)
    row[:9] = [127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5, -126.5]
    c, d = kvq8.quantize_rows_q8(row[None])
    assert d[0] == np.float32(1.0)
    assert c[0, :9].tolist() == [127, 3, -3, 1, -1, 2, -2, 127, -127]


def test_zero_row_equal_row_single_nonzero():
    x = np.zeros((4, 128), np.float32)
    x[1, :] = -0.75
    x[2, 17] = 3.0
    x[3, :] = 1e-9          # below the guard: treated like the zero row
    c, d = kvq8.quantize_rows_q8(x)
    assert np.all(c[0] == 0) and d[0] == np.float32(1) / np.float32(127)
    assert np.all(c[1] == -127) and d[1] == np.float32(0.75) / np.float32(127)
    assert c[2, 17] == 127 and np.count_nonzero(c[2]) == 1 and d[2] == np.float32(3.0) / np.float32(127)
    assert np.all(c[3] == 0) and d[3] == d[0]


@pytest.mark.parametrize("k", [-3, 1, 5])
def test_power_of_two_amplitude_is_exact(k):
    # [P1] Sec. 4 task A: per-row scaling absorbs the amplitude.  For 2**k the
    # float arithmetic is exact, so codes are identical and steps scale exactly.
    r = W.rng(102, k + 10)
    x = W.normal_f32(r, (64, 128))
    c1, d1 = kvq8.quantize_rows_q8(x)
    c2, d2 = kvq8.quantize_rows_q8(x * np.float32(2.0 ** k))
    assert np.array_equal(c1, c2)
    assert np.array_equal(d2, d1 * np.float32(2.0 ** k))


def test_amplitude_x3():
    # [P1] Sec. 4 task A with the page's factor 3: codes move only where the
    # quotient sits within rounding of a half-integer; steps scale by 3.
    r = W.rng(103)
    x = W.normal_f32(r, (2000, 128))
    c1, d1 = kvq8.quantize_rows_q8(x)
    c3, d3 = kvq8.quantize_rows_q8((x * np.float32(3)).astype(np.float32))
    assert np.mean(c1 != c3) < 1e-4
    ratio = d3.astype(np.float64) / d1.astype(np.float64)
    assert np.all(np.abs(ratio - 3.0) <= 3.0 * 2.0 ** -22)


def test_byte_accounting_matches_page():
    g = json.load(open(os.path.join(GOLDEN, "p2_byte_accounting.json")))
    nkv, hd = g["nkv"], g["hd"]
    r = W.rng(104)
    k_tok = W.normal_f32(r, (nkv, hd))
    v_tok = W.normal_f32(r, (nkv, hd))
    kc, kd = kvq8.quantize_rows_q8(k_tok)
    vc, vd = kvq8.quantize_rows_q8(v_tok)
    assert kc.nbytes + vc.nbytes == g["q8_code_bytes_per_token_layer"]
    assert kd.nbytes + vd.nbytes == g["q8_scale_bytes_per_token_layer"]
    total = kc.nbytes + vc.nbytes + kd.nbytes + vd.nbytes
    assert total == g["q8_bytes_per_token_layer"] == kvq8.kv_bytes_per_token_layer(nkv, hd, "q8")
    assert kvq8.kv_bytes_per_token_layer(nkv, hd, "f16") == g["f16_bytes_per_token_layer"]
    assert round(total / g["f16_bytes_per_token_layer"], 2) == g["ratio"]


# ----------------------------------------------------------------------------
# query quantization ([P3] Sec. 2 seg. 1)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_quantize_q_bruteforce(seed):
    r = W.rng(110, seed)
    q = np.concatenate([W.normal_f32(r, (3, 128)), W.normal_f32(r, (1, 128), 40.0)])
    q[0, 32:64] = 0.0                     # a guarded block
    qi, qsc = kvq8.quantize_q_blocks(q)
    inv127 = f32(Fraction(1, 127))
    for i in range(len(q)):
        for b in range(4):
            blk = [fr(v) for v in q[i, 32 * b:32 * b + 32]]
            qm = max(abs(v) for v in blk)
            if qm < fr(np.float32(1e-6)):
                qm = Fraction1
            assert fr(qsc[i, b]) == f32(qm * inv127)
            iq = f32(127 / qm)
            want = [max(-128, min(127, round_half_away(f32(v * iq)))) for v in blk]
            assert qi[i, 32 * b:32 * b + 32].tolist() == want


def test_q_blocks_are_independent():
    r = W.rng(111)
    q = W.normal_f32(r, (1, 128))
    qi1, s1 = kvq8.quantize_q_blocks(q)
    q2 = q.copy()
    q2[0, 64:96] *= 100
    qi2, s2 = kvq8.quantize_q_blocks(q2)
    keep = np.r_[0:64, 96:128]
    assert np.array_equal(qi1[0, keep], qi2[0, keep])
    assert np.array_equal(s1[0, [0, 1, 3]], s2[0, [0, 1, 3]])
    for b in range(4):
        assert np.abs(qi2[0, 32 * b:32 * b + 32]).max() == 127


# ----------------------------------------------------------------------------
# integer block partials ([P3] Sec. 2 seg. 2)
# ----------------------------------------------------------------------------

def test_partials_bruteforce_and_bound():
    r = W.rng(120)
    qi = r.integers(-128, 128, size=(3, 128)).astype(np.int8)
    kq = r.integers(-127, 128, size=(5, 128)).astype(np.int8)
    p = kvq8.qk_block_partials(qi, kq)
    assert p.shape == (3, 5, 4)
    for h in range(3):
        for t in range(5):
            for b in range(4):
                s = sum(int(qi[h, i]) * int(kq[t, i]) for i in range(32 * b, 32 * b + 32))
                assert p[h, t, b] == s
    ext = kvq8.qk_block_partials(np.full((1, 128), -128, np.int8), np.full((1, 128), -127, np.int8))
    assert np.all(ext == 32 * 128 * 127)


# ----------------------------------------------------------------------------
# decode attention: closed forms, invariants, library routine
# ----------------------------------------------------------------------------

def _contiguous_cache(k_codes, k_step, v_codes, v_step, kv_bs=16, r=None):
    """Put [B][L][nkv][128] rows into a paged pool with (optionally shuffled)
    block tables."""
    B, L, nkv, _ = k_codes.shape
    bt, nb = W.paged_block_tables(r, [L] * B, kv_bs)
    pools = [np.zeros((nb, kv_bs, nkv, 128), np.int8) for _ in range(2)]
    steps = [np.zeros((nb, kv_bs, nkv), np.float32) for _ in range(2)]
    for b in range(B):
        for t in range(L):
            blk, off = bt[b, t // kv_bs], t % kv_bs
            pools[0][blk, off] = k_codes[b, t]
            pools[1][blk, off] = v_codes[b, t]
            steps[0][blk, off] = k_step[b, t]
            steps[1][blk, off] = v_step[b, t]
    return pools[0], steps[0], pools[1], steps[1], bt


def _random_quantized(r, B, L, nkv):
    k = W.normal_f32(r, (B, L, nkv, 128))
    v = W.normal_f32(r, (B, L, nkv, 128))
    kc, kd = kvq8.quantize_rows_q8(k)
    vc, vd = kvq8.quantize_rows_q8(v)
    return kc, kd, vc, vd


def test_single_token_returns_its_value_row():
    r = W.rng(130)
    kc, kd, vc, vd = _random_quantized(r, 1, 1, 2)
    kp, ks, vp, vs, bt = _contiguous_cache(kc, kd, vc, vd)
    q = W.normal_f32(r, (1, 4, 128))
    out = kvq8.decode_attention_q8(q, kp, ks, vp, vs, bt, [1], 16, SM)
    for h in range(4):
        want = vc[0, 0, h // 2].astype(np.float64) * np.float64(vd[0, 0, h // 2])
        assert np.array_equal(out[0, h], want)


def test_equal_keys_or_zero_query_give_the_mean_value():
    r = W.rng(131)
    L = 37
    kc, kd, vc, vd = _random_quantized(r, 1, L, 1)
    kc_eq = np.repeat(kc[:, :1], L, axis=1)
    kd_eq = np.repeat(kd[:, :1], L, axis=1)
    mean_v = (vc[0, :, 0].astype(np.float64) * vd[0, :, 0, None].astype(np.float64)).mean(0)
    kp, ks, vp, vs, bt = _contiguous_cache(kc_eq, kd_eq, vc, vd)
    q = W.normal_f32(r, (1, 1, 128))
    out = kvq8.decode_attention_q8(q, kp, ks, vp, vs, bt, [L], 16, SM)
    np.testing.assert_allclose(out[0, 0], mean_v, rtol=0, atol=1e-12)
    kp, ks, vp, vs, bt = _contiguous_cache(kc, kd, vc, vd)
    out0 = kvq8.decode_attention_q8(np.zeros((1, 1, 128), np.float32), kp, ks, vp, vs, bt, [L], 16, SM)
    np.testing.assert_allclose(out0[0, 0], mean_v, rtol=0, atol=1e-12)


def test_dominant_key_selects_its_value():
    # A query parallel to one key row, with a large amplitude, puts almost all
    # weight on that token (softmax of widely separated scores).
    r = W.rng(132)
    L = 50
    kc, kd, vc, vd = _random_quantized(r, 1, L, 1)
    kp, ks, vp, vs, bt = _contiguous_cache(kc, kd, vc, vd)
    target = 17
    q = (kc[0, target, 0].astype(np.float32) * np.float32(40.0))[None, None]
    out = kvq8.decode_attention_q8(q, kp, ks, vp, vs, bt, [L], 16, SM)
    want = vc[0, target, 0].astype(np.float64) * vd[0, target, 0]
    np.testing.assert_allclose(out[0, 0], want, atol=1e-6)


def test_output_is_convex_combination():
    r = W.rng(133)
    L = 300
    kc, kd, vc, vd = _random_quantized(r, 1, L, 1)
    kp, ks, vp, vs, bt = _contiguous_cache(kc, kd, vc, vd)
    q = W.normal_f32(r, (1, 1, 128), 3.0)
    out = kvq8.decode_attention_q8(q, kp, ks, vp, vs, bt, [L], 16, SM)[0, 0]
    V = vc[0, :, 0].astype(np.float64) * vd[0, :, 0, None]
    assert np.all(out <= V.max(0) + 1e-12) and np.all(out >= V.min(0) - 1e-12)


def _grid_exact_inputs(r, B, L, nq, nkv):
    """Keys/values whose rows sit exactly on the int8 grid with power-of-two
    steps (each row has a +-127 code), and queries whose 32-blocks sit on the
    query grid with power-of-two block maxima: quantization returns them
    unchanged (query block scales up to the float32 rounding of 1/127)."""
    def rows(shape):
        c = r.integers(-126, 127, size=shape + (128,))
        j = r.integers(0, 128, size=shape)
        np.put_along_axis(c, j[..., None], np.where(r.random(shape) < .5, 127, -127)[..., None], -1)
        step = 2.0 ** r.integers(-9, -4, size=shape)
        return (c * step[..., None]).astype(np.float32)
    K, V = rows((B, L, nkv)), rows((B, L, nkv))
    qc = r.integers(-126, 127, size=(B, nq, 4, 32))
    qc[..., 0] = 127
    q = (qc * 2.0 ** r.integers(-3, 2, size=(B, nq, 4, 1))).reshape(B, nq, 128).astype(np.float32)
    return q, K, V


@pytest.mark.parametrize("nq,nkv", [(1, 1), (4, 2), (8, 2)])
def test_grid_exact_inputs_match_library_attention(nq, nkv):
    # On exactly representable inputs the quantized pipeline must reduce to
    # plain scaled-dot-product attention; torch's CPU routine (float64, with
    # its own grouped-query convention) serves as the independent reference.
    r = W.rng(134, nq, nkv)
    B, L = 2, 45
    q, K, V = _grid_exact_inputs(r, B, L, nq, nkv)
    kc, kd = kvq8.quantize_rows_q8(K)
    vc, vd = kvq8.quantize_rows_q8(V)
    assert np.array_equal(kc.astype(np.float64) * kd[..., None], K.astype(np.float64))
    kp, ks, vp, vs, bt = _contiguous_cache(kc, kd, vc, vd, r=r)
    out = kvq8.decode_attention_q8(q, kp, ks, vp, vs, bt, [L, L], 16, SM)
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]          # B, nq, 1, D
    kt = torch.from_numpy(K.astype(np.float64)).permute(0, 2, 1, 3)     # B, nkv, L, D
    vt = torch.from_numpy(V.astype(np.float64)).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=SM, enable_gqa=True)
    np.testing.assert_allclose(out, ref[:, :, 0].numpy(), rtol=1e-6, atol=1e-7)


def test_paging_and_batching_do_not_change_results():
    r = W.rng(135)
    B, L, nq, nkv = 3, 70, 4, 2
    kc, kd, vc, vd = _random_quantized(r, B, L, nkv)
    q = W.normal_f32(r, (B, nq, 128))
    lens = [70, 1, 33]
    ident = _contiguous_cache(kc, kd, vc, vd, kv_bs=16, r=None)
    shuf = _contiguous_cache(kc, kd, vc, vd, kv_bs=8, r=r)
    o1 = kvq8.decode_attention_q8(q, *ident[:4], ident[4], lens, 16, SM)
    o2 = kvq8.decode_attention_q8(q, *shuf[:4], shuf[4], lens, 8, SM)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    for b in range(B):
        one = _contiguous_cache(kc[b:b + 1], kd[b:b + 1], vc[b:b + 1], vd[b:b + 1])
        ob = kvq8.decode_attention_q8(q[b:b + 1], *one[:4], one[4], lens[b:b + 1], 16, SM)
        np.testing.assert_allclose(o1[b], ob[0], rtol=1e-13, atol=1e-15)


def test_empty_context_gives_zero_row():
    r = W.rng(136)
    kc, kd, vc, vd = _random_quantized(r, 2, 20, 1)
    kp, ks, vp, vs, bt = _contiguous_cache(kc, kd, vc, vd)
    out = kvq8.decode_attention_q8(W.normal_f32(r, (2, 2, 128)), kp, ks, vp, vs, bt, [0, 20], 16, SM)
    assert np.all(out[0] == 0) and np.all(np.isfinite(out[1])) and np.any(out[1] != 0)


# ----------------------------------------------------------------------------
# single pass == three passes ([P3] Sec. 1 and Sec. 3; exercises of Sec. 4)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("L", [1, 2, 3, 17, 256])
def test_online_single_pass_equals_definition(L):
    r = W.rng(140, L)
    k = W.normal_f32(r, (L, 128))
    v = W.normal_f32(r, (L, 128))
    q = W.normal_f32(r, (128,), 2.0)
    kc, kd = kvq8.quantize_rows_q8(k)
    vc, vd = kvq8.quantize_rows_q8(v)
    trace = []
    on = kvq8.online_decode_q8(q, kc, kd, vc, vd, SM, trace=trace)
    ref = kvq8.decode_attention_q8_contiguous(q, kc, kd, vc, vd, SM)
    np.testing.assert_allclose(on, ref, rtol=2e-5, atol=2e-6)
    assert len(trace) == L                                  # one step per token
    assert all(b >= a for a, b in zip(trace, trace[1:]))    # running max never drops


# ----------------------------------------------------------------------------
# the [P1] Sec. 3 experiment
# ----------------------------------------------------------------------------

def _p1_stats(sigma, rounding, seeds=range(20)):
    mx, mn, sc, pos = [], [], [], []
    for s in seeds:
        q, k, v = W.unit_experiment(s, sigma)
        ref = kvq8.attention_reference(q, k, v, SM)
        got, kd = kvq8.attention_dequant_kv(q, k, v, SM, rounding)
        d = got - ref
        mx.append(np.abs(d).max())
        mn.append(np.abs(d).mean())
        sc.append(kd.mean())
        pos.append(np.mean(d[:4] > 0))
    return np.mean(mx), np.mean(mn), np.mean(sc), np.mean(pos)


def test_p1_magnitudes_round_to_nearest():
    g = json.load(open(os.path.join(GOLDEN, "p1_unit_experiment.json")))
    mx, mn, sc, _ = _p1_stats(1.0, "half_away")
    # the product reading stays within the page's error magnitudes ...
    assert 1e-4 < mx <= g["max_abs_delta"]
    assert 1e-5 < mn <= g["mean_abs_delta"]
    # ... and within half a step on average, as the page argues
    assert mn <= sc / 2
    # step of N(0,1) rows: E[max of 128 |N(0,1)|] / 127 = 2.8/127 ~ 0.0221
    assert abs(sc - 0.0221) < 0.0008


def test_p1_printed_figures_reproduced_by_diagnostic_reading():
    # sigma 0.772 data and add-half-then-truncate rounding reproduce the page's
    # average step, both error magnitudes and the all-positive deltas.
    g = json.load(open(os.path.join(GOLDEN, "p1_unit_experiment.json")))
    mx, mn, sc, pos = _p1_stats(0.772, "trunc_plus_half")
    assert abs(sc / g["avg_k_step"] - 1) < 0.02
    assert abs(mx / g["max_abs_delta"] - 1) < 0.15
    assert abs(mn / g["mean_abs_delta"] - 1) < 0.05
    printed = np.array(g["out_q_first4"]) - np.array(g["out_f_first4"])
    assert np.all(printed > 0) and pos > 0.95


def test_output_depends_on_query_only_through_its_codes():
    # [P3] Sec. 2 seg. 1: the query enters the kernel only as int8 codes and
    # per-block scales.  Two queries with identical codes and scales must give
    # identical outputs; nudging non-maximal elements keeps the codes.
    r = W.rng(137)
    L, nkv = 90, 2
    kc, kd, vc, vd = _random_quantized(r, 1, L, nkv)
    kp, ks, vp, vs, bt = _contiguous_cache(kc, kd, vc, vd)
    q = W.normal_f32(r, (1, 4, 128))
    qi, qsc = kvq8.quantize_q_blocks(q)
    q2 = q.copy()
    blk = np.abs(q.reshape(1, 4, 4, 32))
    notmax = (blk < blk.max(-1, keepdims=True)).reshape(q.shape)
    step = (qsc.repeat(32, axis=-1)).astype(np.float32)
    frac = q / step - np.round(q / step)
    nudge = np.where(notmax & (np.abs(frac) < 0.3), np.float32(0.1) * step, np.float32(0))
    q2 = (q + nudge).astype(np.float32)
    qi2, qsc2 = kvq8.quantize_q_blocks(q2)
    assert np.array_equal(qi, qi2) and np.array_equal(qsc, qsc2) and not np.array_equal(q, q2)
    o1 = kvq8.decode_attention_q8(q, kp, ks, vp, vs, bt, [L], 16, SM)
    o2 = kvq8.decode_attention_q8(q2, kp, ks, vp, vs, bt, [L], 16, SM)
    assert np.array_equal(o1, o2)
    # and the paged definition agrees with the pages' single pass
    on = kvq8.online_decode_q8(q[0, 3], kc[0, :, 1], kd[0, :, 1], vc[0, :, 1], vd[0, :, 1], SM)
    np.testing.assert_allclose(on, o1[0, 3], rtol=2e-5, atol=2e-6)
