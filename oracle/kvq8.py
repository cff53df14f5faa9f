"""Oracle for the int8 (q8) KV path: write-path quantization, query
quantization, integer block dot products and decode attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pins (tests/test_oracle_*.py), one line per function:
  quantize_rows_q8      brute force with exact rationals; argmax code +-127;
                        half-step error bound; tie cases; power-of-two scale
                        invariance; byte accounting against [P2] Sec. 2.
  quantize_q_blocks     brute force with exact rationals; block independence.
  qk_block_partials     brute force with Python integers; |dot| bound.
  decode_attention_q8   closed forms (L=1, equal keys, zero query, two-token
                        softmax), convexity, GQA head mapping, paging
                        invariance, exact-grid inputs vs. plain attention.
  online_decode_q8      equals decode_attention_q8 on small cases ([P3] Sec. 1
                        and Sec. 3 say the two are functionally equivalent);
                        running max is non-decreasing; one step per token.
  attention_reference,
  attention_dequant_kv  [P1] Sec. 3 error statistics (both the round-to-
                        nearest reading and the diagnostic reading that
                        reproduces the printed figures).
"""
from __future__ import annotations

import numpy as np

HD = 128          # head dimension fixed by all four pages
QBLOCK = 32       # query quantization block ([P3] Sec. 2 seg. 1)
F32 = np.float32

# 1/127 as a float32 constant: the engine's dequantization constant for q8
# ([P1] Sec. 2, [P3] Sec. 2 seg. 1).  Computed as an IEEE float32 division.
INV127 = F32(1.0) / F32(127.0)


# ----------------------------------------------------------------------------
# rounding
# ----------------------------------------------------------------------------

def round_half_away(y) -> np.ndarray:
    """C ``roundf`` of float32 values: nearest integer, ties away from zero.

    Exact: widening float32 to float64 and adding 0.5 are both exact for
    |y| < 2**29, and ``floor`` of an exact value is exact."""
    y64 = np.asarray(y, dtype=np.float32).astype(np.float64)
    return np.sign(y64) * np.floor(np.abs(y64) + 0.5)


def trunc_plus_half(y) -> np.ndarray:
    """``(int)(y + 0.5f)`` in C: add one half, then truncate toward zero.

    Diagnostic only.  It rounds negative values half a step upward; together
    with sigma ~ 0.77 data it reproduces every figure printed in [P1] Sec. 3
    (all four printed output deltas are positive, which unbiased rounding does
    not produce).  The product reading is round_half_away."""
    y64 = np.asarray(y, dtype=np.float32).astype(np.float64)
    return np.trunc(y64 + 0.5)


_ROUNDERS = {"half_away": round_half_away, "trunc_plus_half": trunc_plus_half}


# ----------------------------------------------------------------------------
# a1: per-(token, head) K/V quantization  -- [P1] Sec. 2, [P2] Sec. 2
# ----------------------------------------------------------------------------

def quantize_rows_q8(x, rounding: str = "half_away"):
    """Symmetric int8 quantization of each 128-value (token, kv-head) row.

    For each row: amax = max |x|; step d = amax / 127 (float32 division);
    code = round(x / d) (float32 division, then roundf), clamped to
    [-127, 127].  One float32 step per row, shared by its 128 values.

    Reading of a silent point: a row with amax < 1e-6 uses amax = 1, the same
    guard [P3] Sec. 2 seg. 1 applies to query blocks (otherwise d = 0 and
    x / d is undefined).  Such rows get codes 0 and step 1/127.

    Returns (codes int8 [..., 128], d float32 [...]).  The stored per-row
    "scale" is the step d itself, so dequantization is code * d ([P1] Sec. 2).
    """
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] == HD
    amax = np.max(np.abs(x), axis=-1)
    amax = np.where(amax < F32(1e-6), F32(1.0), amax).astype(np.float32)
    d = (amax / F32(127.0)).astype(np.float32)
    y = (x / d[..., None]).astype(np.float32)
    c = np.clip(_ROUNDERS[rounding](y), -127, 127).astype(np.int8)
    return c, d


def dequantize_rows_q8(codes, d) -> np.ndarray:
    """code * step, in float64 ([P1] Sec. 2)."""
    return codes.astype(np.float64) * np.asarray(d, dtype=np.float64)[..., None]


# ----------------------------------------------------------------------------
# a2: query quantization  -- [P3] Sec. 2 seg. 1
# ----------------------------------------------------------------------------

def quantize_q_blocks(q):
    """Quantize each query vector once, in blocks of 32 values.

    Per block: qm = max |q|; if qm < 1e-6 then qm = 1; block scale
    qsc = qm * (1/127) with 1/127 a float32 constant; multiplier
    iq = 127 / qm (float32 division); code = roundf(q * iq) clamped to
    [-128, 127].

    Reading: the page casts without an explicit rounding call; the scheme is
    described as isomorphic to the Q8_0 block format and the K/V rule rounds,
    so codes are rounded to nearest (ties away from zero).  The [-128, 127]
    clamp is kept as printed; it never binds because |q * iq| <= 127.

    Returns (qi int8 [..., 128], qsc float32 [..., 4]).
    """
    q = np.asarray(q, dtype=np.float32)
    assert q.shape[-1] == HD
    qb = q.reshape(q.shape[:-1] + (HD // QBLOCK, QBLOCK))
    qm = np.max(np.abs(qb), axis=-1)
    qm = np.where(qm < F32(1e-6), F32(1.0), qm).astype(np.float32)
    qsc = (qm * INV127).astype(np.float32)
    iq = (F32(127.0) / qm).astype(np.float32)
    y = (qb * iq[..., None]).astype(np.float32)
    qi = np.clip(round_half_away(y), -128, 127).astype(np.int8)
    return qi.reshape(q.shape), qsc


def dequantize_q_blocks(qi, qsc) -> np.ndarray:
    """qi * qsc of its block, in float64."""
    qi = np.asarray(qi)
    b = qi.astype(np.float64).reshape(qi.shape[:-1] + (HD // QBLOCK, QBLOCK))
    return (b * np.asarray(qsc, dtype=np.float64)[..., None]).reshape(qi.shape)


# ----------------------------------------------------------------------------
# a3: integer block dot products  -- [P3] Sec. 2 seg. 2
# ----------------------------------------------------------------------------

def qk_block_partials(qi, kq) -> np.ndarray:
    """dot_b = sum over block b of qi * kq, exact integers.

    qi int8 [..., 128] (one or more query heads), kq int8 [T, 128] (T key
    rows).  Returns int64 [..., T, 4]."""
    a = np.asarray(qi).astype(np.int64)
    a = a.reshape(a.shape[:-1] + (HD // QBLOCK, QBLOCK))
    k = np.asarray(kq).astype(np.int64).reshape(-1, HD // QBLOCK, QBLOCK)
    return np.einsum("...bi,tbi->...tb", a, k)


# ----------------------------------------------------------------------------
# paged cache bookkeeping  -- [P2] Sec. 2, [P3] Sec. 2 seg. 2
# ----------------------------------------------------------------------------
# Layout (the pages' token-major block layout): codes
# [n_blocks][kv_bs][nkv][128]; steps [n_blocks][kv_bs][nkv].  Token t of a
# sequence lives in block table[t // kv_bs], row t % kv_bs, and head kh's
# 128 codes start at kh * 128 inside that row.

def gather_rows(pool, block_table, L: int, kv_bs: int, kh: int):
    """Rows of tokens 0..L-1 for kv-head kh: pool[blk, off, kh]."""
    t = np.arange(L)
    blk = np.asarray(block_table)[t // kv_bs]
    return pool[blk, t % kv_bs, kh]


def quantize_append(k_pool, v_pool, k_step, v_step, k_new, v_new, slots):
    """Write path: quantize each new (token, kv-head) row of K and V and store
    codes and step at cache slot slots[i] = block * kv_bs + offset.

    Pools are modified in place.  Slots outside [0, n_blocks * kv_bs) are
    skipped (a negative slot marks padding).  Returns the pools."""
    kc, kd = quantize_rows_q8(k_new)
    vc, vd = quantize_rows_q8(v_new)
    nb, bs, nkv, hd = k_pool.shape
    flat_kc = k_pool.reshape(nb * bs, nkv, hd)
    flat_vc = v_pool.reshape(nb * bs, nkv, hd)
    flat_ks = k_step.reshape(nb * bs, nkv)
    flat_vs = v_step.reshape(nb * bs, nkv)
    slots = np.asarray(slots, dtype=np.int64)
    ok = (slots >= 0) & (slots < nb * bs)
    flat_kc[slots[ok]] = kc[ok]
    flat_vc[slots[ok]] = vc[ok]
    flat_ks[slots[ok]] = kd[ok]
    flat_vs[slots[ok]] = vd[ok]
    return k_pool, v_pool, k_step, v_step


# ----------------------------------------------------------------------------
# a3-a6: decode attention, the plain definition  -- [P1] Sec. 1-2, [P3] Sec. 1
# ----------------------------------------------------------------------------

def softmax_attention_f64(q_vec, K, V, sm_scale):
    """Three-pass attention for one query: all scores, then max-subtracted
    softmax, then the weighted sum of V rows.  float64 throughout."""
    s = (np.asarray(K, np.float64) @ np.asarray(q_vec, np.float64)) * float(sm_scale)
    w = np.exp(s - s.max())
    w /= w.sum()
    return w @ np.asarray(V, np.float64)


def decode_attention_q8(q, k_pool, k_step, v_pool, v_step, block_tables, ctx_lens,
                        kv_bs: int, sm_scale: float):
    """Decode attention over the int8 paged cache, as defined by the pages.

    q float32 [B][nq][128].  Query head h reads kv-head h // (nq / nkv).  The
    query is quantized once (quantize_q_blocks); keys and values are the
    stored codes times their per-(token, head) step.  The score of token t is
    sm_scale * (sum_b qsc_b * dot_b) * kstep_t, which equals sm_scale times
    the float64 dot product of the dequantized query and key; the output is
    the softmax-weighted sum of dequantized values.  A sequence with
    ctx_len 0 yields a zero row.

    Returns float64 [B][nq][128]."""
    q = np.asarray(q, dtype=np.float32)
    B, nq, hd = q.shape
    nkv = k_pool.shape[2]
    g = nq // nkv
    qi, qsc = quantize_q_blocks(q)
    q_hat = dequantize_q_blocks(qi, qsc)
    out = np.zeros((B, nq, hd), dtype=np.float64)
    for b in range(B):
        L = int(ctx_lens[b])
        if L <= 0:
            continue
        for kh in range(nkv):
            K = dequantize_rows_q8(gather_rows(k_pool, block_tables[b], L, kv_bs, kh),
                                   gather_rows(k_step, block_tables[b], L, kv_bs, kh))
            V = dequantize_rows_q8(gather_rows(v_pool, block_tables[b], L, kv_bs, kh),
                                   gather_rows(v_step, block_tables[b], L, kv_bs, kh))
            for h in range(kh * g, (kh + 1) * g):
                out[b, h] = softmax_attention_f64(q_hat[b, h], K, V, sm_scale)
    return out


def decode_attention_q8_contiguous(q_vec, k_codes, k_step, v_codes, v_step, sm_scale):
    """Single query head over contiguous rows k_codes [L][128] (no paging)."""
    qi, qsc = quantize_q_blocks(np.asarray(q_vec, np.float32)[None])
    q_hat = dequantize_q_blocks(qi, qsc)[0]
    return softmax_attention_f64(q_hat, dequantize_rows_q8(k_codes, k_step),
                                 dequantize_rows_q8(v_codes, v_step), sm_scale)


# ----------------------------------------------------------------------------
# the pages' single pass, step by step  -- [P3] Sec. 2 seg. 1-3
# ----------------------------------------------------------------------------

def online_decode_q8(q_vec, k_codes, k_step, v_codes, v_step, sm_scale, trace=None):
    """One query head, one pass over L key/value rows, in float32, following
    [P3] Sec. 2: quantize q once; for each token take the four integer block
    dot products, scale them by the query block scales, then by the key step
    and sm_scale; keep a running max M and running sum S (online softmax,
    initial M = -1e9); on a new maximum rescale S and the accumulator by
    exp(M_old - M_new) and give the new token weight 1, otherwise weight
    exp(s - M); add weight * step_v * codes_v to the accumulator; finally
    divide by S ([P3] Sec. 2 seg. 3).

    ``trace`` (optional list) receives M after every token.  Small inputs
    only: this is a Python loop."""
    qi, qsc = quantize_q_blocks(np.asarray(q_vec, np.float32)[None])
    qi, qsc = qi[0].astype(np.int64), qsc[0]
    scale = F32(sm_scale)
    M, S = F32(-1e9), F32(0.0)
    acc = np.zeros(HD, dtype=np.float32)
    for t in range(k_codes.shape[0]):
        kt = k_codes[t].astype(np.int64)
        s = F32(0.0)
        for b in range(HD // QBLOCK):
            dot = int(np.dot(qi[b * QBLOCK:(b + 1) * QBLOCK], kt[b * QBLOCK:(b + 1) * QBLOCK]))
            s = F32(s + F32(F32(dot) * qsc[b]))
        s = F32(F32(s * F32(k_step[t])) * scale)
        if s > M:
            r = F32(np.exp(F32(M - s)))
            S = F32(S * r)
            acc = (acc * r).astype(np.float32)
            M = s
            w = F32(1.0)
        else:
            w = F32(np.exp(F32(s - M)))
        S = F32(S + w)
        acc = (acc + v_codes[t].astype(np.float32) * F32(w * F32(v_step[t]))).astype(np.float32)
        if trace is not None:
            trace.append(M)
    return (acc / S).astype(np.float32)


# ----------------------------------------------------------------------------
# the two arms of the [P1] Sec. 1 experiment
# ----------------------------------------------------------------------------

def attention_reference(q_vec, K, V, sm_scale):
    """Baseline arm: unquantized query, keys and values; float64."""
    return softmax_attention_f64(q_vec, K, V, sm_scale)


def attention_dequant_kv(q_vec, K, V, sm_scale, rounding: str = "half_away"):
    """Measured arm: K and V quantized per row by the engine rule, then
    dequantized; the query stays unquantized; same attention formula."""
    kc, kd = quantize_rows_q8(K, rounding)
    vc, vd = quantize_rows_q8(V, rounding)
    return softmax_attention_f64(q_vec, dequantize_rows_q8(kc, kd), dequantize_rows_q8(vc, vd), sm_scale), kd


# ----------------------------------------------------------------------------
# byte accounting  -- [P2] Sec. 2
# ----------------------------------------------------------------------------

def kv_bytes_per_token_layer(nkv: int, hd: int, mode: str) -> int:
    """Cache bytes for one token of one layer, K and V together: 'f16' is two
    bytes per value; 'q8' is one byte per value plus one float32 step per
    (token, head) for K and for V."""
    if mode == "f16":
        return 2 * nkv * hd * 2
    if mode == "q8":
        return 2 * nkv * hd * 1 + 2 * nkv * 4
    raise ValueError(mode)
