"""Oracle for the Q4_0 KV mode: symmetric 4-bit codes in blocks of 32 values
along the head dimension with one float32 step per block, two codes per byte,
and decode attention that scores the query's 8-bit block codes against the
4-bit codes without dequantizing them ([P2] Sec. 1 and Sec. 3: the --kv-q4
switch, a Q4_0 payload cache about 1.65x denser than q8).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Readings (the pages name the format and its density, nothing more):
  * Q4_0 is the 32-value block format whose step is the block's extreme
    value divided by -8, so the extreme lands exactly on code 0 and the codes
    0..15 stand for -8..7 steps.  The page's density fixes the step's width:
    4 blocks x (16 code bytes + 4 step bytes) = 80 B per (token, head)
    against q8's 128 + 4 = 132 B is 1.65x; a float16 step would give 1.83x.
  * extreme = the value of largest magnitude; when a positive and a negative
    value tie for it, the negative one (this makes the choice independent of
    element order).  A block of zeros has step +0 and all codes 8.
  * code = min(15, floor(x / step + 8.5)) in float32 (IEEE division, then one
    float32 addition), i.e. round half up on the code grid; the clamp binds
    only for values above 7.5 steps on the side opposite the extreme.
  * the score needs no dequantization: with query block codes qi and scale
    qsc (the int8 path's query quantization), sum_b qsc_b * step_b *
    (P_b - 8 R_b) where P_b = sum qi * code and R_b = sum qi over block b.
    That is exactly the dot product of the dequantized query and key, which
    is what decode_attention_q4_0 evaluates in float64.
  * storage layouts (two codes per byte) are this library's, chosen so that
    the decode kernel's lanes read contiguous bytes:
      key row (64 B):   byte j holds element j (low nibble) and element
                        64 + j (high nibble);
      value row (64 B): byte 4m + k holds elements 32k + 2m (low nibble) and
                        32k + 2m + 1 (high nibble), k = 0..3, m = 0..15.

Pins (tests/test_oracle_kvq4_0.py):
  quantize_blocks_q4_0  every code is the nearest of all 16 grid points
                        (brute force; ties toward the higher code); the
                        extreme is reproduced exactly; error <= step / 2 except
                        the clamped top, <= one step there; power-of-two
                        scaling moves the step only; zero blocks; tie rule.
  pack / unpack         round trips; single-element placement in both
                        layouts; byte accounting against [P2] (1.65x).
  qk_scores_no_dequant  equals the float64 dot product of the dequantized
                        operands (closed form), and integer P, R by brute
                        force.
  decode_attention_q4_0 closed forms (L = 1, equal keys, zero query,
                        two-token softmax), GQA head mapping, paging
                        invariance.
"""
from __future__ import annotations

import numpy as np

from . import kvq8

HD = 128
BLOCK = 32
NB = HD // BLOCK
F32 = np.float32


# ----------------------------------------------------------------------------
# quantization
# ----------------------------------------------------------------------------

def block_extreme(x) -> np.ndarray:
    """Signed value of largest magnitude of each 32-value block; the negative
    one when a positive and a negative value tie.  x float32 [..., 128] ->
    float32 [..., 4]."""
    b = np.asarray(x, dtype=np.float32).reshape(np.shape(x)[:-1] + (NB, BLOCK))
    mx = b.max(axis=-1)
    mn = b.min(axis=-1)
    return np.where(-mn >= mx, mn, mx).astype(np.float32)


def quantize_blocks_q4_0(x):
    """Q4_0 quantization of each 32-value block of a row (readings in the
    module header).

    x float32 [..., 128].  Returns (codes uint8 [..., 128] in [0, 15],
    step float32 [..., 4]); value = (code - 8) * step."""
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] == HD
    m = block_extreme(x)
    step = (m / F32(-8.0)).astype(np.float32)
    step = np.where(m == 0, F32(0.0), step).astype(np.float32)       # +0 for a zero block
    b = x.reshape(x.shape[:-1] + (NB, BLOCK))
    safe = np.where(step == 0, F32(1.0), step)[..., None]
    with np.errstate(invalid="ignore", divide="ignore"):
        t = ((b / safe).astype(np.float32) + F32(8.5)).astype(np.float32)
    c = np.minimum(np.floor(t), F32(15.0))
    c = np.where((step == 0)[..., None], F32(8.0), c)
    return c.astype(np.uint8).reshape(x.shape), step


def dequantize_blocks_q4_0(codes, step) -> np.ndarray:
    """(code - 8) * step of its block, float64."""
    c = np.asarray(codes).astype(np.float64)
    c = c.reshape(c.shape[:-1] + (NB, BLOCK))
    s = np.asarray(step, dtype=np.float64)[..., None]
    return ((c - 8.0) * s).reshape(np.asarray(codes).shape)


# ----------------------------------------------------------------------------
# storage layouts (two codes per byte)
# ----------------------------------------------------------------------------

def pack_k(codes) -> np.ndarray:
    """Key row: byte j = element j | element (64 + j) << 4.  [..., 128] ->
    uint8 [..., 64]."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., :64] | (c[..., 64:] << 4)).astype(np.uint8)


def unpack_k(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    return np.concatenate([p & 0x0F, p >> 4], axis=-1).astype(np.uint8)


def _v_index():
    """lo[j], hi[j]: elements stored in the low and high nibble of value byte
    j = 4m + k: 32k + 2m and 32k + 2m + 1."""
    j = np.arange(64)
    m, k = j // 4, j % 4
    lo = 32 * k + 2 * m
    return lo, lo + 1


def pack_v(codes) -> np.ndarray:
    """Value row: byte 4m + k = element (32k + 2m) | element (32k + 2m + 1) << 4.
    [..., 128] -> uint8 [..., 64]."""
    c = np.asarray(codes, dtype=np.uint8)
    lo, hi = _v_index()
    return (c[..., lo] | (c[..., hi] << 4)).astype(np.uint8)


def unpack_v(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    lo, hi = _v_index()
    out = np.empty(p.shape[:-1] + (HD,), dtype=np.uint8)
    out[..., lo] = p & 0x0F
    out[..., hi] = p >> 4
    return out


def kv_bytes_per_token_head() -> int:
    """Cache bytes of one (token, kv-head), K and V together: 64 code bytes and
    4 float32 steps each."""
    return 2 * (HD // 2 + NB * 4)


# ----------------------------------------------------------------------------
# write path
# ----------------------------------------------------------------------------

def quantize_append_q4_0(k_pool, v_pool, k_step, v_step, k_new, v_new, slots):
    """Quantize new (token, kv-head) rows of K and V and store them at cache
    slots[i] = block * kv_bs + offset.  Pools: packed codes
    [n_blocks][kv_bs][nkv][64] uint8, steps [n_blocks][kv_bs][nkv][4] float32,
    modified in place.  Slots outside the pool are skipped."""
    kc, ks = quantize_blocks_q4_0(k_new)
    vc, vs = quantize_blocks_q4_0(v_new)
    nb, bs = k_pool.shape[:2]
    slots = np.asarray(slots, dtype=np.int64)
    ok = (slots >= 0) & (slots < nb * bs)
    for pool, val in ((k_pool, pack_k(kc)), (v_pool, pack_v(vc)), (k_step, ks), (v_step, vs)):
        flat = pool.reshape((nb * bs,) + pool.shape[2:])
        flat[slots[ok]] = val[ok]
    return k_pool, v_pool, k_step, v_step


# ----------------------------------------------------------------------------
# scores without dequantization, and decode attention
# ----------------------------------------------------------------------------

def qk_block_terms(qi, codes):
    """Integer block sums P_b = sum qi * code and R_b = sum qi.  qi int8
    [128]; codes uint8 [T, 128] -> (P int64 [T, 4], R int64 [4])."""
    q = np.asarray(qi).astype(np.int64).reshape(NB, BLOCK)
    c = np.asarray(codes).astype(np.int64).reshape(-1, NB, BLOCK)
    return np.einsum("bi,tbi->tb", q, c), q.sum(axis=-1)


def qk_scores_no_dequant(qi, qsc, codes, step) -> np.ndarray:
    """sum_b qsc_b * step_b * (P_b - 8 R_b) per token, float64 ([P2] Sec. 3:
    the q4 decode dot consumes the nibbles directly)."""
    P, R = qk_block_terms(qi, codes)
    return ((P - 8 * R[None, :]).astype(np.float64) * np.asarray(qsc, np.float64)[None, :]
            * np.asarray(step, np.float64)).sum(axis=-1)


def decode_attention_q4_0(q, k_pool, k_step, v_pool, v_step, block_tables, ctx_lens,
                          kv_bs: int, sm_scale: float):
    """Decode attention over the Q4_0 paged cache.

    q float32 [B][nq][128]; query head h reads kv-head h // (nq / nkv).  The
    query is quantized as in the int8 path; keys and values are (code - 8)
    times their block step.  Scores are sm_scale times the dot product of
    the dequantized query and key (equal to the no-dequantization form); the
    output is the softmax-weighted sum of dequantized values, float64.  A
    sequence with ctx_len 0 yields a zero row.  Returns float64 [B][nq][128]."""
    q = np.asarray(q, dtype=np.float32)
    B, nq, hd = q.shape
    nkv = k_pool.shape[2]
    g = nq // nkv
    qi, qsc = kvq8.quantize_q_blocks(q)
    q_hat = kvq8.dequantize_q_blocks(qi, qsc)
    out = np.zeros((B, nq, hd), dtype=np.float64)
    for b in range(B):
        L = int(ctx_lens[b])
        if L <= 0:
            continue
        for kh in range(nkv):
            G = lambda pool: kvq8.gather_rows(pool, block_tables[b], L, kv_bs, kh)  # noqa: E731
            K = dequantize_blocks_q4_0(unpack_k(G(k_pool)), G(k_step))
            V = dequantize_blocks_q4_0(unpack_v(G(v_pool)), G(v_step))
            for h in range(kh * g, (kh + 1) * g):
                out[b, h] = kvq8.softmax_attention_f64(q_hat[b, h], K, V, sm_scale)
    return out
