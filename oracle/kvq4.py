"""Oracle for the int4 group variant: asymmetric 4-bit codes in groups of 64
values along the head dimension, a float16 scale and float16 zero point per
group, two codes per byte; recent tokens kept in the int8 format.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pins (tests/test_oracle_kvq4.py):
  quantize_groups_q4   brute force with exact rationals on small groups;
                       codes in [0, 15]; round-trip error <= half a step
                       ([P4] Sec. 3.2); constant groups are exact.
  pack/unpack_nibbles  round trip; even element in the high nibble.
  pack/unpack_v4       round trip; every pair keeps the page's nibble order;
                       single-pair placement at byte 4m + 2g + k.
  requantize_q8_to_q4  rows whose int8 values lie exactly on an int4 grid give
                       that grid's codes, scale and zero back; the int4 value
                       of every element is within half an int4 step of its
                       int8 value; constant groups take the unit scale.
  decode_attention_mixed
                       with every token in the int8 pool it equals
                       kvq8.decode_attention_q8; on values exactly on the
                       int4 grid it equals plain float64 attention of the
                       dequantized query; token-order invariance across the
                       two pools.
"""
from __future__ import annotations

import numpy as np

from . import kvq8

HD = 128
GROUP = 64        # [P4] Sec. 3.2: group size 64 is the recommended start
F32 = np.float32
F16 = np.float16


def quantize_groups_q4(x):
    """Asymmetric 4-bit quantization of each 64-value group of a row.

    Following [P4] Sec. 3.2, per group: scale = (max - min) / 15, or 1.0 when
    max == min; zero = round(-min / scale); code = clamp(round(x / scale +
    zero), 0, 15); dequantized value = (code - zero) * scale.  round is
    round-half-to-even (the page uses torch.round).

    Readings where the page leaves precision open:
      * arithmetic in float32 with IEEE division;
      * the scale is floored at 1e-7 ([P4] Sec. 5.2 checklist), rounded to
        float16 for storage, and the stored float16 value is the one used to
        compute zero and codes, so stored and used scales agree;
      * zero is clamped to [0, 15] ([P4] Sec. 5.2 says it must lie there) and
        stored as float16, where every such integer is exact; a zero point
        of 0 is stored as +0.0.

    x float32 [..., 128].  Returns (codes uint8 [..., 128] in [0, 15],
    scale float16 [..., 2], zero float16 [..., 2])."""
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] == HD
    g = x.reshape(x.shape[:-1] + (HD // GROUP, GROUP))
    mx = g.max(axis=-1)
    mn = g.min(axis=-1)
    s32 = ((mx - mn).astype(np.float32) / F32(15.0)).astype(np.float32)
    s32 = np.where(mx == mn, F32(1.0), s32)
    s32 = np.maximum(s32, F32(1e-7)).astype(np.float32)
    s16 = s32.astype(F16)
    s = s16.astype(np.float32)
    # the zero point is an integer in [0, 15]; adding +0 stores a zero as +0.0
    # (rint of a small negative quotient is -0.0, the same integer)
    z = (np.clip(np.rint((-mn / s).astype(np.float32)), 0, 15) + F32(0.0)).astype(np.float32)
    y = ((g / s[..., None]).astype(np.float32) + z[..., None]).astype(np.float32)
    c = np.clip(np.rint(y), 0, 15).astype(np.uint8)
    return c.reshape(x.shape), s16, z.astype(F16)


def dequantize_groups_q4(codes, scale, zero) -> np.ndarray:
    """(code - zero) * scale per group, float64."""
    c = np.asarray(codes).astype(np.float64)
    c = c.reshape(c.shape[:-1] + (HD // GROUP, GROUP))
    z = np.asarray(zero, dtype=np.float64)[..., None]
    s = np.asarray(scale, dtype=np.float64)[..., None]
    return ((c - z) * s).reshape(np.asarray(codes).shape)


def pack_nibbles(codes) -> np.ndarray:
    """Two codes per byte, even-indexed code in the high nibble ([P4] Sec. 3.2);
    pair (2i, 2i + 1) in byte i.  The key rows of the int4 pool."""
    c = np.asarray(codes, dtype=np.uint8)
    return ((c[..., 0::2] << 4) | c[..., 1::2]).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p >> 4
    out[..., 1::2] = p & 0x0F
    return out


def _v4_pair_bytes() -> np.ndarray:
    """Byte of each pair (2i, 2i + 1) in a value row: elements 64g + 4m + 2k and
    + 1 (group g, k = 0, 1) sit in byte 4m + 2g + k, so the 4-byte word m holds
    elements 4m .. 4m + 3 of both groups (this library's storage order; the
    pairing and the nibble order are the page's)."""
    e = 2 * np.arange(64)
    g, m, k = e // 64, (e % 64) // 4, (e % 4) // 2
    return 4 * m + 2 * g + k


def pack_v4(codes) -> np.ndarray:
    """Value row of the int4 pool: pairs packed as pack_nibbles, in the byte
    order of _v4_pair_bytes.  [..., 128] -> uint8 [..., 64]."""
    p = pack_nibbles(codes)
    out = np.empty_like(p)
    out[..., _v4_pair_bytes()] = p
    return out


def unpack_v4(packed) -> np.ndarray:
    return unpack_nibbles(np.asarray(packed, dtype=np.uint8)[..., _v4_pair_bytes()])


def quantize_append_q4(k_pool, v_pool, k_scale, k_zero, v_scale, v_zero, k_new, v_new, slots):
    """Write path for the int4 pool: packed codes [n_blocks][kv_bs][nkv][64]
    (keys as pack_nibbles, values as pack_v4),
    scale and zero [n_blocks][kv_bs][nkv][2] float16.  Slots outside the pool
    are skipped.  Pools are modified in place."""
    kc, ks, kz = quantize_groups_q4(k_new)
    vc, vs, vz = quantize_groups_q4(v_new)
    nb, bs, nkv, _ = k_pool.shape
    slots = np.asarray(slots, dtype=np.int64)
    ok = (slots >= 0) & (slots < nb * bs)
    for pool, val in ((k_pool, pack_nibbles(kc)), (v_pool, pack_v4(vc)),
                      (k_scale, ks), (k_zero, kz), (v_scale, vs), (v_zero, vz)):
        flat = pool.reshape((nb * bs,) + pool.shape[2:])
        flat[slots[ok]] = val[ok]
    return k_pool, v_pool, k_scale, k_zero, v_scale, v_zero


def dequantize_rows_q8_f32(codes, d) -> np.ndarray:
    """code * step as the engine computes it: one float32 multiplication."""
    return np.asarray(codes).astype(F32) * np.asarray(d, dtype=F32)[..., None]


def requantize_q8_to_q4(q8_pools, q4_pools, src_slots, dst_slots):
    """Move tokens from the int8 pool to the int4 pool ([P4] Sec. 3.3 practical
    notes: as the sequence grows, the oldest time block is re-quantized from
    8-bit to 4-bit).

    Reading: the float values are gone once a token is in the int8 pool, so
    the int4 codes are those of the int8 values: code * step (float32, the
    engine's precision) goes through quantize_groups_q4.  Pair i moves slot
    src_slots[i] of the int8 pool to slot dst_slots[i] of the int4 pool;
    pairs with either slot outside its pool are skipped.

    q8_pools = (k_codes, k_step, v_codes, v_step) as in kvq8; q4_pools =
    (k_packed, k_scale, k_zero, v_packed, v_scale, v_zero), modified in place.
    """
    kc8, ks8, vc8, vs8 = q8_pools
    k4, k4s, k4z, v4, v4s, v4z = q4_pools
    nb8, bs, nkv, _ = kc8.shape
    nb4 = k4.shape[0]
    src = np.asarray(src_slots, dtype=np.int64)
    dst = np.asarray(dst_slots, dtype=np.int64)
    ok = (src >= 0) & (src < nb8 * bs) & (dst >= 0) & (dst < nb4 * bs)
    src, dst = src[ok], dst[ok]
    flat = lambda a: a.reshape((a.shape[0] * a.shape[1],) + a.shape[2:])
    xk = dequantize_rows_q8_f32(flat(kc8)[src], flat(ks8)[src])
    xv = dequantize_rows_q8_f32(flat(vc8)[src], flat(vs8)[src])
    quantize_append_q4(k4, v4, k4s, k4z, v4s, v4z, xk, xv, dst)
    return q4_pools


def decode_attention_mixed(q, q4_pools, bt4, lens4, q8_pools, bt8, lens8, kv_bs: int, sm_scale: float):
    """Decode attention over a sequence whose older tokens sit in the int4
    pool and whose recent window sits in the int8 pool ([P4] Sec. 2.2 and
    Sec. 3.3: recent tokens keep higher precision).

    q4_pools = (k_packed, k_scale, k_zero, v_packed, v_scale, v_zero);
    q8_pools = (k_codes, k_step, v_codes, v_step).  Sequence b attends over
    lens4[b] int4 tokens (positions 0.. via bt4[b]) and lens8[b] int8 tokens
    (positions 0.. via bt8[b]).  Attention does not depend on token order, so
    the split between the pools only decides each token's precision.

    The query is quantized as in the int8 path; scores are sm_scale times the
    dot product of the dequantized query and dequantized key; float64.
    Returns float64 [B][nq][128]."""
    q = np.asarray(q, dtype=np.float32)
    B, nq, hd = q.shape
    k4, k4s, k4z, v4, v4s, v4z = q4_pools
    k8, k8s, v8, v8s = q8_pools
    nkv = k4.shape[2]
    g = nq // nkv
    qi, qsc = kvq8.quantize_q_blocks(q)
    q_hat = kvq8.dequantize_q_blocks(qi, qsc)
    out = np.zeros((B, nq, hd), dtype=np.float64)
    for b in range(B):
        n4, n8 = int(lens4[b]), int(lens8[b])
        if n4 + n8 <= 0:
            continue
        for kh in range(nkv):
            Ks, Vs = [], []
            if n4 > 0:
                G = lambda pool: kvq8.gather_rows(pool, bt4[b], n4, kv_bs, kh)  # noqa: E731
                Ks.append(dequantize_groups_q4(unpack_nibbles(G(k4)), G(k4s), G(k4z)))
                Vs.append(dequantize_groups_q4(unpack_v4(G(v4)), G(v4s), G(v4z)))
            if n8 > 0:
                G = lambda pool: kvq8.gather_rows(pool, bt8[b], n8, kv_bs, kh)  # noqa: E731
                Ks.append(kvq8.dequantize_rows_q8(G(k8), G(k8s)))
                Vs.append(kvq8.dequantize_rows_q8(G(v8), G(v8s)))
            K = np.concatenate(Ks)
            V = np.concatenate(Vs)
            for h in range(kh * g, (kh + 1) * g):
                out[b, h] = kvq8.softmax_attention_f64(q_hat[b, h], K, V, sm_scale)
    return out
