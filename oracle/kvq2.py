"""Oracle for the 2-bit far band of the group variant: asymmetric 2-bit codes
in groups of 64 values along the head dimension with a float16 scale and
float16 zero point per group, four codes per byte, for the oldest tokens of a
sequence whose middle band is int4 and whose recent window is int8 ([P4]
Sec. 2.2 time-adaptive bits, Sec. 3.3 band schedule and block re-quantization).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Readings (where the page is open):
  * the 2-bit codes are the page's group quantizer (Sec. 3.2) with bits = 2:
    the code range is 0 .. 2^bits - 1 = 3, so scale = (max - min) / 3 (1.0 when
    max == min), zero = round(-min / scale), code = clamp(round(x / scale +
    zero), 0, 3).  The precision conventions are those of the int4 oracle
    (float32 arithmetic, scale floored at 1e-7 and rounded to float16 before
    use, zero clamped to the code range, round half to even).
  * bands: the page's example schedule has edges at 2048 and 16384 tokens and
    gives 8, 4 and 2 bits; as in the int4 variant, the narrative direction
    (recent tokens keep more precision) decides which end is which: the
    newest 2048 tokens are int8, the 14336 before them int4, all older ones
    2-bit (band_lengths).
  * aging: a block leaving the int4 band is re-quantized from its int4 values
    (the only form left), dequantized in float32 -- (code - zero) * scale is
    exact there -- then quantized to 2 bits (requantize_q4_to_q2).
  * storage layouts are this library's (the page packs only 4-bit codes):
      key row (32 B):   word 2g + h holds d = 64h + 16g + i, i = 4k + j, in
                        bits 8j + 2k .. 8j + 2k + 1;
      value row (32 B): 16-bit word m holds d = 64(s / 4) + 4m + s % 4 for
                        s = 0 .. 7 in bits 2s .. 2s + 1.
  * the variance-driven group size of Sec. 3.2 is not taken: its only formula
    is an example the page marks as not final, and the variance is computed
    but not used; groups stay at 64.

Pins (tests/test_oracle_kvq2.py):
  quantize_groups_q2    exact rational brute force; codes in [0, 3]; round
                        trip within half a step; constant groups exact.
  pack / unpack         round trips; single-code placement in both layouts.
  band_lengths          the page's edges (2048, 16384) at lengths around
                        them; the three bands add up to the length.
  requantize_q4_to_q2   int4 rows whose values lie on a 2-bit grid come back
                        as that grid; the error is within half a 2-bit step
                        of the int4 values.
  decode_attention_banded
                        with no 2-bit tokens it equals the int4 oracle's
                        mixed decode; on grid-exact values it equals library
                        attention; page-order invariance; empty contexts.
"""
from __future__ import annotations

import numpy as np

from . import kvq4, kvq8

HD = 128
GROUP = 64
QMAX = 3                 # 2^bits - 1 for bits = 2
WINDOW8 = 2048           # [P4] Sec. 3.3 schedule: newest tokens in int8
EDGE4 = 16384            # ... and int4 up to this distance from the newest
F32 = np.float32
F16 = np.float16


def band_lengths(L: int, window8: int = WINDOW8, edge4: int = EDGE4):
    """(n2, n4, n8): tokens of a length-L sequence in the 2-bit, int4 and
    int8 bands, oldest first."""
    L = max(int(L), 0)
    n8 = min(L, window8)
    n4 = min(max(L - window8, 0), edge4 - window8)
    return L - n4 - n8, n4, n8


def quantize_groups_q2(x):
    """Asymmetric 2-bit quantization of each 64-value group of a row ([P4]
    Sec. 3.2 with bits = 2; readings in the module header).

    x float32 [..., 128].  Returns (codes uint8 [..., 128] in [0, 3], scale
    float16 [..., 2], zero float16 [..., 2]); value = (code - zero) * scale."""
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] == HD
    g = x.reshape(x.shape[:-1] + (HD // GROUP, GROUP))
    mx = g.max(axis=-1)
    mn = g.min(axis=-1)
    s32 = ((mx - mn).astype(np.float32) / F32(QMAX)).astype(np.float32)
    s32 = np.where(mx == mn, F32(1.0), s32)
    s32 = np.maximum(s32, F32(1e-7)).astype(np.float32)
    s16 = s32.astype(F16)
    s = s16.astype(np.float32)
    z = (np.clip(np.rint((-mn / s).astype(np.float32)), 0, QMAX) + F32(0.0)).astype(np.float32)
    y = ((g / s[..., None]).astype(np.float32) + z[..., None]).astype(np.float32)
    c = np.clip(np.rint(y), 0, QMAX).astype(np.uint8)
    return c.reshape(x.shape), s16, z.astype(F16)


def dequantize_groups_q2(codes, scale, zero) -> np.ndarray:
    """(code - zero) * scale per group, float64."""
    return kvq4.dequantize_groups_q4(codes, scale, zero)


# ----------------------------------------------------------------------------
# storage layouts (four codes per byte)
# ----------------------------------------------------------------------------

def _k_bits():
    """Bit position of element d in a key row: d = 64h + 16g + 4k + j sits in
    word 2g + h at bit 8j + 2k."""
    d = np.arange(HD)
    h, g, i = d // 64, (d % 64) // 16, d % 16
    k, j = i // 4, i % 4
    return 32 * (2 * g + h) + 8 * j + 2 * k


def _v_bits():
    """Bit position of element d in a value row: d = 64(s / 4) + 4m + s % 4
    sits in 16-bit word m at bit 2s."""
    d = np.arange(HD)
    grp, m, r = d // 64, (d % 64) // 4, d % 4
    s = 4 * grp + r
    return 16 * m + 2 * s


def _pack(codes, bits) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    out = np.zeros(c.shape[:-1] + (HD // 4,), dtype=np.uint8)
    for d in range(HD):
        byte, sh = bits[d] // 8, bits[d] % 8
        out[..., byte] |= ((c[..., d] & 3) << sh).astype(np.uint8)
    return out


def _unpack(packed, bits) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (HD,), dtype=np.uint8)
    for d in range(HD):
        out[..., d] = (p[..., bits[d] // 8] >> (bits[d] % 8)) & 3
    return out


def pack_k2(codes):
    return _pack(codes, _k_bits())


def unpack_k2(packed):
    return _unpack(packed, _k_bits())


def pack_v2(codes):
    return _pack(codes, _v_bits())


def unpack_v2(packed):
    return _unpack(packed, _v_bits())


def kv_bytes_per_token_head() -> int:
    """Cache bytes of one (token, kv-head), K and V: 32 code bytes and two
    float16 (scale, zero) pairs each."""
    return 2 * (HD // 4 + 2 * 2 * 2)


# ----------------------------------------------------------------------------
# write paths
# ----------------------------------------------------------------------------

def quantize_append_q2(k_pool, v_pool, k_scale, k_zero, v_scale, v_zero, k_new, v_new, slots):
    """Quantize new rows into the 2-bit pool: packed codes [n_blocks][kv_bs]
    [nkv][32] uint8 (keys pack_k2, values pack_v2), scale and zero
    [n_blocks][kv_bs][nkv][2] float16.  Slots outside the pool are skipped;
    pools are modified in place."""
    kc, ks, kz = quantize_groups_q2(k_new)
    vc, vs, vz = quantize_groups_q2(v_new)
    nb, bs = k_pool.shape[:2]
    slots = np.asarray(slots, dtype=np.int64)
    ok = (slots >= 0) & (slots < nb * bs)
    for pool, val in ((k_pool, pack_k2(kc)), (v_pool, pack_v2(vc)),
                      (k_scale, ks), (k_zero, kz), (v_scale, vs), (v_zero, vz)):
        flat = pool.reshape((nb * bs,) + pool.shape[2:])
        flat[slots[ok]] = val[ok]
    return k_pool, v_pool, k_scale, k_zero, v_scale, v_zero


def dequantize_rows_q4_f32(codes, scale, zero) -> np.ndarray:
    """(code - zero) * scale in float32 (exact: an integer below 16 times a
    binary16 value)."""
    c = np.asarray(codes).astype(F32).reshape(np.shape(codes)[:-1] + (HD // GROUP, GROUP))
    z = np.asarray(zero).astype(F32)[..., None]
    s = np.asarray(scale).astype(F32)[..., None]
    return ((c - z) * s).astype(F32).reshape(np.shape(codes))


def requantize_q4_to_q2(q4_pools, q2_pools, src_slots, dst_slots):
    """Move tokens from the int4 pool to the 2-bit pool ([P4] Sec. 3.3: the
    oldest time block drops to fewer bits): pair i re-quantizes int4 slot
    src_slots[i] into 2-bit slot dst_slots[i]; pairs with either slot outside
    its pool are skipped.

    q4_pools = (k_packed, k_scale, k_zero, v_packed, v_scale, v_zero) as in
    kvq4; q2_pools the same for the 2-bit pool, modified in place."""
    k4, k4s, k4z, v4, v4s, v4z = q4_pools
    k2, k2s, k2z, v2, v2s, v2z = q2_pools
    nb4, bs = k4.shape[:2]
    nb2 = k2.shape[0]
    src = np.asarray(src_slots, dtype=np.int64)
    dst = np.asarray(dst_slots, dtype=np.int64)
    ok = (src >= 0) & (src < nb4 * bs) & (dst >= 0) & (dst < nb2 * bs)
    src, dst = src[ok], dst[ok]
    flat = lambda a: a.reshape((a.shape[0] * a.shape[1],) + a.shape[2:])  # noqa: E731
    xk = dequantize_rows_q4_f32(kvq4.unpack_nibbles(flat(k4)[src]), flat(k4s)[src], flat(k4z)[src])
    xv = dequantize_rows_q4_f32(kvq4.unpack_v4(flat(v4)[src]), flat(v4s)[src], flat(v4z)[src])
    quantize_append_q2(k2, v2, k2s, k2z, v2s, v2z, xk, xv, dst)
    return q2_pools


# ----------------------------------------------------------------------------
# decode attention over the three bands
# ----------------------------------------------------------------------------

def decode_attention_banded(q, q2_pools, bt2, lens2, q4_pools, bt4, lens4, q8_pools, bt8, lens8,
                            kv_bs: int, sm_scale: float):
    """Decode attention over a sequence split into a 2-bit band, an int4 band
    and an int8 window ([P4] Sec. 2.2 and 3.3).

    q2_pools / q4_pools = (k_packed, k_scale, k_zero, v_packed, v_scale,
    v_zero); q8_pools = (k_codes, k_step, v_codes, v_step).  Sequence b
    attends over lens2[b], lens4[b] and lens8[b] tokens of the three pools
    (positions 0.. via its block tables).  The query is quantized as in the
    int8 path; scores are sm_scale times the dot product of the dequantized
    query and key; softmax and the weighted sum of dequantized values in
    float64.  Returns float64 [B][nq][128] (zero rows for empty contexts)."""
    q = np.asarray(q, dtype=np.float32)
    B, nq, hd = q.shape
    k2, k2s, k2z, v2, v2s, v2z = q2_pools
    k4, k4s, k4z, v4, v4s, v4z = q4_pools
    k8, k8s, v8, v8s = q8_pools
    nkv = k2.shape[2]
    g = nq // nkv
    qi, qsc = kvq8.quantize_q_blocks(q)
    q_hat = kvq8.dequantize_q_blocks(qi, qsc)
    out = np.zeros((B, nq, hd), dtype=np.float64)
    for b in range(B):
        n2, n4, n8 = int(lens2[b]), int(lens4[b]), int(lens8[b])
        if n2 + n4 + n8 <= 0:
            continue
        for kh in range(nkv):
            Ks, Vs = [], []
            if n2 > 0:
                G = lambda pool: kvq8.gather_rows(pool, bt2[b], n2, kv_bs, kh)  # noqa: E731
                Ks.append(dequantize_groups_q2(unpack_k2(G(k2)), G(k2s), G(k2z)))
                Vs.append(dequantize_groups_q2(unpack_v2(G(v2)), G(v2s), G(v2z)))
            if n4 > 0:
                G = lambda pool: kvq8.gather_rows(pool, bt4[b], n4, kv_bs, kh)  # noqa: E731
                Ks.append(kvq4.dequantize_groups_q4(kvq4.unpack_nibbles(G(k4)), G(k4s), G(k4z)))
                Vs.append(kvq4.dequantize_groups_q4(kvq4.unpack_v4(G(v4)), G(v4s), G(v4z)))
            if n8 > 0:
                G = lambda pool: kvq8.gather_rows(pool, bt8[b], n8, kv_bs, kh)  # noqa: E731
                Ks.append(kvq8.dequantize_rows_q8(G(k8), G(k8s)))
                Vs.append(kvq8.dequantize_rows_q8(G(v8), G(v8s)))
            K = np.concatenate(Ks)
            V = np.concatenate(Vs)
            for h in range(kh * g, (kh + 1) * g):
                out[b, h] = kvq8.softmax_attention_f64(q_hat[b, h], K, V, sm_scale)
    return out
