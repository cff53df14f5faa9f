"""Write paths on rows built to put x / step on or next to half-integers.

Every quantizer rounds the quotient of a value by its row's (block's,
group's) step to an integer; the kernels take the product with a reciprocal
and divide only where that product is near a half-integer.  These rows put
the quotient exactly on half-integers (steps that are powers of two), one ulp
beside them, and within a few ulps of them for steps that are not, so that
both the fast path and the division are exercised.  Codes and steps are
compared bit for bit with the oracle.
"""
import numpy as np
import pytest

import workloads as W
from oracle import kvq8 as O8
from tests.helpers import Q8Cache, dev, host
from tests.test_gpu_kvq4 import Q4Pool
from tests.test_gpu_kvq4_0 import Q40Cache

pytestmark = pytest.mark.gpu

F32 = np.float32


def _ulp_neighbours(v, r):
    """v, or one of its float32 neighbours, chosen per element."""
    v = np.asarray(v, F32)
    pick = r.integers(0, 3, size=v.shape)
    up = np.nextafter(v, F32(np.inf))
    dn = np.nextafter(v, F32(-np.inf))
    return np.where(pick == 0, v, np.where(pick == 1, up, dn)).astype(F32)


def _int8_rows(r, n):
    """Rows of 128 values whose quotients by the row step (max |x| / 127) lie
    on or beside half-integers."""
    rows = []
    k = np.arange(-63, 64, dtype=F32)[:127]                     # 127 half-integers k + 0.5
    for i in range(n):
        kind = i % 4
        if kind == 0:        # step exactly a power of two: quotients exactly k + 0.5
            step = F32(2.0) ** int(r.integers(-12, 3))
            x = (k + F32(0.5)) * step
        elif kind == 1:      # the same, one ulp beside
            step = F32(2.0) ** int(r.integers(-12, 3))
            x = _ulp_neighbours((k + F32(0.5)) * step, r)
        else:                # a step that is not a power of two: within a few ulps of k + 0.5
            amax = F32(r.uniform(0.1, 50.0))
            step = F32(amax / F32(127.0))
            x = _ulp_neighbours(((k + F32(0.5)) * step).astype(F32), r)
        x = np.clip(x, -F32(126.9) * step, F32(126.9) * step)
        row = np.concatenate([[F32(127.0) * step], x]).astype(F32)  # the row maximum gives the step
        rows.append(r.permutation(row) * (F32(-1.0) if r.integers(0, 2) else F32(1.0)))
    return np.stack(rows).astype(F32)


def test_int8_write_ties():
    import torch
    r = W.rng(600)
    n, nkv, bs, nb = 96, 4, 16, 8
    x = _int8_rows(r, n * nkv).reshape(n, nkv, 128)
    y = _int8_rows(r, n * nkv).reshape(n, nkv, 128)
    c = Q8Cache(nb, bs, nkv)
    c.append(x, y, r.permutation(nb * bs)[:n].astype(np.int32))
    torch.cuda.synchronize()
    c.assert_device_matches_host()


def test_int8_fused_write_ties():
    """The fused write path of the decode (its own quantizer layout) on the
    same rows: cache bytes equal the oracle's."""
    import torch
    import decode_attention_int8_amd as K
    r = W.rng(601)
    B, nkv, bs, nq = 64, 2, 16, 4
    lens = r.integers(1, 200, size=B).astype(np.int32)
    bt, nb = W.paged_block_tables(r, lens, bs)
    c = Q8Cache(nb, bs, nkv)
    kn = _int8_rows(r, B * nkv).reshape(B, nkv, 128)
    vn = _int8_rows(r, B * nkv).reshape(B, nkv, 128)
    sl = np.array([bt[b, (lens[b] - 1) // bs] * bs + (lens[b] - 1) % bs for b in range(B)], np.int32)
    q = W.normal_f32(r, (B, nq, 128))
    out = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq8_append_decode_attn(out, dev(q), dev(kn), dev(vn), c.gk, c.gv, c.gks, c.gvs, dev(bt), dev(lens),
                              int(lens.max()))
    torch.cuda.synchronize()
    O8.quantize_append(c.kp, c.vp, c.ks, c.vs, kn, vn, sl)
    c.assert_device_matches_host()


def _q40_rows(r, n):
    """Rows of four 32-value blocks whose quotients by the block step
    (extreme / -8) lie on or beside half-integers."""
    k = np.arange(-8, 8, dtype=F32)                              # codes 0 .. 15 around k + 0.5
    out = np.empty((n, 128), F32)
    for i in range(n):
        for b in range(4):
            kind = (i + b) % 3
            if kind == 0:
                step = F32(2.0) ** int(r.integers(-10, 3))
                v = (k + F32(0.5)) * step
            elif kind == 1:
                step = F32(2.0) ** int(r.integers(-10, 3))
                v = _ulp_neighbours((k + F32(0.5)) * step, r)
            else:
                step = F32(F32(-r.uniform(0.2, 9.0)) * F32(-0.125))
                v = _ulp_neighbours(((k + F32(0.5)) * step).astype(F32), r)
            v = np.clip(v, F32(-7.99) * step, F32(7.99) * step)
            blk = np.concatenate([[F32(-8.0) * step], v, r.choice(v, 15)]).astype(F32)   # extreme -8 step
            out[i, 32 * b:32 * b + 32] = r.permutation(blk)
    return out


def test_q40_write_ties():
    import torch
    import decode_attention_int8_amd as K  # noqa: F401  (loads the library for the cache helper)
    r = W.rng(602)
    n, nkv, bs, nb = 64, 4, 16, 8
    x = _q40_rows(r, n * nkv).reshape(n, nkv, 128)
    y = _q40_rows(r, n * nkv).reshape(n, nkv, 128)
    c = Q40Cache(nb, bs, nkv)
    c.append(x, y, r.permutation(nb * bs)[:n].astype(np.int32))
    torch.cuda.synchronize()
    c.assert_device_matches_host()


def _q4_rows(r, n):
    """Rows of two 64-value groups whose quotients by the group scale lie on
    or beside half-integers: min and max chosen so that (max - min) / 15 is
    exact in binary16, or not."""
    out = np.empty((n, 128), F32)
    for i in range(n):
        for g in range(2):
            kind = (i + g) % 3
            if kind < 2:
                s = F32(2.0) ** int(r.integers(-6, 2))
                z0 = int(r.integers(0, 16))                       # min = -z0 s - s/2 .. max = min + 15 s
            else:
                s = F32(np.float16(r.uniform(0.05, 3.0)))
                z0 = int(r.integers(0, 16))
            mn = F32(-(z0 + 0.5)) * s
            mx = F32(mn + F32(15.0) * s)
            half = (np.arange(-z0 - 1, 15 - z0, dtype=F32) + F32(0.5)) * s   # x / s = k + 0.5 in [min, max]
            v = half if kind == 0 else _ulp_neighbours(half, r)
            v = np.clip(v, mn, mx)
            grp = np.concatenate([[mn, mx], v, r.choice(v, 64 - 2 - len(v))]).astype(F32)
            out[i, 64 * g:64 * g + 64] = r.permutation(grp)
    return out


def test_q4_write_ties():
    import torch
    import decode_attention_int8_amd as K
    r = W.rng(603)
    n, nkv, bs, nb = 64, 4, 16, 8
    x = _q4_rows(r, n * nkv).reshape(n, nkv, 128)
    y = _q4_rows(r, n * nkv).reshape(n, nkv, 128)
    p = Q4Pool(nb, bs, nkv)
    p.append(K, x, y, r.permutation(nb * bs)[:n].astype(np.int32))
    torch.cuda.synchronize()
    p.assert_same()


@pytest.mark.parametrize("nkv", [1, 3, 5, 6, 12])
def test_write_paths_head_counts(nkv):
    """Every write path (int8, Q4_0, int4, int8 -> int4 re-quantization) with
    head counts that are not powers of two: the row index is divided by the
    head count with a multiply and a shift."""
    import torch
    import decode_attention_int8_amd as K
    from oracle import kvq4 as O4
    r = W.rng(604, nkv)
    n, bs = 203, 16
    nb = (2 * n) // bs + 2
    x = W.normal_f32(r, (n, nkv, 128))
    y = W.student_t3_f32(r, (n, nkv, 128), 0.5)
    slots = r.permutation(nb * bs)[:n].astype(np.int32)
    slots[5] = -1
    c8 = Q8Cache(nb, bs, nkv)
    c8.append(x, y, slots)
    c40 = Q40Cache(nb, bs, nkv)
    c40.append(x, y, slots)
    p4 = Q4Pool(nb, bs, nkv)
    p4.append(K, x, y, slots)
    # re-quantize the int8 rows of some tokens into other int4 slots
    src = slots[:100].copy()
    dst = r.permutation(nb * bs)[:100].astype(np.int32)
    O4.requantize_q8_to_q4((c8.kp, c8.ks, c8.vp, c8.vs), p4.oracle_pools(), src, dst)
    K.kvq4_requantize_q8(p4.g, (c8.gk, c8.gv, c8.gks, c8.gvs), dev(src), dev(dst))
    torch.cuda.synchronize()
    c8.assert_device_matches_host()
    c40.assert_device_matches_host()
    p4.assert_same()


def _query_rows(r, n):
    """Query rows whose 32-blocks put q * (127 / qm) on or beside
    half-integers: qm = 127 * 2^k makes the multiplier 2^-k exact, so
    (j + 1/2) 2^k lands exactly on j + 1/2; other blocks sit one ulp beside
    such values, or within a few ulps of them for a multiplier that is not a
    power of two."""
    out = np.empty((n, 128), F32)
    j = np.arange(-126, 126, dtype=F32)
    for i in range(n):
        for b in range(4):
            kind = (i + b) % 3
            if kind < 2:
                unit = F32(2.0) ** int(r.integers(-8, 4))
                vals = (r.choice(j, 31) + F32(0.5)) * unit
                if kind == 1:
                    vals = _ulp_neighbours(vals, r)
            else:
                unit = F32(F32(r.uniform(0.05, 20.0)) / F32(127.0))
                vals = _ulp_neighbours(((r.choice(j, 31) + F32(0.5)) * unit).astype(F32), r)
            vals = np.clip(vals, F32(-126.9) * unit, F32(126.9) * unit)
            blk = np.concatenate([[F32(127.0) * unit * (F32(-1.0) if r.integers(0, 2) else F32(1.0))], vals])
            out[i, 32 * b:32 * b + 32] = r.permutation(blk.astype(F32))
    return out


def test_query_ties_codes_partials_and_decode():
    """The query quantizer on rows with exact half-integer products (ties away
    from zero): the exported codes and scales, the decode's int32 block dots
    and the decode output all follow the oracle."""
    import torch
    import decode_attention_int8_amd as K
    from tests.helpers import SM, assert_attn_close, fill_sequences
    r = W.rng(605)
    q = _query_rows(r, 240)
    qi = torch.empty((len(q), 128), dtype=torch.int8, device="cuda")
    qs = torch.empty((len(q), 4), dtype=torch.float32, device="cuda")
    K.kvq8_quantize_q(qi, qs, dev(q))
    want_i, want_s = O8.quantize_q_blocks(q)
    # the rows do hold exact ties, and at least one where rounding half to even differs
    y = q.reshape(-1, 4, 32) * (F32(127.0) / np.abs(q.reshape(-1, 4, 32)).max(-1, keepdims=True))
    assert np.sum(np.abs(y - np.floor(y)) == 0.5) > 1000
    assert np.any(np.rint(y).astype(np.int64) != want_i.reshape(-1, 4, 32))
    assert np.array_equal(host(qi), want_i)
    assert np.array_equal(host(qs).view(np.uint32), want_s.view(np.uint32))

    B, nkv, nq, bs = 6, 2, 8, 16
    lens = np.array([1, 300, 64, 777, 5, 256], np.int32)
    Lm = int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, bs)
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    v = W.normal_f32(r, (B, Lm, nkv, 128))
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, lens, k, v)
    qd = q[:B * nq].reshape(B, nq, 128)
    part = torch.full((B, nq, Lm, 4), -7, dtype=torch.int32, device="cuda")
    K.kvq8_qk_partials(part, dev(qd), c.gk, dev(bt), dev(lens), Lm)
    out = torch.empty((B, nq, 128), dtype=torch.float32, device="cuda")
    K.kvq8_decode_attn(out, dev(qd), c.gk, c.gv, c.gks, c.gvs, dev(bt), dev(lens), Lm, SM)
    torch.cuda.synchronize()
    got = host(part)
    qiq, _ = O8.quantize_q_blocks(qd)
    for b in range(B):
        for h in range(nq):
            rows = O8.gather_rows(c.kp, bt[b], lens[b], bs, h // (nq // nkv))
            assert np.array_equal(got[b, h, :lens[b]], O8.qk_block_partials(qiq[b, h], rows)), (b, h)
    ref = O8.decode_attention_q8(qd, c.kp, c.ks, c.vp, c.vs, bt, lens, bs, SM)
    assert_attn_close(host(out), ref, "tie queries")
