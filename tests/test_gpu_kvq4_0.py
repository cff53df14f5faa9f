"""GPU parity of the Q4_0 mode against the CPU oracle, through the C ABI.

Bit-exact: packed codes and block steps of the write path.  Float outputs:
|gpu - oracle| <= 1e-4 + 1e-4 |oracle| elementwise.  Sizes span several
tiles and chunks with ragged tails, GQA groups 1-8 and block sizes 8-128.
"""
import numpy as np
import pytest

import workloads as W
from oracle import kvq4_0 as Q, kvq8 as O8
from tests.helpers import SM, assert_attn_close, dev, head_major, host, slot_major

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


@pytest.fixture(scope="module")
def K():
    import decode_attention_int8_amd as K
    return K


class Q40Cache:
    """A Q4_0 paged cache held both on the host (oracle) and on the GPU."""

    def __init__(self, n_blocks, kv_bs, nkv):
        import torch
        self.kv_bs, self.nkv = kv_bs, nkv
        shp, gshp = (n_blocks, kv_bs, nkv), (n_blocks, nkv, kv_bs)   # oracle slot-major, device head-major
        self.kp = np.zeros(shp + (64,), np.uint8)
        self.vp = np.zeros(shp + (64,), np.uint8)
        self.ks = np.zeros(shp + (4,), np.float32)
        self.vs = np.zeros(shp + (4,), np.float32)
        self.gk = torch.zeros(gshp + (64,), dtype=torch.uint8, device="cuda")
        self.gv = torch.zeros(gshp + (64,), dtype=torch.uint8, device="cuda")
        self.gks = torch.zeros(gshp + (4,), dtype=torch.float32, device="cuda")
        self.gvs = torch.zeros(gshp + (4,), dtype=torch.float32, device="cuda")

    def device_expect(self):
        """The oracle's pool in the device's order (k, v, k_step, v_step)."""
        return [head_major(x) for x in (self.kp, self.vp, self.ks, self.vs)]

    def append(self, k_new, v_new, slots, gk_new=None, gv_new=None):
        import decode_attention_int8_amd as K
        Q.quantize_append_q4_0(self.kp, self.vp, self.ks, self.vs, k_new, v_new, slots)
        K.kvq4_0_quantize_append(self.gk, self.gv, self.gks, self.gvs,
                                 dev(k_new) if gk_new is None else gk_new,
                                 dev(v_new) if gv_new is None else gv_new, dev(np.asarray(slots, np.int32)))

    def assert_device_matches_host(self):
        assert np.array_equal(slot_major(host(self.gk)), self.kp), "K codes differ"
        assert np.array_equal(slot_major(host(self.gv)), self.vp), "V codes differ"
        assert np.array_equal(slot_major(host(self.gks)).view(np.uint32), self.ks.view(np.uint32)), "K steps differ"
        assert np.array_equal(slot_major(host(self.gvs)).view(np.uint32), self.vs.view(np.uint32)), "V steps differ"


def _fill(cache, bt, lens, k, v):
    for b, L in enumerate(lens):
        if L == 0:
            continue
        sl = W.slots_for_positions(bt, [b] * L, np.arange(L), cache.kv_bs)
        cache.append(np.ascontiguousarray(k[b, :L]), np.ascontiguousarray(v[b, :L]), sl)


def _decode(K, c, q, bt, lens, max_len, chunk=0):
    torch = _torch()
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    K.kvq4_0_decode_attn(out, dev(q), c.gk, c.gv, c.gks, c.gvs, dev(bt), dev(lens), max_len, SM, chunk=chunk)
    torch.cuda.synchronize()
    return host(out)


def _ref(q, c, bt, lens):
    return Q.decode_attention_q4_0(q, c.kp, c.ks, c.vp, c.vs, bt, lens, c.kv_bs, SM)


# ----------------------------------------------------------------------------
# write path
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_quantize_append_bit_exact(K, dtype):
    torch = _torch()
    r = W.rng(500, ["f32", "bf16", "f16"].index(dtype))
    n, nkv, bs, nb = 777, 4, 16, 64
    x = np.concatenate([W.normal_f32(r, (n // 2, nkv, 128)),
                        W.student_t3_f32(r, (n - n // 2, nkv, 128), 0.5)]).astype(np.float32)
    y = W.outlier_normal_bf16(r, (n, nkv, 128))
    x[3, 1] = 0.0                                   # zero row: steps +0, codes 8
    x[4, 0, 32:64] = -0.0
    x[5, 0, :] = 2.5                                # constant row (positive extreme)
    x[6, 2, :] = 0.25
    x[6, 2, 3], x[6, 2, 17] = 8.0, -8.0             # sign tie: the negative extreme
    x[6, 2, 4], x[6, 2, 5] = 0.5, -0.5              # exact midpoints
    x[7, 3, 64:96] = np.linspace(-1, 3, 32, dtype=np.float32)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    gx, gy = dev(x).to(tdt), dev(y).to(tdt)
    xh = gx.float().cpu().numpy()                   # exact values the kernel sees
    yh = gy.float().cpu().numpy()
    slots = r.permutation(nb * bs)[:n].astype(np.int32)
    slots[10] = -1                                  # padding token: skipped
    slots[11] = nb * bs + 5                         # out of the pool: skipped
    c = Q40Cache(nb, bs, nkv)
    c.append(xh, yh, slots, gx, gy)
    torch.cuda.synchronize()
    c.assert_device_matches_host()


def test_quantize_append_large_and_overwrite(K):
    torch = _torch()
    r = W.rng(501)
    n, nkv, bs, nb = 20011, 8, 16, 1400
    x = W.normal_f32(r, (n, nkv, 128))
    slots = r.permutation(nb * bs)[:n].astype(np.int32)
    c = Q40Cache(nb, bs, nkv)
    c.append(x, x[::-1].copy(), slots)
    b = W.normal_f32(r, (3, nkv, 128), 9.0)
    c.append(b[:2], b[:2], slots[[5, 7]])           # rewrite two slots
    c.append(b[2:], b[2:], slots[[5]])              # and one again: the later call wins
    K.kvq4_0_quantize_append(c.gk, c.gv, c.gks, c.gvs, dev(b[:0]), dev(b[:0]), dev(np.zeros(0, np.int32)))
    torch.cuda.synchronize()
    c.assert_device_matches_host()


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("g", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("bs", [8, 16, 128])
def test_decode_ragged_batch(K, g, bs):
    r = W.rng(510, g, bs)
    nkv = 2 if g < 8 else 1
    nq = g * nkv
    lens = np.array([1, 63, 64, 65, 300, 1025, 0, 2049], np.int32)
    B, Lm = len(lens), int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, bs, spare_blocks=2)
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    v = W.student_t3_f32(r, (B, Lm, nkv, 128), 0.5)
    c = Q40Cache(nb, bs, nkv)
    _fill(c, bt, lens, k, v)
    q = W.normal_f32(r, (B, nq, 128), 2.0)
    got = _decode(K, c, q, bt, lens, Lm)
    assert_attn_close(got, _ref(q, c, bt, lens), f"g={g} bs={bs}")
    assert np.all(got[6] == 0.0)                          # empty context


@pytest.mark.parametrize("chunk", [256, 512, 2048, 16384])
def test_decode_chunk_sizes_agree(K, chunk):
    r = W.rng(511, chunk)
    nq, nkv, bs = 8, 2, 16
    lens = np.array([5000, 257, 4096], np.int32)
    B, Lm = len(lens), int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, bs)
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    v = W.per_unit_sigma_normal(r, (B, Lm, nkv, 128), 1, 0.2, 5.0)
    c = Q40Cache(nb, bs, nkv)
    _fill(c, bt, lens, k, v)
    q = W.normal_f32(r, (B, nq, 128), 3.0)
    assert_attn_close(_decode(K, c, q, bt, lens, Lm, chunk=chunk), _ref(q, c, bt, lens), f"chunk {chunk}")


def test_decode_single_token_and_peaked_softmax(K):
    r = W.rng(512)
    nq, nkv, bs = 4, 1, 16
    lens = np.array([1, 500], np.int32)
    bt, nb = W.paged_block_tables(r, lens, bs)
    k = W.normal_f32(r, (2, 500, nkv, 128))
    v = W.normal_f32(r, (2, 500, nkv, 128))
    c = Q40Cache(nb, bs, nkv)
    _fill(c, bt, lens, k, v)
    q = W.normal_f32(r, (2, nq, 128))
    q[1, 0] = k[1, 321, 0] * 30.0                   # one dominant token
    got = _decode(K, c, q, bt, lens, 500)
    assert_attn_close(got, _ref(q, c, bt, lens), "single / peaked")
    # L = 1: the dequantized value row itself (weight 1)
    row = Q.dequantize_blocks_q4_0(Q.unpack_v(c.vp[bt[0, 0], 0, 0]), c.vs[bt[0, 0], 0, 0])
    np.testing.assert_allclose(got[0], np.repeat(row[None], nq, 0), rtol=1e-6, atol=1e-7)


def test_decode_clamps_lengths_and_skips_bad_blocks(K):
    r = W.rng(513)
    nq, nkv, bs = 4, 2, 16
    lens = np.array([100, 100, 100], np.int32)
    bt, nb = W.paged_block_tables(r, lens, bs)
    k = W.normal_f32(r, (3, 100, nkv, 128))
    c = Q40Cache(nb, bs, nkv)
    _fill(c, bt, lens, k, k)
    q = W.normal_f32(r, (3, nq, 128))
    glens = np.array([100, 100 + 1000, -5], np.int32)      # beyond max_ctx / negative
    bt_bad = bt.copy()
    bt_bad[0, 2] = nb + 100                               # block id outside the pool
    got = _decode(K, c, q, bt_bad, glens, 100)
    keep = np.r_[0:32, 48:100]                            # tokens of block index 2 are skipped
    qi, qsc = O8.quantize_q_blocks(q[0])
    q_hat = O8.dequantize_q_blocks(qi, qsc)
    ref0 = []
    for h in range(nq):
        G = lambda pool: O8.gather_rows(pool, bt[0], 100, bs, h // 2)  # noqa: E731
        Kd = Q.dequantize_blocks_q4_0(Q.unpack_k(G(c.kp)), G(c.ks))[keep]
        Vd = Q.dequantize_blocks_q4_0(Q.unpack_v(G(c.vp)), G(c.vs))[keep]
        ref0.append(O8.softmax_attention_f64(q_hat[h], Kd, Vd, SM))
    assert_attn_close(got[0], np.stack(ref0), "bad block skipped")
    assert_attn_close(got[1:2], _ref(q[1:2], c, bt[1:2], [100]), "length clamped to max_ctx")
    assert np.all(got[2] == 0.0)


def test_decode_8k_layer_and_long_batch(K):
    """The 8K-token batch-1 layer shape (16 / 8 heads) and a batch of long
    contexts (32 / 8 heads), full outputs against the oracle."""
    r = W.rng(514)
    for B, nq, nkv, lens in [(1, 16, 8, np.array([8192], np.int32)),
                             (4, 32, 8, W.uniform_lengths(r, 4, 1024, 32768).astype(np.int32))]:
        bs = 16
        Lm = int(lens.max())
        bt, nb = W.paged_block_tables(r, lens, bs)
        k = W.student_t3_f32(r, (B, Lm, nkv, 128), 0.5)
        v = W.student_t3_f32(r, (B, Lm, nkv, 128), 0.5)
        c = Q40Cache(nb, bs, nkv)
        _fill(c, bt, lens, k, v)
        q = W.normal_f32(r, (B, nq, 128))
        assert_attn_close(_decode(K, c, q, bt, lens, Lm), _ref(q, c, bt, lens), f"B={B} nq={nq}")
