"""kvq8_decode_attn_noalloc: the int8 decode without a caller workspace (its
chunk partials live in the library's own device array).  Called through the
C ABI, it must give exactly what kvq8_decode_attn gives with a workspace, on
consecutive calls that share that array, the second with a smaller input."""
import numpy as np
import pytest

import workloads as W
from oracle import kvq8 as O8
from tests.helpers import SM, Q8Cache, assert_attn_close, dev, fill_sequences, host

pytestmark = pytest.mark.gpu


def _case(seed, lens, nq, nkv, bs):
    r = W.rng(900, seed)
    lens = np.asarray(lens, np.int32)
    B, Lm = len(lens), int(lens.max())
    bt, nb = W.paged_block_tables(r, lens, bs, spare_blocks=2)
    k = W.normal_f32(r, (B, Lm, nkv, 128))
    v = W.student_t3_f32(r, (B, Lm, nkv, 128), 0.5)
    c = Q8Cache(nb, bs, nkv)
    fill_sequences(c, bt, lens, k, v)
    q = W.normal_f32(r, (B, nq, 128))
    return c, q, bt, lens


def _both(K, c, q, bt, lens, chunk):
    import torch
    Lm = int(lens.max())
    qd, btd, ld = dev(q), dev(bt), dev(lens)
    want = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    K.kvq8_decode_attn(want, qd, c.gk, c.gv, c.gks, c.gvs, btd, ld, Lm, SM, chunk=chunk)
    K.kvq8_decode_attn_noalloc(got, qd, c.gk, c.gv, c.gks, c.gvs, btd, ld, Lm, SM, chunk=chunk)
    torch.cuda.synchronize()
    return host(got), host(want)


@pytest.mark.parametrize("chunk", [0, 256])
def test_noalloc_equals_workspace_decode_on_consecutive_calls(chunk):
    import decode_attention_int8_amd as K
    big = _case(1, [5000, 1, 0, 3333, 2048, 777], 16, 4, 16)
    small = _case(2, [300, 65], 8, 2, 8)
    for c, q, bt, lens in (big, small):
        got, want = _both(K, c, q, bt, lens, chunk)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        ref = O8.decode_attention_q8(q, c.kp, c.ks, c.vp, c.vs, bt, lens, c.kv_bs, SM)
        assert_attn_close(got, ref, f"noalloc chunk={chunk} B={len(lens)}")
