"""The head-major pools (int4, 2-bit, Q4_0: slot s of kv-head kh at row
(s / kv_bs * nkv + kh) * kv_bs + s % kv_bs) through their decodes with
kv-head counts that are not powers of two and both tile forms (kv_bs 8: a
16-token group spans two blocks; kv_bs 16: one).  Every pool is written by
the library and compared with the oracle's bit for bit; outputs within
1e-4 + 1e-4 |oracle|."""
import numpy as np
import pytest

import workloads as W
from oracle import kvq4 as O4
from oracle import kvq4_0 as O40
from tests.helpers import SM, Q8Cache, assert_attn_close, dev, host
from tests.test_gpu_kvq2 import _banded, _decode_and_check
from tests.test_gpu_kvq4 import Q4Pool
from tests.test_gpu_kvq4_0 import Q40Cache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import decode_attention_int8_amd as K
    return K


def _fill(r, pool_append, lens, bt, bs, nkv):
    for b, L in enumerate(lens):
        if L:
            k = W.per_unit_sigma_normal(r, (int(L), nkv, 128), 0, 0.5, 2.0)
            pool_append(k, W.normal_f32(r, k.shape), W.slots_for_positions(bt, [b] * L, np.arange(L), bs))


@pytest.mark.parametrize("nkv", [3, 5])
@pytest.mark.parametrize("bs", [8, 16])
def test_int4_decode_odd_head_counts(K, nkv, bs):
    import torch
    r = W.rng(970, nkv, bs)
    g = 2
    nq = g * nkv
    lens4 = np.array([333, 0, 70, 1029], np.int32)
    lens8 = np.array([17, 64, 0, 200], np.int32)
    bt4, nb4 = W.paged_block_tables(r, lens4, bs, spare_blocks=1)
    bt8, nb8 = W.paged_block_tables(r, lens8, bs, spare_blocks=1)
    p4, c8 = Q4Pool(nb4, bs, nkv), Q8Cache(nb8, bs, nkv)
    _fill(r, lambda k, v, s: p4.append(K, k, v, s), lens4, bt4, bs, nkv)
    _fill(r, c8.append, lens8, bt8, bs, nkv)
    q = W.normal_f32(r, (len(lens4), nq, 128), 2.0)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    K.kvq4_decode_attn(out, dev(q), p4.g, dev(bt4), dev(lens4), int(lens4.max()),
                       (c8.gk, c8.gv, c8.gks, c8.gvs), dev(bt8), dev(lens8), int(lens8.max()), SM)
    torch.cuda.synchronize()
    p4.assert_same()
    ref = O4.decode_attention_mixed(q, p4.oracle_pools(), bt4, lens4, (c8.kp, c8.ks, c8.vp, c8.vs), bt8, lens8,
                                    bs, SM)
    assert_attn_close(host(out), ref, f"int4 nkv={nkv} bs={bs}")


@pytest.mark.parametrize("nkv", [3, 5])
@pytest.mark.parametrize("bs", [8, 16])
def test_banded_decode_odd_head_counts(K, nkv, bs):
    r = W.rng(971, nkv, bs)
    nq = 2 * nkv
    lens2 = np.array([900, 1, 0, 257], np.int32)
    lens4 = np.array([100, 0, 33, 64], np.int32)
    lens8 = np.array([5, 80, 0, 1], np.int32)
    bands = _banded(K, r, lens2, lens4, lens8, nq, nkv, bs)
    bands[0][0].assert_same("2-bit fill")
    bands[1][0].assert_same()
    q = W.normal_f32(r, (len(lens2), nq, 128), 2.0)
    got, ref = _decode_and_check(K, q, bands, (lens2, lens4, lens8), "odd heads")
    assert_attn_close(got, ref, f"banded nkv={nkv} bs={bs}")


@pytest.mark.parametrize("nkv", [3, 5])
@pytest.mark.parametrize("bs", [8, 16])
def test_q40_decode_odd_head_counts(K, nkv, bs):
    import torch
    r = W.rng(972, nkv, bs)
    nq = 2 * nkv
    lens = np.array([515, 0, 64, 1200], np.int32)
    bt, nb = W.paged_block_tables(r, lens, bs, spare_blocks=1)
    c = Q40Cache(nb, bs, nkv)
    _fill(r, c.append, lens, bt, bs, nkv)
    q = W.normal_f32(r, (len(lens), nq, 128), 2.0)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    K.kvq4_0_decode_attn(out, dev(q), c.gk, c.gv, c.gks, c.gvs, dev(bt), dev(lens), int(lens.max()), SM)
    torch.cuda.synchronize()
    c.assert_device_matches_host()
    ref = O40.decode_attention_q4_0(q, c.kp, c.ks, c.vp, c.vs, bt, lens, bs, SM)
    assert_attn_close(host(out), ref, f"Q4_0 nkv={nkv} bs={bs}")
