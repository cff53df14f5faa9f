"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and its host-side validation and sizing behave as the
header documents.  No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

from decode_attention_int8_amd import kvq8 as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq8.h")
OK, EINVAL, ESHAPE, EWORKSPACE, EHIP = 0, -1, -2, -3, -4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kvq[248]_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 24, names
    lib = K.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in K._SIGNATURES, f"binding lacks {n}"


def test_status_strings_and_version():
    assert K.kvq8_status_string(OK) == "ok"
    for st in (EINVAL, ESHAPE, EWORKSPACE, EHIP):
        assert K.kvq8_status_string(st) not in ("ok", "unknown status")
    assert K.kvq8_status_string(7) == "unknown status"
    assert "gfx950" in K.kvq8_version()


def _fake(addr=4096):
    """An aligned non-null address; validation never dereferences it."""
    return ctypes.c_void_p(addr)


def _decode(**kw):
    a = dict(out=_fake(), q=_fake(), batch=2, nq=16, kc=_fake(), vc=_fake(), ks=_fake(), vs=_fake(), n_blocks=64,
             kv_bs=16, nkv=8, hd=128, bt=_fake(), mb=32, lens=_fake(), max_ctx=512, sm=0.088, chunk=0,
             ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return K.lib().kvq8_decode_attn(*a.values())


def test_decode_validation():
    assert _decode(hd=64) == ESHAPE
    assert _decode(nq=12, nkv=8) == ESHAPE            # not a multiple
    assert _decode(nq=72, nkv=8) == ESHAPE            # group of 9
    assert _decode(kv_bs=12) == ESHAPE
    assert _decode(kv_bs=4) == ESHAPE
    assert _decode(kv_bs=2048) == ESHAPE
    assert _decode(chunk=100) == ESHAPE
    assert _decode(max_ctx=-1) == EINVAL
    assert _decode(q=None) == EINVAL
    assert _decode(q=_fake(4100)) == EINVAL           # misaligned
    assert _decode() == EWORKSPACE                    # missing workspace
    need = K.kvq8_decode_workspace_size(2, 16, 8, 512, 0)
    assert _decode(ws=_fake(), ws_bytes=need - 1) == EWORKSPACE
    assert _decode(batch=0) == OK                     # nothing to do


def test_decode_score_scale_argument():
    """sm_scale: a NaN or infinite value is rejected before anything runs;
    0 and negative values select the library's default 1 / sqrt(hd) and pass
    validation (here they stop at the missing workspace)."""
    for bad in (float("nan"), float("inf"), float("-inf")):
        assert _decode(sm=bad) == EINVAL
    for ok in (0.0, -1.0, 0.088, 3.0):
        assert _decode(sm=ok) == EWORKSPACE
    # the binding passes 0 for "no scale given": the default is the library's
    assert K._scale(None) == 0.0 and K._scale(0.5) == 0.5


def test_write_validation():
    lib = K.lib()
    args = [_fake(), _fake(), _fake(), _fake(), 64, 16, 8, 128, _fake(), _fake(), K.F32, 10, _fake(), None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.kvq8_quantize_append(*a)
    assert call(a7=96) == ESHAPE
    assert call(a5=24) == ESHAPE
    assert call(a10=5) == EINVAL
    assert call(a11=-1) == EINVAL
    assert call(a11=0) == OK
    assert call(a12=None) == EINVAL
    assert call(a8=_fake(4104)) == EINVAL
    assert lib.kvq4_quantize_append(_fake(), _fake(), _fake(), _fake(), _fake(), _fake(), 64, 16, 8, 128,
                                    _fake(), _fake(), K.BF16, 0, _fake(), None) == OK
    assert lib.kvq4_quantize_append(_fake(), _fake(), _fake(), _fake(), _fake(), _fake(), 64, 16, 8, 100,
                                    _fake(), _fake(), K.BF16, 3, _fake(), None) == ESHAPE


def test_chunk_and_workspace_sizing():
    # one-CU-per-chunk latency case: 8 kv-heads x 8K tokens
    assert K.kvq8_decode_chunk_tokens(1, 8, 8192) == 256
    # long batched contexts grow the chunk, capped at 8 tiles per wave
    c = K.kvq8_decode_chunk_tokens(32, 8, 32768)
    assert c % 256 == 0 and 256 < c <= 2048
    for B, nq, nkv, L, ch in [(1, 16, 8, 8192, 0), (32, 32, 8, 32768, 0), (3, 8, 2, 1000, 512), (1, 1, 1, 0, 0)]:
        chunk = ch or K.kvq8_decode_chunk_tokens(B, nkv, L)
        n = B * nq * -(-L // chunk)
        want = -(-n * 128 * 4 // 256) * 256 + 2 * (-(-n * 4 // 256) * 256)
        assert K.kvq8_decode_workspace_size(B, nq, nkv, L, ch) == want
    assert K.kvq8_decode_workspace_size(1, 16, 8, 100, 300) == 0        # bad chunk
    n4 = K.kvq4_decode_workspace_size(4, 32, 4, 129024, 2048, 1024)
    chunks = -(-129024 // 1024) + 2
    assert n4 == -(-4 * 32 * chunks * 512 // 256) * 256 + 2 * (-(-4 * 32 * chunks * 4 // 256) * 256)


def test_binding_requires_gpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros((4, 16, 2, 128), dtype=torch.int8)
    s = torch.zeros((4, 16, 2), dtype=torch.float32)
    kn = torch.zeros((3, 2, 128), dtype=torch.float32)
    with pytest.raises(ValueError):
        K.kvq8_quantize_append(x, x, s, s, kn, kn, torch.zeros(3, dtype=torch.int32))


def test_binding_checks_every_buffer_shape():
    """The C entry points see one set of sizes (taken from the key cache);
    every other buffer is checked against them in the binding, before any
    pointer is taken, so a short buffer never reaches a kernel."""
    torch = pytest.importorskip("torch")
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt)  # noqa: E731
    i8, u8, f16, i32 = torch.int8, torch.uint8, torch.float16, torch.int32
    nb, bs, nkv, B, nq = 4, 16, 2, 3, 4
    k8, s8 = z(nb, bs, nkv, 128, dt=i8), z(nb, bs, nkv)
    q, bt, ln = z(B, nq, 128), z(B, 2, dt=i32), z(B, dt=i32)

    def raises(fn, *a, match, **kw):
        with pytest.raises(ValueError, match=match):
            fn(*a, **kw)

    raises(K.kvq8_decode_attn, q, q, k8, k8[:2], s8, s8, bt, ln, 32, match="v_cache")
    raises(K.kvq8_decode_attn, q, q, k8, k8, s8, s8[:, :8], bt, ln, 32, match="v_scale")
    raises(K.kvq8_decode_attn, z(B, nq, 64), z(B, nq, 64), k8, k8, s8, s8, bt, ln, 32, match="q must")
    raises(K.kvq8_decode_attn, q[:, :2], q, k8, k8, s8, s8, bt, ln, 32, match="out")
    raises(K.kvq8_decode_attn, q, q, k8, k8, s8, s8, bt[:2], ln, 32, match="block_tables")
    raises(K.kvq8_decode_attn, q, q, k8, k8, s8, s8, bt, ln[:2], 32, match="ctx_lens")
    kn = z(B, nkv, 128)
    raises(K.kvq8_append_decode_attn, q, q, kn, kn, k8, k8, z(nb, bs, 1), s8, bt, ln, 32, match="k_scale")
    raises(K.kvq8_append_decode_attn, q, q, kn[:2], kn[:2], k8, k8, s8, s8, bt, ln, 32, match="k_new")
    raises(K.kvq8_quantize_append, k8, k8, s8, s8, z(5, nkv, 128), z(5, nkv, 128), z(4, dt=i32), match="slots")
    raises(K.kvq8_quantize_q, z(10, 128, dt=i8), z(10, 3), z(10, 128), match="qsc")
    raises(K.kvq8_qk_partials, z(B, nq, 32, 4, dt=i32), q, k8, bt, ln[:1], 32, match="ctx_lens")
    raises(K.kvq8_qk_partials, z(B, nq, 31, 4, dt=i32), q, k8, bt, ln, 32, match="partials")

    c4, g4 = z(nb, nkv, bs, 64, dt=u8), z(nb, nkv, bs, 2, dt=f16)     # head-major inside a block
    pool4, pool8 = (c4, c4, g4, g4, g4, g4), (k8, k8, s8, s8)
    raises(K.kvq4_decode_attn, q, q, (c4, c4, g4, g4, g4[:1], g4), bt, ln, 32, pool8, bt, ln, 16, match="v4_scale")
    raises(K.kvq4_decode_attn, q, q, pool4, bt, ln, 32, (k8, k8, s8, s8[:1]), bt, ln, 16, match="v_scale")
    raises(K.kvq4_decode_attn, q, q, pool4, bt, ln, 32, pool8, bt[:1], ln, 16, match="block_tables8")
    raises(K.kvq4_decode_attn, q[:1], q, pool4, bt, ln, 32, pool8, bt, ln, 16, match="out")
    raises(K.kvq4_requantize_q8, pool4, (k8[:, :8], k8[:, :8], s8[:, :8], s8[:, :8]), ln, ln, match="share")
    raises(K.kvq4_requantize_q8, (c4[:, :1],) * 2 + (g4[:, :1],) * 4, pool8, ln, ln, match="share")
    raises(K.kvq4_quantize_append, c4, c4[:1], g4, g4, g4, g4, kn, kn, ln, match="v4")
    c40, s40 = z(nb, nkv, bs, 64, dt=u8), z(nb, nkv, bs, 4)     # head-major inside a block
    raises(K.kvq4_0_decode_attn, q, q, c40, c40, s40, s40[..., :2], bt, ln, 32, match="v_step")
    raises(K.kvq4_0_quantize_append, c40, c40, s40, s40, kn, kn, ln[:1], match="slots")


def _decode4(**kw):
    a = dict(out=_fake(), q=_fake(), batch=2, nq=32, k4=_fake(), v4=_fake(), k4s=_fake(), k4z=_fake(), v4s=_fake(),
             v4z=_fake(), n4=64, bt4=_fake(), mb4=32, l4=_fake(), ml4=512, k8=_fake(), v8=_fake(), k8s=_fake(),
             v8s=_fake(), n8=8, bt8=_fake(), mb8=4, l8=_fake(), ml8=64, kv_bs=16, nkv=4, hd=128, sm=0.088, chunk=0,
             ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return K.lib().kvq4_decode_attn(*a.values())


def test_decode4_validation():
    need = K.kvq4_decode_workspace_size(2, 32, 4, 512, 64, 0)
    ws = dict(ws=_fake(), ws_bytes=need)
    # the binary16 scale / zero arrays are read two groups per word
    for name in ("k4s", "k4z", "v4s", "v4z"):
        assert _decode4(**ws, **{name: _fake(4098)}) == EINVAL, name
    assert _decode4(hd=64, **ws) == ESHAPE
    assert _decode4(nq=36, **ws) == ESHAPE            # group of 9
    assert _decode4(**ws, n4=1 << 30) == ESHAPE       # more than 2^32 - 1 rows
    assert _decode4(ws=None, ws_bytes=0) == EWORKSPACE


def test_requantize_validation():
    lib = K.lib()
    base = [_fake(), _fake(), _fake(), _fake(), _fake(), _fake(), 8, _fake(), _fake(), _fake(), _fake(), 4,
            16, 4, 128, 10, _fake(), _fake(), None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.kvq4_requantize_q8(*a)
    assert call(a15=0) == OK
    assert call(a14=96) == ESHAPE
    assert call(a12=12) == ESHAPE
    assert call(a6=0) == ESHAPE
    assert call(a15=-1) == EINVAL
    assert call(a16=None) == EINVAL
    assert call(a7=_fake(4104)) == EINVAL             # int8 cache not 16-byte aligned


def _decode40(**kw):
    a = dict(out=_fake(), q=_fake(), batch=2, nq=16, kc=_fake(), vc=_fake(), ks=_fake(), vs=_fake(), n_blocks=64,
             kv_bs=16, nkv=8, hd=128, bt=_fake(), mb=32, lens=_fake(), max_ctx=512, sm=0.088, chunk=0,
             ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return K.lib().kvq4_0_decode_attn(*a.values())


def test_q4_0_validation_and_sizing():
    lib = K.lib()
    need = K.kvq4_0_decode_workspace_size(2, 16, 8, 512, 0)
    assert need == K.kvq8_decode_workspace_size(2, 16, 8, 512, 0)
    assert K.kvq4_0_decode_chunk_tokens(1, 8, 8192) == K.kvq8_decode_chunk_tokens(1, 8, 8192)
    ws = dict(ws=_fake(), ws_bytes=need)
    assert _decode40(hd=64, **ws) == ESHAPE
    assert _decode40(nq=72, **ws) == ESHAPE           # group of 9
    assert _decode40(kv_bs=4, **ws) == ESHAPE
    assert _decode40(chunk=100, **ws) == ESHAPE
    assert _decode40(max_ctx=-1, **ws) == EINVAL
    assert _decode40(ks=_fake(4104), **ws) == EINVAL  # steps are read 16 bytes at a time
    assert _decode40(vc=None, **ws) == EINVAL
    assert _decode40(n_blocks=1 << 30, **ws) == ESHAPE
    assert _decode40() == EWORKSPACE
    assert _decode40(ws=_fake(), ws_bytes=need - 1) == EWORKSPACE
    assert _decode40(batch=0) == OK
    args = [_fake(), _fake(), _fake(), _fake(), 64, 16, 8, 128, _fake(), _fake(), K.F32, 10, _fake(), None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.kvq4_0_quantize_append(*a)
    assert call(a7=96) == ESHAPE
    assert call(a5=24) == ESHAPE
    assert call(a4=0) == ESHAPE
    assert call(a10=5) == EINVAL
    assert call(a11=-1) == EINVAL
    assert call(a11=0) == OK
    assert call(a12=None) == EINVAL
    assert call(a2=_fake(4104)) == EINVAL             # step array not 16-byte aligned
    assert call(a11=1 << 27) == ESHAPE                # 2^31 rows: beyond 32-bit row indexing
    assert call(a4=1 << 25) == ESHAPE                 # 2^25 x 16 slots x 8 heads: pool rows beyond 32 bits


def test_write_row_limit():
    """Every write path indexes rows in 32 bits and rejects larger calls before
    launching anything."""
    lib = K.lib()
    big = 1 << 27                                     # x 8 heads x 2 = 2^31 rows
    assert lib.kvq8_quantize_append(_fake(), _fake(), _fake(), _fake(), 64, 16, 8, 128, _fake(), _fake(), K.F32,
                                    big, _fake(), None) == ESHAPE
    # a pool of 2^25 x 16 slots x 8 heads = 2^32 rows: beyond 32-bit pool rows
    assert lib.kvq8_quantize_append(_fake(), _fake(), _fake(), _fake(), 1 << 25, 16, 8, 128, _fake(), _fake(),
                                    K.F32, 10, _fake(), None) == ESHAPE
    assert lib.kvq4_quantize_append(_fake(), _fake(), _fake(), _fake(), _fake(), _fake(), 64, 16, 8, 128,
                                    _fake(), _fake(), K.BF16, big, _fake(), None) == ESHAPE
    assert lib.kvq4_0_quantize_append(_fake(), _fake(), _fake(), _fake(), 64, 16, 8, 128, _fake(), _fake(), K.BF16,
                                      big, _fake(), None) == ESHAPE
    assert lib.kvq4_requantize_q8(_fake(), _fake(), _fake(), _fake(), _fake(), _fake(), 64, _fake(), _fake(),
                                  _fake(), _fake(), 64, 16, 8, 128, big, _fake(), _fake(), None) == ESHAPE
    # pools of 2^25 blocks x 16 slots x 8 heads = 2^32 rows: beyond the 32-bit
    # pool rows of the int4, 2-bit and Q4_0 writers and re-quantizations
    huge = 1 << 25
    assert lib.kvq4_quantize_append(_fake(), _fake(), _fake(), _fake(), _fake(), _fake(), huge, 16, 8, 128,
                                    _fake(), _fake(), K.BF16, 10, _fake(), None) == ESHAPE
    assert lib.kvq2_quantize_append(_fake(), _fake(), _fake(), _fake(), _fake(), _fake(), huge, 16, 8, 128,
                                    _fake(), _fake(), K.BF16, 10, _fake(), None) == ESHAPE
    assert lib.kvq4_0_quantize_append(_fake(), _fake(), _fake(), _fake(), huge, 16, 8, 128, _fake(), _fake(),
                                      K.BF16, 10, _fake(), None) == ESHAPE
    assert lib.kvq4_requantize_q8(_fake(), _fake(), _fake(), _fake(), _fake(), _fake(), huge, _fake(), _fake(),
                                  _fake(), _fake(), 64, 16, 8, 128, 10, _fake(), _fake(), None) == ESHAPE
    assert lib.kvq2_requantize_q4(_fake(), _fake(), _fake(), _fake(), _fake(), _fake(), huge, _fake(), _fake(),
                                  _fake(), _fake(), _fake(), _fake(), 64, 16, 8, 128, 10, _fake(), _fake(),
                                  None) == ESHAPE
    assert lib.kvq2_requantize_q4(_fake(), _fake(), _fake(), _fake(), _fake(), _fake(), 64, _fake(), _fake(),
                                  _fake(), _fake(), _fake(), _fake(), huge, 16, 8, 128, 10, _fake(), _fake(),
                                  None) == ESHAPE


def _decode2(**kw):
    a = dict(out=_fake(), q=_fake(), batch=2, nq=32,
             k2=_fake(), v2=_fake(), k2s=_fake(), k2z=_fake(), v2s=_fake(), v2z=_fake(), n2=64, bt2=_fake(),
             mb2=64, l2=_fake(), ml2=1024,
             k4=_fake(), v4=_fake(), k4s=_fake(), k4z=_fake(), v4s=_fake(), v4z=_fake(), n4=64, bt4=_fake(),
             mb4=32, l4=_fake(), ml4=512,
             k8=_fake(), v8=_fake(), k8s=_fake(), v8s=_fake(), n8=8, bt8=_fake(), mb8=4, l8=_fake(), ml8=64,
             kv_bs=16, nkv=4, hd=128, sm=0.088, chunk=0, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return K.lib().kvq2_decode_attn(*a.values())


def test_decode2_validation_and_sizing():
    need = K.kvq2_decode_workspace_size(2, 32, 4, 1024, 512, 64, 0)
    ch = K.kvq2_decode_chunk_tokens(2, 4, 1024, 512, 64)
    assert ch == K.kvq4_decode_chunk_tokens(2, 4, 1024 + 512, 64)       # the same rule over all bands
    n = 2 * 32 * (-(-1024 // ch) + -(-512 // ch) + -(-64 // ch))
    assert need == -(-n * 512 // 256) * 256 + 2 * (-(-n * 4 // 256) * 256)
    assert K.kvq2_decode_workspace_size(2, 32, 4, 1024, 512, 64, 300) == 0      # bad chunk
    ws = dict(ws=_fake(), ws_bytes=need)
    for name in ("k2s", "k2z", "v2s", "v2z", "k4s", "v4z"):
        assert _decode2(**ws, **{name: _fake(4098)}) == EINVAL, name
    for name in ("k2", "v2", "bt2", "l2"):
        assert _decode2(**ws, **{name: None}) == EINVAL, name
    assert _decode2(k2=_fake(4104), **ws) == EINVAL                      # codes 16-byte aligned
    assert _decode2(hd=64, **ws) == ESHAPE
    assert _decode2(nq=36, **ws) == ESHAPE
    assert _decode2(n2=0, **ws) == ESHAPE
    assert _decode2(mb2=0, **ws) == ESHAPE
    assert _decode2(n2=1 << 30, **ws) == ESHAPE                          # more than 2^32 - 1 rows
    assert _decode2(ml2=-1, **ws) == EINVAL
    assert _decode2(ws=_fake(), ws_bytes=need - 1) == EWORKSPACE
    assert _decode2(batch=0, **ws) == OK


def test_write2_and_requant2_validation():
    lib = K.lib()
    w = [_fake()] * 6 + [8, 16, 4, 128, _fake(), _fake(), 0, 10, _fake(), None]
    assert lib.kvq2_quantize_append(*w[:9], 64, *w[10:]) == ESHAPE
    assert lib.kvq2_quantize_append(*w[:7], 12, *w[8:]) == ESHAPE        # kv_bs not a power of two
    assert lib.kvq2_quantize_append(*w[:12], 3, *w[13:]) == EINVAL       # dtype
    assert lib.kvq2_quantize_append(*w[:13], -1, *w[14:]) == EINVAL
    assert lib.kvq2_quantize_append(*w[:13], 0, *w[14:]) == OK
    assert lib.kvq2_quantize_append(*w[:10], _fake(4100), *w[11:]) == EINVAL
    assert lib.kvq2_quantize_append(*w[:13], 1 << 28, *w[14:]) == ESHAPE  # 2^31 rows
    r = [_fake()] * 6 + [8] + [_fake()] * 6 + [4, 16, 4, 128, 10, _fake(), _fake(), None]
    assert lib.kvq2_requantize_q4(*r[:6], 0, *r[7:]) == ESHAPE
    assert lib.kvq2_requantize_q4(*r[:13], 0, *r[14:]) == ESHAPE
    assert lib.kvq2_requantize_q4(*r[:17], -1, *r[18:]) == EINVAL
    assert lib.kvq2_requantize_q4(*r[:17], 0, *r[18:]) == OK
    assert lib.kvq2_requantize_q4(*r[:17], 1 << 28, *r[18:]) == ESHAPE
    assert lib.kvq2_requantize_q4(*r[:18], None, *r[19:]) == EINVAL


def test_binding_checks_two_bit_pools():
    torch = pytest.importorskip("torch")
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt)  # noqa: E731
    u8, f16, i8, i32 = torch.uint8, torch.float16, torch.int8, torch.int32
    nb, bs, nkv, B, nq = 4, 16, 2, 3, 4
    c2, g = z(nb, nkv, bs, 32, dt=u8), z(nb, nkv, bs, 2, dt=f16)     # head-major inside a block
    c4 = z(nb, nkv, bs, 64, dt=u8)
    p2, p4 = (c2, c2, g, g, g, g), (c4, c4, g, g, g, g)
    p8 = (z(nb, bs, nkv, 128, dt=i8), z(nb, bs, nkv, 128, dt=i8), z(nb, bs, nkv), z(nb, bs, nkv))
    q, bt, ln = z(B, nq, 128), z(B, 2, dt=i32), z(B, dt=i32)
    with pytest.raises(ValueError, match="v2_zero"):
        K.kvq2_decode_attn(q, q, (c2, c2, g, g, g, g[:1]), bt, ln, 32, p4, bt, ln, 32, p8, bt, ln, 32)
    with pytest.raises(ValueError, match="share"):
        K.kvq2_decode_attn(q, q, p2, bt, ln, 32, (c4[:, :, :8],) * 2 + (g[:, :, :8],) * 4, bt, ln, 32, p8, bt, ln, 32)
    with pytest.raises(ValueError, match="lens2"):
        K.kvq2_decode_attn(q, q, p2, bt, ln[:1], 32, p4, bt, ln, 32, p8, bt, ln, 32)
    with pytest.raises(ValueError, match="share"):
        K.kvq2_requantize_q4(p2, (c4[:, :, :8],) * 2 + (g[:, :, :8],) * 4, ln, ln)
    kn = z(5, nkv, 128)
    with pytest.raises(ValueError, match="slots"):
        K.kvq2_quantize_append(*p2, kn, kn, ln)


def test_noalloc_decode_validation():
    """kvq8_decode_attn_noalloc checks its arguments as kvq8_decode_attn does
    and rejects sizes whose partials exceed the library's scratch array
    (KVQ8_DECODE_SCRATCH_BYTES, 16 MiB) before touching the device."""
    lib = K.lib()
    limit = 16 << 20

    def call(batch=2, nq=16, nkv=8, max_ctx=512, chunk=0, sm=0.088, q=_fake(), hd=128):
        return lib.kvq8_decode_attn_noalloc(_fake(), q, batch, nq, _fake(), _fake(), _fake(), _fake(), 64 << 10,
                                            16, nkv, hd, _fake(), 4096, _fake(), max_ctx, sm, chunk, None)
    assert call(hd=64) == ESHAPE
    assert call(chunk=100) == ESHAPE
    assert call(q=None) == EINVAL
    assert call(sm=float("nan")) == EINVAL
    assert call(batch=0) == OK
    assert K.kvq8_decode_workspace_size(64, 64, 8, 65536, 0) > limit
    assert call(batch=64, nq=64, max_ctx=65536) == EWORKSPACE
