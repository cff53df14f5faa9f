"""Python binding of ``libkvq8.so`` (ctypes).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, checks their dtype / shape / layout, passes raw device
pointers and the current HIP stream to the C entry point of the same name,
and raises on a non-zero status.  No computation happens here, and there is
no fallback: if the library is not built, every call raises.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch has already loaded (same soname), and the stream handle
torch hands out is valid in it.
"""
from __future__ import annotations

import ctypes
import os

import torch

HD = 128
F32, BF16, F16 = 0, 1, 2
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq8.so")

_c_int, _c_size, _p, _f = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float

# name -> (restype, argtypes); mirrors include/kvq8.h
_SIGNATURES = {
    "kvq8_status_string": (ctypes.c_char_p, [_c_int]),
    "kvq8_version": (ctypes.c_char_p, []),
    "kvq8_quantize_append": (_c_int, [_p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _p, _p, _c_int, _c_int,
                                      _p, _p]),
    "kvq8_decode_chunk_tokens": (_c_int, [_c_int, _c_int, _c_int]),
    "kvq8_decode_workspace_size": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "kvq8_decode_attn": (_c_int, [_p, _p, _c_int, _c_int, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _p,
                                  _c_int, _p, _c_int, _f, _c_int, _p, _c_size, _p]),
    "kvq8_decode_attn_noalloc": (_c_int, [_p, _p, _c_int, _c_int, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int,
                                          _p, _c_int, _p, _c_int, _f, _c_int, _p]),
    "kvq8_append_decode_attn": (_c_int, [_p, _p, _c_int, _c_int, _p, _p, _c_int, _p, _p, _p, _p, _c_int, _c_int,
                                         _c_int, _c_int, _p, _c_int, _p, _c_int, _f, _c_int, _p, _c_size, _p]),
    "kvq8_quantize_q": (_c_int, [_p, _p, _p, _c_int, _c_int, _p]),
    "kvq8_qk_partials": (_c_int, [_p, _p, _c_int, _c_int, _p, _c_int, _c_int, _c_int, _c_int, _p, _c_int, _p,
                                  _c_int, _p]),
    "kvq4_quantize_append": (_c_int, [_p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _p, _p, _c_int,
                                      _c_int, _p, _p]),
    "kvq4_requantize_q8": (_c_int, [_p, _p, _p, _p, _p, _p, _c_int, _p, _p, _p, _p, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _p, _p, _p]),
    "kvq4_decode_chunk_tokens": (_c_int, [_c_int, _c_int, _c_int, _c_int]),
    "kvq4_decode_workspace_size": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "kvq4_decode_attn": (_c_int, [_p, _p, _c_int, _c_int,
                                  _p, _p, _p, _p, _p, _p, _c_int, _p, _c_int, _p, _c_int,
                                  _p, _p, _p, _p, _c_int, _p, _c_int, _p, _c_int,
                                  _c_int, _c_int, _c_int, _f, _c_int, _p, _c_size, _p]),
    "kvq2_quantize_append": (_c_int, [_p, _p, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _p, _p, _c_int,
                                      _c_int, _p, _p]),
    "kvq2_requantize_q4": (_c_int, [_p, _p, _p, _p, _p, _p, _c_int, _p, _p, _p, _p, _p, _p, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _p, _p, _p]),
    "kvq2_decode_chunk_tokens": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "kvq2_decode_workspace_size": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "kvq2_decode_attn": (_c_int, [_p, _p, _c_int, _c_int,
                                  _p, _p, _p, _p, _p, _p, _c_int, _p, _c_int, _p, _c_int,
                                  _p, _p, _p, _p, _p, _p, _c_int, _p, _c_int, _p, _c_int,
                                  _p, _p, _p, _p, _c_int, _p, _c_int, _p, _c_int,
                                  _c_int, _c_int, _c_int, _f, _c_int, _p, _c_size, _p]),
    "kvq4_0_quantize_append": (_c_int, [_p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _p, _p, _c_int, _c_int,
                                        _p, _p]),
    "kvq4_0_decode_chunk_tokens": (_c_int, [_c_int, _c_int, _c_int]),
    "kvq4_0_decode_workspace_size": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "kvq4_0_decode_attn": (_c_int, [_p, _p, _c_int, _c_int, _p, _p, _p, _p, _c_int, _c_int, _c_int, _c_int, _p,
                                    _c_int, _p, _c_int, _f, _c_int, _p, _c_size, _p]),
}

_lib = None


class KVQ8Error(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KVQ8Error(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                            f"g.build()'` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int, what: str):
    if status != 0:
        msg = lib().kvq8_status_string(status).decode()
        raise KVQ8Error(f"{what} failed: {msg} ({status})")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _scale(sm_scale):
    """The score scale argument: None passes 0, which the library reads as
    its default 1 / sqrt(hd)."""
    return 0.0 if sm_scale is None else float(sm_scale)


def _ptr(t: torch.Tensor | None, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t: torch.Tensor, shape, name: str):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(map(str, devs))}")


def _int8_pool(k_cache, v_cache, k_scale, v_scale):
    """[n_blocks][kv_bs][nkv][128] codes and [n_blocks][kv_bs][nkv] steps, K and V alike."""
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [n_blocks][kv_bs][nkv][hd]")
    _shape(v_cache, k_cache.shape, "v_cache")
    _shape(k_scale, k_cache.shape[:3], "k_scale")
    _shape(v_scale, k_cache.shape[:3], "v_scale")
    return tuple(k_cache.shape)


def _query(out, q, hd: int):
    if q.dim() != 3 or q.shape[2] != hd:
        raise ValueError(f"q must be [B][nq][{hd}]")
    _shape(out, q.shape, "out")


def _tables(block_tables, ctx_lens, B: int, suffix=""):
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError(f"block_tables{suffix} must be [B][max_blocks]")
    _shape(ctx_lens, (B,), "ctx_lens" if not suffix else f"lens{suffix}")


def _group_pool(pool, codes_per_byte: int, names):
    """Packed codes [n_blocks][nkv][kv_bs][hd / codes_per_byte] (head-major
    inside a block), K and V alike, and four [n_blocks][nkv][kv_bs][hd / 64]
    scale / zero tensors.  Returns (n_blocks, kv_bs, nkv, hd)."""
    kc, vc, ks, kz, vs, vz = pool
    if kc.dim() != 4:
        raise ValueError(f"{names[0]} must be [n_blocks][nkv][kv_bs][hd / {codes_per_byte}]")
    _shape(vc, kc.shape, names[1])
    n, nkv, bs, row = kc.shape
    hd = codes_per_byte * row
    for t, nm in zip((ks, kz, vs, vz), names[2:]):
        _shape(t, (n, nkv, bs, hd // 64), nm)
    return n, bs, nkv, hd


def _int2_pool(pool2):
    return _group_pool(pool2, 4, ("k2", "v2", "k2_scale", "k2_zero", "v2_scale", "v2_zero"))


def _int4_pool(pool4):
    return _group_pool(pool4, 2, ("k4", "v4", "k4_scale", "k4_zero", "v4_scale", "v4_zero"))


def kvq8_status_string(status: int) -> str:
    return lib().kvq8_status_string(status).decode()


def kvq8_version() -> str:
    return lib().kvq8_version().decode()


# ----------------------------------------------------------------------------
# int8 path
# ----------------------------------------------------------------------------

def kvq8_quantize_append(k_cache, v_cache, k_scale, v_scale, k_new, v_new, slots, stream=None):
    """Quantize k_new / v_new [n_tokens][nkv][128] (f32, bf16 or f16) into the
    int8 cache [n_blocks][kv_bs][nkv][128] at ``slots`` (int32)."""
    n_blocks, kv_bs, nkv, hd = _int8_pool(k_cache, v_cache, k_scale, v_scale)
    if k_new.dtype not in _DTYPES or v_new.dtype != k_new.dtype:
        raise ValueError("k_new / v_new must share one of float32, bfloat16, float16")
    if k_new.dim() != 3 or tuple(k_new.shape[1:]) != (nkv, hd) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [n_tokens][nkv][hd]")
    if slots.shape != (k_new.shape[0],):
        raise ValueError("slots must be [n_tokens]")
    _same_device(k_cache, v_cache, k_scale, v_scale, k_new, v_new, slots)
    st = lib().kvq8_quantize_append(
        _ptr(k_cache, torch.int8, "k_cache"), _ptr(v_cache, torch.int8, "v_cache"),
        _ptr(k_scale, torch.float32, "k_scale"), _ptr(v_scale, torch.float32, "v_scale"),
        n_blocks, kv_bs, nkv, hd, _ptr(k_new, name="k_new"), _ptr(v_new, name="v_new"), _DTYPES[k_new.dtype],
        k_new.shape[0], _ptr(slots, torch.int32, "slots"), _stream(stream))
    _check(st, "kvq8_quantize_append")


def kvq8_decode_chunk_tokens(batch: int, nkv: int, max_ctx_len: int) -> int:
    return lib().kvq8_decode_chunk_tokens(batch, nkv, max_ctx_len)


def kvq8_decode_workspace_size(batch: int, nq: int, nkv: int, max_ctx_len: int, chunk: int = 0) -> int:
    return lib().kvq8_decode_workspace_size(batch, nq, nkv, max_ctx_len, chunk)


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """Device bytes for a workspace argument (16-byte aligned by torch)."""
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def kvq8_decode_attn(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, max_ctx_len: int,
                     sm_scale: float | None = None, chunk: int = 0, workspace=None, stream=None):
    """Decode attention: out [B][nq][128] (float32) from q [B][nq][128] over
    the int8 cache.  ``workspace`` (uint8) is allocated when not given."""
    n_blocks, kv_bs, nkv, hd = _int8_pool(k_cache, v_cache, k_scale, v_scale)
    _query(out, q, hd)
    B, nq, _ = q.shape
    _tables(block_tables, ctx_lens, B)
    _same_device(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, workspace)
    need = kvq8_decode_workspace_size(B, nq, nkv, max_ctx_len, chunk)
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    st = lib().kvq8_decode_attn(
        _ptr(out, torch.float32, "out"), _ptr(q, torch.float32, "q"), B, nq,
        _ptr(k_cache, torch.int8, "k_cache"), _ptr(v_cache, torch.int8, "v_cache"),
        _ptr(k_scale, torch.float32, "k_scale"), _ptr(v_scale, torch.float32, "v_scale"),
        n_blocks, kv_bs, nkv, hd, _ptr(block_tables, torch.int32, "block_tables"), block_tables.shape[1],
        _ptr(ctx_lens, torch.int32, "ctx_lens"), max_ctx_len, _scale(sm_scale), chunk,
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "kvq8_decode_attn")
    return out


def kvq8_decode_attn_noalloc(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, max_ctx_len: int,
                             sm_scale: float | None = None, chunk: int = 0, stream=None):
    """kvq8_decode_attn without a workspace: the library keeps the chunk
    partials in its own device array (KVQ8_DECODE_SCRATCH_BYTES per device),
    so the call allocates nothing.  Calls that overlap on one device race on
    that array; order them on one stream."""
    n_blocks, kv_bs, nkv, hd = _int8_pool(k_cache, v_cache, k_scale, v_scale)
    _query(out, q, hd)
    B, nq, _ = q.shape
    _tables(block_tables, ctx_lens, B)
    _same_device(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens)
    st = lib().kvq8_decode_attn_noalloc(
        _ptr(out, torch.float32, "out"), _ptr(q, torch.float32, "q"), B, nq,
        _ptr(k_cache, torch.int8, "k_cache"), _ptr(v_cache, torch.int8, "v_cache"),
        _ptr(k_scale, torch.float32, "k_scale"), _ptr(v_scale, torch.float32, "v_scale"),
        n_blocks, kv_bs, nkv, hd, _ptr(block_tables, torch.int32, "block_tables"), block_tables.shape[1],
        _ptr(ctx_lens, torch.int32, "ctx_lens"), max_ctx_len, _scale(sm_scale), chunk, _stream(stream))
    _check(st, "kvq8_decode_attn_noalloc")
    return out


def kvq8_append_decode_attn(out, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens,
                            max_ctx_len: int, sm_scale: float | None = None, chunk: int = 0, workspace=None,
                            stream=None):
    """Write each sequence's newest token (k_new / v_new [B][nkv][128] at
    position ctx_lens[b] - 1) into the int8 cache, then decode attention over
    the whole context, in one pass."""
    n_blocks, kv_bs, nkv, hd = _int8_pool(k_cache, v_cache, k_scale, v_scale)
    _query(out, q, hd)
    B, nq, _ = q.shape
    if k_new.dtype not in _DTYPES or v_new.dtype != k_new.dtype:
        raise ValueError("k_new / v_new must share one of float32, bfloat16, float16")
    if tuple(k_new.shape) != (B, nkv, hd) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [B][nkv][hd]")
    _tables(block_tables, ctx_lens, B)
    _same_device(out, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables, ctx_lens, workspace)
    need = kvq8_decode_workspace_size(B, nq, nkv, max_ctx_len, chunk)
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    st = lib().kvq8_append_decode_attn(
        _ptr(out, torch.float32, "out"), _ptr(q, torch.float32, "q"), B, nq, _ptr(k_new, name="k_new"),
        _ptr(v_new, name="v_new"), _DTYPES[k_new.dtype], _ptr(k_cache, torch.int8, "k_cache"),
        _ptr(v_cache, torch.int8, "v_cache"), _ptr(k_scale, torch.float32, "k_scale"),
        _ptr(v_scale, torch.float32, "v_scale"), n_blocks, kv_bs, nkv, hd,
        _ptr(block_tables, torch.int32, "block_tables"), block_tables.shape[1],
        _ptr(ctx_lens, torch.int32, "ctx_lens"), max_ctx_len, _scale(sm_scale), chunk,
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "kvq8_append_decode_attn")
    return out


def kvq8_quantize_q(qi, qsc, q, stream=None):
    """Query codes qi [n][128] int8 and block scales qsc [n][4] float32 of
    q [..., 128] (n = q.numel() / 128 vectors; any shapes of those sizes)."""
    if q.dim() < 1 or q.shape[-1] != HD:
        raise ValueError(f"q must be [..., {HD}]")
    n = q.numel() // HD
    if qi.numel() != n * HD or qsc.numel() != n * (HD // 32):
        raise ValueError(f"qi must hold {n} x {HD} codes and qsc {n} x {HD // 32} scales")
    _same_device(qi, qsc, q)
    st = lib().kvq8_quantize_q(_ptr(qi, torch.int8, "qi"), _ptr(qsc, torch.float32, "qsc"),
                               _ptr(q, torch.float32, "q"), n, HD, _stream(stream))
    _check(st, "kvq8_quantize_q")


def kvq8_qk_partials(partials, q, k_cache, block_tables, ctx_lens, max_ctx_len: int, stream=None):
    """int32 block partials [B][nq][max_ctx_len][4]."""
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [n_blocks][kv_bs][nkv][hd]")
    n_blocks, kv_bs, nkv, hd = k_cache.shape
    if q.dim() != 3 or q.shape[2] != hd:
        raise ValueError(f"q must be [B][nq][{hd}]")
    B, nq, _ = q.shape
    _shape(partials, (B, nq, max_ctx_len, 4), "partials")
    _tables(block_tables, ctx_lens, B)
    _same_device(partials, q, k_cache, block_tables, ctx_lens)
    st = lib().kvq8_qk_partials(
        _ptr(partials, torch.int32, "partials"), _ptr(q, torch.float32, "q"), B, nq,
        _ptr(k_cache, torch.int8, "k_cache"), n_blocks, kv_bs, nkv, hd,
        _ptr(block_tables, torch.int32, "block_tables"), block_tables.shape[1],
        _ptr(ctx_lens, torch.int32, "ctx_lens"), max_ctx_len, _stream(stream))
    _check(st, "kvq8_qk_partials")


# ----------------------------------------------------------------------------
# int4 group variant
# ----------------------------------------------------------------------------

def kvq4_quantize_append(k_cache, v_cache, k_scale, k_zero, v_scale, v_zero, k_new, v_new, slots, stream=None):
    """Quantize into the int4 pool: packed codes [n_blocks][nkv][kv_bs][64]
    uint8, scale / zero [n_blocks][nkv][kv_bs][2] float16."""
    n_blocks, kv_bs, nkv, hd = _int4_pool((k_cache, v_cache, k_scale, k_zero, v_scale, v_zero))
    if k_new.dtype not in _DTYPES or v_new.dtype != k_new.dtype:
        raise ValueError("k_new / v_new must share one of float32, bfloat16, float16")
    if k_new.dim() != 3 or tuple(k_new.shape[1:]) != (nkv, hd) or v_new.shape != k_new.shape or \
            slots.shape != (k_new.shape[0],):
        raise ValueError("k_new / v_new must be [n_tokens][nkv][hd], slots [n_tokens]")
    _same_device(k_cache, v_cache, k_scale, k_zero, v_scale, v_zero, k_new, v_new, slots)
    st = lib().kvq4_quantize_append(
        _ptr(k_cache, torch.uint8, "k_cache"), _ptr(v_cache, torch.uint8, "v_cache"),
        _ptr(k_scale, torch.float16, "k_scale"), _ptr(k_zero, torch.float16, "k_zero"),
        _ptr(v_scale, torch.float16, "v_scale"), _ptr(v_zero, torch.float16, "v_zero"),
        n_blocks, kv_bs, nkv, hd, _ptr(k_new, name="k_new"), _ptr(v_new, name="v_new"), _DTYPES[k_new.dtype],
        k_new.shape[0], _ptr(slots, torch.int32, "slots"), _stream(stream))
    _check(st, "kvq4_quantize_append")


def kvq4_requantize_q8(pool4, pool8, src_slots, dst_slots, stream=None):
    """Move tokens from the int8 pool (k, v, k_scale, v_scale) into the int4
    pool (k, v, k_scale, k_zero, v_scale, v_zero): pair i takes int8 slot
    src_slots[i] to int4 slot dst_slots[i] (int32 device tensors)."""
    k4, v4, k4s, k4z, v4s, v4z = pool4
    k8, v8, k8s, v8s = pool8
    n4, kv_bs, nkv, hd = _int4_pool(pool4)
    n8 = _int8_pool(k8, v8, k8s, v8s)[0]
    if tuple(k8.shape[1:]) != (kv_bs, nkv, hd):
        raise ValueError("the int8 and int4 pools must share kv_bs, nkv and hd")
    if src_slots.shape != dst_slots.shape or src_slots.dim() != 1:
        raise ValueError("src_slots and dst_slots must be [n_tokens]")
    _same_device(*pool4, *pool8, src_slots, dst_slots)
    st = lib().kvq4_requantize_q8(
        _ptr(k4, torch.uint8, "k4"), _ptr(v4, torch.uint8, "v4"), _ptr(k4s, torch.float16, "k4_scale"),
        _ptr(k4z, torch.float16, "k4_zero"), _ptr(v4s, torch.float16, "v4_scale"),
        _ptr(v4z, torch.float16, "v4_zero"), n4, _ptr(k8, torch.int8, "k8"), _ptr(v8, torch.int8, "v8"),
        _ptr(k8s, torch.float32, "k8_scale"), _ptr(v8s, torch.float32, "v8_scale"), n8, kv_bs, nkv, hd,
        src_slots.shape[0], _ptr(src_slots, torch.int32, "src_slots"), _ptr(dst_slots, torch.int32, "dst_slots"),
        _stream(stream))
    _check(st, "kvq4_requantize_q8")


def kvq4_decode_chunk_tokens(batch: int, nkv: int, max_len4: int, max_len8: int) -> int:
    return lib().kvq4_decode_chunk_tokens(batch, nkv, max_len4, max_len8)


def kvq4_decode_workspace_size(batch: int, nq: int, nkv: int, max_len4: int, max_len8: int, chunk: int = 0) -> int:
    return lib().kvq4_decode_workspace_size(batch, nq, nkv, max_len4, max_len8, chunk)


def kvq4_decode_attn(out, q, pool4, block_tables4, lens4, max_len4: int, pool8, block_tables8, lens8,
                     max_len8: int, sm_scale: float | None = None, chunk: int = 0, workspace=None, stream=None):
    """Decode attention over an int4 pool (k, v, k_scale, k_zero, v_scale,
    v_zero) plus an int8 recent-window pool (k, v, k_scale, v_scale)."""
    k4, v4, k4s, k4z, v4s, v4z = pool4
    k8, v8, k8s, v8s = pool8
    n4, kv_bs, nkv, hd = _int4_pool(pool4)
    n8 = _int8_pool(k8, v8, k8s, v8s)[0]
    if tuple(k8.shape[1:]) != (kv_bs, nkv, hd):
        raise ValueError("int8 pool must share kv_bs, nkv and hd with the int4 pool")
    _query(out, q, hd)
    B, nq, _ = q.shape
    _tables(block_tables4, lens4, B, "4")
    _tables(block_tables8, lens8, B, "8")
    _same_device(out, q, *pool4, *pool8, block_tables4, lens4, block_tables8, lens8, workspace)
    need = kvq4_decode_workspace_size(B, nq, nkv, max_len4, max_len8, chunk)
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    st = lib().kvq4_decode_attn(
        _ptr(out, torch.float32, "out"), _ptr(q, torch.float32, "q"), B, nq,
        _ptr(k4, torch.uint8, "k4"), _ptr(v4, torch.uint8, "v4"), _ptr(k4s, torch.float16, "k4_scale"),
        _ptr(k4z, torch.float16, "k4_zero"), _ptr(v4s, torch.float16, "v4_scale"),
        _ptr(v4z, torch.float16, "v4_zero"), n4, _ptr(block_tables4, torch.int32, "block_tables4"),
        block_tables4.shape[1], _ptr(lens4, torch.int32, "lens4"), max_len4,
        _ptr(k8, torch.int8, "k8"), _ptr(v8, torch.int8, "v8"), _ptr(k8s, torch.float32, "k8_scale"),
        _ptr(v8s, torch.float32, "v8_scale"), n8, _ptr(block_tables8, torch.int32, "block_tables8"),
        block_tables8.shape[1], _ptr(lens8, torch.int32, "lens8"), max_len8,
        kv_bs, nkv, hd, _scale(sm_scale), chunk, _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream(stream))
    _check(st, "kvq4_decode_attn")
    return out


# ----------------------------------------------------------------------------
# Q4_0 mode
# ----------------------------------------------------------------------------

def _q40_pool(k_cache, v_cache, k_step, v_step):
    """Packed codes [n_blocks][nkv][kv_bs][hd / 2] (head-major inside a
    block), K and V alike, and steps [n_blocks][nkv][kv_bs][hd / 32].
    Returns (n_blocks, kv_bs, nkv, hd)."""
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [n_blocks][nkv][kv_bs][hd / 2]")
    _shape(v_cache, k_cache.shape, "v_cache")
    n, nkv, bs, half = k_cache.shape
    _shape(k_step, (n, nkv, bs, 2 * half // 32), "k_step")
    _shape(v_step, (n, nkv, bs, 2 * half // 32), "v_step")
    return n, bs, nkv, 2 * half


def kvq4_0_quantize_append(k_cache, v_cache, k_step, v_step, k_new, v_new, slots, stream=None):
    """Quantize k_new / v_new [n_tokens][nkv][128] (f32, bf16 or f16) into the
    Q4_0 pool: packed codes [n_blocks][nkv][kv_bs][64] uint8, steps
    [n_blocks][nkv][kv_bs][4] float32, at ``slots`` (int32)."""
    n_blocks, kv_bs, nkv, hd = _q40_pool(k_cache, v_cache, k_step, v_step)
    if k_new.dtype not in _DTYPES or v_new.dtype != k_new.dtype:
        raise ValueError("k_new / v_new must share one of float32, bfloat16, float16")
    if k_new.dim() != 3 or tuple(k_new.shape[1:]) != (nkv, hd) or v_new.shape != k_new.shape or \
            slots.shape != (k_new.shape[0],):
        raise ValueError("k_new / v_new must be [n_tokens][nkv][hd], slots [n_tokens]")
    _same_device(k_cache, v_cache, k_step, v_step, k_new, v_new, slots)
    st = lib().kvq4_0_quantize_append(
        _ptr(k_cache, torch.uint8, "k_cache"), _ptr(v_cache, torch.uint8, "v_cache"),
        _ptr(k_step, torch.float32, "k_step"), _ptr(v_step, torch.float32, "v_step"),
        n_blocks, kv_bs, nkv, hd, _ptr(k_new, name="k_new"), _ptr(v_new, name="v_new"), _DTYPES[k_new.dtype],
        k_new.shape[0], _ptr(slots, torch.int32, "slots"), _stream(stream))
    _check(st, "kvq4_0_quantize_append")


def kvq4_0_decode_chunk_tokens(batch: int, nkv: int, max_ctx_len: int) -> int:
    return lib().kvq4_0_decode_chunk_tokens(batch, nkv, max_ctx_len)


def kvq4_0_decode_workspace_size(batch: int, nq: int, nkv: int, max_ctx_len: int, chunk: int = 0) -> int:
    return lib().kvq4_0_decode_workspace_size(batch, nq, nkv, max_ctx_len, chunk)


def kvq4_0_decode_attn(out, q, k_cache, v_cache, k_step, v_step, block_tables, ctx_lens, max_ctx_len: int,
                       sm_scale: float | None = None, chunk: int = 0, workspace=None, stream=None):
    """Decode attention: out [B][nq][128] (float32) from q [B][nq][128] over
    the Q4_0 cache.  ``workspace`` (uint8) is allocated when not given."""
    n_blocks, kv_bs, nkv, hd = _q40_pool(k_cache, v_cache, k_step, v_step)
    _query(out, q, hd)
    B, nq, _ = q.shape
    _tables(block_tables, ctx_lens, B)
    _same_device(out, q, k_cache, v_cache, k_step, v_step, block_tables, ctx_lens, workspace)
    need = kvq4_0_decode_workspace_size(B, nq, nkv, max_ctx_len, chunk)
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    st = lib().kvq4_0_decode_attn(
        _ptr(out, torch.float32, "out"), _ptr(q, torch.float32, "q"), B, nq,
        _ptr(k_cache, torch.uint8, "k_cache"), _ptr(v_cache, torch.uint8, "v_cache"),
        _ptr(k_step, torch.float32, "k_step"), _ptr(v_step, torch.float32, "v_step"),
        n_blocks, kv_bs, nkv, hd, _ptr(block_tables, torch.int32, "block_tables"), block_tables.shape[1],
        _ptr(ctx_lens, torch.int32, "ctx_lens"), max_ctx_len, _scale(sm_scale), chunk,
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "kvq4_0_decode_attn")
    return out


# ----------------------------------------------------------------------------
# 2-bit band of the group variant
# ----------------------------------------------------------------------------

def _pool_ptrs(pool, codes_dtype, prefix):
    kc, vc, ks, kz, vs, vz = pool
    return (_ptr(kc, codes_dtype, f"k{prefix}"), _ptr(vc, codes_dtype, f"v{prefix}"),
            _ptr(ks, torch.float16, f"k{prefix}_scale"), _ptr(kz, torch.float16, f"k{prefix}_zero"),
            _ptr(vs, torch.float16, f"v{prefix}_scale"), _ptr(vz, torch.float16, f"v{prefix}_zero"))


def kvq2_quantize_append(k_cache, v_cache, k_scale, k_zero, v_scale, v_zero, k_new, v_new, slots, stream=None):
    """Quantize into the 2-bit pool: packed codes [n_blocks][nkv][kv_bs][32]
    uint8, scale / zero [n_blocks][nkv][kv_bs][2] float16."""
    pool = (k_cache, v_cache, k_scale, k_zero, v_scale, v_zero)
    n_blocks, kv_bs, nkv, hd = _int2_pool(pool)
    if k_new.dtype not in _DTYPES or v_new.dtype != k_new.dtype:
        raise ValueError("k_new / v_new must share one of float32, bfloat16, float16")
    if k_new.dim() != 3 or tuple(k_new.shape[1:]) != (nkv, hd) or v_new.shape != k_new.shape or \
            slots.shape != (k_new.shape[0],):
        raise ValueError("k_new / v_new must be [n_tokens][nkv][hd], slots [n_tokens]")
    _same_device(*pool, k_new, v_new, slots)
    st = lib().kvq2_quantize_append(
        *_pool_ptrs(pool, torch.uint8, "2"), n_blocks, kv_bs, nkv, hd, _ptr(k_new, name="k_new"),
        _ptr(v_new, name="v_new"), _DTYPES[k_new.dtype], k_new.shape[0], _ptr(slots, torch.int32, "slots"),
        _stream(stream))
    _check(st, "kvq2_quantize_append")


def kvq2_requantize_q4(pool2, pool4, src_slots, dst_slots, stream=None):
    """Move tokens from the int4 pool (k, v, k_scale, k_zero, v_scale,
    v_zero) into the 2-bit pool (same order): pair i takes int4 slot
    src_slots[i] to 2-bit slot dst_slots[i] (int32 device tensors)."""
    n2, kv_bs, nkv, hd = _int2_pool(pool2)
    n4 = _int4_pool(pool4)[0]
    if tuple(pool4[0].shape[1:3]) != (nkv, kv_bs) or 2 * pool4[0].shape[3] != hd:
        raise ValueError("the int4 and 2-bit pools must share kv_bs, nkv and hd")
    if src_slots.shape != dst_slots.shape or src_slots.dim() != 1:
        raise ValueError("src_slots and dst_slots must be [n_tokens]")
    _same_device(*pool2, *pool4, src_slots, dst_slots)
    st = lib().kvq2_requantize_q4(
        *_pool_ptrs(pool2, torch.uint8, "2"), n2, *_pool_ptrs(pool4, torch.uint8, "4"), n4, kv_bs, nkv, hd,
        src_slots.shape[0], _ptr(src_slots, torch.int32, "src_slots"), _ptr(dst_slots, torch.int32, "dst_slots"),
        _stream(stream))
    _check(st, "kvq2_requantize_q4")


def kvq2_decode_chunk_tokens(batch: int, nkv: int, max_len2: int, max_len4: int, max_len8: int) -> int:
    return lib().kvq2_decode_chunk_tokens(batch, nkv, max_len2, max_len4, max_len8)


def kvq2_decode_workspace_size(batch: int, nq: int, nkv: int, max_len2: int, max_len4: int, max_len8: int,
                               chunk: int = 0) -> int:
    return lib().kvq2_decode_workspace_size(batch, nq, nkv, max_len2, max_len4, max_len8, chunk)


def kvq2_decode_attn(out, q, pool2, block_tables2, lens2, max_len2: int, pool4, block_tables4, lens4,
                     max_len4: int, pool8, block_tables8, lens8, max_len8: int, sm_scale: float | None = None,
                     chunk: int = 0, workspace=None, stream=None):
    """Decode attention over a 2-bit band (pool2: k, v, k_scale, k_zero,
    v_scale, v_zero), an int4 band (pool4, the same order) and an int8
    window (pool8: k, v, k_scale, v_scale)."""
    n2, kv_bs, nkv, hd = _int2_pool(pool2)
    n4 = _int4_pool(pool4)[0]
    k8, v8, k8s, v8s = pool8
    n8 = _int8_pool(k8, v8, k8s, v8s)[0]
    if tuple(pool4[0].shape[1:3]) != (nkv, kv_bs) or 2 * pool4[0].shape[3] != hd or \
            tuple(k8.shape[1:]) != (kv_bs, nkv, hd):
        raise ValueError("the three pools must share kv_bs, nkv and hd")
    _query(out, q, hd)
    B, nq, _ = q.shape
    _tables(block_tables2, lens2, B, "2")
    _tables(block_tables4, lens4, B, "4")
    _tables(block_tables8, lens8, B, "8")
    _same_device(out, q, *pool2, *pool4, *pool8, block_tables2, lens2, block_tables4, lens4, block_tables8, lens8,
                 workspace)
    need = kvq2_decode_workspace_size(B, nq, nkv, max_len2, max_len4, max_len8, chunk)
    if workspace is None:
        workspace = alloc_workspace(need, q.device)
    st = lib().kvq2_decode_attn(
        _ptr(out, torch.float32, "out"), _ptr(q, torch.float32, "q"), B, nq,
        *_pool_ptrs(pool2, torch.uint8, "2"), n2, _ptr(block_tables2, torch.int32, "block_tables2"),
        block_tables2.shape[1], _ptr(lens2, torch.int32, "lens2"), max_len2,
        *_pool_ptrs(pool4, torch.uint8, "4"), n4, _ptr(block_tables4, torch.int32, "block_tables4"),
        block_tables4.shape[1], _ptr(lens4, torch.int32, "lens4"), max_len4,
        _ptr(k8, torch.int8, "k8"), _ptr(v8, torch.int8, "v8"), _ptr(k8s, torch.float32, "k8_scale"),
        _ptr(v8s, torch.float32, "v8_scale"), n8, _ptr(block_tables8, torch.int32, "block_tables8"),
        block_tables8.shape[1], _ptr(lens8, torch.int32, "lens8"), max_len8,
        kv_bs, nkv, hd, _scale(sm_scale), chunk, _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream(stream))
    _check(st, "kvq2_decode_attn")
    return out
