"""Shared pieces of the GPU parity tests: device copies of seeded inputs,
oracle-side cache construction and the output tolerance of the float path."""
from __future__ import annotations

import numpy as np

import workloads as W
from oracle import kvq8 as O8

SM = float(np.float32(1.0) / np.sqrt(np.float32(128.0)))
ATOL = 1e-4
RTOL = 1e-4


def dev(x, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def assert_attn_close(got, ref, what=""):
    """|gpu - oracle| <= 1e-4 + 1e-4 |oracle| elementwise (float32
    accumulation against the float64 definition)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    excess = np.abs(got - ref) - (ATOL + RTOL * np.abs(ref))
    i = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess.max() <= 0, (f"{what}: |gpu-oracle| = {abs(got[i] - ref[i]):.3e} at {i} "
                               f"(oracle {ref[i]:.6f}); max abs err {np.abs(got - ref).max():.3e}")
    return float(np.abs(got - ref).max())


def pool_columns(n_slots, nkv):
    """The library's storage order of the int8 code pool: the
    column of head kh in the row of slot s (within each aligned group of P
    heads, P the largest power of two dividing nkv, at most 8, the heads
    rotate with the slot).  Steps are not rotated."""
    p = min(nkv & -nkv, 8)
    s = np.arange(n_slots)[:, None]
    kh = np.arange(nkv)[None, :]
    return (kh & ~(p - 1)) | ((kh + s) & (p - 1))


def pool_pages_order(pool):
    """A code pool [n_blocks][kv_bs][nkv][row bytes] as the library stores it
    -> the pages' layout (head kh at column kh), as the oracle keeps it."""
    pool = np.asarray(pool)
    nb, bs, nkv, w = pool.shape
    flat = pool.reshape(nb * bs, nkv, w)
    col = pool_columns(nb * bs, nkv)
    return np.take_along_axis(flat, col[:, :, None], axis=1).reshape(pool.shape)


def pool_library_order(pool):
    """The inverse of pool_pages_order: a pool in the pages' layout -> the
    library's storage order."""
    pool = np.asarray(pool)
    nb, bs, nkv, w = pool.shape
    flat = pool.reshape(nb * bs, nkv, w)
    out = np.empty_like(flat)
    col = pool_columns(nb * bs, nkv)
    np.put_along_axis(out, col[:, :, None], flat, axis=1)
    return out.reshape(pool.shape)


# The library's storage order of an int4 key row: 8-byte part 2c + h holds the
# pages' part 4h + c (pairs 32h + 8c .. +7, codes 64h + 16c .. +15).
Q4_KEY_PAGES_PART = np.array([2 * (p % 4) + p // 4 for p in range(8)])     # pages part p <- library part
Q4_KEY_LIBRARY_PART = np.array([4 * (p % 2) + p // 2 for p in range(8)])   # library part p <- pages part


def q4_key_pages_order(pool):
    """An int4 key pool [..][64] as the library stores it -> the pages' row
    layout (pair i in byte i), as the oracle keeps it."""
    pool = np.asarray(pool)
    return pool.reshape(pool.shape[:-1] + (8, 8))[..., Q4_KEY_PAGES_PART, :].reshape(pool.shape)


def q4_key_library_order(pool):
    """The inverse of q4_key_pages_order."""
    pool = np.asarray(pool)
    return pool.reshape(pool.shape[:-1] + (8, 8))[..., Q4_KEY_LIBRARY_PART, :].reshape(pool.shape)


def head_major(pool):
    """A pool [n_blocks][kv_bs][nkv][..] in the pages' slot-major order (as
    the oracle keeps it) -> the device order of the int4 and 2-bit pools,
    [n_blocks][nkv][kv_bs][..] (the rows of one block and kv-head contiguous)."""
    return np.ascontiguousarray(np.swapaxes(np.asarray(pool), 1, 2))


def slot_major(pool):
    """The inverse of head_major."""
    return np.ascontiguousarray(np.swapaxes(np.asarray(pool), 1, 2))


class Q8Cache:
    """An int8 paged cache held both on the host (oracle) and on the GPU."""

    def __init__(self, n_blocks, kv_bs, nkv, device="cuda"):
        import torch
        self.kv_bs, self.nkv = kv_bs, nkv
        shp = (n_blocks, kv_bs, nkv, 128)
        self.kp = np.zeros(shp, np.int8)
        self.vp = np.zeros(shp, np.int8)
        self.ks = np.zeros(shp[:3], np.float32)
        self.vs = np.zeros(shp[:3], np.float32)
        self.gk = torch.zeros(shp, dtype=torch.int8, device=device)
        self.gv = torch.zeros(shp, dtype=torch.int8, device=device)
        self.gks = torch.zeros(shp[:3], dtype=torch.float32, device=device)
        self.gvs = torch.zeros(shp[:3], dtype=torch.float32, device=device)

    def append(self, k_new, v_new, slots, gk_new=None, gv_new=None):
        """Write the same new rows through the oracle and through the GPU.
        k_new / v_new are float32 host arrays (exact values of the device
        inputs); gk_new / gv_new the device tensors (default: k_new as f32)."""
        import decode_attention_int8_amd as K
        O8.quantize_append(self.kp, self.vp, self.ks, self.vs, k_new, v_new, slots)
        K.kvq8_quantize_append(self.gk, self.gv, self.gks, self.gvs,
                               dev(k_new) if gk_new is None else gk_new,
                               dev(v_new) if gv_new is None else gv_new, dev(np.asarray(slots, np.int32)))

    def assert_device_matches_host(self):
        assert np.array_equal(pool_pages_order(host(self.gk)), self.kp), "K codes differ"
        assert np.array_equal(pool_pages_order(host(self.gv)), self.vp), "V codes differ"
        assert np.array_equal(host(self.gks).view(np.uint32), self.ks.view(np.uint32)), "K steps differ"
        assert np.array_equal(host(self.gvs).view(np.uint32), self.vs.view(np.uint32)), "V steps differ"

    def pull(self):
        """Adopt the device cache as the host cache (after a device-only fill)."""
        self.kp, self.vp = pool_pages_order(host(self.gk)), pool_pages_order(host(self.gv))
        self.ks, self.vs = host(self.gks), host(self.gvs)


def fill_sequences(cache: Q8Cache, bt, lens, k, v):
    """k, v float32 [B][Lmax][nkv][128]: append sequence b's first lens[b]
    tokens at their paged slots."""
    for b, L in enumerate(lens):
        if L == 0:
            continue
        sl = W.slots_for_positions(bt, [b] * L, np.arange(L), cache.kv_bs)
        cache.append(np.ascontiguousarray(k[b, :L]), np.ascontiguousarray(v[b, :L]), sl)
