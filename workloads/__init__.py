"""Seeded synthetic inputs for int8 / int4 KV-cache decode attention.

This module only draws random numbers and lays out paged-cache bookkeeping
(block tables, slot indices).  It holds none of the method's arithmetic: no
quantization, no dot products, no softmax.  Both the CPU oracle's callers and
the GPU path's callers take their inputs from here, so the two sides always see
the same bytes.

Shapes follow the source pages' models (head dim 128; Qwen3-VL-2B-like 28
layers x 16 query / 8 kv heads; Qwen3-VL-8B-like 36 layers x 32 / 8) and the
pages' unit experiment (one head, 256 tokens, N(0, 1) data).

Every generator takes explicit integer seeds.  numpy generators use
``default_rng(SeedSequence(key))``; torch generators use a ``torch.Generator``
seeded from the same key, so a given key always yields the same tensor on a
given device type.
"""
from __future__ import annotations

import numpy as np

HD = 128


# ----------------------------------------------------------------------------
# numpy (host) generators
# ----------------------------------------------------------------------------

def rng(*key: int) -> np.random.Generator:
    """A numpy Generator keyed by a tuple of non-negative integers."""
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def normal_f32(r: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    """i.i.d. N(0, sigma^2), drawn in float64 and rounded once to float32."""
    return (sigma * r.standard_normal(shape)).astype(np.float32)


def student_t3_f32(r: np.random.Generator, shape, scale: float = 0.5) -> np.ndarray:
    """scale * Student-t(nu=3), built as Z / sqrt(chi2_3 / 3) from normals."""
    shape = tuple(np.atleast_1d(shape)) if not isinstance(shape, tuple) else shape
    z = r.standard_normal(shape)
    c = (r.standard_normal(shape + (3,)) ** 2).sum(-1) / 3.0
    return (scale * z / np.sqrt(c)).astype(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as
    float32 holding exactly those bfloat16 values.  Used to make bf16 inputs
    whose float32 widening is exact on both sides."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x_bf16_valued: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are exact bfloat16 numbers."""
    u = np.ascontiguousarray(x_bf16_valued, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


def outlier_normal_bf16(r: np.random.Generator, shape, p: float = 0.01, factor: float = 20.0) -> np.ndarray:
    """N(0, 1) with each element independently multiplied by ``factor`` with
    probability ``p``; rounded once to bf16 (returned as float32)."""
    x = r.standard_normal(shape)
    m = r.random(shape) < p
    x = np.where(m, x * factor, x)
    return round_to_bf16(x.astype(np.float32))


def per_unit_sigma_normal(r: np.random.Generator, shape, unit_axes: int, lo: float, hi: float) -> np.ndarray:
    """N(0, 1) scaled by a sigma drawn U[lo, hi] per leading index over the
    first ``unit_axes`` axes (e.g. per (sequence, kv-head))."""
    sig = r.uniform(lo, hi, size=shape[:unit_axes])
    x = r.standard_normal(shape)
    return (x * sig.reshape(sig.shape + (1,) * (len(shape) - unit_axes))).astype(np.float32)


def uniform_lengths(r: np.random.Generator, batch: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths drawn uniformly from the integers in [lo, hi]."""
    return r.integers(lo, hi + 1, size=batch).astype(np.int32)


# ----------------------------------------------------------------------------
# paged-cache bookkeeping
# ----------------------------------------------------------------------------

def paged_block_tables(r: np.random.Generator | None, ctx_lens, kv_bs: int, spare_blocks: int = 0,
                       capacity_tokens: int | None = None):
    """Assign physical cache blocks to sequences.

    Each sequence b gets ceil(cap_b / kv_bs) blocks, cap_b = max(ctx_lens[b],
    capacity_tokens or 0).  Physical ids are a random permutation when ``r`` is
    given (pages scattered through the pool), else identity order.  Unused
    table entries are -1.

    Returns (block_tables int32 [B][max_blocks_per_seq], n_blocks).
    """
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    caps = np.maximum(ctx_lens, capacity_tokens or 0)
    nb = (caps + kv_bs - 1) // kv_bs
    total = int(nb.sum()) + spare_blocks
    ids = r.permutation(total) if r is not None else np.arange(total)
    mb = max(1, int(nb.max()) if len(nb) else 1)
    bt = np.full((len(ctx_lens), mb), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(nb):
        bt[b, :n] = ids[pos:pos + n]
        pos += n
    return bt, total


def slots_for_positions(block_tables: np.ndarray, seq_ids, positions, kv_bs: int) -> np.ndarray:
    """Cache slot (block_id * kv_bs + offset) of token ``positions[i]`` of
    sequence ``seq_ids[i]`` under ``block_tables``."""
    seq_ids = np.asarray(seq_ids, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    blk = block_tables[seq_ids, positions // kv_bs].astype(np.int64)
    return (blk * kv_bs + positions % kv_bs).astype(np.int32)


# ----------------------------------------------------------------------------
# torch (device) generators, for the full-size workloads
# ----------------------------------------------------------------------------

def torch_generator(device, *key: int):
    import torch
    g = torch.Generator(device=device)
    s = np.random.SeedSequence([int(k) for k in key]).generate_state(2, dtype=np.uint32)
    g.manual_seed(int(s[0]) << 32 | int(s[1]))
    return g


def torch_normal(shape, device, key, sigma: float = 1.0, dtype=None):
    import torch
    g = torch_generator(device, *key)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x if dtype is None else x.to(dtype)


def torch_student_t3(shape, device, key, scale: float = 0.5):
    import torch
    g = torch_generator(device, *key)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    c = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(3):
        e = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        c.addcmul_(e, e)
    return z.mul_(scale).div_(torch.sqrt(c.div_(3.0)))


def torch_outlier_normal_bf16(shape, device, key, p: float = 0.01, factor: float = 20.0):
    import torch
    g = torch_generator(device, *key)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    m = torch.rand(shape, generator=g, device=device) < p
    x = torch.where(m, x * factor, x)
    return x.to(torch.bfloat16)


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

# Pages' unit experiment: 1 query head / 1 kv head, L = 256, N(0, 1).
UNIT = dict(nq=1, nkv=1, L=256)
# Qwen3-VL-2B-shaped decode, batch 1, 8K context.
QWEN2B_8K = dict(layers=28, nq=16, nkv=8, batch=1, L=8192, kv_bs=16)
# Qwen3-VL-8B-shaped batched decode, 32 sequences with lengths in [1024, 32768].
QWEN8B_B32 = dict(layers=36, nq=32, nkv=8, batch=32, L_lo=1024, L_hi=32768, kv_bs=16)
# Write path: 65536 new tokens x 8 kv heads, then one GQA-4 decode step over them.
APPEND_64K = dict(n_tok=65536, nq=32, nkv=8, kv_bs=16)
# int4 group variant: 32 / 4 heads, batch 4, 128K context, last 2048 tokens int8.
Q4_128K = dict(nq=32, nkv=4, batch=4, L=131072, window=2048, kv_bs=16, group=64)
# The same shape with the page's three-band schedule: the newest 2048 tokens
# int8, those up to 16384 from the newest int4, all older ones 2-bit.
Q2_128K = dict(nq=32, nkv=4, batch=4, L=131072, window=2048, edge4=16384, kv_bs=16, group=64)


def unit_experiment(seed: int = 0, sigma: float = 1.0):
    """q [128], k, v [256][128] float32 i.i.d. N(0, sigma^2) (q is N(0, 1))."""
    r = rng(1, seed)
    q = normal_f32(r, (HD,))
    k = normal_f32(r, (UNIT["L"], HD), sigma)
    v = normal_f32(r, (UNIT["L"], HD), sigma)
    return q, k, v


def qwen8b_lengths(seed: int = 0) -> np.ndarray:
    return uniform_lengths(rng(3, seed), QWEN8B_B32["batch"], QWEN8B_B32["L_lo"], QWEN8B_B32["L_hi"])
