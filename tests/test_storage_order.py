"""The library's storage orders, as the header states them, against the test
helpers that convert device pools to the pages' layout (CPU only):

* int4 key rows: the pair starting at element 64h + 16c + 2j (h = 0, 1;
  c = 0..3; j = 0..7) sits in byte 16c + 8h + j, even element in the high
  nibble; the pages' layout (the oracle's) keeps pair i in byte i.
* int8 code pools: head kh of slot s at column (kh & ~(P-1)) |
  ((kh + s) & (P-1)), P the largest power of two dividing nkv, at most 8.
* int4, 2-bit and Q4_0 pools: head-major inside each block, slot s of head
  kh at row (s / kv_bs * nkv + kh) * kv_bs + s % kv_bs."""
import numpy as np

from oracle import kvq4 as O4
from tests.helpers import (head_major, pool_columns, pool_library_order, pool_pages_order, q4_key_library_order,
                           q4_key_pages_order, slot_major)


def test_q4_key_order_matches_header_formula():
    codes = (np.arange(128) * 7 + 3) % 16                    # every pair distinct enough to locate
    pages = O4.pack_nibbles(codes.astype(np.uint8))          # pair i in byte i
    lib = q4_key_library_order(pages[None])[0]
    for h in range(2):
        for c in range(4):
            for j in range(8):
                e = 64 * h + 16 * c + 2 * j
                assert lib[16 * c + 8 * h + j] == (codes[e] << 4 | codes[e + 1]), (h, c, j)
    assert np.array_equal(q4_key_pages_order(lib[None])[0], pages)


def test_q4_key_order_round_trip():
    r = np.random.default_rng(3)
    x = r.integers(0, 256, (5, 16, 3, 64), dtype=np.uint8)
    assert np.array_equal(q4_key_pages_order(q4_key_library_order(x)), x)
    assert np.array_equal(q4_key_library_order(q4_key_pages_order(x)), x)
    assert not np.array_equal(q4_key_library_order(x), x)


def test_int8_rotation_matches_header_formula():
    for nkv in range(1, 17):
        p = 1
        while nkv % (2 * p) == 0 and 2 * p <= 8:
            p *= 2
        col = pool_columns(40, nkv)
        for s in range(40):
            assert sorted(col[s]) == list(range(nkv))        # a permutation of the row's columns
            for kh in range(nkv):
                assert col[s, kh] == (kh & ~(p - 1)) | ((kh + s) & (p - 1))
        x = np.random.default_rng(nkv).integers(-127, 128, (5, 8, nkv, 128)).astype(np.int8)
        assert np.array_equal(pool_pages_order(pool_library_order(x)), x)


def test_head_major_rows_match_header_formula():
    """The int4 / 2-bit pools keep slot s = block * kv_bs + offset of kv-head
    kh in row (block * nkv + kh) * kv_bs + offset (include/kvq8.h); the tests'
    conversion from the oracle's slot-major arrays must put it there."""
    nb, bs, nkv = 3, 8, 5
    slot = np.arange(nb * bs).reshape(nb, bs, 1)
    kh = np.arange(nkv).reshape(1, 1, nkv)
    x = (slot * 100 + kh).astype(np.int64)              # [n_blocks][kv_bs][nkv], one value per (slot, head)
    rows = head_major(x).reshape(-1)
    for s in range(nb * bs):
        for h in range(nkv):
            assert rows[((s // bs) * nkv + h) * bs + s % bs] == s * 100 + h
    assert np.array_equal(slot_major(head_major(x)), x)
