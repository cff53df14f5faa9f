"""The seeded input generators: determinism, shapes and bookkeeping."""
import numpy as np

import workloads as W


def test_seeded_and_distinct():
    a = W.unit_experiment(3)
    b = W.unit_experiment(3)
    c = W.unit_experiment(4)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[1], c[1])
    assert a[0].shape == (128,) and a[1].shape == (256, 128) and a[1].dtype == np.float32


def test_bf16_rounding_is_exact_bf16():
    r = W.rng(9)
    x = W.outlier_normal_bf16(r, (1000, 128))
    bits = x.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    assert 0.003 < np.mean(np.abs(x) > 6) < 0.02          # about 1% outliers x20
    assert W.round_to_bf16(np.array([1.0 + 2 ** -8], np.float32))[0] == 1.0          # tie -> even
    assert W.round_to_bf16(np.array([1.0 + 3 * 2 ** -8], np.float32))[0] == 1.0 + 2 ** -6


def test_block_tables_and_slots():
    r = W.rng(10)
    lens = np.array([5, 0, 33])
    bt, nb = W.paged_block_tables(r, lens, 16, spare_blocks=2)
    assert nb == 1 + 0 + 3 + 2 and bt.shape == (3, 3)
    used = bt[bt >= 0]
    assert len(set(used.tolist())) == len(used) == 4
    assert np.all(bt[1] == -1)
    s = W.slots_for_positions(bt, [2, 2], [0, 17], 16)
    assert s.tolist() == [bt[2, 0] * 16, bt[2, 1] * 16 + 1]


def test_lengths_in_range():
    L = W.qwen8b_lengths(0)
    assert L.shape == (32,) and L.min() >= 1024 and L.max() <= 32768
