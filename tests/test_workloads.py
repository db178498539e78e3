"""The seeded synthetic workloads: determinism, shapes and length distributions."""
import math

import numpy as np

import workloads as W
from oracle import replay


def test_deterministic():
    a, b = W.make_config(3, small=True), W.make_config(3, small=True)
    assert a.ops == b.ops and np.array_equal(a.free_order, b.free_order)
    for (ka, va), (kb, vb) in zip(a.kv, b.kv):
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    assert all(np.array_equal(x, y) for x, y in zip(a.q, b.q))


def test_script_without_values_matches():
    for k in (2, 4):
        a = W.make_config(k, small=True)
        b = W.make_config(k, small=True, draw_values=False)
        assert a.ops == b.ops and np.array_equal(a.free_order, b.free_order)


def test_config1_lengths_and_shapes():
    w = W.make_config(1)
    assert sorted(w.final_lengths().values()) == [7, 16, 33, 100]
    assert (w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype, w.num_blocks) == (4, 4, 64, "f32", 64)
    assert w.scale == np.float32(0.125)
    assert sorted(w.free_order.tolist()) == list(range(64))
    att = w.attend_ops()
    assert len(att) == 1 and w.q[att[0][2]].shape == (4, 4, 64)


def test_full_size_length_distributions():
    L2 = np.array(list(W.make_config(2, draw_values=False).final_lengths().values()))
    assert len(L2) == 64 and L2.min() >= 512 and L2.max() <= 4096
    L3 = np.array(list(W.make_config(3, draw_values=False).final_lengths().values()))
    assert len(L3) == 128 and L3.min() >= 1 and L3.max() <= 8192
    assert 1500 < np.median(L3) < 2700
    w4 = W.make_config(4, draw_values=False)
    L4 = np.array(list(w4.final_lengths().values()))
    assert len(L4) == 256 and L4.min() >= 2056 + 64 and L4.max() <= 2056 + 512
    w5 = W.make_config(5, draw_values=False)
    L5 = np.array(list(w5.final_lengths().values()))
    assert len(L5) == 16 and L5.min() >= 16384 + 8 and L5.max() <= 32768 + 8
    assert len(w5.attend_ops()) == 8


def test_pool_sized_with_headroom():
    for k in (2, 3, 5):
        w = W.make_config(k, draw_values=False)
        need = sum(math.ceil(L / 16) for L in w.final_lengths().values())
        assert need <= w.num_blocks <= math.ceil(1.25 * need) + 1


def test_small_configs_replay_on_oracle():
    for k in (1, 2, 3, 4, 5):
        w = W.make_config(k, small=True, draw_values=False)
        r = replay.run(w, compute_attention=False)
        assert r.allocator.num_used() <= w.num_blocks
        for lens, tab in zip(r.context_lens, r.tables):
            assert np.all(lens >= 1)
            nb = -(-lens // 16)
            for row, n in zip(tab, nb):
                assert np.all(row[:n] >= 0) and np.all(row[n:] == -1)
        if k == 4:
            assert sum(len(c) for c in r.copies) == 2 * 7
