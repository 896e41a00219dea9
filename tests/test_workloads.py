"""The seeded input generator: determinism and the structure the recipes ask for."""
import numpy as np

from paged_fp8_split_amd import workloads as W


def test_same_seed_same_bytes():
    a = W.config(1)
    b = W.config(1)
    for f in ("q_fp16", "k_pool", "v_pool", "k_scale", "v_scale", "block_table", "live_len", "head_map"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = W.config(1, seed=99)
    assert not np.array_equal(a.k_pool, c.k_pool)


def test_config1_shape_and_scale_recipe():
    w = W.config(1)
    assert (w.batch, w.q, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size) == (1, 8, 4, 1, 64, 16)
    assert int(w.live_len[0]) == 1024 + 8
    # one per-tensor scale = absmax / 448; the largest live code is 448 (0x7E or 0xFE)
    view = w.pool_view(w.k_pool)
    t = np.arange(1032)
    live = view[w.block_table[0, t // 16], t % 16]
    assert (live & 0x7F).max() == 0x7E
    assert w.k_scale.dtype == np.float32 and w.k_scale.shape == (1,)
    # pages are a permutation: no physical page is used twice
    used = w.block_table[0, : -(-1032 // 16)]
    assert len(set(used.tolist())) == len(used)


def test_config4_lengths_and_retired_rows():
    L = W._cfg4_lengths(4)
    assert L.shape == (32,) and (L == 0).sum() == 2
    nz = L[L > 0]
    assert nz.min() >= 1024 and nz.max() <= 32768


def test_relocate_keeps_logical_content():
    w = W.build(seed=1, batch=2, q=4, num_q_heads=2, num_kv_heads=1, head_dim=16, page_size=16, lengths=[40, 17])
    r = W.relocate(w, 5)
    for b, L in enumerate(w.live_len):
        t = np.arange(L)
        a = w.pool_view(w.k_pool)[w.block_table[b, t // 16], t % 16]
        c = r.pool_view(r.k_pool)[r.block_table[b, t // 16], t % 16]
        assert np.array_equal(a, c)
    assert not np.array_equal(w.block_table, r.block_table)


def test_midpoint_slot_counts():
    w = W.build(seed=2, batch=1, q=1, num_q_heads=2, num_kv_heads=1, head_dim=8, page_size=64, lengths=[1024],
                midpoint={"b": 0, "g": 0, "counts": [4, 12]})
    t = np.arange(1024)
    v = w.pool_view(w.v_pool)[w.block_table[0, t // 64], t % 64, 0]
    k = w.pool_view(w.k_pool)[w.block_table[0, t // 64], t % 64, 0]
    assert np.all(k == 0)
    assert set(np.unique(v).tolist()) == {0x38, 0x39}
    assert [(v[:, d] == 0x39).sum() for d in range(4)] == [4, 12, 4, 12]


def test_outlier_fraction():
    w = W.build(seed=3, batch=1, q=8, num_q_heads=2, num_kv_heads=1, head_dim=32, page_size=16, lengths=[2000],
                outlier_frac=0.01)
    # outlier tokens dominate the per-head absmax, so ordinary tokens quantize
    # to small codes; about 1% of tokens hold codes of 128 or more
    t = np.arange(2000)
    k = w.pool_view(w.k_pool)[w.block_table[0, t // 16], t % 16, 0].view(np.int8)
    big = (k.view(np.uint8) & 0x7F) >= 0x70  # |code| >= 128: about 9 sigma of an ordinary token
    frac = big.any(axis=1).mean()
    assert 0.005 < frac < 0.02
