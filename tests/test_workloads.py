"""The seeded input generators: determinism, shapes and the recipes' structure."""
import numpy as np
import pytest
import torch

from workloads import configs as W


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125 + 2**-8, -2.5], dtype=np.float32)
    bits = W.f32_to_bf16_bits(x)
    back = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    # 1 + 2^-8 and 1 + 3*2^-8 are ties: the even mantissa wins (1.0, then 1 + 2^-6)
    np.testing.assert_array_equal(back, np.array([1.0, 1.0, 1.0078125, 1.015625, -2.5], np.float32))


def test_config1_matches_its_recipe():
    w = W.make_workload(1)
    assert (w.B, w.H, w.H_kv, w.d, w.dtype, w.num_blocks) == (2, 2, 2, 64, "f32", 16)
    s = w.steps[0]
    assert list(s.context_lens) == [17, 33]
    used = w.block_tables[w.block_tables != W.TABLE_SENTINEL]
    assert len(used) == 5 and len(set(used.tolist())) == 5
    assert w.scale == 0.125


def test_workloads_are_deterministic_per_seed():
    a = W.make_workload(1)
    b = W.make_workload(1)
    c = W.make_workload(1, seed=99)
    np.testing.assert_array_equal(a.k_pool, b.k_pool)
    np.testing.assert_array_equal(a.steps[0].q, b.steps[0].q)
    assert not np.array_equal(a.k_pool, c.k_pool)


def test_scattered_tables_use_distinct_blocks():
    w = W.scattered_workload("t", "bf16", 5, 4, 2, 64, [1, 16, 17, 100, 33], seed=3)
    used = w.block_tables[w.block_tables != W.TABLE_SENTINEL]
    assert len(set(used.tolist())) == len(used) == 1 + 1 + 2 + 7 + 3
    assert used.max() < w.num_blocks


@pytest.mark.slow
def test_shared_prefix_recipe():
    w = W.shared_prefix_workload(5, B=16, steps=50)
    assert np.all(w.block_tables[:, :64] == w.block_tables[0, :64])
    for s, st in enumerate(w.steps):
        assert np.all(st.context_lens >= 1024 + 16 + s + 1)
        assert np.all(st.context_lens <= 1024 + 300 + s + 1)
    last = w.steps[-1].context_lens
    for b in range(w.B):
        nb = -(-int(last[b]) // 16)
        assert np.all(w.block_tables[b, :nb] != W.TABLE_SENTINEL)
    used = w.block_tables[w.block_tables != W.TABLE_SENTINEL]
    private = w.block_tables[:, 64:][w.block_tables[:, 64:] != W.TABLE_SENTINEL]
    assert len(set(private.tolist())) == len(private)      # private blocks not shared
    assert used.max() < w.num_blocks


def test_fp8_workload_shares_shapes_and_draws_valid_codes():
    w8 = W.make_workload(4, kv_dtype="fp8")
    w = W.make_workload(4)
    assert w8.kv_dtype == "fp8" and w8.dtype == "bf16" and w8.name.endswith("-fp8kv")
    assert w8.k_pool.dtype == np.uint8 and w8.kv_elem_bytes == 1
    # same lengths, tables and activations as the bf16 workload
    np.testing.assert_array_equal(w8.block_tables, w.block_tables)
    np.testing.assert_array_equal(w8.steps[0].context_lens, w.steps[0].context_lens)
    np.testing.assert_array_equal(w8.steps[0].q, w.steps[0].q)
    np.testing.assert_array_equal(w8.steps[0].new_k, w.steps[0].new_k)
    # the byte recipe: magnitude codes 0x00..0x3F with either sign, never NaN
    mag = w8.k_pool & 0x7F
    assert int(mag.max()) == W.FP8_MAG_CODES - 1
    assert set(np.unique(w8.v_pool & 0x80).tolist()) == {0, 0x80}
    assert w8.k_scale == 1.0 and w8.v_scale == 1.0
    with pytest.raises(ValueError):
        W.make_workload(1, kv_dtype="fp8")
