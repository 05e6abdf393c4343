"""Pins of the oracle's sliding-window attention (a query at position p sees
positions max(0, p - W + 1) .. p; "MLSys Engineer - Inference Systems Q&A",
Q3 item 4 and Q4's tile-skipping rule).  CPU only.

Each pin checks the window against something other than the oracle's own
slicing: PyTorch's scaled_dot_product_attention with an explicit boolean mask
over the whole context, the closed form of a one-key window, the invariance
to every row outside the window (NaN there changes nothing), and the split
partials merged by the reduce.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from workloads import configs as W

CTX = [1, 15, 16, 17, 40, 129, 300]


def _work(H=8, H_kv=2, d=64, ctx=CTX, seed=3, kv="bf16"):
    return W.scattered_workload("win", "bf16", len(ctx), H, H_kv, d, ctx, seed=seed,
                                kv_dtype=kv, k_scale=0.5 if kv == "fp8" else 1.0,
                                v_scale=1.5 if kv == "fp8" else 1.0)


def _dense(w, b):
    """De-paged K, V [H_kv, ctx, d] of sequence b (float64)."""
    c = int(w.steps[0].context_lens[b])
    KV = [O.gather_sequence(w.k_pool, w.v_pool, w.block_tables[b], c, h, w.H_kv, w.d,
                            w.kv_dtype, w.k_scale, w.v_scale) for h in range(w.H_kv)]
    return np.stack([k for k, _ in KV]), np.stack([v for _, v in KV])


@pytest.mark.parametrize("window", [1, 7, 16, 17, 100])
def test_window_equals_sdpa_with_a_banded_mask(window):
    w = _work()
    st, g = w.steps[0], w.group
    for b, c in enumerate(CTX):
        K, V = _dense(w, b)
        q = O.bits_to_f64(st.q[b], "bf16")                          # [H, d]
        pos = np.arange(c)
        mask = (pos >= c - window)[None, None, :]                   # [1, 1, ctx]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[:, None, :], torch.from_numpy(K).repeat_interleave(g, 0),
            torch.from_numpy(V).repeat_interleave(g, 0),
            attn_mask=torch.from_numpy(mask), scale=w.scale)[:, 0].numpy()
        got = O.decode_sequence(w.k_pool, w.v_pool, st.q[b], w.block_tables[b], c, w.H, w.H_kv,
                                w.d, "bf16", w.scale, window=window)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_window_of_one_key_is_the_newest_value_row():
    w = _work()
    st, g = w.steps[0], w.group
    for b, c in enumerate(CTX):
        _, V = _dense(w, b)
        got = O.decode_sequence(w.k_pool, w.v_pool, st.q[b], w.block_tables[b], c, w.H, w.H_kv,
                                w.d, "bf16", w.scale, window=1)
        np.testing.assert_array_equal(got, np.repeat(V[:, c - 1], g, axis=0))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_window_covering_the_context_is_the_full_decode(kv):
    w = _work(kv=kv)
    st = w.steps[0]
    full = O.decode(w.k_pool, w.v_pool, st.q, w.block_tables, st.context_lens, w.H, w.H_kv, w.d,
                    kv, w.scale, w.k_scale, w.v_scale)
    for window in (max(CTX), max(CTX) + 5, 1 << 20):
        got = O.decode(w.k_pool, w.v_pool, st.q, w.block_tables, st.context_lens, w.H, w.H_kv,
                       w.d, kv, w.scale, w.k_scale, w.v_scale, window=window)
        np.testing.assert_array_equal(got, full)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_rows_before_the_window_are_never_read(kv):
    """NaN in every row before the window leaves the output bit-identical;
    NaN in the window's first row does not."""
    w = _work(kv=kv)
    st = w.steps[0]
    nan = {"bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}[kv]
    xs = np.arange(w.d)
    window = 9
    for b, c in enumerate(CTX):
        if c <= window:
            continue
        kp, vp = w.k_pool.copy(), w.v_pool.copy()
        for pos in range(c - window):
            blk = int(w.block_tables[b][pos // 16])
            for h in range(w.H_kv):
                kp[O.k_offset(blk, h, pos % 16, xs, w.H_kv, w.d, kv)] = nan
                vp[O.v_offset(blk, h, pos % 16, xs, w.H_kv, w.d, kv)] = nan
        args = (st.q[b], w.block_tables[b], c, w.H, w.H_kv, w.d, kv, w.scale, w.k_scale,
                w.v_scale)
        clean = O.decode_sequence(w.k_pool, w.v_pool, *args, window=window)
        np.testing.assert_array_equal(O.decode_sequence(kp, vp, *args, window=window), clean)
        pos = c - window                                    # the window's first row
        blk = int(w.block_tables[b][pos // 16])
        vp[O.v_offset(blk, 0, pos % 16, xs, w.H_kv, w.d, kv)] = nan
        assert np.isnan(O.decode_sequence(kp, vp, *args, window=window)).any()


@pytest.mark.parametrize("P", [16, 32, 64])
@pytest.mark.parametrize("window", [5, 16, 33, 120])
def test_windowed_partials_reduce_to_the_windowed_decode(P, window):
    w = _work(seed=8)
    st = w.steps[0]
    args = (w.k_pool, w.v_pool, st.q, w.block_tables, st.context_lens, w.H, w.H_kv, w.d, "bf16",
            w.scale)
    o, m, l, counts = O.partials(*args, partition_size=P, window=window)
    ref = O.decode(*args, window=window)
    np.testing.assert_allclose(O.reduce(o, m, l, counts), ref, rtol=1e-12, atol=1e-14)
    for b, c in enumerate(CTX):
        first = max(0, c - window)
        r = first // 16 * 16                            # the block holding the first position
        # brute force: the partitions [r + kP, r + (k+1)P) that hold a visible position
        want = sum(1 for k in range(c // P + 2) if r + k * P < c)
        assert counts[b] == want
        assert np.isfinite(m[b, :, :counts[b]]).all()   # no partition is wholly masked


@pytest.mark.parametrize("window", [1, 6, 16, 40])
def test_windowed_chunk_rows_equal_sdpa_and_decodes(window):
    ctx, n = [20, 50, 33], [4, 17, 33]
    wk = W.multi_token_workload("mw", "bf16", 3, 8, 2, 64, ctx, n, seed=12)
    m, g = wk.multi, wk.group
    sl = O.chunk_slots(wk.block_tables, m.context_lens, m.query_start)
    kp, vp = O.reshape_and_cache(wk.k_pool, wk.v_pool, m.new_k, m.new_v, sl, 2, 64, "bf16",
                                 wk.num_blocks)
    out = O.decode_multi(kp, vp, m.q, m.query_start, wk.block_tables, m.context_lens, 8, 2, 64,
                         "bf16", wk.scale, window=window)
    for b, (c, k) in enumerate(zip(ctx, n)):
        KV = [O.gather_sequence(kp, vp, wk.block_tables[b], c, h, 2, 64, "bf16") for h in (0, 1)]
        K = np.stack([x for x, _ in KV])
        V = np.stack([y for _, y in KV])
        Q = O.bits_to_f64(m.q[m.query_start[b]:m.query_start[b + 1]], "bf16")   # [k, H, d]
        p = c - k + np.arange(k)
        t = np.arange(c)
        mask = (t[None, :] <= p[:, None]) & (t[None, :] > p[:, None] - window)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q).permute(1, 0, 2), torch.from_numpy(K).repeat_interleave(g, 0),
            torch.from_numpy(V).repeat_interleave(g, 0), attn_mask=torch.from_numpy(mask),
            scale=wk.scale).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-13)
        for j in range(k):
            one = O.decode_sequence(kp, vp, m.q[m.query_start[b] + j], wk.block_tables[b],
                                    c - k + j + 1, 8, 2, 64, "bf16", wk.scale, window=window)
            np.testing.assert_array_equal(out[b][j], one)


def test_planted_off_by_one_windows_are_caught(monkeypatch):
    real = O.pagedkv_oracle.window_first
    for wrong in (lambda pos, w: max(0, int(pos) - int(w)) if w > 0 else 0,       # W + 1 keys
                  lambda pos, w: max(0, int(pos) - int(w) + 2) if w > 0 else 0):  # W - 1 keys
        monkeypatch.setattr(O.pagedkv_oracle, "window_first", wrong)
        with pytest.raises(AssertionError):
            test_window_equals_sdpa_with_a_banded_mask(7)
        with pytest.raises((AssertionError, ValueError)):   # W - 1 = 0 keys cannot reduce
            test_window_of_one_key_is_the_newest_value_row()
    monkeypatch.setattr(O.pagedkv_oracle, "window_first", real)
