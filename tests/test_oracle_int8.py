"""Pins of the oracle's int8 KV cache with per-token scales ("MLSys Engineer -
Inference Systems Q&A", Q3 item 1: scale = the row's largest magnitude / 127,
dequantise before the softmax).  CPU only.

The quantiser is pinned by closed forms that do not restate it: rows built
from integer codes times a power-of-two scale come back exactly; exact ties
go to the even code; negation, power-of-two rescaling and zero rows behave as
the definition forces; every element lies within half a scale of its value.
The cache and decode are pinned against torch: SDPA over rows dequantised as
code * scale, and the bytes the write touches.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from workloads import configs as W


def _bf16(x):
    return W.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_rows_of_integer_codes_times_a_power_of_two_come_back_exactly():
    rng = np.random.default_rng(1)
    for e in (-9, -3, 0, 2):
        codes = rng.integers(-127, 128, size=(50, 64))
        codes[:, 7] = np.where(rng.random(50) < 0.5, 127, -127)   # the row max is 127
        x = codes.astype(np.float32) * np.float32(2.0 ** e)       # exact in bf16 (8 bits)
        got, s = O.int8_quantize_rows(_bf16(x), "bf16")
        assert np.array_equal(got.view(np.int8).astype(np.int64), codes)
        assert np.all(s == np.float32(127 * 2.0 ** e) / np.float32(127))


def test_exact_ties_go_to_the_even_code():
    # scale 1 (row max 127): x = k + 1/2 is an exact tie between k and k + 1
    ks = np.arange(-126, 126)
    x = np.concatenate([[127.0], ks + 0.5]).astype(np.float32)
    got, s = O.int8_quantize_rows(_bf16(x[None, :]), "bf16")
    assert s[0] == 1.0
    want = np.where(ks % 2 == 0, ks, ks + 1)                       # the even neighbour
    assert np.array_equal(got.view(np.int8)[0, 1:].astype(np.int64), want)


def test_negation_rescaling_zero_rows_and_non_finite_elements():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((40, 128)).astype(np.float32)
    c, s = O.int8_quantize_rows(_bf16(x), "bf16")
    cn, sn = O.int8_quantize_rows(_bf16(-x), "bf16")
    assert np.array_equal(cn.view(np.int8), -c.view(np.int8)) and np.array_equal(sn, s)
    c4, s4 = O.int8_quantize_rows(_bf16(x * 4), "bf16")            # power of two: exact
    assert np.array_equal(c4, c) and np.array_equal(s4, s * 4)
    assert np.all(np.abs(c.view(np.int8)).max(axis=1) == 127)     # the largest maps to +-127
    z, sz = O.int8_quantize_rows(_bf16(np.zeros((3, 16))), "bf16")
    assert np.all(z == 0) and np.all(sz == 0)
    y = x[:2].copy()
    y[0, 5], y[1, 9] = np.inf, np.nan
    cy, sy = O.int8_quantize_rows(_bf16(y), "bf16")
    assert cy[0, 5] == 0 and cy[1, 9] == 0                        # non-finite: code 0
    finite_max = np.abs(np.where(np.isfinite(O.bits_to_f64(_bf16(y), "bf16")),
                                 O.bits_to_f64(_bf16(y), "bf16"), 0)).max(axis=1)
    assert np.allclose(sy, finite_max / 127, rtol=1e-7)


def test_every_element_is_within_half_a_scale():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((200, 128)) * rng.uniform(0.01, 100, size=(200, 1))).astype(np.float32)
    xb = O.bits_to_f64(_bf16(x), "bf16")
    c, s = O.int8_quantize_rows(_bf16(x), "bf16")
    err = np.abs(c.view(np.int8) * s[:, None].astype(np.float64) - xb)
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))


@pytest.mark.parametrize("window", [0, 20])
def test_int8_decode_equals_sdpa_over_dequantised_rows(window):
    w = W.scattered_workload("i8", "bf16", 4, 8, 2, 64, [1, 17, 40, 300], seed=4, kv_dtype="int8")
    st, g = w.steps[0], w.group
    slots = O.slot_mapping(w.block_tables, st.context_lens)
    kp, vp = O.reshape_and_cache(w.k_pool, w.v_pool, st.new_k, st.new_v, slots, 2, 64, "int8",
                                 w.num_blocks)
    codes_len = O.int8_codes_bytes(len(kp), 64)
    assert codes_len == w.num_blocks * 2 * 16 * 64
    for b, c in enumerate(st.context_lens):
        c = int(c)
        K = np.zeros((2, c, 64))
        V = np.zeros((2, c, 64))
        for h in range(2):                                         # dequantise through torch
            for t in range(c):
                blk, off = int(w.block_tables[b][t // 16]), t % 16
                kc = torch.from_numpy(kp[O.k_offset(blk, h, off, np.arange(64), 2, 64, "int8")]
                                      .view(np.int8).copy()).double()
                vc = torch.from_numpy(vp[O.v_offset(blk, h, off, np.arange(64), 2, 64, "int8")]
                                      .view(np.int8).copy()).double()
                srow = codes_len + 4 * ((blk * 2 + h) * 16 + off)
                ks = torch.from_numpy(kp[srow:srow + 4].copy()).view(torch.float32).double()
                vs = torch.from_numpy(vp[srow:srow + 4].copy()).view(torch.float32).double()
                K[h, t] = (kc * ks).numpy()
                V[h, t] = (vc * vs).numpy()
        q = O.bits_to_f64(st.q[b], "bf16")
        mask = (np.arange(c) >= (c - window if window else 0))[None, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[:, None, :], torch.from_numpy(K).repeat_interleave(g, 0),
            torch.from_numpy(V).repeat_interleave(g, 0), attn_mask=torch.from_numpy(mask),
            scale=w.scale)[:, 0].numpy()
        got = O.decode_sequence(kp, vp, st.q[b], w.block_tables[b], c, 8, 2, 64, "int8", w.scale,
                                window=window)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_the_write_touches_codes_and_one_scale_per_row():
    """A write of N tokens changes at most N * H_kv * (d + 4) bytes of each
    cache: d one-byte codes and one 4-byte scale per (token, KV head) row, the
    KV-cache size formula with b = 1 plus the row scale."""
    w = W.scattered_workload("i8w", "bf16", 5, 4, 2, 128, [3, 16, 17, 64, 90], seed=5,
                             kv_dtype="int8")
    st = w.steps[0]
    slots = O.slot_mapping(w.block_tables, st.context_lens)
    kp, vp = O.reshape_and_cache(w.k_pool, w.v_pool, st.new_k, st.new_v, slots, 2, 128, "int8",
                                 w.num_blocks)
    for old, new in ((w.k_pool, kp), (w.v_pool, vp)):
        assert np.count_nonzero(old != new) <= 5 * 2 * (128 + 4)
        assert len(new) == w.num_blocks * 2 * 16 * (128 + 4)


def test_planted_quantiser_mistakes_are_caught(monkeypatch):
    real = O.pagedkv_oracle.int8_quantize_rows

    def per_tensor(bits, dtype):                 # one scale for the whole batch
        c, s = real(bits, dtype)
        x = O.bits_to_f64(bits, dtype).astype(np.float32)
        st = np.float32(np.abs(x).max() / 127)
        q = np.clip(np.rint(x / st), -127, 127).astype(np.int8).view(np.uint8)
        return q, np.full_like(s, st)

    def truncating(bits, dtype):                 # rounds toward zero
        x = O.bits_to_f64(bits, dtype).astype(np.float32)
        a = np.abs(x).max(axis=-1)
        s = (a / np.float32(127)).astype(np.float32)
        q = np.trunc(x / s[..., None])
        return np.clip(q, -127, 127).astype(np.int8).view(np.uint8), s

    def by_128(bits, dtype):                     # 128 levels instead of 127
        x = O.bits_to_f64(bits, dtype).astype(np.float32)
        a = np.abs(x).max(axis=-1)
        s = (a / np.float32(128)).astype(np.float32)
        q = np.rint(x / s[..., None])
        return np.clip(q, -127, 127).astype(np.int8).view(np.uint8), s

    for wrong in (per_tensor, truncating, by_128):
        monkeypatch.setattr(O, "int8_quantize_rows", wrong)
        monkeypatch.setattr(O.pagedkv_oracle, "int8_quantize_rows", wrong)
        with pytest.raises(AssertionError):
            test_rows_of_integer_codes_times_a_power_of_two_come_back_exactly()
            test_exact_ties_go_to_the_even_code()
            test_negation_rescaling_zero_rows_and_non_finite_elements()
    monkeypatch.setattr(O, "int8_quantize_rows", real)
    monkeypatch.setattr(O.pagedkv_oracle, "int8_quantize_rows", real)
