"""Pins of the oracle's multi-token attention (a prefill chunk or a block of
draft tokens per sequence, causal within it) and of its chunk slot mapping.
CPU only."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from workloads import configs as W


def _step(w):
    """The oracle's write of the step's rows, then its multi-token output."""
    m = w.multi
    slots = O.chunk_slots(w.block_tables, m.context_lens, m.query_start)
    kp, vp = O.reshape_and_cache(w.k_pool, w.v_pool, m.new_k, m.new_v, slots, w.H_kv, w.d,
                                 w.kv_dtype, w.num_blocks, w.k_scale, w.v_scale)
    out = O.decode_multi(kp, vp, m.q, m.query_start, w.block_tables, m.context_lens, w.H,
                         w.H_kv, w.d, w.kv_dtype, w.scale, w.k_scale, w.v_scale)
    return kp, vp, out


CASES = [
    dict(H=4, H_kv=4, d=64, ctx=[20, 5, 40, 33], n=[4, 5, 1, 16]),
    dict(H=8, H_kv=2, d=128, ctx=[17, 64, 3], n=[17, 3, 2]),
    dict(H=6, H_kv=3, d=64, ctx=[50], n=[32]),
]


@pytest.mark.parametrize("c", CASES)
def test_chunk_equals_sdpa_with_an_explicit_causal_mask(c):
    w = W.multi_token_workload("m", "bf16", len(c["ctx"]), c["H"], c["H_kv"], c["d"], c["ctx"],
                               c["n"], seed=5)
    kp, vp, out = _step(w)
    m, g = w.multi, c["H"] // c["H_kv"]
    for b, (ctx, n) in enumerate(zip(c["ctx"], c["n"])):
        K = np.stack([O.gather_sequence(kp, vp, w.block_tables[b], ctx, kvh, w.H_kv, w.d, "bf16")[0]
                      for kvh in range(w.H_kv)])                       # [H_kv, ctx, d]
        V = np.stack([O.gather_sequence(kp, vp, w.block_tables[b], ctx, kvh, w.H_kv, w.d, "bf16")[1]
                      for kvh in range(w.H_kv)])
        Q = O.bits_to_f64(m.q[m.query_start[b]:m.query_start[b + 1]], "bf16")   # [n, H, d]
        mask = np.arange(ctx)[None, :] <= (ctx - n + np.arange(n))[:, None]     # [n, ctx]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q).permute(1, 0, 2),                                # [H, n, d]
            torch.from_numpy(K).repeat_interleave(g, 0),
            torch.from_numpy(V).repeat_interleave(g, 0),
            attn_mask=torch.from_numpy(mask), scale=w.scale).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-13)


def test_each_chunk_row_equals_a_decode_at_its_own_position():
    c = CASES[1]
    w = W.multi_token_workload("m", "bf16", 3, c["H"], c["H_kv"], c["d"], c["ctx"], c["n"], seed=6)
    kp, vp, out = _step(w)
    m = w.multi
    for b, (ctx, n) in enumerate(zip(c["ctx"], c["n"])):
        for j in range(n):
            one = O.decode_sequence(kp, vp, m.q[m.query_start[b] + j], w.block_tables[b],
                                    ctx - n + j + 1, w.H, w.H_kv, w.d, "bf16", w.scale)
            np.testing.assert_array_equal(out[b][j], one)


def test_one_token_chunks_are_the_decode_step():
    w = W.multi_token_workload("m", "bf16", 4, 8, 2, 64, [1, 16, 17, 90], [1, 1, 1, 1], seed=7)
    kp, vp, out = _step(w)
    m = w.multi
    assert np.array_equal(O.chunk_slots(w.block_tables, m.context_lens, m.query_start),
                          O.slot_mapping(w.block_tables, m.context_lens))
    ref = O.decode(kp, vp, m.q.reshape(4, 1, 8, 64)[:, 0], w.block_tables, m.context_lens, 8, 2,
                   64, "bf16", w.scale)
    for b in range(4):
        np.testing.assert_array_equal(out[b][0], ref[b])


def test_chunk_slots_follow_each_position_through_the_table():
    w = W.multi_token_workload("m", "bf16", 3, 4, 4, 64, [40, 7, 33], [20, 7, 0], seed=8)
    m = w.multi
    got = O.chunk_slots(w.block_tables, m.context_lens, m.query_start)
    want = []
    for b, (ctx, n) in enumerate(zip([40, 7, 33], [20, 7, 0])):
        for pos in range(ctx - n, ctx):                 # brute force: walk the table
            blk = w.block_tables[b][pos // 16]
            want.append(int(blk) * 16 + pos % 16)
    assert got.tolist() == want


def test_fp8_chunk_matches_the_dequantized_definition():
    w = W.multi_token_workload("m8", "bf16", 2, 8, 2, 128, [30, 19], [6, 19], seed=9,
                               kv_dtype="fp8", k_scale=0.5, v_scale=1.5)
    kp, vp, out = _step(w)
    m = w.multi
    for b, (ctx, n) in enumerate(zip([30, 19], [6, 19])):
        for j in range(n):
            one = O.decode_sequence(kp, vp, m.q[m.query_start[b] + j], w.block_tables[b],
                                    ctx - n + j + 1, 8, 2, 128, "fp8", w.scale, 0.5, 1.5)
            np.testing.assert_array_equal(out[b][j], one)


def test_planted_mistakes_are_caught(monkeypatch):
    """A chunk that sees every key (no causal mask) or misses its own position
    breaks the SDPA pin."""
    c = CASES[0]
    w = W.multi_token_workload("m", "bf16", len(c["ctx"]), c["H"], c["H_kv"], c["d"], c["ctx"],
                               c["n"], seed=5)
    real = O.pagedkv_oracle.decode_multi

    def no_mask(kp, vp, q_rows, qs, tables, ctx, H, H_kv, d, dtype, scale, *a, **k):
        # every row attends to the whole context
        return {b: np.stack([O.decode_sequence(kp, vp, q_rows[qs[b] + j], tables[b], int(ctx[b]),
                                                H, H_kv, d, dtype, scale)
                             for j in range(int(qs[b + 1] - qs[b]))]) for b in range(len(ctx))}

    def exclusive(kp, vp, q_rows, qs, tables, ctx, H, H_kv, d, dtype, scale, *a, **k):
        # a row sees positions 0..p-1 only (the first row of a sequence keeps one key)
        return {b: np.stack([O.decode_sequence(kp, vp, q_rows[qs[b] + j], tables[b],
                                                max(int(ctx[b]) - int(qs[b + 1] - qs[b]) + j, 1),
                                                H, H_kv, d, dtype, scale)
                             for j in range(int(qs[b + 1] - qs[b]))]) for b in range(len(ctx))}

    for wrong in (no_mask, exclusive):
        monkeypatch.setattr(O, "decode_multi", wrong)
        with pytest.raises(AssertionError):
            test_chunk_equals_sdpa_with_an_explicit_causal_mask(c)
    monkeypatch.setattr(O, "decode_multi", real)
