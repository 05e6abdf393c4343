"""GPU parity of sliding-window attention ("MLSys Engineer - Inference Systems
Q&A", Q3 item 4 and Q4): the decode query sees the last `window` positions,
each multi-token row the `window` positions ending at its own.

Every case checks the step's writes bit for bit, then the outputs against the
float64 oracle (bf16: rel-L2 <= 5e-3, max-abs <= 1e-2; fp32: max-abs <= 1e-5).
What lies before the window is made unusable on the GPU side: every position
before the first visible one holds NaN, and the table entries of blocks wholly
before the window hold an index outside the pool, so a kernel that loaded such
a block would report NaN for the sequence.  The oracle keeps the real table
(it reads only the window's rows).
"""
import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_33_amd as P
from workloads import configs as W

from _harness import (NAN_BITS, assert_close, from_dev, log, poison, to_dev, upload)
from test_gpu_multi import assert_rows_close

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 250, 700, 1100]
WINDOWS = [1, 7, 16, 17, 128, 1000]


def _hide_before(w, kp, vp, tables, first):
    """NaN in every position < first[b] (an int8 pool: NaN row scales, its
    codes cannot be NaN); table entries of blocks wholly before it set outside
    the pool (GPU copies only)."""
    xs = np.arange(w.d)
    tables = tables.copy()
    for b in range(w.B):
        f = int(first[b])
        for pos in range((f // 16) * 16, f):          # the window's first block, before it
            blk = int(w.block_tables[b][pos // 16])
            for h in range(w.H_kv):
                if w.kv_dtype == "int8":
                    for pool in (kp, vp):
                        O.int8_write_scales(pool, O.int8_scale_offset(blk, h, pos % 16, w.H_kv,
                                                                      w.d, len(pool)), [np.nan])
                    continue
                nan = NAN_BITS[w.kv_dtype]
                kp[O.k_offset(blk, h, pos % 16, xs, w.H_kv, w.d, w.kv_dtype)] = nan
                vp[O.v_offset(blk, h, pos % 16, xs, w.H_kv, w.d, w.kv_dtype)] = nan
        tables[b, :f // 16] = w.num_blocks + 1000
    return tables


def _decode_case(w, window, part, label):
    st = w.steps[0]
    ctx = st.context_lens.astype(np.int64)
    kp0, vp0 = poison(w, np.maximum(ctx - 1, 0))
    slots = O.slot_mapping(w.block_tables, st.context_lens)
    kp, vp = O.reshape_and_cache(kp0, vp0, st.new_k, st.new_v, slots, w.H_kv, w.d, w.kv_dtype,
                                 w.num_blocks, w.k_scale, w.v_scale)
    first = np.array([O.window_first(c - 1, window) if c > 0 else 0 for c in ctx])
    gk, gv = kp0.copy(), vp0.copy()
    gtab = _hide_before(w, gk, gv, w.block_tables, first)
    dw = upload(w, gk, gv)
    tables = torch.from_numpy(gtab).cuda()
    log(f"[gpu] window {label}: W={window} P={part} B={w.B} H={w.H} H_kv={w.H_kv} d={w.d} "
        f"{w.kv_dtype} kernel={P.kv_decode_kernel_kind(dw.pool, w.H)}")
    ctx_t = torch.from_numpy(st.context_lens).cuda()
    out_slots = torch.empty(w.B, dtype=torch.int64, device="cuda")
    P.kv_cache_append(dw.pool, to_dev(st.new_k), to_dev(st.new_v), tables, ctx_t, out_slots)
    q = to_dev(st.q)
    out = torch.empty_like(q)
    L = int(max(ctx.max(), 1))
    ws = None
    if part:
        ws = torch.empty(P.paged_attention_workspace_bytes(w.B, w.H, w.d, L, part),
                         dtype=torch.uint8, device="cuda")
    P.paged_attention_decode(dw.pool, out, q, tables, ctx_t, L, w.scale, part, ws, window=window)
    if part:
        P.paged_attention_reduce(out, ws, ctx_t, L, part, w.dtype, window=window)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out_slots.cpu().numpy(), slots)
    # the write's bytes: the oracle's pool with the same positions hidden
    ek, ev = kp.copy(), vp.copy()
    _hide_before(w, ek, ev, w.block_tables, first)
    assert np.array_equal(from_dev(dw.pool.k_cache, w.kv_dtype), ek), f"{label}: K pool"
    assert np.array_equal(from_dev(dw.pool.v_cache, w.kv_dtype), ev), f"{label}: V pool"
    ref = {b: O.decode_sequence(kp, vp, st.q[b], w.block_tables[b], int(ctx[b]), w.H, w.H_kv, w.d,
                                w.kv_dtype, w.scale, w.k_scale, w.v_scale, window=window)
           for b in range(w.B)}
    return assert_close(from_dev(out, w.dtype), ref, w.dtype, label)


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("part", [0, 32, 512])
@pytest.mark.parametrize("dtype,kv,H,H_kv,d", [
    ("bf16", "bf16", 4, 4, 128),     # vector-ALU kernel
    ("f32", "f32", 2, 2, 64),
    ("bf16", "fp8", 4, 4, 128),
    ("bf16", "bf16", 16, 2, 128),    # matrix-core kernel
    ("bf16", "fp8", 32, 8, 64),
])
def test_windowed_decode_matches_oracle(window, part, dtype, kv, H, H_kv, d):
    w = W.scattered_workload("win", dtype, len(LENS), H, H_kv, d, LENS, seed=70 + H + d,
                             kv_dtype=kv, k_scale=0.5 if kv == "fp8" else 1.0,
                             v_scale=1.5 if kv == "fp8" else 1.0)
    _decode_case(w, window, part, f"{dtype}/{kv}")


MULTI = [
    ("g8-verify", 32, 4, 128, [700, 33, 129, 1500, 20, 260], [2, 4, 5, 4, 1, 3]),
    ("g4-chunk", 16, 4, 64, [40, 90, 200, 31], [40, 17, 32, 31]),
    ("mha", 4, 4, 128, [5, 40, 300, 17, 64, 1000], [5, 4, 16, 17, 33, 1]),
    ("g8-verify8", 32, 4, 64, [900, 450, 1300], [8, 6, 7]),
]


@pytest.mark.parametrize("window", [1, 5, 16, 33, 128])
@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("case", MULTI, ids=[c[0] for c in MULTI])
def test_windowed_multi_matches_oracle(case, kv, window):
    windowed_multi_case(case, kv, window)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("case", [
    # g = 8 with 64 and 40 rows (the LDS-staged kernel, two tiles per wave):
    # the work-groups' first blocks are odd and even in turn, and each walks
    # more than 32 blocks, past the wrap of the per-block validity bits
    ("g8-long", 64, 8, 128, [1500, 2100], [64, 40]),
    # 8 and 6 draft tokens at g = 8 (one tile per wave): the pipelined pairs
    # start inside the window
    ("g8-verify-long", 32, 4, 128, [1500, 2100], [8, 6]),
], ids=["two-tiles", "one-tile"])
def test_windowed_long_chunk_matches_oracle(case, kv):
    windowed_multi_case(case, kv, 1000)


def windowed_multi_case(case, kv, window):
    name, H, H_kv, d, ctx, n = case
    w = W.multi_token_workload(name, "bf16", len(ctx), H, H_kv, d, ctx, n, seed=500 + H,
                               kv_dtype=kv, k_scale=0.5 if kv == "fp8" else 1.0,
                               v_scale=1.5 if kv == "fp8" else 1.0)
    m = w.multi
    nq = np.diff(m.query_start).astype(np.int64)
    cl = m.context_lens.astype(np.int64)
    kp0, vp0 = poison(w, np.maximum(cl - nq, 0))
    sl = O.chunk_slots(w.block_tables, m.context_lens, m.query_start)
    kp, vp = O.reshape_and_cache(kp0, vp0, m.new_k, m.new_v, sl, w.H_kv, w.d, w.kv_dtype,
                                 w.num_blocks, w.k_scale, w.v_scale)
    # the first row's window starts earliest
    first = np.array([O.window_first(c - k, window) for c, k in zip(cl, nq)])
    gk, gv = kp0.copy(), vp0.copy()
    gtab = _hide_before(w, gk, gv, w.block_tables, first)
    dw = upload(w, gk, gv)
    tables = torch.from_numpy(gtab).cuda()
    log(f"[gpu] windowed multi {name}-{kv} W={window}")
    qs = torch.from_numpy(m.query_start).cuda()
    ctx_t = torch.from_numpy(m.context_lens).cuda()
    mq = int(nq.max())
    P.kv_cache_append_chunk(dw.pool, to_dev(m.new_k), to_dev(m.new_v), qs, mq, tables, ctx_t)
    q = to_dev(m.q)
    out = torch.empty_like(q)
    P.paged_attention_multi(dw.pool, out, q, qs, mq, tables, ctx_t, w.scale, window=window)
    torch.cuda.synchronize()
    ref = O.decode_multi(kp, vp, m.q, m.query_start, w.block_tables, m.context_lens, w.H, w.H_kv,
                         w.d, w.kv_dtype, w.scale, w.k_scale, w.v_scale, window=window)
    rows = {int(m.query_start[b]) + j: r[j] for b, r in ref.items() for j in range(len(r))}
    assert_rows_close(from_dev(out, "bf16"), rows, f"{name}-{kv}-W{window}")


@pytest.mark.parametrize("kv_dtype", ["", "fp8"])
@pytest.mark.parametrize("window", [128, 1024])
def test_full_size_windowed_decode(window, kv_dtype):
    """The GQA batch-256 workload with a gpt-oss-like 128-token band and a
    1,024-token window; 16 sampled sequences checked (shortest, longest, 14
    at random)."""
    w = W.make_workload(3, kv_dtype=kv_dtype)
    st = w.steps[0]
    ctx = st.context_lens.astype(np.int64)
    kp0, vp0 = poison(w, ctx - 1)
    dw = upload(w, kp0, vp0)
    log(f"[gpu] full-size window W={window} {w.kv_dtype}")
    tables = dw.tables
    ctx_t = torch.from_numpy(st.context_lens).cuda()
    P.kv_cache_append(dw.pool, to_dev(st.new_k), to_dev(st.new_v), tables, ctx_t)
    q = to_dev(st.q)
    out = torch.empty_like(q)
    P.paged_attention_decode(dw.pool, out, q, tables, ctx_t, int(ctx.max()), w.scale,
                             window=window)
    torch.cuda.synchronize()
    slots = O.slot_mapping(w.block_tables, st.context_lens)
    kp, vp = O.reshape_and_cache(kp0, vp0, st.new_k, st.new_v, slots, w.H_kv, w.d, w.kv_dtype,
                                 w.num_blocks, w.k_scale, w.v_scale)
    rng = np.random.default_rng(9)
    seqs = sorted({int(ctx.argmin()), int(ctx.argmax()),
                   *rng.choice(w.B, size=14, replace=False).tolist()})
    ref = {b: O.decode_sequence(kp, vp, st.q[b], w.block_tables[b], int(ctx[b]), w.H, w.H_kv, w.d,
                                w.kv_dtype, w.scale, w.k_scale, w.v_scale, window=window)
           for b in seqs}
    assert_close(from_dev(out, "bf16"), ref, "bf16", f"config3-W{window}-{w.kv_dtype}")
