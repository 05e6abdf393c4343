"""GPU parity of the multi-token path: several new tokens per sequence (a
prefill chunk, or draft tokens to verify), written with kv_cache_append_chunk
and attended with paged_attention_multi, causal within each sequence's rows.

For every case: the chunk slot mapping and the whole K and V pools after the
write equal the oracle's bit for bit (fp8: code for code), and the output rows
are within the bf16 tolerances of the float64 oracle: rel-L2 <= 5e-3 over all
compared rows, and max-abs <= 1e-2 * max(1, max |row|) per row.  The scale
applies only to rows whose outputs exceed 1 in magnitude: the first rows of a
first chunk average one to a few keys, so their outputs are as large as single
V rows, and both the bf16 rounding of the output (up to 2^-8 of its
magnitude) and that of the softmax weights the matrix cores take (up to 2^-8
of the spread of the V values) grow with them.  Decode outputs average many
keys and stay well below 1, where the bound is the fixed 1e-2.  The slots the step writes, the tails of the last blocks and
the unused blocks hold NaN before the step, so a row that read a slot it must
not (a later position, a slot past its context, a stale one) comes out NaN.
"""
import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_33_amd as P
from workloads import configs as W

from _harness import (BF16_MAX_ABS, BF16_REL_L2, from_dev, log, poison, to_dev, upload)

pytestmark = pytest.mark.gpu

NAN16 = np.uint16(0x7FC0)
SENT16 = np.uint16(0x1234)   # out rows no call may write


def _gpu_multi(dw, m, max_query_len=None, num_rows=None, write=True, out_fill=None):
    T = int(m.q.shape[0])
    qs = torch.from_numpy(m.query_start).cuda()
    ctx = torch.from_numpy(m.context_lens).cuda()
    mq = int(np.diff(m.query_start).max(initial=0)) if max_query_len is None else max_query_len
    slots = torch.full((T,), -7, dtype=torch.int64, device="cuda")
    if write:
        P.kv_cache_append_chunk(dw.pool, to_dev(m.new_k), to_dev(m.new_v), qs, mq, dw.tables, ctx,
                                slots)
    q = to_dev(m.q)
    out = torch.empty_like(q)
    if out_fill is not None:
        out.fill_(int(np.int16(out_fill.view(np.int16))))
    P.paged_attention_multi(dw.pool, out, q, qs, mq, dw.tables, ctx, dw.w.scale)
    return slots, out


def _ref_rows(w, kp, vp, seqs=None):
    m = w.multi
    ref = O.decode_multi(kp, vp, m.q, m.query_start, w.block_tables, m.context_lens, w.H, w.H_kv,
                         w.d, w.kv_dtype, w.scale, w.k_scale, w.v_scale, seqs=seqs)
    rows = {}
    for b, r in ref.items():
        for j in range(r.shape[0]):
            rows[int(m.query_start[b]) + j] = r[j]
    return rows


def assert_rows_close(got_bits, ref_rows, label):
    """GPU rows (bits [T, H, d]) against oracle rows {row: float64 [H, d]}."""
    rs = sorted(ref_rows)
    got = O.bits_to_f64(got_bits[rs], "bf16")
    want = np.stack([ref_rows[r] for r in rs])
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    assert rel <= BF16_REL_L2, f"{label}: rel-L2 {rel:.3e}"
    err = np.abs(got - want).reshape(len(rs), -1).max(axis=1)
    amp = np.maximum(1.0, np.abs(want).reshape(len(rs), -1).max(axis=1))
    worst = int(np.argmax(err / amp))
    assert err[worst] <= BF16_MAX_ABS * amp[worst], (
        f"{label}: row {rs[worst]} max-abs {err[worst]:.3e} (row magnitude {amp[worst]:.2f})")
    return float(err.max()), rel


def multi_case(w, label, seqs=None):
    """Write + attend on the GPU; slots and pools bit-exact, rows in tolerance."""
    m = w.multi
    n = np.diff(m.query_start).astype(np.int64)
    first = np.maximum(m.context_lens.astype(np.int64) - n, 0)
    kp0, vp0 = poison(w, first)
    dw = upload(w, kp0, vp0)
    log(f"[gpu] multi {label}: B={w.B} H={w.H} H_kv={w.H_kv} d={w.d} {w.kv_dtype} "
        f"n={n.tolist()[:8]}{'...' if w.B > 8 else ''} rows={int(m.q.shape[0])}")
    slots, out = _gpu_multi(dw, m)
    torch.cuda.synchronize()
    oslots = O.chunk_slots(w.block_tables, m.context_lens, m.query_start)
    np.testing.assert_array_equal(slots.cpu().numpy(), oslots, err_msg=f"{label}: slots")
    kp, vp = O.reshape_and_cache(kp0, vp0, m.new_k, m.new_v, oslots, w.H_kv, w.d, w.kv_dtype,
                                 w.num_blocks, w.k_scale, w.v_scale)
    assert np.array_equal(from_dev(dw.pool.k_cache, w.kv_dtype), kp), f"{label}: K pool"
    assert np.array_equal(from_dev(dw.pool.v_cache, w.kv_dtype), vp), f"{label}: V pool"
    ref = _ref_rows(w, kp, vp, seqs)
    err, rel = assert_rows_close(from_dev(out, "bf16"), ref, label)
    log(f"[gpu]   max-abs {err:.2e} rel-L2 {rel:.2e}")
    return dw, out


# (H, H_kv, d, context lengths, new tokens per sequence)
CASES = [
    # MHA: 16 tokens of one head per tile
    ("mha", 4, 4, 128, [5, 40, 300, 17, 64, 1000], [5, 4, 16, 17, 33, 1]),
    # group 8, draft verification shapes: 1, 2 and 3 tiles per KV head
    ("g8-verify", 32, 4, 128, [700, 33, 129, 1500, 20, 260], [2, 4, 5, 4, 1, 3]),
    # group 4, d 64: up to 10 tiles (groups of 4, 4 and 2)
    ("g4-chunk", 16, 4, 64, [40, 90, 200, 31], [40, 17, 32, 31]),
    # group 16: one token per tile; group 3 and 24: tiles cross token borders
    ("g16", 32, 2, 128, [100, 47, 16], [3, 7, 16]),
    ("g3", 6, 2, 64, [50, 18, 77, 9], [11, 18, 6, 9]),
    ("g24", 48, 2, 128, [60, 33], [5, 2]),
    # sequences with no new token this step next to others
    ("idle-rows", 16, 2, 128, [30, 64, 65, 10], [0, 8, 0, 3]),
    # 6 to 8 draft tokens at g = 8 (3 or 4 tiles, one per wave) over contexts
    # long enough for the pipelined pairs, d 64 and 128
    ("g8-verify8", 32, 4, 64, [900, 450, 1300], [8, 6, 7]),
    ("g8-verify8-d128", 16, 2, 128, [700, 260], [8, 8]),
    # group 4, d 64, chunks of 33-40 rows (two tiles per wave) over long
    # contexts: many pipelined pairs per work-group
    ("g4-chunk-long", 16, 4, 64, [700, 1000], [40, 33]),
]


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_multi_matches_oracle(case, kv_dtype):
    name, H, H_kv, d, ctx, n = case
    w = W.multi_token_workload(name, "bf16", len(ctx), H, H_kv, d, ctx, n, seed=300 + H + d,
                               kv_dtype=kv_dtype, k_scale=0.5 if kv_dtype == "fp8" else 1.0,
                               v_scale=1.5 if kv_dtype == "fp8" else 1.0)
    multi_case(w, f"{name}-{kv_dtype}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "int8"])
def test_prefill_chunk_of_512_tokens(kv_dtype):
    """Chunked prefill: a 512-token chunk on top of earlier ones, a first chunk
    (the whole context is new), and a short tail chunk, batched with decodes."""
    ctx = [1536, 512, 700, 2000, 90]
    n = [512, 512, 188, 1, 1]
    w = W.multi_token_workload("prefill", "bf16", len(ctx), 32, 8, 128, ctx, n, seed=41,
                               kv_dtype=kv_dtype, k_scale=0.5 if kv_dtype == "fp8" else 1.0,
                               v_scale=1.5 if kv_dtype == "fp8" else 1.0)
    multi_case(w, f"prefill-{kv_dtype}")


def test_one_token_rows_match_the_decode_kernel_closely():
    """n_b = 1 is the decode step: the two kernels agree within a bf16 ulp-scale
    tolerance (same products, different order)."""
    ctx = [17, 300, 1024, 2047]
    w = W.multi_token_workload("n1", "bf16", 4, 64, 8, 128, ctx, [1, 1, 1, 1], seed=12)
    dw, out = multi_case(w, "n1")
    m = w.multi
    dec = torch.empty_like(out)
    ctx_t = torch.from_numpy(m.context_lens).cuda()
    P.paged_attention_decode(dw.pool, dec, to_dev(m.q), dw.tables, ctx_t, int(max(ctx)), w.scale)
    torch.cuda.synchronize()
    a = O.bits_to_f64(from_dev(out, "bf16"), "bf16")
    b = O.bits_to_f64(from_dev(dec, "bf16"), "bf16")
    assert np.abs(a - b).max() <= BF16_MAX_ABS


def test_bad_lengths_tables_and_rows_are_contained():
    """n_b > ctx_b, n_b > max_query_len and ctx_b > max_nb*16 give NaN rows
    (only below max_query_len); a bad table entry in block 0 makes every row of
    its sequence NaN; n_b = 0 and a sequence whose rows lie outside the buffer
    write nothing; the good sequences are unaffected."""
    H, H_kv, d = 16, 4, 128
    ctx = [40, 5, 30, 20, 64, 33]
    n = [4, 8, 6, 3, 0, 2]
    w = W.multi_token_workload("bad", "bf16", len(ctx), H, H_kv, d, ctx, n, seed=77, max_nb=4)
    m = w.multi
    # sequence 1: n = 8 > ctx = 5; sequence 2: n = 6 > max_query_len = 5;
    # sequence 3: a table entry outside the pool at block 0;
    # sequence 5: ctx raised past max_nb*16 on the device side
    w.block_tables[3, 0] = w.num_blocks + 5
    ctx_dev = m.context_lens.copy()
    ctx_dev[5] = 4 * 16 + 1
    dw = upload(w, w.k_pool, w.v_pool)
    qs = m.query_start
    T = int(qs[-1])
    log("[gpu] multi bad-input containment")
    m2 = W.MultiStep(context_lens=ctx_dev, query_start=qs, q=m.q, new_k=m.new_k, new_v=m.new_v)
    _, out = _gpu_multi(dw, m2, max_query_len=5, write=False, out_fill=SENT16)
    torch.cuda.synchronize()
    got = from_dev(out, "bf16").reshape(T, H, d)
    rows = lambda b: slice(int(qs[b]), int(qs[b + 1]))
    assert np.all(np.isnan(O.bits_to_f64(got[rows(1)][:5], "bf16")))
    assert np.all(got[rows(1)][5:] == SENT16)           # past max_query_len: untouched
    assert np.all(np.isnan(O.bits_to_f64(got[rows(2)][:5], "bf16")))
    assert np.all(got[rows(2)][5:] == SENT16)
    assert np.all(np.isnan(O.bits_to_f64(got[rows(3)], "bf16")))
    assert np.all(np.isnan(O.bits_to_f64(got[rows(5)], "bf16")))
    ref = _ref_rows(w, w.k_pool, w.v_pool, seqs=[0])
    assert_rows_close(got, ref, "good sequence next to bad ones")

    # a sequence whose rows lie outside [0, num_rows): nothing is written, the
    # other sequences are computed as usual
    qs_bad = qs.copy()
    qs_bad[-1] = T + 100
    m3 = W.MultiStep(context_lens=m.context_lens, query_start=qs_bad, q=m.q, new_k=m.new_k,
                     new_v=m.new_v)
    dw = upload(w, w.k_pool, w.v_pool)
    slots, out = _gpu_multi(dw, m3, max_query_len=8, out_fill=SENT16, write=True)
    torch.cuda.synchronize()
    got = from_dev(out, "bf16").reshape(T, H, d)
    assert np.all(got[rows(5)] == SENT16)
    assert np.all(slots.cpu().numpy()[rows(5)] == -7)    # the write skipped it too
    assert np.all(np.isfinite(O.bits_to_f64(got[rows(0)], "bf16")))


@pytest.mark.parametrize("kv_dtype", ["", "fp8", "int8"])
@pytest.mark.parametrize("config,K", [(2, 4), (3, 4), (3, 8)])
def test_full_size_draft_verification(config, K, kv_dtype):
    """Draft verification at the full shapes of the 7B-like batch-64 and the GQA
    batch-256 workloads: every sequence verifies K tokens.  Pools and slots are
    compared whole; outputs on 12 sampled sequences (the shortest, the longest
    and 10 drawn at random)."""
    w = W.make_workload(config, kv_dtype=kv_dtype)
    W.add_multi_step(w, [K] * w.B, seed=900 + config)
    ctx = w.multi.context_lens
    rng = np.random.default_rng(5)
    seqs = sorted({int(ctx.argmin()), int(ctx.argmax()),
                   *rng.choice(w.B, size=10, replace=False).tolist()})
    multi_case(w, f"config{config}-K{K}-{w.kv_dtype}", seqs=seqs)


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8", "int8"])
@pytest.mark.parametrize("d", [64, 128])
def test_chunk_write_alone_is_bit_exact(kv, d):
    """kv_cache_append_chunk for every pool dtype: chunks that start and end
    inside blocks, fill whole blocks, cross several, a first chunk, one row, a
    sequence with no row, one with more rows than context (its first rows get
    slot -1) and one with more rows than max_query_len (rows past it are not
    written).  Slots and both pools equal the oracle's bit for bit; the slots
    the chunk does not cover keep their bits (NaN payloads included)."""
    ctx = [40, 16, 100, 7, 33, 5, 60]
    n = [13, 16, 70, 1, 0, 9, 44]
    act = "f32" if kv == "f32" else "bf16"
    w = W.multi_token_workload("cw", act, len(ctx), 8, 2, d, ctx, n, seed=61 + d, kv_dtype=kv,
                               k_scale=0.5 if kv == "fp8" else 1.0,
                               v_scale=1.5 if kv == "fp8" else 1.0)
    m = w.multi
    mq = 40                                   # sequences 2 (70 rows) and 6 (44) exceed it
    kp0, vp0 = poison(w, np.zeros(w.B, dtype=np.int64))   # every slot NaN before the write
    dw = upload(w, kp0, vp0)
    log(f"[gpu] chunk write {kv} d={d}")
    T = int(m.query_start[-1])
    slots = torch.full((T,), -7, dtype=torch.int64, device="cuda")
    P.kv_cache_append_chunk(dw.pool, to_dev(m.new_k), to_dev(m.new_v),
                            torch.from_numpy(m.query_start).cuda(), mq, dw.tables,
                            torch.from_numpy(m.context_lens).cuda(), slots)
    torch.cuda.synchronize()
    want = O.chunk_slots(w.block_tables, m.context_lens, m.query_start)
    for b in range(w.B):                      # rows at or past max_query_len: untouched
        for j in range(mq, int(m.query_start[b + 1] - m.query_start[b])):
            want[m.query_start[b] + j] = -7
    np.testing.assert_array_equal(slots.cpu().numpy(), want)
    written = np.where(want >= 0, want, -1)
    kp, vp = O.reshape_and_cache(kp0, vp0, m.new_k, m.new_v, written, w.H_kv, w.d, kv,
                                 w.num_blocks, w.k_scale, w.v_scale)
    assert np.array_equal(from_dev(dw.pool.k_cache, kv), kp)
    assert np.array_equal(from_dev(dw.pool.v_cache, kv), vp)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "int8"])
def test_long_chunk_kernel_contains_bad_inputs(kv_dtype):
    """The same containment for the long-chunk kernel (g * max_query_len of 320
    columns, ten column sets): n > ctx, n > max_query_len and ctx > max_nb*16
    give NaN rows below max_query_len, a bad table entry in block 0 gives NaN
    rows, the good sequence is unaffected."""
    H, H_kv, d = 32, 4, 128
    ctx = [300, 10, 200, 120, 400]
    n = [40, 30, 45, 33, 20]
    w = W.multi_token_workload("badc", "bf16", len(ctx), H, H_kv, d, ctx, n, seed=78, max_nb=25,
                               kv_dtype=kv_dtype)
    m = w.multi
    w.block_tables[3, 0] = w.num_blocks + 3
    ctx_dev = m.context_lens.copy()
    ctx_dev[4] = 25 * 16 + 1
    dw = upload(w, w.k_pool, w.v_pool)
    qs = m.query_start
    T = int(qs[-1])
    log(f"[gpu] long-chunk bad-input containment ({kv_dtype})")
    m2 = W.MultiStep(context_lens=ctx_dev, query_start=qs, q=m.q, new_k=m.new_k, new_v=m.new_v)
    _, out = _gpu_multi(dw, m2, max_query_len=40, write=False, out_fill=SENT16)
    torch.cuda.synchronize()
    got = from_dev(out, "bf16").reshape(T, H, d)
    rows = lambda b: slice(int(qs[b]), int(qs[b + 1]))
    assert np.all(np.isnan(O.bits_to_f64(got[rows(1)], "bf16")))          # n > ctx
    assert np.all(np.isnan(O.bits_to_f64(got[rows(2)][:40], "bf16")))     # n > max_query_len
    assert np.all(got[rows(2)][40:] == SENT16)
    assert np.all(np.isnan(O.bits_to_f64(got[rows(3)], "bf16")))          # bad entry, block 0
    assert np.all(np.isnan(O.bits_to_f64(got[rows(4)], "bf16")))          # ctx > max_nb * 16
    ref = _ref_rows(w, w.k_pool, w.v_pool, seqs=[0])
    assert_rows_close(got, ref, "good sequence next to bad ones")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("shape", [
    # (H, H_kv, d, context lengths, rows per sequence)
    (64, 8, 128, [1500, 2100, 900, 3000], [8, 8, 8, 8]),      # one tile per wave
    (64, 8, 128, [1200, 2600], [64, 48]),                      # two tiles per wave
], ids=["verify", "chunk"])
def test_repeated_calls_are_bit_identical(kv_dtype, shape):
    """The LDS-staged kernel's pipelined pairs share each block between waves
    through barriers; the same call repeated on the same pool gives the same
    bits every time (a wave reading a stage before it is complete, or after
    it is reused, would show as run-to-run differences), and the rows agree
    with the oracle."""
    H, H_kv, d, ctx, n = shape
    w = W.multi_token_workload("rep", "bf16", len(ctx), H, H_kv, d, ctx, n, seed=91 + n[0],
                               kv_dtype=kv_dtype)
    m = w.multi
    dw = upload(w, w.k_pool, w.v_pool)
    log(f"[gpu] repeated multi {kv_dtype} rows={n}")
    _, out0 = _gpu_multi(dw, m, write=True)
    first = from_dev(out0, "bf16").copy()
    for rep in range(4):
        _, out = _gpu_multi(dw, m, write=False)
        torch.cuda.synchronize()
        got = from_dev(out, "bf16")
        assert np.array_equal(got, first), f"call {rep + 2} differs from the first"
    sl = O.chunk_slots(w.block_tables, m.context_lens, m.query_start)
    kp, vp = O.reshape_and_cache(w.k_pool, w.v_pool, m.new_k, m.new_v, sl, w.H_kv, w.d,
                                 w.kv_dtype, w.num_blocks, w.k_scale, w.v_scale)
    assert_rows_close(first, _ref_rows(w, kp, vp, seqs=[0, len(ctx) - 1]), "repeated calls")
