"""kv_decode_step, the whole decode step in one launch: the newest rows are
written by extra work-groups and the attention takes the newest position from
the rows themselves.

Every check of the two-call step holds for it: slots and whole pools bit-exact
with the oracle after the step, outputs within the stated tolerances (fp32
max-abs <= 1e-5; bf16 rel-L2 <= 5e-3 and max-abs <= 1e-2).  The slot of the
newest position holds NaN before the step (poisoned), so a decode that read
it would fail.  Covered: the vector-ALU kernel (MHA, fp32 any g) and the
matrix-core kernel, single pass and splits of 16, 32 and 512 tokens, windows,
the newest position opening a fresh block (ctx % 16 == 1), ctx = 1 (the
output is the new value row exactly), a bad table entry for the newest block,
zero-length sequences, the full-size workloads in the bench's launch
configuration.  fp8 (E4M3, per-tensor scales) and int8 (per-token row scales)
pools too: the newest position enters the attention as the codes the write
stores, so the pools must still equal the oracle's bit for bit and the
outputs meet the same bounds (int8: the per-row bound of its other tests).
"""
import numpy as np
import pytest
import torch

from workloads import configs as W

from _harness import (assert_close, from_dev, gpu_step, log, oracle_step, poison,
                      single_step_case, upload)

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 33, 250, 700, 1100]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("P_", [0, 16, 512])
def test_mha_bf16(d, P_):
    w = W.scattered_workload("step-mha", "bf16", B=len(LENS), H=4, H_kv=4, d=d,
                             context_lens=LENS, seed=201 + d)
    single_step_case(w, P_, label=f"step-mha-d{d}", one_launch=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,H_kv", [(2, 2), (8, 2)])
@pytest.mark.parametrize("P_", [0, 32])
def test_fp32(d, H, H_kv, P_):
    w = W.scattered_workload("step-f32", "f32", B=len(LENS), H=H, H_kv=H_kv, d=d,
                             context_lens=LENS, seed=211 + d + H)
    single_step_case(w, P_, label=f"step-f32-d{d}-H{H}", one_launch=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,H_kv", [(4, 2), (8, 1), (32, 8), (64, 2), (6, 2)])
@pytest.mark.parametrize("P_", [0, 32, 512])
def test_gqa_bf16(d, H, H_kv, P_):
    w = W.scattered_workload("step-gqa", "bf16", B=len(LENS), H=H, H_kv=H_kv, d=d,
                             context_lens=LENS, seed=221 + H + d)
    single_step_case(w, P_, label=f"step-gqa-d{d}-g{H // H_kv}", one_launch=True)


@pytest.mark.parametrize("H,H_kv", [(4, 4), (32, 8)])
@pytest.mark.parametrize("window", [1, 7, 16, 100])
@pytest.mark.parametrize("P_", [0, 32])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "int8"])
def test_windows(H, H_kv, window, P_, kv_dtype):
    w = W.scattered_workload("step-win", "bf16", B=len(LENS), H=H, H_kv=H_kv, d=128,
                             context_lens=LENS, seed=231 + window, kv_dtype=kv_dtype)
    single_step_case(w, P_, label=f"step-window{window}-{kv_dtype}", one_launch=True,
                     window=window, per_row=kv_dtype == "int8")


@pytest.mark.parametrize("H,H_kv,dtype", [(4, 4, "bf16"), (16, 2, "bf16"), (2, 2, "f32")])
@pytest.mark.parametrize("P_", [0, 16])
def test_single_token_context_returns_the_new_value_row(H, H_kv, dtype, P_):
    w = W.scattered_workload("step-one", dtype, B=3, H=H, H_kv=H_kv, d=128,
                             context_lens=[1, 1, 1], seed=241)
    step = w.steps[0]
    kp, vp = poison(w, step.context_lens.astype(np.int64) - 1)
    dw = upload(w, kp, vp)
    _, out = gpu_step(dw, step, P_, one_launch=True)
    got = from_dev(out, dtype).reshape(3, H_kv, H // H_kv, 128)
    want = step.new_v.reshape(3, H_kv, 1, 128)
    np.testing.assert_array_equal(got, np.broadcast_to(want, got.shape))


@pytest.mark.parametrize("H,H_kv", [(4, 4), (16, 2)])
@pytest.mark.parametrize("P_", [0, 32])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "int8"])
def test_bad_entry_for_the_newest_block(H, H_kv, P_, kv_dtype):
    # sequence 1's newest position opens block 2 (ctx 33); sequence 2's sits
    # inside block 1 (ctx 30); both blocks' entries point outside the pool
    lens = [40, 33, 30, 17]
    w = W.scattered_workload("step-bad", "bf16", B=4, H=H, H_kv=H_kv, d=128,
                             context_lens=lens, seed=251, kv_dtype=kv_dtype)
    step = w.steps[0]
    kp, vp = poison(w, step.context_lens.astype(np.int64) - 1)
    good_tables = w.block_tables.copy()
    w.block_tables[1, 2] = w.num_blocks + 3
    w.block_tables[2, 1] = -5
    dw = upload(w, kp, vp)
    slots, out = gpu_step(dw, step, P_, one_launch=True)
    got = from_dev(out, "bf16")
    assert slots.cpu().numpy()[1] == -1 and slots.cpu().numpy()[2] == -1
    gotf = got.astype(np.uint32) << 16
    assert np.all(np.isnan(gotf[[1, 2]].view(np.float32)))
    # sequences 0 and 3 own other blocks: the oracle step over the intact
    # tables gives their outputs
    w.block_tables[:] = good_tables
    _, _, _, ref = oracle_step(w, kp, vp, step, seqs=[0, 3])
    assert_close(got, ref, "bf16", f"step-bad-entry-{kv_dtype}", per_row=kv_dtype == "int8")


@pytest.mark.parametrize("H,H_kv", [(4, 4), (8, 2)])
@pytest.mark.parametrize("P_", [0, 16])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "int8"])
def test_empty_contexts(H, H_kv, P_, kv_dtype):
    lens = [0, 20, 0, 33]
    w = W.scattered_workload("step-empty", "bf16", B=4, H=H, H_kv=H_kv, d=128,
                             context_lens=lens, seed=261, kv_dtype=kv_dtype)
    step = w.steps[0]
    kp, vp = poison(w, np.maximum(step.context_lens.astype(np.int64) - 1, 0))
    dw = upload(w, kp, vp)
    slots, out = gpu_step(dw, step, P_, one_launch=True)
    got = from_dev(out, "bf16")
    assert list(slots.cpu().numpy()[[0, 2]]) == [-1, -1]
    assert np.all(got[[0, 2]] == 0)
    _, _, _, ref = oracle_step(w, kp, vp, step, seqs=[1, 3])
    assert_close(got, ref, "bf16", f"step-empty-{kv_dtype}", per_row=kv_dtype == "int8")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("H,H_kv", [(4, 4), (32, 8)])
def test_agrees_with_the_two_call_step(kv_dtype, H, H_kv):
    """The write inside the launch stores what kv_cache_append stores (the
    pools equal bit for bit), and the outputs agree within rounding."""
    w = W.scattered_workload("step-vs-two", "bf16", B=len(LENS), H=H, H_kv=H_kv, d=128,
                             context_lens=LENS, seed=271 + H, kv_dtype=kv_dtype,
                             k_scale=0.5 if kv_dtype == "fp8" else 1.0,
                             v_scale=1.5 if kv_dtype == "fp8" else 1.0)
    step = w.steps[0]
    kp, vp = poison(w, step.context_lens.astype(np.int64) - 1)
    a = upload(w, kp, vp)
    b = upload(w, kp, vp)
    _, out_a = gpu_step(a, step, 0, fused=True)
    _, out_b = gpu_step(b, step, 0, one_launch=True)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(a.pool.k_cache, kv_dtype), from_dev(b.pool.k_cache, kv_dtype))
    assert np.array_equal(from_dev(a.pool.v_cache, kv_dtype), from_dev(b.pool.v_cache, kv_dtype))
    ga = (from_dev(out_a, "bf16").astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    gb = (from_dev(out_b, "bf16").astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    diff = np.abs(ga - gb)
    if kv_dtype == "int8":
        # each is within int8's per-row bound of the exact result (1e-2 of the
        # row's largest magnitude, at least 1e-2), so they agree within twice it
        bound = 2e-2 * np.maximum(1.0, np.abs(ga).max(axis=-1, keepdims=True))
        assert np.all(diff <= bound), float((diff / bound).max())
    else:
        assert diff.max() <= 1e-2


@pytest.mark.parametrize("kv_dtype", ["fp8", "int8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,H_kv", [(4, 4), (8, 2), (32, 8)])
@pytest.mark.parametrize("P_", [0, 16, 512])
def test_byte_code_pools(kv_dtype, d, H, H_kv, P_):
    """One-launch steps over fp8 and int8 pools, through both kernels (MHA:
    the vector-ALU kernel; GQA: the matrix-core kernel, single pass, the
    item-by-item split and the streamed split), against the oracle: slots and
    pools bit for bit, outputs within the bounds."""
    w = W.scattered_workload("step-bytes", "bf16", B=len(LENS), H=H, H_kv=H_kv, d=d,
                             context_lens=LENS, seed=281 + H + d, kv_dtype=kv_dtype,
                             k_scale=0.5 if kv_dtype == "fp8" else 1.0,
                             v_scale=1.5 if kv_dtype == "fp8" else 1.0)
    single_step_case(w, P_, label=f"step-{kv_dtype}-d{d}-H{H}/{H_kv}", one_launch=True,
                     per_row=kv_dtype == "int8")


@pytest.mark.parametrize("kv_dtype", ["fp8", "int8"])
def test_byte_code_single_token_context(kv_dtype):
    """ctx = 1: only the newest position is seen, as the cache holds it."""
    w = W.scattered_workload("step-bytes-one", "bf16", B=3, H=8, H_kv=2, d=128,
                             context_lens=[1, 1, 1], seed=291, kv_dtype=kv_dtype,
                             k_scale=0.5 if kv_dtype == "fp8" else 1.0,
                             v_scale=1.5 if kv_dtype == "fp8" else 1.0)
    single_step_case(w, 0, label=f"step-{kv_dtype}-one", one_launch=True,
                     per_row=kv_dtype == "int8")
    single_step_case(w, 16, label=f"step-{kv_dtype}-one-split", one_launch=True,
                     per_row=kv_dtype == "int8")


BENCH_PARTITION = {2: 0, 3: 0, 4: 512, 5: 0}


@pytest.mark.parametrize("config,kv_dtype", [(1, ""), (2, ""), (3, ""), (4, ""),
                                             (2, "fp8"), (3, "int8"), (4, "fp8"), (4, "int8")])
def test_full_size(config, kv_dtype):
    w = W.make_workload(config, kv_dtype=kv_dtype)
    step = w.steps[0]
    P_ = BENCH_PARTITION.get(config, 0)
    log(f"[gpu] one-launch step, full-size config {config}: B={w.B} H={w.H} H_kv={w.H_kv} "
        f"sum ctx={int(step.context_lens.sum())} partition={P_}")
    kp0, vp0 = poison(w, step.context_lens.astype(np.int64) - 1)
    dw = upload(w, kp0, vp0)
    slots, out = gpu_step(dw, step, P_, one_launch=True)
    torch.cuda.synchronize()
    oslots, kp, vp, ref = oracle_step(w, kp0, vp0, step)
    np.testing.assert_array_equal(slots.cpu().numpy(), oslots)
    assert np.array_equal(from_dev(dw.pool.k_cache, w.kv_dtype), kp)
    assert np.array_equal(from_dev(dw.pool.v_cache, w.kv_dtype), vp)
    err, rel = assert_close(from_dev(out, w.dtype), ref, w.dtype,
                            f"step-config{config}{kv_dtype}", per_row=kv_dtype == "int8")
    log(f"[gpu] config {config} {w.kv_dtype}: max-abs {err:.2e} rel-L2 {rel:.2e}")


def test_full_size_shared_prefix_50_steps():
    w = W.make_workload(5)
    kp, vp = poison(w, w.steps[0].context_lens.astype(np.int64) - 1)
    dw = upload(w, kp, vp)
    check_at = {0, 1, 24, len(w.steps) - 1}
    for s, step in enumerate(w.steps):
        slots, out = gpu_step(dw, step, 0, one_launch=True)
        got = from_dev(out, w.dtype) if s in check_at else None
        oslots, kp, vp, ref = oracle_step(w, kp, vp, step, seqs=range(w.B) if s in check_at else [])
        np.testing.assert_array_equal(slots.cpu().numpy(), oslots, err_msg=f"step {s}")
        if got is not None:
            err, rel = assert_close(got, ref, w.dtype, f"step-config5-step{s}")
            log(f"[gpu] one-launch config 5 step {s}: max-abs {err:.2e} rel-L2 {rel:.2e}")
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dw.pool.k_cache, w.kv_dtype), kp)
    assert np.array_equal(from_dev(dw.pool.v_cache, w.kv_dtype), vp)
