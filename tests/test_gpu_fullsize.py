"""GPU parity at the full sizes of the five workloads, in the launch
configuration bench.py times (single pass for configs 2, 3, 5; 512-token split
plus the log-sum-exp reduce for config 4).

For each: the slot mapping and the whole K and V pools after the cache write
are compared bit for bit with the oracle's, and every sequence's output is
compared with the float64 oracle (bf16: rel-L2 <= 5e-3, max-abs <= 1e-2; for
an int8 cache the max-abs bound scales with each row's magnitude, as in the
int8 parity tests).
Config 5 runs its 50 write+decode steps in order on the GPU; outputs are
checked at four of the steps and the pools after the last one.  Configs 2-5
also run with an fp8 (E4M3) cache and with an int8 cache (per-token row
scales): the pools are then compared code for code (and scale for scale)
after the quantising write.
"""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import configs as W

from _harness import (assert_close, from_dev, gpu_step, log, oracle_step, poison, upload)

pytestmark = pytest.mark.gpu

BENCH_PARTITION = {2: 0, 3: 0, 4: 512, 5: 0}


def _check_single_step(config: int, kv_dtype: str = ""):
    w = W.make_workload(config, kv_dtype=kv_dtype)
    step = w.steps[0]
    P_ = BENCH_PARTITION[config]
    log(f"[gpu] full-size config {config} ({w.kv_dtype} cache): B={w.B} H={w.H} H_kv={w.H_kv} "
        f"sum ctx={int(step.context_lens.sum())} partition={P_}")
    kp0, vp0 = poison(w, step.context_lens.astype(np.int64) - 1)
    dw = upload(w, kp0, vp0)
    slots, out = gpu_step(dw, step, P_)
    torch.cuda.synchronize()
    got = from_dev(out, w.dtype)
    gk = from_dev(dw.pool.k_cache, w.kv_dtype)
    gv = from_dev(dw.pool.v_cache, w.kv_dtype)
    oslots, kp, vp, ref = oracle_step(w, kp0, vp0, step)
    np.testing.assert_array_equal(slots.cpu().numpy(), oslots)
    assert np.array_equal(gk, kp), "K pool differs from the oracle's after the write"
    assert np.array_equal(gv, vp), "V pool differs from the oracle's after the write"
    err, rel = assert_close(got, ref, w.dtype, f"config{config}-{w.kv_dtype}",
                            per_row=w.kv_dtype == "int8")
    log(f"[gpu] config {config} ({w.kv_dtype}): max-abs {err:.2e} rel-L2 {rel:.2e}")


@pytest.mark.parametrize("kv_dtype", ["", "fp8", "int8"])
@pytest.mark.parametrize("config", [2, 3, 4])
def test_full_size_single_step(config, kv_dtype):
    _check_single_step(config, kv_dtype)


@pytest.mark.parametrize("kv_dtype", ["", "fp8", "int8"])
def test_full_size_shared_prefix_50_steps(kv_dtype):
    w = W.make_workload(5, kv_dtype=kv_dtype)
    first = w.steps[0].context_lens.astype(np.int64) - 1
    kp, vp = poison(w, first)
    dw = upload(w, kp, vp)
    check_at = {0, 1, 24, len(w.steps) - 1}
    log(f"[gpu] full-size config 5 ({w.kv_dtype} cache): B={w.B} steps={len(w.steps)}")
    for s, step in enumerate(w.steps):
        slots, out = gpu_step(dw, step, BENCH_PARTITION[5])
        oslots = O.slot_mapping(w.block_tables, step.context_lens)
        np.testing.assert_array_equal(slots.cpu().numpy(), oslots, err_msg=f"step {s}")
        got = from_dev(out, w.dtype) if s in check_at else None
        _, kp, vp, ref = oracle_step(w, kp, vp, step, seqs=range(w.B) if s in check_at else [])
        if got is not None:
            err, rel = assert_close(got, ref, w.dtype, f"config5-step{s}",
                                    per_row=w.kv_dtype == "int8")
            log(f"[gpu] config 5 step {s}: max-abs {err:.2e} rel-L2 {rel:.2e}")
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dw.pool.k_cache, w.kv_dtype), kp)
    assert np.array_equal(from_dev(dw.pool.v_cache, w.kv_dtype), vp)


def test_config1_at_its_full_size():
    w = W.make_workload(1)
    step = w.steps[0]
    kp0, vp0 = poison(w, step.context_lens.astype(np.int64) - 1)
    dw = upload(w, kp0, vp0)
    _, out = gpu_step(dw, step, 0)
    _, _, _, ref = oracle_step(w, kp0, vp0, step)
    assert_close(from_dev(out, w.dtype), ref, w.dtype, "config1")
