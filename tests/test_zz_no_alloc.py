"""The allocation-free split decode (paged_attention_decode_noalloc) against
the split decode with a caller workspace followed by the reduce, through the
C ABI: the same kernels on the same inputs, so the outputs must agree bit for
bit, and both must meet the oracle's tolerances.  Two calls in a row, the
second smaller and with another partition layout, so whatever the first left
in the library's scratch must not leak into the second.  Sizes beyond the
scratch are refused before anything runs.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_33_amd as P
from workloads import configs as W

from _harness import (assert_close, from_dev, gpu_step, log, oracle_step, poison, to_dev,
                      upload)

pytestmark = pytest.mark.gpu


def _case(name, H, H_kv, lens, seed, kv_dtype=None):
    w = W.scattered_workload(name, "bf16", B=len(lens), H=H, H_kv=H_kv, d=128,
                             context_lens=lens, seed=seed, kv_dtype=kv_dtype)
    step = w.steps[0]
    kp, vp = poison(w, np.maximum(step.context_lens.astype(np.int64) - 1, 0))
    return w, step, kp, vp


def _noalloc(dw, step, partition_size, L):
    ctx = torch.from_numpy(step.context_lens).cuda()
    q = to_dev(step.q)
    out = torch.full_like(q, -1)
    P.paged_attention_decode_noalloc(dw.pool, out, q, dw.tables, ctx, L, dw.w.scale,
                                     partition_size)
    return out


@pytest.mark.parametrize("kv_dtype", [None, "int8"])
def test_noalloc_equals_the_workspace_path_on_two_calls(kv_dtype):
    calls = [
        # a long-context mix at 512-token partitions, then a smaller batch split at 32
        ("noalloc-long", 32, 8, [20000, 6000, 1100, 513, 300, 17, 1, 0], 101, 512),
        ("noalloc-small", 16, 4, [700, 33, 1], 102, 32),
    ]
    for name, H, H_kv, lens, seed, Ps in calls:
        w, step, kp, vp = _case(name, H, H_kv, lens, seed, kv_dtype)
        dw = upload(w, kp, vp)
        L = int(max(lens))
        log(f"[gpu] {name} {w.kv_dtype} B={w.B} H={H} P={Ps}: workspace path")
        _, ref_out = gpu_step(dw, step, Ps)                  # write + decode + reduce
        torch.cuda.synchronize()
        log(f"[gpu] {name}: allocation-free path")
        got = _noalloc(dw, step, Ps, L)                      # the cache already holds the row
        torch.cuda.synchronize()
        np.testing.assert_array_equal(from_dev(got, w.dtype), from_dev(ref_out, w.dtype),
                                      err_msg=f"{name}: differs from the workspace path")
        _, _, _, ref = oracle_step(w, kp, vp, step, seqs=[b for b in range(w.B) if lens[b] > 0])
        assert_close(from_dev(got, w.dtype), ref, w.dtype, name, per_row=kv_dtype == "int8")
        assert np.all(from_dev(got, w.dtype)[[b for b in range(w.B) if lens[b] == 0]] == 0)


def test_noalloc_single_pass_and_size_limit():
    w, step, kp, vp = _case("noalloc-single", 8, 2, [300, 17, 1], 103)
    dw = upload(w, kp, vp)
    _, ref_out = gpu_step(dw, step, 0)
    got = _noalloc(dw, step, 0, 300)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev(got, "bf16"), from_dev(ref_out, "bf16"))
    # partials beyond the scratch: refused on the host, nothing enqueued
    big_B, H, L, Ps = 64, 64, 1 << 16, 16
    need = P.paged_attention_workspace_bytes(big_B, H, 128, L, Ps)
    assert need > 32 << 20
    q = torch.zeros((big_B, H, 128), dtype=torch.int16, device="cuda")
    tables = torch.zeros((big_B, L // 16), dtype=torch.int32, device="cuda")
    ctx = torch.ones(big_B, dtype=torch.int32, device="cuda")
    with pytest.raises(P.PagedKVError, match="at most"):
        P.paged_attention_decode_noalloc(dw.pool, torch.empty_like(q), q, tables, ctx, L,
                                         w.scale, Ps)
