"""The split workspace contract on the GPU, and the long-walk code paths.

paged_attention_decode in split mode leaves, per (sequence, query head,
partition), a partial result (o, m, l) in the workspace, in base-2 units: m a
reference value within 8 of the partition's largest score s2 = scale * log2(e)
* q.k, l = sum 2^(s2 - m), o the normalised partial output.  These are the
running max and denominator the Q&A page's Q4 keeps while it walks K/V tiles,
taken per partition; the oracle's `partials` computes them in natural units
(m_k = max s, l_k = sum e^(s - m_k)).  Converted, l * 2^m must equal
l_k * e^(m_k), and o must equal o_k element by element.

Also covered: repeated split steps give the same bits (the work list's
dealing and the streamed worker's prefetch of its next item), the vector-ALU
kernel's refill of its 64-entry table window (a
wave walks more than 64 blocks: contexts beyond 8,192 tokens in one pass) and
the item-by-item split path taken by partitions longer than one streamed
item (partition_size beyond 64 blocks per wave).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_33_amd as P
from workloads import configs as W

from _harness import from_dev, gpu_step, log, poison, single_step_case, to_dev, upload

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)


def _workspace_regions(ws: torch.Tensor, B, H, d, L, Psize):
    n_part = -(-L // Psize)
    n = B * H * n_part
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    o_bytes, ml_bytes = a256(n * d * 4), a256(n * 4)
    raw = ws.cpu().numpy()
    o = raw[:n * d * 4].view(np.float32).reshape(B, H, n_part, d)
    m = raw[o_bytes:o_bytes + n * 4].view(np.float32).reshape(B, H, n_part)
    l = raw[o_bytes + ml_bytes:o_bytes + ml_bytes + n * 4].view(np.float32).reshape(B, H, n_part)
    return o.astype(np.float64), m.astype(np.float64), l.astype(np.float64)


CASES = [
    # name, kv dtype, H, H_kv, d, lengths, partition sizes
    ("long-context-shape", "bf16", 32, 8, 128, [5000, 2100, 1100, 517, 300, 17, 1], (512, 32)),
    ("mha", "bf16", 4, 4, 128, [1100, 700, 250, 17, 16, 1], (512, 32)),
    ("gqa-fp8", "fp8", 16, 4, 128, [2100, 700, 33, 1], (512, 32)),
    ("gqa-int8", "int8", 16, 4, 128, [2100, 700, 33, 1], (512, 32)),
    ("gqa-d64", "bf16", 8, 2, 64, [1300, 513, 64, 2], (256,)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_partials_match_the_oracle(case):
    name, kvd, H, H_kv, d, lens, psizes = case
    act = "bf16"
    w = W.scattered_workload(name, act, B=len(lens), H=H, H_kv=H_kv, d=d, context_lens=lens,
                             seed=71 + H + d, kv_dtype=None if kvd == act else kvd)
    step = w.steps[0]
    kp0, vp0 = poison(w, np.maximum(step.context_lens.astype(np.int64) - 1, 0))
    dw = upload(w, kp0, vp0)
    ctx = torch.from_numpy(step.context_lens).cuda()
    slots = P.kv_slot_mapping(dw.tables, ctx)
    P.reshape_and_cache(dw.pool, to_dev(step.new_k), to_dev(step.new_v), slots)
    q = to_dev(step.q)
    kp, vp = O.reshape_and_cache(kp0, vp0, step.new_k, step.new_v,
                                 O.slot_mapping(w.block_tables, step.context_lens),
                                 w.H_kv, w.d, w.kv_dtype, w.num_blocks, w.k_scale, w.v_scale)
    L = int(max(lens))
    for Ps in psizes:
        log(f"[gpu] partials {name} {kvd} H={H} H_kv={H_kv} d={d} P={Ps}")
        nbytes = P.paged_attention_workspace_bytes(w.B, H, d, L, Ps)
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN everywhere
        out = torch.empty_like(q)
        P.paged_attention_decode(dw.pool, out, q, dw.tables, ctx, L, w.scale, Ps, ws)
        torch.cuda.synchronize()
        go, gm, gl = _workspace_regions(ws, w.B, H, d, L, Ps)
        oo, om, ol, counts = O.partials(kp, vp, step.q, w.block_tables, step.context_lens, H,
                                        H_kv, d, w.kv_dtype, w.scale, Ps, w.k_scale, w.v_scale)
        checked = 0
        for b in range(w.B):
            if counts[b] < 2:            # one partition: the decode writes out directly
                continue
            k = int(counts[b])
            # base-2 reference within 8 of the partition's largest score
            s2max = om[b, :, :k] * LOG2E
            assert np.all(np.isfinite(gm[b, :, :k])), f"{name} P={Ps} b={b}: m not finite"
            assert np.all(gm[b, :, :k] <= s2max + 1e-3), f"{name} P={Ps} b={b}: m above max"
            assert np.all(gm[b, :, :k] >= s2max - 8 - 1e-3), f"{name} P={Ps} b={b}: m below max-8"
            # denominators: l * 2^m == l_k * e^(m_k), compared in log space
            lhs = np.log(gl[b, :, :k]) + gm[b, :, :k] * math.log(2.0)
            rhs = np.log(ol[b, :, :k]) + om[b, :, :k]
            rel = np.abs(np.expm1(lhs - rhs))
            assert rel.max() <= 5e-3, f"{name} P={Ps} b={b}: l*2^m off by {rel.max():.2e}"
            # normalised partial outputs, element by element
            err = np.abs(go[b, :, :k] - oo[b, :, :k])
            assert err.max() <= 1e-2, f"{name} P={Ps} b={b}: o max-abs {err.max():.2e}"
            rl2 = np.linalg.norm(go[b, :, :k] - oo[b, :, :k]) / np.linalg.norm(oo[b, :, :k])
            assert rl2 <= 5e-3, f"{name} P={Ps} b={b}: o rel-L2 {rl2:.2e}"
            checked += k
        assert checked > 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_vector_alu_walk_refills_its_table_window(dtype):
    # one pass, 8 waves: a wave's window of 64 entries covers 512 blocks = 8,192
    # tokens; these lengths make the waves refill it once and twice
    lens = [20000, 9000, 8193, 8192, 17]
    w = W.scattered_workload("valu-long", dtype, B=len(lens), H=2, H_kv=2, d=128,
                             context_lens=lens, seed=81)
    single_step_case(w, 0, label=f"valu-long-{dtype}")


@pytest.mark.parametrize("kvd,Ps", [("bf16", 16384), ("bf16", 8208), ("int8", 8192),
                                    ("fp8", 16384)])
def test_long_partitions_take_the_item_by_item_path(kvd, Ps):
    lens = [40000, 16385, 16384, 8209, 100, 1]
    w = W.scattered_workload("long-part", "bf16", B=len(lens), H=8, H_kv=2, d=128,
                             context_lens=lens, seed=83,
                             kv_dtype=None if kvd == "bf16" else kvd)
    single_step_case(w, Ps, label=f"long-partitions-{kvd}-P{Ps}", per_row=kvd == "int8")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("one_launch", [False, True], ids=["two-calls", "one-launch"])
def test_repeated_split_steps_are_bit_identical(kv_dtype, one_launch):
    """Resident workers deal the (sequence, partition) items among themselves
    (bf16 and int8 pools: each streams its items back to back, requesting the
    next item's table window and first tiles while it merges; fp8: item by
    item), and the reduce merges the partials.  The same step repeated on the
    same pool (its write stores the same rows again) gives the same output
    bits every time."""
    ctx = [20000, 9000, 3000, 700, 17]
    w = W.scattered_workload("rep-split", "bf16", B=len(ctx), H=32, H_kv=8, d=128,
                             context_lens=ctx, seed=123, kv_dtype=kv_dtype)
    dw = upload(w, w.k_pool, w.v_pool)
    log(f"[gpu] repeated split steps {kv_dtype} one_launch={one_launch}")
    outs = []
    for _ in range(4):
        _, out = gpu_step(dw, w.steps[0], partition_size=512, fused=not one_launch,
                          one_launch=one_launch)
        torch.cuda.synchronize()
        outs.append(from_dev(out, "bf16").copy())
    assert np.all(np.isfinite(O.bits_to_f64(outs[0], "bf16")))
    for rep, o in enumerate(outs[1:]):
        assert np.array_equal(o, outs[0]), f"step {rep + 2} differs from the first"
