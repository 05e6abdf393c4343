"""Throughput of the paged decode-attention step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config N] [--partition P]

A step is the whole hot path for one batch: slot mapping, cache write of one
new token per sequence, decode attention (and the log-sum-exp reduce when
split), all through libpagedkv's C ABI on the current torch stream.  Inputs
are seeded and synthetic (workloads/), resident in HBM before timing starts.

Prints one JSON line.  `value` is HBM GB/s of the step's algorithmic bytes
(cached K/V read once, query, output, table and length reads, plus the
cache write's bytes); `roofline` prices the decode kernel alone against the
8 TB/s HBM3E peak; `cpu_baseline` times the float64 CPU oracle on a bounded
sample of the same workload (and checks the GPU output against it).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode-attn HBM GB/s (% of peak) + decode steps/sec, 7B-shape batch 64"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD's published peak
DEFAULT_PARTITION = {1: 0, 2: 0, 3: 0, 4: 512, 5: 0}


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (default 2: the headline)")
    ap.add_argument("--partition", type=int, default=None,
                    help="split-KV partition size in tokens (0 = single pass)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--decode-only", action="store_true",
                    help="launch only the decode kernel repeatedly (for counter runs)")
    ap.add_argument("--unfused", action="store_true",
                    help="run the step as three calls (slot map, cache write, decode) instead "
                         "of kv_cache_append + decode")
    return ap.parse_args(argv)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "paged_kv_cache_33_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()


def step_bytes(w, step) -> dict:
    """Algorithmic bytes of one step (each byte the method must move, once)."""
    e = w.elem_bytes
    ctx = step.context_lens.astype(np.int64)
    ctx = np.maximum(ctx, 0)
    nb = (ctx + 15) // 16
    kv = int(ctx.sum()) * w.H_kv * w.d * 2 * e
    qo = 2 * w.B * w.H * w.d * e
    decode = kv + qo + 4 * int(nb.sum()) + 4 * w.B
    write = 2 * (2 * w.B * w.H_kv * w.d * e) + 8 * w.B      # K,V rows in and out, slots read
    slots = 4 * w.B + 4 * w.B + 8 * w.B                    # lengths, table entries, slots out
    return {"decode": decode, "kv": kv, "step": decode + write + slots}


def traffic_from_profile(kernel: str, workload: str, launches_per_step: int = 1):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return float(rec["hbm_bytes_per_dispatch"]) / launches_per_step


def calib_copy(mib: int, iters: int = 5) -> None:
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(iters):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n, "iters": iters}), flush=True)


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(sequences, KV heads and context partitions shard without exchange, but no "
              "multi-GPU path is built)", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.calib_copy_mib:
        calib_copy(args.calib_copy_mib)
        return 0

    import paged_kv_cache_33_amd as P
    from workloads import configs as W

    t0 = time.time()
    w = W.make_workload(args.config)
    part = DEFAULT_PARTITION[args.config] if args.partition is None else args.partition
    print(f"[bench] workload {w.name}: B={w.B} H={w.H} H_kv={w.H_kv} d={w.d} pool={w.num_blocks} "
          f"blocks, generated in {time.time() - t0:.1f}s; partition={part}", file=sys.stderr,
          flush=True)

    view = np.int16 if w.dtype == "bf16" else np.int32

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(view)).cuda()

    pool = P.KVPool(dev(w.k_pool), dev(w.v_pool), w.num_blocks, w.H_kv, w.d, w.dtype)
    tables = torch.from_numpy(w.block_tables).cuda()
    steps_dev = []
    for st in w.steps:
        steps_dev.append(dict(ctx=torch.from_numpy(st.context_lens).cuda(), q=dev(st.q),
                              k=dev(st.new_k), v=dev(st.new_v),
                              slots=torch.empty(w.B, dtype=torch.int64, device="cuda"),
                              L=int(st.context_lens.max())))
    L_max = max(s["L"] for s in steps_dev)
    out = torch.empty_like(steps_dev[0]["q"])
    ws = None
    if part:
        ws = torch.empty(P.paged_attention_workspace_bytes(w.B, w.H, w.d, L_max, part),
                         dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def run_step(i, ev=None):
        s = steps_dev[i % len(steps_dev)]
        if args.unfused:
            P.kv_slot_mapping(tables, s["ctx"], s["slots"], stream)
            P.reshape_and_cache(pool, s["k"], s["v"], s["slots"], stream)
        else:
            P.kv_cache_append(pool, s["k"], s["v"], tables, s["ctx"], s["slots"], stream)
        if ev is not None:
            ev[0].record(stream)
        P.paged_attention_decode(pool, out, s["q"], tables, s["ctx"], L_max, w.scale, part, ws,
                                 stream)
        if ev is not None:
            ev[1].record(stream)
        if part:
            P.paged_attention_reduce(out, ws, s["ctx"], L_max, part, w.dtype, stream)

    if args.decode_only:
        s = steps_dev[0]
        for _ in range(args.warmup + args.steps):
            P.paged_attention_decode(pool, out, s["q"], tables, s["ctx"], L_max, w.scale, part,
                                     ws, stream)
        torch.cuda.synchronize()
        print(json.dumps({"decode_only_launches": args.warmup + args.steps}), flush=True)
        return 0

    # one step, kept for the parity check against the CPU oracle
    run_step(0)
    torch.cuda.synchronize()
    first_out = out.cpu().numpy().copy()

    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        run_step(i, evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    dec_ms = [a.elapsed_time(b) for a, b in evs]
    dec_avg = float(np.mean(dec_ms))

    by = [step_bytes(w, st) for st in w.steps]
    used = [by[i % len(by)] for i in range(args.steps)]
    step_b = float(np.mean([u["step"] for u in used]))
    dec_b = float(np.mean([u["decode"] for u in used]))
    gbs = step_b / (ms_step * 1e-3) / 1e9
    dec_gbs = dec_b / (dec_avg * 1e-3) / 1e9
    kernel = "decode_mfma" if P.kv_decode_kernel_kind(pool, w.H) == 1 else "decode_valu"
    traffic = traffic_from_profile(kernel, w.name)

    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.B,
            "query_heads": w.H,
            "kv_heads": w.H_kv,
            "head_dim": w.d,
            "block_size": 16,
            "sum_context_tokens": int(w.steps[0].context_lens.astype(np.int64).sum()),
            "max_context_tokens": L_max,
            "partition_size": part,
            "seed": w.seed,
            "step": ("kv_slot_mapping + reshape_and_cache" if args.unfused else "kv_cache_append")
                    + " + paged_attention_decode" + (" + paged_attention_reduce" if part else ""),
        },
        "decode_steps_per_sec": round(1000.0 / ms_step, 1),
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "step_bytes": int(step_b),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(dec_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "bytes_per_launch": int(dec_b),
            "avg_launch_ms": round(dec_avg, 5),
        },
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, first_out, args.cpu_seconds)

    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline(w, gpu_out_bits: np.ndarray, budget_s: float) -> dict:
    """Time the float64 oracle on a bounded sample of sequences (one thread) and
    check the GPU's first-step output on the same sample."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    step = w.steps[0]
    slots = O.slot_mapping(w.block_tables, step.context_lens)
    kp, vp = O.reshape_and_cache(w.k_pool, w.v_pool, step.new_k, step.new_v, slots, w.H_kv, w.d,
                                 w.dtype, w.num_blocks)
    rng = np.random.default_rng(1234)
    order = rng.permutation(w.B)
    done, tokens, elapsed = [], 0, 0.0
    max_abs, num, den = 0.0, 0.0, 0.0
    for b in order:
        t = time.perf_counter()
        ref = O.decode_sequence(kp, vp, step.q[b], w.block_tables[b], int(step.context_lens[b]),
                                w.H, w.H_kv, w.d, w.dtype, w.scale)
        elapsed += time.perf_counter() - t
        done.append(int(b))
        tokens += int(step.context_lens[b])
        got = O.bits_to_f64(gpu_out_bits[b].view(np.uint16 if w.dtype == "bf16" else np.uint32),
                            w.dtype)
        max_abs = max(max_abs, float(np.abs(got - ref).max()))
        num += float(((got - ref) ** 2).sum())
        den += float((ref ** 2).sum())
        if elapsed >= budget_s:
            break
    if limiter is not None:
        limiter.unregister()
    total_tokens = int(np.maximum(step.context_lens, 0).sum())
    full_step_s = elapsed / max(tokens, 1) * total_tokens
    dec_bytes = step_bytes(w, step)["decode"]
    rel = math.sqrt(num / den) if den > 0 else 0.0
    ok = max_abs <= (1e-5 if w.dtype == "f32" else 1e-2) and (w.dtype == "f32" or rel <= 5e-3)
    if not ok:
        print(f"[bench] PARITY FAILURE on the oracle sample: max-abs {max_abs:.3e} rel-L2 {rel:.3e}",
              file=sys.stderr, flush=True)
    return {
        "value": round(dec_bytes / full_step_s / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{len(done)} of {w.B} sequences ({tokens} of {total_tokens} context tokens) of "
                  f"the first step, float64 NumPy, one BLAS thread; "
                  f"{elapsed:.1f}s, scaled to the whole step",
        "steps_per_sec": round(1.0 / full_step_s, 4),
        "parity": {"max_abs": max_abs, "rel_l2": rel, "ok": bool(ok)},
    }


if __name__ == "__main__":
    sys.exit(main())
