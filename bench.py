"""Throughput of the paged decode-attention step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config N] [--partition P] [--cold]

A step is the whole hot path for one batch: the new token's slot mapping and
cache write (kv_cache_append), decode attention, and the log-sum-exp reduce
when split, all through libpagedkv's C ABI on the current torch stream.
Inputs are seeded and synthetic (workloads/), resident in HBM before timing
starts.

Order of work:
  1. the workload is generated on the host;
  2. the CPU baseline (unless --no-cpu-baseline): the float64 oracle on a
     bounded sample of the first step, one thread, then a pool of processes
     over the host cores; this runs before the GPU is touched, and the one-
     thread sample's outputs are kept as the parity reference;
  3. one GPU step, compared with that reference (a mismatch makes the exit
     status 3, after the JSON line);
  4. W warm-up steps, then the timed region: exactly K steps between two
     events, nothing else inside -> ms_per_step and `value`;
  5. K more steps with events around every kernel -> the decode kernel's
     average duration (`roofline`) and the step-time distribution;
  6. the read ceiling: kv_read_tiles over exactly the tiles the first step's
     decode reads (same loads, no arithmetic), timed over 10 launches; the
     decode's rate as a fraction of it is `roofline.frac_of_read_ceiling`.
With --cold every step is instead preceded by a 512 MiB write that evicts the
caches (outside the timed range) and timed alone.

Prints one JSON line.  `value` is HBM GB/s of the step's algorithmic bytes
(cached K/V read once, query, output, table and length reads, plus the cache
write's bytes) over ms_per_step; `roofline` prices the decode kernel alone
against the 8 TB/s HBM3E peak.
"""
from __future__ import annotations

import argparse
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
FLUSH_BYTES = 512 << 20  # twice the 256 MiB last-level cache
MAX_CPU_WORKERS = 16     # host cores a one-GPU share may use


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--ramp-ms", type=float, default=150.0,
                    help="untimed steps for this long before the warm-up steps, so the shader "
                         "clock has left its idle level (0: none)")
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (default 2: the headline)")
    ap.add_argument("--partition", type=int, default=None,
                    help="split-KV partition size in tokens (0 = single pass)")
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8", "int8"],
                    help="cache element type: bf16 (the workloads as configured), fp8 "
                         "(E4M3 codes, scales 1.0) or int8 (codes with per-token row scales); "
                         "activations stay bf16")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window in tokens (0 = whole context): each decode query "
                         "attends to its last W positions (paged_attention_decode_window)")
    ap.add_argument("--cold", action="store_true",
                    help="evict the caches before every step and time steps one by one")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the one-thread CPU oracle sample")
    ap.add_argument("--cpu-parallel-seconds", type=float, default=6.0,
                    help="wall-time budget of the multi-process CPU oracle run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--decode-only", action="store_true",
                    help="launch only the decode kernel repeatedly (for counter runs)")
    ap.add_argument("--serve", action="store_true",
                    help="a serving loop driven by the native block manager (prefix-cached "
                         "admission, forked samples, copy-on-write appends) at the 7B shape; "
                         "prints its own JSON line")
    ap.add_argument("--verify", type=int, default=0, metavar="K",
                    help="draft verification: K new tokens per sequence of --config (2 or 3), "
                         "written with kv_cache_append_chunk and attended with "
                         "paged_attention_multi; prints its own JSON line")
    ap.add_argument("--prefill", action="store_true",
                    help="chunked prefill: a 512-token chunk for each of 16 sequences "
                         "(64 query heads over 8 KV heads); prints its own JSON line")
    ap.add_argument("--unfused", action="store_true",
                    help="run the step as kv_slot_mapping + reshape_and_cache + the decode "
                         "instead of one kv_decode_step launch")
    ap.add_argument("--two-launch", action="store_true",
                    help="run the step as kv_cache_append + the decode instead of one "
                         "kv_decode_step launch")
    return ap.parse_args(argv)


# Sources each timed kernel is compiled from (its own file and the headers it
# includes); a counter summary stays valid while these hash the same.
KERNEL_SOURCES = {
    "decode_valu": ["decode_valu.hip", "device_common.h", "launch.h", "work_list.h"],
    "decode_mfma": ["decode_mfma.hip", "mfma_tile.h", "device_common.h", "launch.h",
                    "work_list.h"],
    "multi_mfma": ["multi_mfma.hip", "mfma_tile.h", "device_common.h", "launch.h",
                   "work_list.h"],
}


def kernel_source_hash(kernel: str = "") -> str:
    """SHA-256 over the sources of `kernel` (all kernel sources if empty)."""
    csrc = os.path.join(ROOT, "paged_kv_cache_33_amd", "csrc")
    names = KERNEL_SOURCES.get(kernel) or sorted(os.listdir(csrc))
    h = hashlib.sha256()
    for name in sorted(names):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def step_bytes(w, step, window: int = 0) -> dict:
    """Algorithmic bytes of one step (each byte the method must move, once).
    With a sliding window only the visible positions' K/V count (and the
    table entries of their blocks)."""
    e = w.elem_bytes            # query, output, rows handed to the write
    ec = w.kv_elem_bytes        # cache elements
    ctx = step.context_lens.astype(np.int64)
    ctx = np.maximum(ctx, 0)
    first = np.maximum(ctx - window, 0) if window > 0 else np.zeros_like(ctx)
    nb = (ctx + 15) // 16 - first // 16
    ctx = ctx - first
    kv = int(ctx.sum()) * w.H_kv * (w.d * ec + w.kv_row_extra_bytes) * 2
    qo = 2 * w.B * w.H * w.d * e
    decode = kv + qo + 4 * int(nb.sum()) + 4 * w.B
    write = 2 * w.B * w.H_kv * (w.d * (e + ec) + w.kv_row_extra_bytes)  # rows in, cache out
    slots = 4 * w.B + 4 * w.B + 8 * w.B                    # lengths, table entries, slots out
    return {"decode": decode, "kv": kv, "step": decode + write + slots}


def visible_tiles(w, step, window: int = 0) -> np.ndarray:
    """The (block, KV head) tiles a decode step reads, as tile indices
    p * H_kv + h, sequence by sequence in table order (each once per
    sequence, so a block shared by several sequences appears once for each)."""
    out = []
    hs = np.arange(w.H_kv, dtype=np.int64)
    for b, c in enumerate(step.context_lens.astype(np.int64)):
        if c <= 0:
            continue
        first = max(int(c) - window, 0) if window > 0 else 0
        blocks = w.block_tables[b][first // 16:(int(c) + 15) // 16].astype(np.int64)
        out.append((blocks[:, None] * w.H_kv + hs[None, :]).reshape(-1))
    return np.concatenate(out).astype(np.int32) if out else np.zeros(0, np.int32)


def read_ceiling(P, torch, pool, w, step, window, stream, launches: int = 10) -> dict:
    """Time kv_read_tiles over exactly the tiles the decode reads: the rate
    that access pattern reaches with no arithmetic (the decode's own ceiling)."""
    tiles = visible_tiles(w, step, window)
    tile_bytes = 16 * w.d * w.kv_elem_bytes
    groups = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    t = torch.from_numpy(tiles).cuda()
    sink = torch.empty(groups, dtype=torch.int32, device="cuda")
    for _ in range(3):
        P.kv_read_tiles(pool, t, sink, stream)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(launches):
        P.kv_read_tiles(pool, t, sink, stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / launches
    nbytes = 2 * int(tiles.size) * tile_bytes
    unique = 2 * int(np.unique(tiles).size) * (tile_bytes + 16 * w.kv_row_extra_bytes)
    return {"kernel": "read_tiles", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "unit": "GB/s", "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_per_launch": nbytes, "avg_launch_ms": round(ms, 5),
            "tiles": int(tiles.size), "unique_kv_bytes": unique}


def gpu_clocks(torch) -> dict:
    """Current shader and memory clock levels of device 0 from sysfs (the
    lines marked '*' of pp_dpm_sclk / pp_dpm_mclk), when the files are
    readable; empty otherwise."""
    try:
        p = torch.cuda.get_device_properties(0)
        base = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (
            int(getattr(p, "pci_domain_id", 0)), int(p.pci_bus_id), int(p.pci_device_id))
        out = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            path = os.path.join(base, name)
            if os.path.exists(path):
                with open(path) as f:
                    cur = [l.split(":", 1)[1].replace("*", "").strip()
                           for l in f.read().splitlines() if l.strip().endswith("*")]
                if cur:
                    out[name[7:]] = cur[0]
        return out
    except Exception:  # best effort: the clocks are context, not a result
        return {}


def ramp_clock(torch, step, ms: float) -> None:
    """Run `step` untimed until `ms` of wall time have passed (the shader
    clock climbs from its idle level over tens of milliseconds of load)."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step()
        torch.cuda.synchronize()


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return float(rec["hbm_bytes_per_dispatch"])


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


# --------------------------------------------------------------------------
# CPU baseline: the oracle, run before the GPU is initialised.

_CPU = {}  # state the forked workers read (shared copy-on-write)


def _cpu_prepare(w, window: int = 0):
    import oracle as O
    step = w.steps[0]
    slots = O.slot_mapping(w.block_tables, step.context_lens)
    kp, vp = O.reshape_and_cache(w.k_pool, w.v_pool, step.new_k, step.new_v, slots, w.H_kv, w.d,
                                 w.kv_dtype, w.num_blocks, w.k_scale, w.v_scale)
    _CPU.update(w=w, kp=kp, vp=vp, window=window)


def _cpu_one(b: int) -> np.ndarray:
    import oracle as O
    w = _CPU["w"]
    step = w.steps[0]
    return O.decode_sequence(_CPU["kp"], _CPU["vp"], step.q[b], w.block_tables[b],
                             int(step.context_lens[b]), w.H, w.H_kv, w.d, w.kv_dtype, w.scale,
                             w.k_scale, w.v_scale, window=_CPU["window"])


def _visible(ctx, window: int) -> int:
    """Context tokens a decode query attends to."""
    c = max(int(ctx), 0)
    return min(c, window) if window > 0 else c


def _cpu_worker(args):
    """Decode the sequences of `seqs` over and over (at least once) until
    budget_s has passed; return (context tokens decoded, seconds)."""
    seqs, budget_s = args
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        tokens = 0
        while True:
            for b in seqs:
                _cpu_one(int(b))
                tokens += _visible(_CPU["w"].steps[0].context_lens[b], _CPU["window"])
                if time.perf_counter() - t0 >= budget_s:
                    return tokens, time.perf_counter() - t0


def _host_info() -> dict:
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def cpu_baseline(w, budget_s: float, par_budget_s: float, window: int = 0):
    """Oracle throughput on a bounded sample of the first step.  Returns the
    record and {sequence: float64 output [H, d]} of the one-thread sample."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    _cpu_prepare(w, window)
    step = w.steps[0]
    order = np.random.default_rng(1234).permutation(w.B)
    # one thread: the sampled sequences' outputs are the parity reference; once
    # every sequence is done the walk starts again, until budget_s has passed
    refs, tokens, elapsed = {}, 0, 0.0
    with threadpool_limits(limits=1):
        while elapsed < budget_s:
            for b in order:
                t = time.perf_counter()
                ref = _cpu_one(int(b))
                elapsed += time.perf_counter() - t
                refs.setdefault(int(b), ref)
                tokens += _visible(step.context_lens[b], window)
                if elapsed >= budget_s:
                    break
    total_tokens = sum(_visible(c, window) for c in step.context_lens)
    dec_bytes = step_bytes(w, step, window)["decode"]
    one_step_s = elapsed / max(tokens, 1) * total_tokens

    host = _host_info()
    n_proc = max(1, min(MAX_CPU_WORKERS, host["affinity_cores"]))
    par = None
    if n_proc > 1 and par_budget_s > 0:
        # every worker walks its own share of a second seeded order of sequences
        order2 = np.random.default_rng(4321).permutation(w.B)
        shares = [order2[i::n_proc] for i in range(n_proc)]
        shares = [s for s in shares if len(s)]
        ctx = mp.get_context("fork")
        t0 = time.perf_counter()
        with ctx.Pool(len(shares)) as pool:
            res = pool.map(_cpu_worker, [(s, par_budget_s) for s in shares])
        wall = time.perf_counter() - t0
        par_tokens = sum(r[0] for r in res)
        par = {"procs": len(shares), "tokens": par_tokens, "wall_s": wall,
               "step_s": wall / max(par_tokens, 1) * total_tokens}
    _CPU.clear()

    if par is not None and par["step_s"] < one_step_s:
        best_s, cores = par["step_s"], par["procs"]
        sample = (f"first step of the workload ({w.B} sequences, {total_tokens} context "
                  f"tokens), float64 NumPy oracle, one BLAS thread per process: "
                  f"{par['procs']} processes over disjoint seeded shares of the sequences, each "
                  f"repeating its share until {par_budget_s:.0f}s had passed, decoded "
                  f"{par['tokens']} context tokens in {par['wall_s']:.1f}s wall; scaled to one "
                  f"step.  One process alone: {tokens} context tokens in {elapsed:.1f}s")
    else:
        best_s, cores = one_step_s, 1
        sample = (f"{len(refs)} of {w.B} sequences of the first step ({tokens} context tokens "
                  f"decoded, {total_tokens} in the step), float64 NumPy, one BLAS thread; "
                  f"{elapsed:.1f}s, scaled to the whole step"
                  + ("" if par is None else f" (faster than {par['procs']} processes here)"))
    rec = {
        "value": round(dec_bytes / best_s / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": sample,
        "steps_per_sec": round(1.0 / best_s, 4),
        "one_core_value": round(dec_bytes / one_step_s / 1e9, 4),
        "host": host,
    }
    return rec, refs


def parity_vs_refs(w, gpu_out_bits: np.ndarray, refs: dict) -> dict:
    import oracle as O
    max_abs, num, den = 0.0, 0.0, 0.0
    view = np.uint16 if w.dtype == "bf16" else np.uint32
    for b, ref in refs.items():
        got = O.bits_to_f64(gpu_out_bits[b].view(view), w.dtype)
        max_abs = max(max_abs, float(np.abs(got - ref).max()))
        num += float(((got - ref) ** 2).sum())
        den += float((ref ** 2).sum())
    rel = math.sqrt(num / den) if den > 0 else 0.0
    ok = max_abs <= (1e-5 if w.dtype == "f32" else 1e-2) and (w.dtype == "f32" or rel <= 5e-3)
    return {"sequences": len(refs), "max_abs": max_abs, "rel_l2": rel, "ok": bool(ok)}


# --------------------------------------------------------------------------
# Serving loop on the native block manager

def serve(args) -> int:
    """B sequences share a 1,024-token system prompt (found in the prefix cache
    after the first admission) plus 16..300 private tokens; every fourth
    sequence is forked once (a second sample).  Each step appends one token to
    every sequence (one kv_bm_append_batch call), copies the shared last blocks
    that the appends name (one kv_copy_blocks), writes the new rows at the
    manager's slots, uploads the batch tables and decodes; every eighth step
    four samples are released and forked again, so copies on write keep
    happening.  Step time covers all of it, host included."""
    import torch
    import paged_kv_cache_33_amd as P
    torch.cuda.set_device(0)
    H = H_kv = 32
    d, B0, system_len = 128, 48, 1024
    rng = np.random.default_rng(5)
    system = rng.integers(0, 32000, size=system_len).tolist()
    private = rng.integers(16, 301, size=B0)
    num_blocks = 8192
    elem = 2
    n = num_blocks * H_kv * 16 * d
    kc = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    vc = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    kc.normal_()
    vc.normal_()
    pool = P.KVPool(kc, vc, num_blocks, H_kv, d, "bf16")
    bm = P.BlockManager(num_blocks)
    seqs, hits_total = [], 0
    for b in range(B0):
        prompt = system + rng.integers(0, 32000, size=int(private[b])).tolist()
        hits_total += bm.admit(b, prompt)
        seqs.append(b)
    for b in range(0, B0, 4):
        bm.fork(b, 1000 + b)
        seqs.append(1000 + b)
    B = len(seqs)
    max_nb = 128
    q = torch.randn(B, H, d, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    rows = torch.randn(B, H_kv, d, device="cuda").to(torch.bfloat16)
    stream = torch.cuda.current_stream()
    scale = 1.0 / math.sqrt(d)

    parents = list(range(0, B0, 4))
    children = {p: 1000 + p for p in parents}
    next_child = 2000
    state = {"i": 0}

    def step():
        nonlocal next_child
        t0 = time.perf_counter()
        if state["i"] % 8 == 7:                # re-sample: four forks replace their children
            for p in parents[:4]:
                old = children[p]
                bm.release(old)
                bm.fork(p, next_child)
                seqs[seqs.index(old)] = next_child
                children[p] = next_child
                next_child += 1
            for _ in range(4):                 # the next four parents go next time
                parents.append(parents.pop(0))
        state["i"] += 1
        slots, copies = bm.append_batch(seqs, rng.integers(0, 32000, size=B))
        tables, lens = bm.batch_tables(seqs, max_nb)
        host = time.perf_counter() - t0
        if len(copies):
            cp = torch.from_numpy(np.ascontiguousarray(copies.T)).cuda(non_blocking=True)
            P.kv_copy_blocks(pool, cp[0], cp[1], stream)
        P.reshape_and_cache(pool, rows, rows, torch.from_numpy(slots).cuda(non_blocking=True),
                            stream)
        tt = torch.from_numpy(tables).cuda(non_blocking=True)
        cl = torch.from_numpy(lens).cuda(non_blocking=True)
        P.paged_attention_decode(pool, out, q, tt, cl, int(lens.max()), scale, 0, None, stream)
        return host, len(copies), int(lens.sum())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    host_s, copies, ctx_tokens = 0.0, 0, 0
    t0 = time.perf_counter()
    for _ in range(args.steps):
        h, c, ct = step()
        host_s += h
        copies += c
        ctx_tokens += ct
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall / args.steps * 1e3
    kv = ctx_tokens / args.steps * H_kv * d * 2 * elem
    print(json.dumps({
        "metric": "serving step on the native block manager, 7B shape",
        "value": round(1000.0 / ms, 1), "unit": "steps/s", "ms_per_step": round(ms, 4),
        "steps": args.steps, "warmup": args.warmup, "batch": B,
        "forked_samples": B - B0, "prefix_tokens_found_at_admission": hits_total,
        "host_block_manager_us_per_step": round(host_s / args.steps * 1e6, 1),
        "copy_on_write_blocks_per_step": round(copies / args.steps, 2),
        "kv_GBs": round(kv / (ms * 1e-3) / 1e9, 1),
        "dtype": "bf16", "data": "synthetic",
        "step": "kv_bm_append_batch + kv_bm_batch_tables + kv_copy_blocks + reshape_and_cache "
                "+ table upload + paged_attention_decode",
    }), flush=True)
    return 0


# --------------------------------------------------------------------------
# Several new tokens per sequence: draft verification and chunked prefill

PEAK_MFMA_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
PREFILL_CHUNK = 512


def multi_workload(args):
    from workloads import configs as W
    kv = args.kv_dtype if args.kv_dtype != "bf16" else ""
    if args.prefill:
        # chunk k of a prompt: the chunk is the last 512 of 512..4096 context tokens
        rng = np.random.default_rng(2024)
        ctx = rng.integers(PREFILL_CHUNK, 4097, size=16)
        w = W.multi_token_workload(f"prefill-chunk{PREFILL_CHUNK}-b16-gqa64x8", "bf16", 16, 64, 8,
                                   128, ctx, [PREFILL_CHUNK] * 16, seed=2024,
                                   kv_dtype=kv or None)
        return w
    if args.config not in (2, 3):
        raise SystemExit("--verify runs on --config 2 or 3")
    w = W.make_workload(args.config, kv_dtype=kv)
    W.add_multi_step(w, [args.verify] * w.B, seed=900 + args.config)
    w.name = f"{w.name}-verify{args.verify}"
    return w


def multi_bytes_flops(w) -> dict:
    """Algorithmic bytes and flops of one multi-token step."""
    m = w.multi
    ctx = m.context_lens.astype(np.int64)
    n = np.diff(m.query_start).astype(np.int64)
    T = int(n.sum())
    e, ec = w.elem_bytes, w.kv_elem_bytes
    kv = int(ctx.sum()) * w.H_kv * (w.d * ec + w.kv_row_extra_bytes) * 2  # every cached row once
    nb = (ctx + 15) // 16
    attn = kv + 2 * T * w.H * w.d * e + 4 * int(nb.sum()) + 4 * (2 * w.B + 1)
    write = 2 * T * w.H_kv * (w.d * (e + ec) + w.kv_row_extra_bytes) + 8 * T
    # row at position p: q.k and p.v over p + 1 keys, per query head
    seen = sum(int(((c - k + 1) + c) * k // 2) for c, k in zip(ctx, n))
    flops = 4 * w.H * w.d * seen
    return {"attn": attn, "kv": kv, "write": write, "step": attn + write, "flops": flops,
            "rows": T}


def multi(args) -> int:
    """Time the multi-token step (chunk write + causal multi-row attention) and,
    on the same pool, the one-token decode step of the same sequences."""
    import torch
    import oracle as O
    import paged_kv_cache_33_amd as P
    w = multi_workload(args)
    m = w.multi
    print(f"[bench] {w.name} ({w.kv_dtype} cache): B={w.B} H={w.H} H_kv={w.H_kv} rows="
          f"{int(m.query_start[-1])}", file=sys.stderr, flush=True)
    torch.cuda.set_device(0)
    views = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32}

    def dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(views.get(a.dtype, a.dtype))).cuda()

    pool = P.KVPool(dev(w.k_pool), dev(w.v_pool), w.num_blocks, w.H_kv, w.d, w.kv_dtype,
                    w.k_scale, w.v_scale)
    tables = torch.from_numpy(w.block_tables).cuda()
    ctx = torch.from_numpy(m.context_lens).cuda()
    qs = torch.from_numpy(m.query_start).cuda()
    mq = int(np.diff(m.query_start).max())
    q, nk, nv = dev(m.q), dev(m.new_k), dev(m.new_v)
    out = torch.empty_like(q)
    slots = torch.empty(q.shape[0], dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    st = w.steps[0]
    dq, dk, dv = dev(st.q), dev(st.new_k), dev(st.new_v)
    dout = torch.empty_like(dq)
    L = int(m.context_lens.max())

    def run(ev=None):
        if ev is not None:
            ev[0].record(stream)
        P.kv_cache_append_chunk(pool, nk, nv, qs, mq, tables, ctx, slots, stream)
        if ev is not None:
            ev[1].record(stream)
        P.paged_attention_multi(pool, out, q, qs, mq, tables, ctx, w.scale, stream)
        if ev is not None:
            ev[2].record(stream)

    def run_decode():
        P.kv_cache_append(pool, dk, dv, tables, ctx, None, stream)
        P.paged_attention_decode(pool, dout, dq, tables, ctx, L, w.scale, 0, None, stream)

    # parity of three sequences' rows against the oracle
    run()
    torch.cuda.synchronize()
    sl = O.chunk_slots(w.block_tables, m.context_lens, m.query_start)
    kp, vp = O.reshape_and_cache(w.k_pool, w.v_pool, m.new_k, m.new_v, sl, w.H_kv, w.d,
                                 w.kv_dtype, w.num_blocks, w.k_scale, w.v_scale)
    seqs = [int(np.argmin(m.context_lens)), int(np.argmax(m.context_lens)), w.B // 2]
    ref = O.decode_multi(kp, vp, m.q, m.query_start, w.block_tables, m.context_lens, w.H, w.H_kv,
                         w.d, w.kv_dtype, w.scale, w.k_scale, w.v_scale, seqs=seqs)
    got = out.cpu().numpy().view(np.uint16)
    worst, num, den = 0.0, 0.0, 0.0
    for b, r in ref.items():
        g = O.bits_to_f64(got[m.query_start[b]:m.query_start[b + 1]], "bf16")
        amp = np.maximum(1.0, np.abs(r).reshape(len(r), -1).max(axis=1))
        worst = max(worst, float((np.abs(g - r).reshape(len(r), -1).max(axis=1) / amp).max()))
        num += float(((g - r) ** 2).sum())
        den += float((r ** 2).sum())
    rel = math.sqrt(num / den)
    parity = {"sequences": seqs, "max_abs_over_row_scale": worst, "rel_l2": rel,
              "ok": bool(worst <= 1e-2 and rel <= 5e-3)}

    ramp_clock(torch, run, args.ramp_ms)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        run()
    b_.record(stream)
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b_) / args.steps
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
           for _ in range(args.steps)]
    for i in range(args.steps):
        run(evs[i])
    torch.cuda.synchronize()
    attn_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    write_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    for _ in range(args.warmup):
        run_decode()
    a.record(stream)
    for _ in range(args.steps):
        run_decode()
    b_.record(stream)
    torch.cuda.synchronize()
    dec_ms = a.elapsed_time(b_) / args.steps

    bf = multi_bytes_flops(w)
    attn_avg = float(attn_ms.mean())
    if args.prefill:
        achieved = bf["flops"] / (attn_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_BF16_TFLOPS, 4)}
    else:
        achieved = bf["attn"] / (attn_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof.update({"kernel": "multi_mfma", "traffic": None, "bytes_per_launch": bf["attn"],
                 "flops_per_launch": bf["flops"], "avg_launch_ms": round(attn_avg, 5)})
    rows = bf["rows"]
    print(json.dumps({
        "metric": ("chunked-prefill attention over a paged KV cache" if args.prefill else
                   "draft verification over a paged KV cache (K new tokens per sequence)"),
        "value": round(rows / (ms_step * 1e-3), 1), "unit": "query tokens/s",
        "ms_per_step": round(ms_step, 5), "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "n_gpus": 1,
        "dtype": "bf16" if w.kv_dtype == "bf16" else f"{w.kv_dtype} cache, bf16 activations",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "query_heads": w.H, "kv_heads": w.H_kv,
                   "head_dim": w.d, "rows": rows,
                   "sum_context_tokens": int(m.context_lens.astype(np.int64).sum()),
                   "step": "kv_cache_append_chunk + paged_attention_multi"},
        "step_GBs": round(bf["step"] / (ms_step * 1e-3) / 1e9, 1),
        "write_ms_avg": round(float(write_ms.mean()), 5),
        "decode_step_ms_same_pool": round(dec_ms, 5),
        "step_over_decode_step": round(ms_step / dec_ms, 3),
        "roofline": roof,
        "parity": parity,
    }), flush=True)
    return 0 if parity["ok"] else 3


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(sequences, KV heads and context partitions shard without exchange, but no "
              "multi-GPU path is built)", file=sys.stderr)
        return 2

    if args.calib_copy_mib:
        import torch
        torch.cuda.set_device(0)
        calib_copy(args.calib_copy_mib)
        return 0
    if args.serve:
        return serve(args)
    if args.verify or args.prefill:
        return multi(args)

    from workloads import configs as W
    t0 = time.time()
    w = W.make_workload(args.config, kv_dtype=args.kv_dtype if args.kv_dtype != "bf16" else "")
    part = DEFAULT_PARTITION[args.config] if args.partition is None else args.partition
    print(f"[bench] workload {w.name} ({w.kv_dtype} cache): B={w.B} H={w.H} H_kv={w.H_kv} d={w.d} pool={w.num_blocks} "
          f"blocks, generated in {time.time() - t0:.1f}s; partition={part}", file=sys.stderr,
          flush=True)

    cpu_rec, refs = None, None
    if not (args.no_cpu_baseline or args.decode_only):
        t0 = time.time()
        cpu_rec, refs = cpu_baseline(w, args.cpu_seconds, args.cpu_parallel_seconds, args.window)
        print(f"[bench] cpu baseline done in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)

    import paged_kv_cache_33_amd as P

    views = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32}

    def dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(views.get(a.dtype, a.dtype))).cuda()

    pool = P.KVPool(dev(w.k_pool), dev(w.v_pool), w.num_blocks, w.H_kv, w.d, w.kv_dtype,
                    w.k_scale, w.v_scale)
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
    kernel = "decode_mfma" if P.kv_decode_kernel_kind(pool, w.H) == 1 else "decode_valu"

    # The step: one kv_decode_step launch (the write on extra work-groups, the
    # attention taking the newest position from the new rows, as the write
    # stores them), or the write and the decode as separate launches.
    one_launch = not (args.unfused or args.two_launch)

    def run_step(i, ev=None):
        """One step; ev = (before write, before decode, after decode, after step)
        events (with one launch the first two coincide)."""
        s = steps_dev[i % len(steps_dev)]
        if ev is not None:
            ev[0].record(stream)
        if one_launch:
            if ev is not None:
                ev[1].record(stream)
            P.kv_decode_step(pool, out, s["q"], s["k"], s["v"], tables, s["ctx"], L_max, w.scale,
                             part, ws, s["slots"], stream, window=args.window)
        else:
            if args.unfused:
                P.kv_slot_mapping(tables, s["ctx"], s["slots"], stream)
                P.reshape_and_cache(pool, s["k"], s["v"], s["slots"], stream)
            else:
                P.kv_cache_append(pool, s["k"], s["v"], tables, s["ctx"], s["slots"], stream)
            if ev is not None:
                ev[1].record(stream)
            P.paged_attention_decode(pool, out, s["q"], tables, s["ctx"], L_max, w.scale, part,
                                     ws, stream, window=args.window)
        if ev is not None:
            ev[2].record(stream)
        if part:
            P.paged_attention_reduce(out, ws, s["ctx"], L_max, part, w.dtype, stream,
                                     window=args.window)
        if ev is not None:
            ev[3].record(stream)

    if args.decode_only:
        # decode launches alone (for counter runs); with --cold each one follows
        # a write of twice the last-level cache, so it starts from HBM
        s = steps_dev[0]
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda") if args.cold else None
        for i in range(args.warmup + args.steps):
            if flush is not None:
                flush.fill_(i & 0xFF)
            if one_launch:
                P.kv_decode_step(pool, out, s["q"], s["k"], s["v"], tables, s["ctx"], L_max,
                                 w.scale, part, ws, s["slots"], stream, window=args.window)
            else:
                P.paged_attention_decode(pool, out, s["q"], tables, s["ctx"], L_max, w.scale,
                                         part, ws, stream, window=args.window)
        torch.cuda.synchronize()
        print(json.dumps({"decode_only_launches": args.warmup + args.steps}), flush=True)
        return 0

    # 3. parity of the first step against the oracle sample
    run_step(0)
    torch.cuda.synchronize()
    parity = parity_vs_refs(w, out.cpu().numpy(), refs) if refs else None
    if parity is not None and not parity["ok"]:
        print(f"[bench] PARITY FAILURE on the oracle sample: {parity}", file=sys.stderr, flush=True)

    def new_events(n):
        return [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(n)]

    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda") if args.cold else None

    # 4. clock ramp, warm-up, then the timed region.  From idle the shader
    # clock climbs over tens of milliseconds of load (sysfs samples: 1.2-1.3
    # GHz at the first launch, above 2 GHz after about 100 ms), and launches
    # in the first ~20 ms run up to 40% slower; steps run untimed until
    # --ramp-ms of wall time have passed, so the timed steps see the clock a
    # sustained decode loop runs at.
    ramp_clock(torch, lambda: run_step(0), args.ramp_ms)
    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    if not args.cold:
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(args.steps):
            run_step(i)
        end.record(stream)
        torch.cuda.synchronize()
        ms_step = start.elapsed_time(end) / args.steps

    # 5. the instrumented pass (the timed pass itself with --cold)
    evs = new_events(args.steps)
    for i in range(args.steps):
        if args.cold:
            flush_buf.fill_(i & 0xFF)
        run_step(i, evs[i])
    torch.cuda.synchronize()
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    write_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    step_ms = np.array([e[0].elapsed_time(e[3]) for e in evs])
    if args.cold:
        ms_step = float(step_ms.mean())
    dec_avg = float(dec_ms.mean())

    by = [step_bytes(w, st, args.window) for st in w.steps]
    used = [by[i % len(by)] for i in range(args.steps)]
    step_b = float(np.mean([u["step"] for u in used]))
    # the timed kernel: the decode, or with one launch the decode and the write
    dec_b = float(np.mean([u["step"] if one_launch else u["decode"] for u in used]))
    gbs = step_b / (ms_step * 1e-3) / 1e9
    dec_gbs = dec_b / (dec_avg * 1e-3) / 1e9
    wname = w.name + (f"-window{args.window}" if args.window else "")
    traffic = traffic_from_profile(kernel, wname + ("-cold" if args.cold else ""))
    ceiling = read_ceiling(P, torch, pool, w, w.steps[0], args.window, stream)
    clocks = gpu_clocks(torch)

    def pct(a, q):
        return round(float(np.percentile(a, q)), 5)

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
        "dtype": w.dtype if w.kv_dtype == w.dtype else f"{w.kv_dtype} cache, {w.dtype} activations",
        "data": "synthetic",
        "config": {
            "workload": wname,
            "batch": w.B,
            "query_heads": w.H,
            "kv_heads": w.H_kv,
            "head_dim": w.d,
            "block_size": 16,
            "sum_context_tokens": int(w.steps[0].context_lens.astype(np.int64).sum()),
            "max_context_tokens": L_max,
            "partition_size": part,
            "window": args.window,
            "seed": w.seed,
            "kv_cache": w.kv_dtype,
            "step": ("kv_decode_step (cache write and attention in one launch)" if one_launch
                     else ("kv_slot_mapping + reshape_and_cache" if args.unfused
                           else "kv_cache_append")
                     + (" + paged_attention_decode_window" if args.window else
                        " + paged_attention_decode"))
                    + ((" + paged_attention_reduce_window" if args.window else
                        " + paged_attention_reduce") if part else ""),
            "caches": "evicted before every step" if args.cold else "warm (steps back to back)",
        },
        "decode_steps_per_sec": round(1000.0 / ms_step, 1),
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "step_bytes": int(step_b),
        "step_ms_instrumented": {"p10": pct(step_ms, 10), "median": pct(step_ms, 50),
                                 "p90": pct(step_ms, 90)},
        "write_ms_avg": round(float(write_ms.mean()), 5),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel + (" (with the cache write: kv_decode_step)" if one_launch else ""),
            "achieved": round(dec_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "bytes_per_launch": int(dec_b),
            "avg_launch_ms": round(dec_avg, 5),
            "launch_ms_p10_median_p90": [pct(dec_ms, 10), pct(dec_ms, 50), pct(dec_ms, 90)],
            "frac_of_read_ceiling": round(dec_gbs / ceiling["achieved"], 4),
        },
        "read_ceiling": ceiling,
        "kv_bytes_logical": int(np.mean([u["kv"] for u in used])),
        "kv_bytes_unique": ceiling["unique_kv_bytes"],
        "decode_gbps_unique_kv": round(ceiling["unique_kv_bytes"] / (dec_avg * 1e-3) / 1e9, 1),
        "gpu_clocks": clocks,
    }
    if cpu_rec is not None:
        cpu_rec["parity"] = parity
        result["cpu_baseline"] = cpu_rec

    print(json.dumps(result), flush=True)
    return 3 if (parity is not None and not parity["ok"]) else 0


if __name__ == "__main__":
    sys.exit(main())
