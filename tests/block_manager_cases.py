"""Drivers shared by the block-manager tests: the page's demo, replayed from
tests/golden/block_manager_demo.json, and seeded random operation sequences.

`bm` is any object with admit(seq, prompt, salt) -> hits, append(seq, token)
-> (slot, copy), fork(seq, child), release(seq), num_free(), table(seq) -> ids,
num_tokens(seq); failures for lack of blocks raise the given exception type.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_manager_demo.json")


def load_demo():
    with open(GOLDEN) as f:
        return json.load(f)


def _prompt(spec, system):
    out = []
    for part in spec:
        if part == "system":
            out += system
        elif part == "system[1:]":
            out += system[1:]
        else:
            out += list(part)
    return out


def replay_demo(bm):
    """Run the demo on bm; return the list of printed values."""
    d = load_demo()
    system = list(range(*d["system"]))
    ids = {}
    seq_id = lambda name: ids.setdefault(name, len(ids) + 1)  # noqa: E731
    printed = []
    for st in d["steps"]:
        op = st["op"]
        if op == "admit":
            printed.append(bm.admit(seq_id(st["seq"]), _prompt(st["prompt"], system), st["salt"]))
        elif op == "fork":
            bm.fork(seq_id(st["seq"]), seq_id(st["child"]))
        elif op == "append":
            bm.append(seq_id(st["seq"]), st["token"])
        elif op == "free":
            printed.append(bm.num_free())
        elif op == "release":
            bm.release(seq_id(st["seq"]))
    return printed


def random_ops(seed: int, n_ops: int, vocab: int = 6):
    """A seeded list of operations over a small token vocabulary (so that
    prefixes repeat and hit the cache)."""
    rng = np.random.default_rng(seed)
    ops = []
    live = []
    next_id = 1
    prefixes = [list(rng.integers(0, vocab, size=rng.integers(16, 80))) for _ in range(4)]
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.3 or not live:
            base = prefixes[rng.integers(0, len(prefixes))]
            cut = int(rng.integers(0, len(base) + 1))
            tail = list(rng.integers(0, vocab, size=int(rng.integers(0, 40))))
            salt = ["", "", "t1"][int(rng.integers(0, 3))]
            ops.append(("admit", next_id, [int(t) for t in base[:cut] + tail], salt))
            live.append(next_id)
            next_id += 1
        elif r < 0.65:
            ops.append(("append", live[int(rng.integers(0, len(live)))], int(rng.integers(0, vocab))))
        elif r < 0.8:
            ops.append(("fork", live[int(rng.integers(0, len(live)))], next_id))
            live.append(next_id)
            next_id += 1
        else:
            s = live.pop(int(rng.integers(0, len(live))))
            ops.append(("release", s))
    return ops


def run_ops(bm, ops, no_blocks_exc):
    """Apply ops; return the trace of results (NoBlocks recorded, state unchanged)."""
    trace = []
    live = set()
    for op in ops:
        kind = op[0]
        try:
            if kind == "admit":
                if op[1] in live:
                    continue
                trace.append(("admit", op[1], bm.admit(op[1], op[2], op[3])))
                live.add(op[1])
            elif kind == "append":
                if op[1] not in live:
                    continue
                trace.append(("append", op[1], bm.append(op[1], op[2])))
            elif kind == "fork":
                if op[1] not in live or op[2] in live:
                    continue
                bm.fork(op[1], op[2])
                live.add(op[2])
                trace.append(("fork", op[1], op[2]))
            elif kind == "release":
                if op[1] not in live:
                    continue
                bm.release(op[1])
                live.discard(op[1])
                trace.append(("release", op[1]))
        except no_blocks_exc:
            trace.append((kind, op[1], "no-blocks"))
        trace.append(("free", bm.num_free()))
        trace.append(("tables", tuple((s, tuple(bm.table(s)), bm.num_tokens(s)) for s in sorted(live))))
    return trace
