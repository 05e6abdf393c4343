"""Oracle of the host-side block bookkeeping of a paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by tests, never by the product path.

What it models ("Forward Deployed Engineering Interview", Ch.2 section 8, the
block-manager teaching model and its demo; "Anthropic Interview: Design an LLM
Inference API with GPU Batching", 4.1/4.2 data model: block tables, a free
stack, reference counts):

  * blocks of 16 token slots; each has a reference count, the token ids it
    holds and, once full, a prefix key;
  * the prefix key of a full block covers its parent's key (the block before it
    in the table) and its own tokens; a sequence's first block starts from its
    salt, so another salt, or one changed early token, changes every key after
    it; only full blocks get keys and enter the prefix cache;
  * admitting a prompt reuses cached blocks for an unbroken run of full blocks
    from the start of the prompt and takes fresh blocks for the rest; a cached
    block that was released but not yet reused is taken back out of the free
    queue;
  * taking a block pops the front of the free queue (the least recently freed)
    and drops the cache entry the block still carried;
  * appending a token opens a fresh block when the last one is full, and copies
    the last block first when it is shared (copy-on-write): a shared block is
    never written;
  * forking gives the child the parent's table, every block's count + 1;
  * releasing drops one reference from each block, last block first; a block
    whose count reaches zero joins the back of the free queue and keeps its
    cache entry until it is taken again.

Readings where the page is silent: an operation that needs more free blocks
than there are fails with NoBlocks and changes nothing (the page's model raises
part-way); the prefix key is SHA-256 over an encoding of the parent key (or the
salt) and the token ids (only key equality matters).

Parity status: pinned by the demo's printed results (tests/golden) and by
bookkeeping invariants (tests/test_block_manager.py).
"""
from __future__ import annotations

import hashlib
from collections import deque
from typing import Dict, List, Optional, Tuple

BLOCK = 16


class NoBlocks(Exception):
    """Not enough free blocks for the operation (nothing was changed)."""


class _Block:
    __slots__ = ("id", "refs", "tokens", "key")

    def __init__(self, bid: int):
        self.id = bid
        self.refs = 0
        self.tokens: List[int] = []
        self.key: Optional[bytes] = None


def prefix_key(parent: Optional[bytes], tokens: List[int], salt: str) -> bytes:
    """Key of a full block: SHA-256 of the parent's key (the salt for a first
    block) followed by the block's token ids."""
    h = hashlib.sha256()
    if parent is None:
        h.update(b"S" + salt.encode("utf-8"))
    else:
        h.update(b"P" + parent)
    h.update(b"|" + ",".join(str(int(t)) for t in tokens).encode())
    return h.digest()


class BlockManagerModel:
    def __init__(self, num_blocks: int):
        self.blocks = [_Block(i) for i in range(num_blocks)]
        self.free: deque = deque(self.blocks)         # front = taken first
        self.cache: Dict[bytes, _Block] = {}
        self.seqs: Dict[int, Tuple[List[_Block], str]] = {}

    # ---------------------------------------------------------------- helpers
    def _take(self, tokens: List[int]) -> _Block:
        b = self.free.popleft()
        if b.key is not None and self.cache.get(b.key) is b:
            del self.cache[b.key]
        b.refs, b.tokens, b.key = 1, list(tokens), None
        return b

    def _seal(self, b: _Block, parent: Optional[bytes], salt: str) -> None:
        if len(b.tokens) == BLOCK:
            b.key = prefix_key(parent, b.tokens, salt)
            self.cache.setdefault(b.key, b)

    def _plan_admit(self, prompt: List[int], salt: str):
        """Cached blocks an admit would reuse (in order) and fresh blocks it needs."""
        reuse: List[_Block] = []
        parent = None
        n_chunks = -(-len(prompt) // BLOCK)
        for c in range(n_chunks):
            chunk = prompt[c * BLOCK:(c + 1) * BLOCK]
            if len(chunk) < BLOCK:
                break
            b = self.cache.get(prefix_key(parent, chunk, salt))
            if b is None:
                break
            reuse.append(b)
            parent = b.key
        return reuse, n_chunks - len(reuse)

    # ---------------------------------------------------------------- operations
    def admit(self, seq: int, prompt: List[int], salt: str = "") -> int:
        """Build seq's table for a new prompt; return the prompt tokens found cached."""
        if seq in self.seqs:
            raise ValueError(f"sequence {seq} exists")
        reuse, fresh = self._plan_admit(prompt, salt)
        revived = sum(1 for b in reuse if b.refs == 0)
        if fresh > len(self.free) - revived:
            raise NoBlocks
        table: List[_Block] = []
        for b in reuse:
            if b.refs == 0:
                self.free.remove(b)
            b.refs += 1
            table.append(b)
        for c in range(len(reuse), len(reuse) + fresh):
            chunk = prompt[c * BLOCK:(c + 1) * BLOCK]
            b = self._take(chunk)
            self._seal(b, table[-1].key if table else None, salt)
            table.append(b)
        self.seqs[seq] = (table, salt)
        return len(reuse) * BLOCK

    def append(self, seq: int, token: int):
        """Write one token.  Returns (slot, copy) where copy is (src, dst) when the
        shared last block was copied first, else None."""
        table, salt = self.seqs[seq]
        copy = None
        last = table[-1] if table else None
        if last is None or len(last.tokens) == BLOCK:
            if not self.free:
                raise NoBlocks
            table.append(self._take([]))
        elif last.refs > 1:
            if not self.free:
                raise NoBlocks
            last.refs -= 1
            nb = self._take(last.tokens)
            copy = (last.id, nb.id)
            table[-1] = nb
        b = table[-1]
        b.tokens.append(int(token))
        self._seal(b, table[-2].key if len(table) > 1 else None, salt)
        slot = b.id * BLOCK + len(b.tokens) - 1
        return slot, copy

    def fork(self, seq: int, child: int) -> None:
        if child in self.seqs:
            raise ValueError(f"sequence {child} exists")
        table, salt = self.seqs[seq]
        for b in table:
            b.refs += 1
        self.seqs[child] = (list(table), salt)

    def release(self, seq: int) -> None:
        table, _ = self.seqs.pop(seq)
        for b in reversed(table):
            b.refs -= 1
            if b.refs == 0:
                self.free.append(b)

    # ---------------------------------------------------------------- views
    def num_free(self) -> int:
        return len(self.free)

    def table(self, seq: int) -> List[int]:
        return [b.id for b in self.seqs[seq][0]]

    def num_tokens(self, seq: int) -> int:
        t = self.seqs[seq][0]
        return 0 if not t else (len(t) - 1) * BLOCK + len(t[-1].tokens)

    def refs(self) -> List[int]:
        return [b.refs for b in self.blocks]

    def free_order(self) -> List[int]:
        return [b.id for b in self.free]
