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
  * taking a block takes the least recently freed one and drops the cache
    entry the block still carried;
  * appending a token opens a fresh block when the last one is full, and copies
    the last block first when it is shared (copy-on-write): a shared block is
    never written;
  * forking gives the child the parent's table, every block's count + 1;
  * releasing drops one reference from each block, last block first; a block
    whose count reaches zero becomes the most recently freed one and keeps its
    cache entry until it is taken again.

Form.  The state is a set of plain arrays indexed by block id (reference
count, contents, key, and the time at which a block was last freed, absent
while it is referenced) plus the prefix index and the tables.  The free queue
is not stored as a list: the free blocks are those with a free-time, taken in
increasing free-time order.  Every operation first derives the complete change
it would make (which blocks it revives, takes, and what it writes), checks it
against the free count, and only then applies it, so a failed operation
leaves the state untouched by construction.

Readings where the page is silent: an operation that needs more free blocks
than there are fails with NoBlocks and changes nothing (the page's model raises
part-way); the prefix key is SHA-256 over an encoding of the parent key (or the
salt) and the token ids (only key equality matters).

Parity status: pinned by the demo's printed results (tests/golden) and by
bookkeeping invariants (tests/test_block_manager.py).
"""
from __future__ import annotations

import hashlib
from typing import Dict, List, Optional, Sequence, Tuple

BLOCK = 16


class NoBlocks(Exception):
    """Not enough free blocks for the operation (nothing was changed)."""


def prefix_key(parent: Optional[bytes], tokens: Sequence[int], salt: str) -> bytes:
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
        n = num_blocks
        self.refcount: List[int] = [0] * n
        self.content: List[Tuple[int, ...]] = [()] * n
        self.key: List[Optional[bytes]] = [None] * n
        # free-time of every unreferenced block (block i starts free at time i)
        self.freed_at: Dict[int, int] = {i: i for i in range(n)}
        self.clock = n
        self.index: Dict[bytes, int] = {}          # prefix key -> block id
        self.tables: Dict[int, List[int]] = {}
        self.salt: Dict[int, str] = {}

    # ------------------------------------------------------------ derived facts
    def _key_of(self, table: List[int], pos: int, salt: str) -> Optional[bytes]:
        """Key the block at table position `pos` gets if it is full."""
        b = table[pos]
        if len(self.content[b]) != BLOCK:
            return None
        parent = self.key[table[pos - 1]] if pos > 0 else None
        return prefix_key(parent, self.content[b], salt)

    def _oldest_free(self, count: int, excluded=()) -> List[int]:
        """The `count` least recently freed blocks, skipping `excluded`."""
        order = sorted((t, b) for b, t in self.freed_at.items() if b not in excluded)
        if len(order) < count:
            raise NoBlocks
        return [b for _, b in order[:count]]

    # ------------------------------------------------------------ state changes
    def _reference(self, b: int) -> None:
        self.freed_at.pop(b, None)
        self.refcount[b] += 1

    def _unreference(self, b: int) -> None:
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.freed_at[b] = self.clock
            self.clock += 1

    def _recycle(self, b: int, tokens: Tuple[int, ...]) -> None:
        """Give free block b new contents: its old cache entry goes, it is held once."""
        old = self.key[b]
        if old is not None and self.index.get(old) == b:
            del self.index[old]
        self.key[b] = None
        self.content[b] = tuple(tokens)
        self._reference(b)

    def _publish(self, table: List[int], pos: int, salt: str) -> None:
        """Key a block that has just become full and enter it in the prefix index
        (an existing entry for the same key is kept)."""
        k = self._key_of(table, pos, salt)
        if k is not None:
            self.key[table[pos]] = k
            self.index.setdefault(k, table[pos])

    # ------------------------------------------------------------ operations
    def admit(self, seq: int, prompt: List[int], salt: str = "") -> int:
        """Build seq's table for a new prompt; return the prompt tokens found cached."""
        if seq in self.tables:
            raise ValueError(f"sequence {seq} exists")
        chunks = [tuple(int(t) for t in prompt[i:i + BLOCK]) for i in range(0, len(prompt), BLOCK)]
        # longest run of full leading chunks already in the prefix index
        hits: List[int] = []
        parent: Optional[bytes] = None
        for chunk in chunks:
            b = self.index.get(prefix_key(parent, chunk, salt)) if len(chunk) == BLOCK else None
            if b is None:
                break
            hits.append(b)
            parent = self.key[b]
        fresh = self._oldest_free(len(chunks) - len(hits), excluded=set(hits))
        # apply
        for b in hits:
            self._reference(b)
        table = list(hits)
        for chunk, b in zip(chunks[len(hits):], fresh):
            self._recycle(b, chunk)
            table.append(b)
            self._publish(table, len(table) - 1, salt)
        self.tables[seq] = table
        self.salt[seq] = salt
        return len(hits) * BLOCK

    def append(self, seq: int, token: int):
        """Write one token.  Returns (slot, copy) where copy is (src, dst) when the
        shared last block was copied first, else None."""
        table = self.tables[seq]
        last = table[-1] if table else None
        opens = last is None or len(self.content[last]) == BLOCK
        copies = not opens and self.refcount[last] > 1
        target = self._oldest_free(1)[0] if (opens or copies) else last
        copy = None
        if opens:
            self._recycle(target, ())
            table.append(target)
        elif copies:
            self._unreference(last)
            self._recycle(target, self.content[last])
            table[-1] = target
            copy = (last, target)
        self.content[target] = self.content[target] + (int(token),)
        self._publish(table, len(table) - 1, self.salt[seq])
        return target * BLOCK + len(self.content[target]) - 1, copy

    def fork(self, seq: int, child: int) -> None:
        if child in self.tables:
            raise ValueError(f"sequence {child} exists")
        for b in self.tables[seq]:
            self._reference(b)
        self.tables[child] = list(self.tables[seq])
        self.salt[child] = self.salt[seq]

    def release(self, seq: int) -> None:
        table = self.tables.pop(seq)
        self.salt.pop(seq)
        for pos in range(len(table) - 1, -1, -1):
            self._unreference(table[pos])

    # ------------------------------------------------------------ views
    def num_free(self) -> int:
        return len(self.freed_at)

    def table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def num_tokens(self, seq: int) -> int:
        return sum(len(self.content[b]) for b in self.tables[seq])

    def refs(self) -> List[int]:
        return list(self.refcount)

    def free_order(self) -> List[int]:
        return [b for _, b in sorted((t, b) for b, t in self.freed_at.items())]
