"""Model of prefix caching by block keys.

TEST INFRASTRUCTURE (see the package docstring): the native prefix cache
(kv_prefix_cache_* in include/kvpaged.h) must match this model bit for bit
on every operation trace.

What the explainer says ["PagedAttention Nedir?" (bitcanli.com), section
"Prefix Sharing Nasıl Çalışır?"]: requests that start with the same tokens
can reuse the K/V computed for that start, but only when the token sequence
itself matches (and the model, adapter and other context that shape the
cache do); the keys that find reusable data take both a block's contents and
the context before it into account; the gain is in prefill, and only while
the blocks are still cached.

Readings (the pages give no formula; one rule is fixed so both
implementations agree exactly):
  * only full blocks are keyed; the key of block i of a prompt is
    FNV-1a-64 over the bytes of (key of block i-1, or 0 for the first block;
    the salt; the block's B token ids), as little-endian u64, u64 and int32s.
    The salt stands for "the model, adapter and other context";
  * an entry stores its block id, parent key and token ids; a lookup or an
    insert accepts a key only if the stored parent and tokens are equal (a
    hash collision is a miss, never a wrong reuse);
  * lookup walks a prompt's full blocks from the first and stops at the
    first miss; every block found gets one more reference for the caller;
  * insert walks the same chain over the caller's blocks: a missing key is
    inserted with one reference held by the cache; an existing equal entry
    is kept (the caller's block is not cached); a colliding key ends the
    walk;
  * every block a lookup or insert passes is "used": a tick counter is
    advanced over the chain from its last block to its first, so the blocks
    of a chain age tail first;
  * evict frees cached blocks that only the cache references (refcount 1),
    least recently used first, and drops their entries. A child whose
    parent was evicted is unreachable until it is evicted in turn.
"""
from __future__ import annotations

import struct
from typing import Dict, List, Optional, Sequence, Tuple

from .allocator import ModelPool

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """FNV-1a, 64-bit (Fowler, Noll, Vo): per byte, xor then multiply."""
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_key(parent: int, salt: int, tokens: Sequence[int]) -> int:
    data = struct.pack("<QQ", parent & MASK64, salt & MASK64)
    data += b"".join(struct.pack("<i", int(t)) for t in tokens)
    return fnv1a64(data)


class _Entry:
    __slots__ = ("block", "parent", "tokens", "last_use")

    def __init__(self, block: int, parent: int, tokens: Tuple[int, ...]):
        self.block = block
        self.parent = parent
        self.tokens = tokens
        self.last_use = 0


class ModelPrefixCache:
    def __init__(self, pool: ModelPool, salt: int, key_fn=block_key):
        self.pool = pool
        self.B = pool.block_size
        self.salt = salt & MASK64
        self.key_fn = key_fn
        self.entries: Dict[int, _Entry] = {}
        self.tick = 0

    def _chain(self, tokens: Sequence[int]):
        """(key, parent, block tokens) of each full block, first to last."""
        out, parent = [], 0
        for i in range(len(tokens) // self.B):
            toks = tuple(int(t) for t in tokens[i * self.B:(i + 1) * self.B])
            k = self.key_fn(parent, self.salt, toks)
            out.append((k, parent, toks))
            parent = k
        return out

    def _match(self, k: int, parent: int, toks) -> Optional[_Entry]:
        e = self.entries.get(k)
        if e is None or e.parent != parent or e.tokens != toks:
            return None
        return e

    def _touch(self, entries: List[_Entry]) -> None:
        for e in reversed(entries):
            self.tick += 1
            e.last_use = self.tick

    def lookup(self, tokens: Sequence[int]) -> List[int]:
        found: List[_Entry] = []
        for k, parent, toks in self._chain(tokens):
            e = self._match(k, parent, toks)
            if e is None:
                break
            found.append(e)
        blocks = [e.block for e in found]
        if blocks:
            assert self.pool.share(blocks) == 0
        self._touch(found)
        return blocks

    def insert(self, tokens: Sequence[int], blocks: Sequence[int]) -> int:
        """The caller's blocks hold the K/V of `tokens` (blocks[i] = its
        block i). Returns the number of entries added."""
        passed: List[_Entry] = []
        added = 0
        for i, (k, parent, toks) in enumerate(self._chain(tokens)):
            e = self.entries.get(k)
            if e is None:
                b = int(blocks[i])
                assert self.pool.share([b]) == 0
                e = _Entry(b, parent, toks)
                self.entries[k] = e
                added += 1
            elif e.parent != parent or e.tokens != toks:
                break
            passed.append(e)
        self._touch(passed)
        return added

    def evict(self, n: int) -> List[int]:
        """Free up to n cache-only blocks, least recently used first;
        returns them in the order freed."""
        cands = sorted((e.last_use, k) for k, e in self.entries.items()
                       if self.pool.refcount(e.block) == 1)
        freed = []
        for _, k in cands[:max(0, n)]:
            b = self.entries.pop(k).block
            assert self.pool.free_blocks([b]) == 0
            freed.append(b)
        return freed

    def size(self) -> int:
        return len(self.entries)
