"""CPU oracle for prefix-block matching (host side of the prefix cache).

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: imported by tests/ and
bench.py's CPU leg, never by the library.

What it follows: "Qwen3-4B / 8B / 32B", intro and Architecture Notes (paged
KV cache, prefix caching on by default, prefix matching against the GPU KV
cache) and section Warm Prefix-Cache TTFT (a repeated prompt lands as a
warm prefix hit and skips most of its prefill).  The pages give no
mechanism; the plainest reading, used here:

  * Only sealed (full, 16-token) blocks are cached.  A cached block is
    identified by the token ids of the whole prefix that ends with it, so
    block i of a sequence can be reused only if blocks 0..i-1 match as well.
  * A lookup returns the longest run of leading full blocks whose prefixes
    are all cached, and the physical blocks holding them.
  * Registering a sequence's sealed blocks adds the prefixes not yet cached;
    a prefix already cached keeps its first block.  A block id already
    cached under another prefix means the block was reused for other
    tokens: that entry, and every entry extending it, is dropped first.
    Ids given for blocks already cached are ignored; an id that appears
    twice among the blocks to register, or that already holds one of the
    sequence's own cached blocks, is an error (nothing changes).  A negative
    id stops the registration there; so does a full index.
  * Removing a block drops its entry and every entry extending it.

Everything is a plain dict keyed by prefix tuples: slow and obviously
correct.  Parity with the library is exact (integers).
"""
from __future__ import annotations

BLOCK = 16


class PrefixCache:
    def __init__(self, capacity: int):
        self.capacity = int(capacity)
        self.entries: dict[tuple, int] = {}      # full-prefix token tuple -> block id

    def _key(self, tokens, i):
        return tuple(int(t) for t in tokens[:BLOCK * (i + 1)])

    def match(self, tokens) -> list:
        """Block ids of the longest cached run of leading full blocks."""
        out = []
        for i in range(len(tokens) // BLOCK):
            key = self._key(tokens, i)
            if key not in self.entries:
                break
            out.append(self.entries[key])
        return out

    def remove(self, block: int) -> int:
        """Drop the entry held by `block` and every entry extending it."""
        roots = [k for k, v in self.entries.items() if v == block]
        gone = [k for k in self.entries if any(k[:len(r)] == r for r in roots)]
        for k in gone:
            del self.entries[k]
        return len(gone)

    def insert(self, tokens, block_ids):
        """Register the sealed blocks of a sequence; returns the number of
        new entries, or None for an invalid call (nothing changed)."""
        n = min(len(tokens) // BLOCK, len(block_ids))
        path, i = [], 0
        while i < n and self._key(tokens, i) in self.entries:
            path.append(self.entries[self._key(tokens, i)])
            i += 1
        new = []
        for j in range(i, n):
            if block_ids[j] < 0:
                break
            new.append(int(block_ids[j]))
        if len(set(new)) != len(new) or set(new) & set(path):
            return None
        added = 0
        for j, b in enumerate(new, start=i):
            if len(self.entries) >= self.capacity and b not in self.entries.values():
                break
            self.remove(b)
            if len(self.entries) >= self.capacity:
                break
            self.entries[self._key(tokens, j)] = b
            added += 1
        return added

    def __len__(self):
        return len(self.entries)
