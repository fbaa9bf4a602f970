"""Automatic prefix caching over the block pool (oracle).

Test infrastructure only; see the package docstring for who may use it.

[lesson] "Sharing, and the reference counting it needs": hash each
block-aligned prefix of token ids, look it up in a global table and reuse
the block on a hit; two prefixes share a block only if every token id is
equal.  [claims] "Paged Attention": because blocks are hashed by their token
sequence, a hit needs an unbroken matching prefix (the first differing token
ends the chain).  [arch] "Production PyTorch Implementation", Step 3: two
prompts with the same 16-token system prefix share its block (count 2).

Readings taken where the pages stop:

* Only full blocks of a prompt are cached; the key of logical block j is the
  whole token prefix 0 .. (j+1)B - 1 (here the exact tuple, so the oracle
  has no hash collisions by construction).  The walk stops at the first
  block whose prefix is not cached.
* A cached block whose count falls to 0 keeps its entry and waits, oldest
  first, in an evictable list (the LRU eviction the [lesson] section names
  for RadixAttention): a later hit revives it (count 1); an allocation that
  finds the free list empty evicts the oldest one, dropping its entry.
  Uncached blocks go back to the free list as in the plain pool.
* The blocks allocated for the uncached part of an admitted prompt are
  entered under their prefixes at once: the caller writes those positions
  (paged_kv_append_tokens) before any attention reads them.  A prefix that
  is already cached under another block (its parent was evicted, so the walk
  could not reach it) keeps its first block.
"""

from __future__ import annotations

from .block_manager import NoFreeBlock, OracleBlockPool, OracleSequence


class OraclePrefixPool(OracleBlockPool):
    def __init__(self, num_blocks: int, block_size: int):
        super().__init__(num_blocks, block_size)
        self.key_of: dict[int, tuple] = {}     # cached block -> its prefix
        self.block_of: dict[tuple, int] = {}   # prefix -> cached block
        self.lru: list[int] = []               # cached blocks with count 0, oldest first

    def num_free(self) -> int:
        """Blocks an allocation can take: free ones and evictable cached ones."""
        return len(self.free) + len(self.lru)

    def alloc(self) -> int:
        if self.free:
            i = self.free.pop()
        elif self.lru:
            i = self.lru.pop(0)
            del self.block_of[self.key_of.pop(i)]
        else:
            raise NoFreeBlock("no free block: preempt a sequence")
        self.ref[i] = 1
        return i

    def release(self, i: int) -> None:
        if self.ref[i] <= 0:
            raise ValueError(f"block {i} is not allocated")
        self.ref[i] -= 1
        if self.ref[i] == 0:
            if i in self.key_of:
                self.lru.append(i)
            else:
                self.free.append(i)

    def num_cached(self) -> int:
        return len(self.block_of)


def admit_prompt(seq: OracleSequence, tokens) -> int:
    """Admit an empty sequence with the given prompt token ids; returns the
    number of leading tokens whose keys and values are already in the cache
    (a multiple of B).  All or none: on NoFreeBlock nothing changes."""
    pool = seq.pool
    if not isinstance(pool, OraclePrefixPool):
        raise TypeError("prefix caching needs an OraclePrefixPool")
    if seq.table or seq.len or seq.swapped:
        raise ValueError("admit_prompt is for an empty sequence")
    tokens = [int(t) for t in tokens]
    b = pool.block_size
    full = len(tokens) // b
    hits = []
    for j in range(full):
        blk = pool.block_of.get(tuple(tokens[: (j + 1) * b]))
        if blk is None:
            break
        hits.append(blk)
    need = -(-len(tokens) // b) - len(hits)
    revived = sum(1 for blk in hits if pool.ref[blk] == 0)
    if need > pool.num_free() - revived:
        raise NoFreeBlock("not enough free blocks for the prompt")
    for blk in hits:
        if pool.ref[blk] == 0:
            pool.lru.remove(blk)
            pool.ref[blk] = 1
        else:
            pool.ref[blk] += 1
    new = [pool.alloc() for _ in range(need)]
    for j in range(len(hits), full):
        key = tuple(tokens[: (j + 1) * b])
        if key not in pool.block_of:
            blk = new[j - len(hits)]
            pool.block_of[key] = blk
            pool.key_of[blk] = key
    seq.table = hits + new
    seq.len = len(tokens)
    return len(hits) * b
