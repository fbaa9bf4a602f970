"""Free list, reference counts, block tables, fork and copy-on-write (oracle).

Test infrastructure only; see the package docstring for who may use it.

Semantics follow [pofe] "Minimal implementation" (``BlockPool`` and
``Sequence``) and the decode-step pseudocode of [pofe] "How it works":

* the free list starts as ids 0..N-1 and hands out the id at its end
  (last in, first out); a released block goes back on the end;
* alloc sets the count to 1, share adds 1, release subtracts 1 and frees the
  block when the count reaches 0 ([pofe] "on finish" pseudocode;
  [note] "Shared prefixes can share physical storage");
* fork gives the child a table that shares every parent block
  ([pofe] "Sharing and copy-on-write");
* append: if len mod B == 0 a new block is allocated and appended to the
  table; otherwise if the last block is shared (count > 1) a new block is
  allocated, the old block's contents are to be copied into it, the old block
  is released and the table's last entry is remapped (copy-on-write,
  [arch] 4. steps 1-4; [pofe] ``Sequence.append``).  The slot written is
  len mod B of the last entry; len then grows by one.

Preemption by swapping ([pofe] "When memory runs out") moves a whole
sequence out (every block released, its contents to be copied to host
memory) and back in (fresh blocks, all or none).

Running out of blocks raises :class:`NoFreeBlock` ([pofe] raises MemoryError
asking for a preemption; [arch] Step 1 raises MemoryError as well) and leaves
every table and count as it was.  The data movement itself (block copy,
slot write) is left to :mod:`oracle.cache_ops`; this module only decides.
"""

from __future__ import annotations


class NoFreeBlock(Exception):
    """The pool has no free block left (a preemption would be needed)."""


class OracleBlockPool:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(range(num_blocks))
        self.ref = [0] * num_blocks

    def alloc(self) -> int:
        if not self.free:
            raise NoFreeBlock("no free block: preempt a sequence")
        i = self.free.pop()
        self.ref[i] = 1
        return i

    def share(self, i: int) -> int:
        if self.ref[i] <= 0:
            raise ValueError(f"block {i} is not allocated")
        self.ref[i] += 1
        return i

    def release(self, i: int) -> None:
        if self.ref[i] <= 0:
            raise ValueError(f"block {i} is not allocated")
        self.ref[i] -= 1
        if self.ref[i] == 0:
            self.free.append(i)

    def num_free(self) -> int:
        return len(self.free)


class OracleSequence:
    def __init__(self, pool: OracleBlockPool):
        self.pool = pool
        self.table: list[int] = []
        self.len = 0
        self.swapped = False

    def reserve_prompt(self, n_tokens: int) -> None:
        """Admission: allocate ceil(n / B) blocks for an n-token prompt
        ([pofe] "How it works", admit pseudocode); prefill fills them."""
        if self.table or self.len:
            raise ValueError("reserve_prompt is for an empty sequence")
        need = -(-n_tokens // self.pool.block_size)
        if need > self.pool.num_free():
            raise NoFreeBlock("not enough free blocks for the prompt")
        self.table = [self.pool.alloc() for _ in range(need)]
        self.len = n_tokens

    def adopt_prefix(self, source: "OracleSequence", n_blocks: int) -> None:
        """Start an empty sequence on the first ``n_blocks`` full blocks of
        ``source``, shared by reference (a prefix hit: [arch] 4. and Step 1's
        prefix cache hands out the cached block and adds 1 to its count;
        [note] "Shared prefixes can share physical storage")."""
        if self.table or self.len:
            raise ValueError("adopt_prefix is for an empty sequence")
        if source.swapped:
            raise ValueError("a swapped-out sequence has no blocks to share")
        if n_blocks * self.pool.block_size > source.len:
            raise ValueError("only full blocks of the source can be adopted")
        self.table = [self.pool.share(i) for i in source.table[:n_blocks]]
        self.len = n_blocks * self.pool.block_size

    def extend_prompt(self, n_tokens: int) -> None:
        """Admit ``n_tokens`` more prompt tokens after the current length,
        allocating the blocks they need; the current last block must not be a
        shared partial block (prefill never writes into shared blocks)."""
        if self.swapped:
            raise ValueError("swap the sequence in first")
        b = self.pool.block_size
        if self.len % b != 0 and self.pool.ref[self.table[-1]] > 1:
            raise ValueError("cannot extend into a shared partial block")
        need = -(-(self.len + n_tokens) // b) - len(self.table)
        if need > self.pool.num_free():
            raise NoFreeBlock("not enough free blocks for the prompt")
        self.table += [self.pool.alloc() for _ in range(need)]
        self.len += n_tokens

    def fork(self) -> "OracleSequence":
        if self.swapped:
            raise ValueError("swap the sequence in first")
        child = OracleSequence(self.pool)
        child.table = [self.pool.share(i) for i in self.table]
        child.len = self.len
        return child

    def append_slot(self):
        """Decide where the next token goes; returns (block, slot, cow) with
        cow = (old, new) when a copy-on-write is needed, else None."""
        if self.swapped:
            raise ValueError("swap the sequence in first")
        b = self.pool.block_size
        cow = None
        if self.len % b == 0:
            self.table.append(self.pool.alloc())
        elif self.pool.ref[self.table[-1]] > 1:
            old = self.table[-1]
            new = self.pool.alloc()
            self.pool.release(old)
            self.table[-1] = new
            cow = (old, new)
        block, slot = self.table[-1], self.len % b
        self.len += 1
        return block, slot, cow

    def swap_out(self) -> list[int]:
        """Preempt by swapping ([pofe] "When memory runs out": whole
        sequences, all or none of their blocks, are copied to CPU memory).
        Returns the table (the blocks to copy out, slot i = logical block i)
        and releases every block; the length is kept.  Reading: shared blocks
        are copied as well and their references dropped, so a swapped-in
        sequence owns private copies."""
        if self.swapped:
            raise ValueError("sequence already swapped out")
        out = list(self.table)
        for i in self.table:
            self.pool.release(i)
        self.table = []
        self.swapped = True
        return out

    def swap_in(self) -> list[int]:
        """Bring a swapped sequence back: allocate ceil(len / B) blocks, all
        or none ([pofe]: whole sequences), and return them in table order
        (host slot i goes to block i)."""
        if not self.swapped:
            raise ValueError("sequence is not swapped out")
        need = -(-self.len // self.pool.block_size)
        if need > self.pool.num_free():
            raise NoFreeBlock("not enough free blocks to swap the sequence in")
        self.table = [self.pool.alloc() for _ in range(need)]
        self.swapped = False
        return list(self.table)

    def free_all(self) -> None:
        for i in self.table:
            self.pool.release(i)
        self.table = []
        self.len = 0
        self.swapped = False
