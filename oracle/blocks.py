"""A refcounted block manager with prefix sharing and copy-on-write.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path imports this module.

[share] §3.1-§3.2, §5.1, §6.1: the KV cache is cut into fixed-size blocks
(16 tokens by default, §5.2); a block table maps each sequence's logical
blocks to physical ones.  Sequences with a common prefix point at the same
physical blocks, each holding a reference count.  Appending a token to a
block that more than one sequence references first copies that block and
makes the copy private (copy-on-write); appending to a full block takes a
new one.  Ending a sequence drops one reference from each of its blocks and
returns a block to the free list only when no sequence references it; every
path that ends a sequence (normal end, cancel, timeout) goes through that
same rule.

Readings where the page is silent:

* Allocation takes the lowest-numbered free block, so the mapping is unique
  and the GPU side can be compared with this one bit for bit.
* share_prefix(src, dst, n) gives an empty dst the first ceil(n / bs) blocks
  of src and length n; the last of them may be only partly used by dst.
* A copy-on-write copy takes the rows the writing sequence already uses in
  that block (its length mod bs); the new token is then written after them.

Besides the table this module keeps, per physical row, what it holds: a
(sequence, position) tag of the token written there.  That is how the
isolation property is checked: every sequence must read back exactly its own
history through its table.

Pins (tests/test_oracle_blocks.py): the page's worked numbers (a 2000-token
prompt shared by 100 requests is stored once: 125 blocks of 16 instead of
12500), refcount = number of table entries naming a block, free list =
blocks with no reference, isolation under random interleavings of
allocate / share / append / free, and block counts ceil(len / bs).
"""

from __future__ import annotations


class BlocksExhausted(ValueError):
    """No free block left for an allocation or a copy-on-write."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be >= 1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.tables: dict = {}   # seq -> [physical block, ...]
        self.lens: dict = {}     # seq -> tokens
        self.rows: dict = {}     # (block, row) -> tag of the token stored there

    # -- allocation ------------------------------------------------------------
    def _take(self) -> int:
        for b in range(self.num_blocks):
            if self.ref[b] == 0:
                self.ref[b] = 1
                return b
        raise BlocksExhausted("no free block")

    def free_count(self) -> int:
        return sum(1 for r in self.ref if r == 0)

    def allocate(self, seq, num_tokens: int, tags=None) -> list:
        """An empty sequence gets room for num_tokens tokens (fresh blocks);
        returns the physical rows of those tokens in order."""
        if self.tables.get(seq):
            raise ValueError(f"sequence {seq} is not empty")
        need = -(-num_tokens // self.block_size)
        if need > self.free_count():
            raise BlocksExhausted(f"{need} blocks needed, {self.free_count()} free")
        self.tables[seq] = [self._take() for _ in range(need)]
        self.lens[seq] = num_tokens
        rows = [self.row_of(seq, i) for i in range(num_tokens)]
        for i, r in enumerate(rows):
            self.rows[r] = tags[i] if tags is not None else (seq, i)
        return rows

    def share_prefix(self, src, dst, prefix_len: int) -> None:
        """The first prefix_len tokens of dst point at src's blocks."""
        if self.tables.get(dst):
            raise ValueError(f"sequence {dst} is not empty")
        if prefix_len > self.lens.get(src, 0):
            raise ValueError("prefix longer than the source")
        n = -(-prefix_len // self.block_size)
        blocks = self.tables[src][:n]
        for b in blocks:
            self.ref[b] += 1
        self.tables[dst] = list(blocks)
        self.lens[dst] = prefix_len

    def append_token(self, seq, tag=None) -> tuple:
        """One token appended to seq; returns (row, copied) where copied is
        (old block, new block, rows copied) when a copy-on-write happened."""
        table = self.tables.setdefault(seq, [])
        n = self.lens.get(seq, 0)
        r = n % self.block_size
        copied = None
        if r == 0:
            table.append(self._take())
        else:
            old = table[-1]
            if self.ref[old] > 1:
                new = self._take()
                for i in range(r):
                    self.rows[(new, i)] = self.rows.get((old, i))
                self.ref[old] -= 1
                table[-1] = new
                copied = (old, new, r)
        row = (table[-1], r)
        self.rows[row] = tag if tag is not None else (seq, n)
        self.lens[seq] = n + 1
        return row, copied

    def free(self, seq) -> None:
        """Drops seq's references; blocks nobody references become free."""
        for b in self.tables.pop(seq, []):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                for i in range(self.block_size):
                    self.rows.pop((b, i), None)
        self.lens.pop(seq, None)

    # -- views -----------------------------------------------------------------
    def row_of(self, seq, i: int) -> tuple:
        return (self.tables[seq][i // self.block_size], i % self.block_size)

    def read(self, seq) -> list:
        """Tags of seq's tokens, read through its table."""
        return [self.rows.get(self.row_of(seq, i)) for i in range(self.lens.get(seq, 0))]
