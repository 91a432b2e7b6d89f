"""Block-manager oracle: the allocation side of paged KV memory, in plain Python.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module; the product's block manager is the
C++ one in libpa.so and shares no code with this file.

What the pages fix [P2 "PagedAttention 机制深度解析": 块表 / 工作流程 /
写时复制; P1 §01 continuous batching; P1 §02 Paged Attention]:

* The KV memory is a pool of equal physical blocks of ``block_size`` token
  slots; each request keeps a block table mapping its logical blocks, in
  order, to physical blocks.
* When a request needs room for a new token, a free block is taken from the
  pool and appended to the end of its block table (only when its last block
  is full: token ``p`` lives in logical block ``p // block_size`` at row
  ``p % block_size``).
* Several candidate sequences generated from one prompt (parallel sampling,
  beam search) share KV by copying only the block table: the copy points at
  the same physical blocks. A new physical block is given to a candidate
  only when it writes something the others do not share.
* The scheduler admits work only while free blocks remain.

Readings where the pages are silent (stated in the design notes too):

* Sharing is counted per physical block (reference count = number of block
  tables holding it); a block returns to the pool when its count drops to 0.
* Writing into a shared block that is only partly filled (the fork's last
  block) first copies it to a fresh block for the writer (copy-on-write): the
  writer's table entry moves to the copy, the old block loses one reference,
  and the (source, destination) pair is queued for the device copy, which
  must run before the new tokens' K/V are written. A full shared block is
  never written again, so it stays shared.
* Allocation order: the pool is a stack. Initially block 0 is on top, then
  1, 2, ...; blocks that come free are pushed on top and so are handed out
  first. A freed sequence releases its blocks from its last logical block to
  its first (so its first block ends on top).
* An append that needs more free blocks than the pool has changes nothing
  and reports the shortfall.
"""

from __future__ import annotations


class OutOfBlocks(Exception):
    """The pool cannot hold the tokens asked for; nothing was changed."""


class UnknownSequence(KeyError):
    """A sequence id that does not exist, or one that already exists."""


class BlockManagerOracle:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError("num_blocks >= 0 and block_size > 0 required")
        self.num_blocks = num_blocks
        self.block_size = block_size
        # stack of free blocks: the end of the list is the top
        self.free = list(range(num_blocks - 1, -1, -1))
        self.refs = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.copies: list[tuple[int, int]] = []

    # -- queries ------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def seq_len(self, seq: int) -> int:
        if seq not in self.lens:
            raise UnknownSequence(seq)
        return self.lens[seq]

    def block_table(self, seq: int) -> list[int]:
        if seq not in self.tables:
            raise UnknownSequence(seq)
        return list(self.tables[seq])

    def ref_count(self, block: int) -> int:
        return self.refs[block]

    def blocks_needed(self, seq: int, n: int) -> int:
        """Free blocks an append of n tokens to seq would take."""
        if n < 0:
            raise ValueError("n >= 0")
        table = self.tables.get(seq, [])
        length = self.lens.get(seq, 0)
        bs = self.block_size
        need = 0
        if n > 0 and length % bs != 0 and self.refs[table[-1]] > 1:
            need += 1  # copy-on-write of the shared, partly filled last block
        have = len(table)
        need += max(0, -(-(length + n) // bs) - have)
        return need

    # -- updates ------------------------------------------------------------
    def _pop(self) -> int:
        b = self.free.pop()
        assert self.refs[b] == 0
        self.refs[b] = 1
        return b

    def append(self, seq: int, n: int) -> list[int]:
        """Room for n new tokens of seq (created if new); returns their slots
        (block * block_size + row), in token order."""
        need = self.blocks_needed(seq, n)
        if need > len(self.free):
            raise OutOfBlocks(need - len(self.free))
        table = self.tables.setdefault(seq, [])
        length = self.lens.setdefault(seq, 0)
        bs = self.block_size
        if n > 0 and length % bs != 0 and self.refs[table[-1]] > 1:
            src = table[-1]
            dst = self._pop()
            self.refs[src] -= 1
            table[-1] = dst
            self.copies.append((src, dst))
        slots = []
        for p in range(length, length + n):
            j = p // bs
            if j == len(table):
                table.append(self._pop())
            slots.append(table[j] * bs + p % bs)
        self.lens[seq] = length + n
        return slots

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.tables or child in self.tables:
            raise UnknownSequence(child if parent in self.tables else parent)
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.refs[b] += 1

    def free_seq(self, seq: int) -> None:
        if seq not in self.tables:
            raise UnknownSequence(seq)
        for b in reversed(self.tables.pop(seq)):
            self.refs[b] -= 1
            if self.refs[b] == 0:
                self.free.append(b)
        del self.lens[seq]

    def take_copies(self, max_pairs: int) -> list[tuple[int, int]]:
        taken, self.copies = self.copies[:max_pairs], self.copies[max_pairs:]
        return taken


def copy_blocks(k_cache, v_cache, pairs):
    """Device-copy oracle: K[dst] = K[src] and V[dst] = V[src] for each
    (src, dst) pair in order, raw bits; pairs naming a block outside the pool
    are skipped. Arrays are numpy [num_blocks, block_size, Hkv, D]."""
    k, v = k_cache.copy(), v_cache.copy()
    nb = k.shape[0]
    for src, dst in pairs:
        if 0 <= src < nb and 0 <= dst < nb:
            k[dst] = k[src]
            v[dst] = v[src]
    return k, v
