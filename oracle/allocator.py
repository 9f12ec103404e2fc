"""Oracle O1: the block allocator and block tables, in exact integers.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Written from:

  [velog] "구현 세부사항 / 메모리 할당자": an allocator hands out a free physical
      block id (allocate_block) and takes one back for reuse (free_block).
  [studynote 223] section II, figure: a request's KV lives in scattered physical
      blocks chained by a block table; when the request grows and runs out of
      room, an empty block is taken on demand and linked into the table.
  [velog] "작동 예시": with 16-token blocks a new block is taken exactly when
      token 17 and token 33 arrive (logical 0->3, 1->7, 2->2).
  [ch.09] "해법: 페이지처럼 나눠 담기": logical blocks look contiguous, physical
      blocks may be anywhere; any free physical block can be used, and internal
      waste is limited to the last block.
  [studynote 223] section II, copy-on-write paragraph and [velog] "메모리 공유
      (Copy-on-Write)": requests with the same prefix point at the same physical
      blocks; a request that starts writing something different gets its own copy.

Readings taken where the pages are silent (each is listed in the design doc):
  * free list order: FIFO.  The pool starts with a given order (default
    0..N-1); allocate takes the head, a block whose reference count falls to
    zero goes to the tail.  Sequence frees release blocks in logical order.
  * copy-on-write trigger: appending into a partially filled last block whose
    reference count is above one.  A full shared block never needs a copy (the
    next token opens a new block).  The copy target is allocated before any new
    block of the same append.  The last holder (count 1) writes in place.
  * an append is all-or-nothing: if the pool cannot supply every block it
    needs, it raises and nothing changes.
  * sequence ids are handed out 0, 1, 2, ... and never reused.
  * slot = physical_block * block_size + (position mod block_size).
  * padded block tables use -1.
"""

from collections import deque


class AllocatorError(Exception):
    """Base class of the oracle's allocator errors."""


class OutOfBlocks(AllocatorError):
    pass


class BadBlock(AllocatorError):
    pass


class BadSequence(AllocatorError):
    pass


class BlockAllocator:
    """Free list + reference counts + per-sequence block tables."""

    def __init__(self, num_blocks, block_size, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of 0..num_blocks-1")
        self.free = deque(order)
        self.refcount = [0] * self.num_blocks
        self.tables = {}    # seq id -> list of physical block ids, logical order
        self.lengths = {}   # seq id -> number of tokens held
        self.next_seq = 0

    # -- the pages' two calls ([velog] 메모리 할당자) ---------------------------
    def allocate_block(self):
        """Take a free physical block; its reference count becomes 1."""
        if not self.free:
            raise OutOfBlocks("no free block")
        b = self.free.popleft()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def free_block(self, block):
        """Drop one reference; at zero the block returns to the free pool."""
        if not (0 <= block < self.num_blocks) or self.refcount[block] == 0:
            raise BadBlock(f"block {block} is not allocated")
        self.refcount[block] -= 1
        if self.refcount[block] == 0:
            self.free.append(block)

    def num_free(self):
        return len(self.free)

    # -- sequences ---------------------------------------------------------------
    def _check_seq(self, seq):
        if seq not in self.tables:
            raise BadSequence(f"unknown sequence {seq}")

    def create_seq(self):
        s = self.next_seq
        self.next_seq += 1
        self.tables[s] = []
        self.lengths[s] = 0
        return s

    def fork(self, parent):
        """New sequence sharing every block of `parent` ([studynote 223] II, COW)."""
        self._check_seq(parent)
        child = self.create_seq()
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for b in self.tables[child]:
            self.refcount[b] += 1
        return child

    def _blocks_for(self, ntokens):
        bs = self.block_size
        return (ntokens + bs - 1) // bs

    def append_slots(self, seq, n):
        """Grow `seq` by n tokens.  Returns (slots, cow_pairs).

        slots[i] is the cache slot of position length+i.  cow_pairs is a list
        of (src, dst) physical blocks whose contents must be copied before the
        new tokens are written (at most one pair: only the last, partially
        filled block can be both shared and written).
        """
        self._check_seq(seq)
        if n < 0:
            raise ValueError("n must be >= 0")
        if n == 0:
            return [], []
        bs = self.block_size
        table = self.tables[seq]
        length = self.lengths[seq]
        needs_cow = (length % bs != 0) and self.refcount[table[-1]] > 1
        new_blocks = self._blocks_for(length + n) - self._blocks_for(length)
        if new_blocks + (1 if needs_cow else 0) > len(self.free):
            raise OutOfBlocks("append needs more blocks than are free")
        cow = []
        if needs_cow:
            src = table[-1]
            dst = self.allocate_block()
            self.refcount[src] -= 1          # stays >= 1: it was > 1
            table[-1] = dst
            cow.append((src, dst))
        slots = []
        for p in range(length, length + n):
            if p % bs == 0:
                table.append(self.allocate_block())
            slots.append(table[p // bs] * bs + p % bs)
        self.lengths[seq] = length + n
        return slots, cow

    def cow_block(self, seq, logical_index):
        """Make logical block `logical_index` of `seq` private.

        If the block is shared (count > 1) a fresh block is allocated, the
        pair (src, dst) is returned and the sequence points at dst; otherwise
        nothing changes and None is returned.
        """
        self._check_seq(seq)
        table = self.tables[seq]
        if not (0 <= logical_index < len(table)):
            raise ValueError("logical block index out of range")
        src = table[logical_index]
        if self.refcount[src] <= 1:
            return None
        dst = self.allocate_block()
        self.refcount[src] -= 1
        table[logical_index] = dst
        return (src, dst)

    def free_seq(self, seq):
        self._check_seq(seq)
        for b in self.tables[seq]:
            self.free_block(b)
        del self.tables[seq]
        del self.lengths[seq]

    # -- outputs -----------------------------------------------------------------
    def block_tables(self, seqs, max_blocks):
        """Rows of physical ids padded with -1, and the context lengths."""
        tables = []
        lens = []
        for s in seqs:
            self._check_seq(s)
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError(f"sequence {s} holds {len(t)} blocks > max_blocks {max_blocks}")
            tables.append(list(t) + [-1] * (max_blocks - len(t)))
            lens.append(self.lengths[s])
        return tables, lens


def run_script(alloc, script):
    """Execute an op script (see workloads) and collect what each op returned.

    Ops: ("create",) -> seq id; ("fork", parent) -> child id;
    ("append", seq, n) -> (slots, cow_pairs); ("cow", seq, logical) -> pair or None;
    ("free", seq) -> None.
    """
    results = []
    for op in script:
        kind = op[0]
        if kind == "create":
            results.append(alloc.create_seq())
        elif kind == "fork":
            results.append(alloc.fork(op[1]))
        elif kind == "append":
            results.append(alloc.append_slots(op[1], op[2]))
        elif kind == "cow":
            results.append(alloc.cow_block(op[1], op[2]))
        elif kind == "free":
            alloc.free_seq(op[1])
            results.append(None)
        else:
            raise ValueError(f"unknown op {kind!r}")
    return results
