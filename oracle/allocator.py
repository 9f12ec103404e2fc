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

Readings taken where the pages are silent:
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
        self.hit_tokens = 0     # tokens found cached (prefix caching only)
        self.evictions = 0      # cached blocks handed to a new owner (prefix caching only)

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

    def _available(self):
        """Blocks an allocation can still obtain."""
        return len(self.free)

    def num_cached(self):
        return 0

    def stats(self):
        """Occupancy counts, for fragmentation accounting ([ch.09] "문제: 연속
        할당의 단편화" and "해법: 페이지처럼 나눠 담기": with paging the only
        waste is the unfilled tail of each sequence's last block).

        stored_tokens is the number of distinct physical slots (block, offset)
        that hold a position of some live sequence -- positions p < length
        map to (table[p // bs], p mod bs) -- so a shared slot counts once."""
        bs = self.block_size
        held = set()
        for s, table in self.tables.items():
            for p in range(self.lengths[s]):
                held.add((table[p // bs], p % bs))
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self.free),
            "cached_blocks": self.num_cached(),
            "used_blocks": sum(1 for c in self.refcount if c >= 1),
            "shared_blocks": sum(1 for c in self.refcount if c >= 2),
            "live_seqs": len(self.tables),
            "logical_tokens": sum(self.lengths.values()),
            "stored_tokens": len(held),
            "hit_tokens": self.hit_tokens,
            "evictions": self.evictions,
        }

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
        if new_blocks + (1 if needs_cow else 0) > self._available():
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
        if self._available() == 0:
            raise OutOfBlocks("no free block")
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


class PrefixCachingAllocator(BlockAllocator):
    """The allocator with automatic prefix caching.

    Written from: [studynote 528] section II, key ideas (requests with the same
    system prompt share its blocks and skip re-computing it) and section IV
    (prefix caching for a shared system prompt lowers the time to first
    token); [ch.09] "09. PagedAttention", closing section (the next chapter's
    subject: finding reusable prompt blocks automatically); [studynote 223]
    section II copy-on-write paragraph (identical prefixes point at the same
    physical blocks).  The pages give the idea, not the rules; the rules taken
    here:

      * A full block's content is identified by (content of the block before
        it, its block_size token ids); the first block's predecessor is the
        empty prefix.  Identity is exact: equal ids mean equal token streams.
      * append_tokens: a new block that the call fills completely, in a
        sequence whose content is known so far, is looked up; if a block with
        that content is cached, the sequence points at it (its count + 1) and
        those tokens get slot -1 (their K/V is already in the pool).  Hits are
        taken before any fresh block of the same call is allocated.
      * A block that becomes full with known content is registered as the
        cached block of that content, unless another block already is.
      * When its count drops to zero, a registered block is kept, with its
        contents, on an evictable list (oldest first) instead of the free
        list.  An allocation takes the free list's head; if that is empty, it
        evicts the oldest evictable block (which forgets its content).
      * append_slots (no token ids) makes the sequence's content unknown: none
        of its later blocks is looked up or registered.
    """

    ROOT = 0

    def __init__(self, num_blocks, block_size, free_order=None):
        super().__init__(num_blocks, block_size, free_order)
        self.content_ids = {}                 # (parent content, tokens) -> content id (1, 2, ...)
        self.cached = {}                      # content id -> physical block
        self.content_of = [0] * num_blocks    # physical block -> content id it is registered under
        self.evictable = []                   # registered blocks with count 0, oldest first
        self.chain = {}                       # seq -> content id of its last full block, -1 unknown
        self.pending = {}                     # seq -> token ids of its partial last block

    def _available(self):
        return len(self.free) + len(self.evictable)

    def num_cached(self):
        return len(self.evictable)

    def allocate_block(self):
        if self.free:
            return super().allocate_block()
        if not self.evictable:
            raise OutOfBlocks("no free block")
        b = self.evictable.pop(0)
        self.evictions += 1
        del self.cached[self.content_of[b]]
        self.content_of[b] = 0
        self.refcount[b] = 1
        return b

    def free_block(self, block):
        if not (0 <= block < self.num_blocks) or self.refcount[block] == 0:
            raise BadBlock(f"block {block} is not allocated")
        self.refcount[block] -= 1
        if self.refcount[block] == 0:
            (self.evictable if self.content_of[block] else self.free).append(block)

    def create_seq(self):
        s = super().create_seq()
        self.chain[s] = self.ROOT
        self.pending[s] = []
        return s

    def fork(self, parent):
        child = super().fork(parent)
        self.chain[child] = self.chain[parent]
        self.pending[child] = list(self.pending[parent])
        return child

    def free_seq(self, seq):
        super().free_seq(seq)
        del self.chain[seq]
        del self.pending[seq]

    def append_slots(self, seq, n):
        out = super().append_slots(seq, n)
        if n:
            self.chain[seq] = -1
            self.pending[seq] = []
        return out

    def _content(self, parent, tokens, create):
        key = (parent, tuple(int(t) for t in tokens))
        cid = self.content_ids.get(key)
        if cid is None and create:
            cid = len(self.content_ids) + 1
            self.content_ids[key] = cid
        return cid

    def append_tokens(self, seq, tokens):
        """Grow `seq` by the given token ids.  Returns (slots, cow_pairs, n_cached):
        slots as append_slots, with -1 for a token whose block was found in
        the cache; n_cached counts those tokens."""
        self._check_seq(seq)
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        if n == 0:
            return [], [], 0
        bs = self.block_size
        table = self.tables[seq]
        length = self.lengths[seq]
        needs_cow = (length % bs != 0) and self.refcount[table[-1]] > 1
        # plan: which new blocks are cache hits
        chain = self.chain[seq]
        pend = list(self.pending[seq])
        hits = {}                             # logical block index -> cached physical block
        new_blocks = 0
        p = length
        while p < length + n:
            i = p - length
            if p % bs == 0:
                new_blocks += 1
                full = p + bs <= length + n
                if full and chain >= 0:
                    cid = self._content(chain, tokens[i:i + bs], create=False)
                    if cid is not None and cid in self.cached:
                        hits[p // bs] = self.cached[cid]
                    chain = self._content(chain, tokens[i:i + bs], create=True)
                elif chain >= 0:
                    pend = tokens[i:]         # a partial new block
                p += bs if full else (length + n - p)
            else:
                # filling the existing partial block
                take = min(bs - p % bs, length + n - p)
                if chain >= 0:
                    pend = pend + tokens[i:i + take]
                    if len(pend) == bs:
                        chain = self._content(chain, pend, create=True)
                        pend = []
                p += take
        pinned = sum(1 for b in hits.values() if self.refcount[b] == 0)
        if new_blocks - len(hits) + (1 if needs_cow else 0) > self._available() - pinned:
            raise OutOfBlocks("append needs more blocks than are free")
        # execute: hits first, then the copy-on-write block, then fresh blocks
        for b in hits.values():
            if self.refcount[b] == 0:
                self.evictable.remove(b)
            self.refcount[b] += 1
        cow = []
        if needs_cow:
            src = table[-1]
            dst = self.allocate_block()
            self.refcount[src] -= 1
            table[-1] = dst
            cow.append((src, dst))
        slots = []
        n_cached = 0
        chain = self.chain[seq]
        pend = list(self.pending[seq])
        for i, p in enumerate(range(length, length + n)):
            lb = p // bs
            if p % bs == 0:
                table.append(hits[lb] if lb in hits else self.allocate_block())
            if lb in hits:
                slots.append(-1)
                n_cached += 1
            else:
                slots.append(table[lb] * bs + p % bs)
            if chain >= 0:
                pend.append(tokens[i])
                if len(pend) == bs:
                    chain = self._content(chain, pend, create=True)
                    pend = []
                    b = table[lb]
                    if chain not in self.cached:      # register (a hit is registered already)
                        self.cached[chain] = b
                        self.content_of[b] = chain
        self.lengths[seq] = length + n
        self.chain[seq] = chain
        self.pending[seq] = pend if chain >= 0 else []
        self.hit_tokens += n_cached
        return slots, cow, n_cached


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
        elif kind == "append_tokens":
            results.append(alloc.append_tokens(op[1], op[2]))
        else:
            raise ValueError(f"unknown op {kind!r}")
    return results
