"""Pins of the oracle's prefix-caching allocator, against things other than itself.

  * worked cases of the rules (shared prompt -> shared blocks and skipped
    writes; a freed prompt stays reusable; oldest cached block evicted first;
    a partial block is never reused; the first differing token stops reuse);
  * a content model: every slot written is given the whole token prefix it
    holds the K/V of (copy-on-write copies it too), and after every operation
    of random scripts each live sequence's block table must read back exactly
    its own history -- reuse may only ever map identical content;
  * bookkeeping invariants recomputed from scratch after every operation;
  * planted mistakes (a block identity that forgets its parent, an eviction
    that keeps the old registration, a cached block sent to the free list)
    that the content model must catch.
"""

import random

import pytest

from oracle.allocator import BlockAllocator, OutOfBlocks, PrefixCachingAllocator


def tokens(*ranges):
    out = []
    for a, b in ranges:
        out += list(range(a, b))
    return out


def test_shared_prompt_reuses_full_blocks_and_skips_their_writes():
    a = PrefixCachingAllocator(8, 4)
    s1 = a.create_seq()
    slots1, cow, n1 = a.append_tokens(s1, tokens((1, 11)))          # 10 tokens: 2 full + 2
    assert n1 == 0 and cow == [] and -1 not in slots1
    s2 = a.create_seq()
    slots2, cow, n2 = a.append_tokens(s2, tokens((1, 11)))
    assert n2 == 8 and slots2[:8] == [-1] * 8 and -1 not in slots2[8:]
    assert a.tables[s2][:2] == a.tables[s1][:2]
    assert a.tables[s2][2] != a.tables[s1][2]                        # partial block: private
    assert [a.refcount[b] for b in a.tables[s1]] == [2, 2, 1]


def test_freed_prompt_stays_cached_and_is_found_again():
    a = PrefixCachingAllocator(8, 4)
    s1 = a.create_seq()
    a.append_tokens(s1, tokens((1, 11)))
    full = a.tables[s1][:2]
    partial = a.tables[s1][2]
    a.free_seq(s1)
    assert a.evictable == full and partial in a.free
    assert a.num_cached() == 2 and a.num_free() == 6
    s2 = a.create_seq()
    _, _, n = a.append_tokens(s2, tokens((1, 9)))
    assert n == 8 and a.tables[s2] == full and a.num_cached() == 0
    st = a.stats()
    assert (st["hit_tokens"], st["evictions"], st["stored_tokens"], st["used_blocks"]) == (8, 0, 8, 2)


def test_oldest_cached_block_is_evicted_first():
    a = PrefixCachingAllocator(4, 2, free_order=[3, 2, 1, 0])
    s1 = a.create_seq()
    a.append_tokens(s1, [1, 2, 3, 4])              # blocks 3, 2 (content A, AB)
    s2 = a.create_seq()
    a.append_tokens(s2, [9, 9, 8, 8])              # blocks 1, 0
    a.free_seq(s1)                                 # 3 then 2 become evictable
    a.free_seq(s2)                                 # then 1, 0
    assert a.evictable == [3, 2, 1, 0] and a.num_free() == 0
    s3 = a.create_seq()
    slots, _, n = a.append_tokens(s3, [5, 5, 9, 9])   # two fresh blocks: evicts 3 and 2
    assert n == 0 and a.tables[s3] == [3, 2]
    s4 = a.create_seq()
    _, _, n = a.append_tokens(s4, [1, 2, 3, 4])       # A was evicted: miss (evicts 1, 0)
    assert n == 0
    s5 = a.create_seq()
    with pytest.raises(OutOfBlocks):
        a.append_tokens(s5, [9, 9, 8, 8])
    assert a.num_cached() == 0
    st = a.stats()
    assert (st["evictions"], st["hit_tokens"], st["used_blocks"], st["cached_blocks"]) == (4, 0, 4, 0)


def test_partial_block_is_never_reused_and_first_difference_stops_reuse():
    a = PrefixCachingAllocator(16, 4)
    s1 = a.create_seq()
    a.append_tokens(s1, tokens((0, 14)))
    s2 = a.create_seq()
    t = tokens((0, 14))
    t[9] = 99                                      # differs inside block 2
    slots, _, n = a.append_tokens(s2, t)
    assert n == 8                                  # blocks 0 and 1 only
    assert a.tables[s2][:2] == a.tables[s1][:2] and a.tables[s2][2] != a.tables[s1][2]
    s3 = a.create_seq()
    _, _, n = a.append_tokens(s3, tokens((0, 3)))     # shorter than a block: no reuse
    assert n == 0


def test_appending_without_token_ids_makes_content_unknown():
    a = PrefixCachingAllocator(16, 4)
    s1 = a.create_seq()
    a.append_slots(s1, 4)                          # content unknown from here on
    a.append_tokens(s1, [1, 2, 3, 4])
    s2 = a.create_seq()
    a.append_tokens(s2, [1, 2, 3, 4])
    assert a.tables[s2][0] != a.tables[s1][1]      # block 1 of s1 was never registered
    s3 = a.create_seq()
    _, _, n = a.append_tokens(s3, [1, 2, 3, 4])
    assert n == 4 and a.tables[s3][0] == a.tables[s2][0]


def test_block_by_block_decode_fills_register_too():
    a = PrefixCachingAllocator(16, 4)
    s1 = a.create_seq()
    for t in range(8):
        a.append_tokens(s1, [t])                   # one token at a time, as in decode
    s2 = a.create_seq()
    _, _, n = a.append_tokens(s2, list(range(8)))
    assert n == 8 and a.tables[s2] == a.tables[s1]


# ---- random scripts against a content model -----------------------------------------------
class ContentModel:
    """What each physical block holds.  A token's K/V depends on every token
    before it, so a slot's content is modelled as the whole prefix ending at
    that token."""

    def __init__(self, alloc):
        self.a = alloc
        self.slot_tok = {}
        self.history = {}

    def after_append(self, seq, toks, slots, cow):
        bs = self.a.block_size
        for src, dst in cow:
            for o in range(bs):
                if (src, o) in self.slot_tok:
                    self.slot_tok[(dst, o)] = self.slot_tok[(src, o)]
                else:
                    self.slot_tok.pop((dst, o), None)
        hist = self.history.get(seq, []) + list(toks)
        base = len(hist) - len(toks)
        for i, sl in enumerate(slots):
            if sl >= 0:
                self.slot_tok[(sl // bs, sl % bs)] = tuple(hist[:base + i + 1])
        self.history[seq] = hist

    def check(self):
        a = self.a
        bs = a.block_size
        for s, hist in self.history.items():
            if s not in a.tables:
                continue
            assert a.lengths[s] == len(hist)
            for p in range(len(hist)):
                b = a.tables[s][p // bs]
                assert self.slot_tok.get((b, p % bs)) == tuple(hist[:p + 1]), (s, p)
        # bookkeeping: every block is exactly one of free / evictable / referenced
        used = {}
        for s, tab in a.tables.items():
            for b in tab:
                used[b] = used.get(b, 0) + 1
        for b in range(a.num_blocks):
            assert a.refcount[b] == used.get(b, 0)
            states = (b in a.free) + (b in a.evictable) + (a.refcount[b] > 0)
            assert states == 1, b
            assert (a.content_of[b] != 0) == (b in a.cached.values())
        for cid, b in a.cached.items():
            assert a.content_of[b] == cid
        for b in a.evictable:
            assert a.content_of[b] != 0


@pytest.mark.parametrize("seed", range(12))
def test_random_scripts_read_back_their_own_tokens(seed):
    rng = random.Random(seed)
    bs = rng.choice([2, 3, 4])
    n = rng.randint(6, 24)
    a = PrefixCachingAllocator(n, bs, free_order=rng.sample(range(n), n))
    m = ContentModel(a)
    prompts = [[rng.randint(0, 3) for _ in range(rng.randint(1, 12))] for _ in range(4)]
    live = []
    hits = 0
    for _ in range(400):
        op = rng.random()
        try:
            if op < 0.25 or not live:
                s = a.create_seq()
                toks = list(rng.choice(prompts))
                slots, cow, n = a.append_tokens(s, toks)
                hits += n
                m.after_append(s, toks, slots, cow)
                live.append(s)
            elif op < 0.55:
                s = rng.choice(live)
                toks = [rng.randint(0, 3) for _ in range(rng.randint(1, 5))]
                slots, cow, n = a.append_tokens(s, toks)
                hits += n
                m.after_append(s, toks, slots, cow)
            elif op < 0.65:
                s = rng.choice(live)
                c = a.fork(s)
                m.history[c] = list(m.history[s])
                live.append(c)
            elif op < 0.72:
                s = rng.choice(live)
                k = rng.randint(1, 3)
                slots, cow = a.append_slots(s, k)
                toks = [1000 + rng.randint(0, 9) for _ in range(k)]   # unknown content
                m.after_append(s, toks, slots, cow)
            else:
                s = rng.choice(live)
                a.free_seq(s)
                live.remove(s)
                del m.history[s]
        except OutOfBlocks:
            pass
        m.check()
    assert hits > 0


# ---- planted mistakes: the content model must catch each -----------------------------------
class _KeyIgnoresParent(PrefixCachingAllocator):
    """Bug: a block's identity forgets what came before it."""

    def _content(self, parent, tokens, create):
        return super()._content(0, tokens, create)


class _EvictionKeepsMapping(PrefixCachingAllocator):
    """Bug: an evicted block stays registered under its old content."""

    def allocate_block(self):
        if self.free:
            return BlockAllocator.allocate_block(self)
        if not self.evictable:
            raise OutOfBlocks("no free block")
        b = self.evictable.pop(0)
        self.refcount[b] = 1
        return b


class _FreedGoesToFreeList(PrefixCachingAllocator):
    """Bug: a cached block whose count drops to zero is freed but stays registered."""

    def free_block(self, block):
        self.refcount[block] -= 1
        if self.refcount[block] == 0:
            self.free.append(block)


def _runs_clean(cls, seed):
    rng = random.Random(seed)
    bs = rng.choice([2, 3, 4])
    n = rng.randint(6, 24)
    a = cls(n, bs, free_order=rng.sample(range(n), n))
    m = ContentModel(a)
    prompts = [[rng.randint(0, 3) for _ in range(rng.randint(1, 12))] for _ in range(4)]
    live = []
    try:
        for _ in range(400):
            op = rng.random()
            try:
                if op < 0.3 or not live:
                    s = a.create_seq()
                    toks = list(rng.choice(prompts))
                    slots, cow, _ = a.append_tokens(s, toks)
                    m.after_append(s, toks, slots, cow)
                    live.append(s)
                elif op < 0.65:
                    s = rng.choice(live)
                    toks = [rng.randint(0, 3) for _ in range(rng.randint(1, 5))]
                    slots, cow, _ = a.append_tokens(s, toks)
                    m.after_append(s, toks, slots, cow)
                else:
                    s = rng.choice(live)
                    a.free_seq(s)
                    live.remove(s)
                    del m.history[s]
            except OutOfBlocks:
                pass
            m.check()
    except (AssertionError, KeyError, ValueError):
        return False
    return True


@pytest.mark.parametrize("mutant", [_KeyIgnoresParent, _EvictionKeepsMapping, _FreedGoesToFreeList])
def test_planted_mistakes_are_caught(mutant):
    assert all(_runs_clean(PrefixCachingAllocator, seed) for seed in range(6))
    assert not all(_runs_clean(mutant, seed) for seed in range(6)), mutant.__doc__
