"""Pins of the oracle's allocator (O1) against what the pages print and fix.

Every check here is independent of the oracle's own code: the expected
tables come from the pages' worked examples (tests/golden, cited there), and
the random-op check recomputes every derived quantity (reference counts, the
free set, table lengths, slots) from first principles after each op.
"""

import json
import os
import random

import pytest

from oracle import accounting, cache
from oracle.allocator import BlockAllocator, OutOfBlocks, BadBlock, BadSequence, run_script

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "allocator_examples.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_velog_worked_example(golden):
    g = golden["velog_worked_example"]
    a = BlockAllocator(g["num_blocks"], g["block_size"], g["free_order"])
    s = a.create_seq()
    opened = []
    for tok in range(1, g["appends_one_at_a_time"] + 1):
        before = len(a.tables[s])
        a.append_slots(s, 1)
        if len(a.tables[s]) > before:
            opened.append(tok)
    assert a.tables[s] == g["expected_table"]
    assert opened == g["first_token_of_block"]


def test_ch09_flowchart(golden):
    g = golden["ch09_flowchart"]
    a = BlockAllocator(g["num_blocks"], g["block_size"], g["free_order"])
    s = a.create_seq()
    for _ in range(g["appends_one_at_a_time"]):
        a.append_slots(s, 1)
    assert a.tables[s] == g["expected_table"]


@pytest.mark.parametrize("key", ["studynote528_diagram", "studynote223_diagram"])
def test_interleaved_requests(golden, key):
    g = golden[key]
    a = BlockAllocator(g["num_blocks"], g["block_size"], g["free_order"])
    ids = {}
    for name, n in g["interleaved_appends"]:
        if name not in ids:
            ids[name] = a.create_seq()
        a.append_slots(ids[name], n)
    want = g.get("expected_tables") or g["expected_tables_before_growth"]
    for name, table in want.items():
        assert a.tables[ids[name]] == table
    if "growth" in g:
        name, n = g["growth"]
        a.append_slots(ids[name], n)
        for nm, table in g["expected_table_after_growth"].items():
            assert a.tables[ids[nm]] == table


def test_velog_beam_fork(golden):
    g = golden["velog_beam_fork"]
    a = BlockAllocator(g["num_blocks"], g["block_size"], g["free_order"])
    prompt = a.create_seq()
    a.append_slots(prompt, g["prompt_tokens"])
    paths = {"A": prompt, "B": a.fork(prompt)}
    for name in ("A", "B"):
        slots, cow = a.append_slots(paths[name], 1)
        assert cow == []            # the prompt's blocks are full: no copy needed
    for name, table in g["expected_tables"].items():
        assert a.tables[paths[name]] == table
    for b, rc in g["expected_refcounts"].items():
        assert a.refcount[int(b)] == rc


def test_studynote223_cow(golden):
    g = golden["studynote223_cow"]
    a = BlockAllocator(g["num_blocks"], g["block_size"], g["free_order"])
    first = a.create_seq()
    a.append_slots(first, g["shared_prompt_tokens"])
    users = [first] + [a.fork(first) for _ in range(g["users"] - 1)]
    shared = a.tables[first][0]
    assert a.refcount[shared] == g["expected_shared_refcount_before"]
    writer = users[3]
    slots, cow = a.append_slots(writer, g["writer_appends"])
    assert len(cow) == g["expected_cow_pairs_for_writer"]
    src, dst = cow[0]
    assert src == shared and dst != shared
    assert a.tables[writer] == [dst]
    assert a.refcount[shared] == g["expected_shared_refcount_after"]
    # the writer's new token lands in its own copy, right after the shared prefix
    assert slots == [dst * g["block_size"] + g["shared_prompt_tokens"]]
    # every other user still points at the shared block
    for u in users:
        if u != writer:
            assert a.tables[u] == [shared]


def test_last_holder_writes_in_place():
    a = BlockAllocator(8, 4)
    s0 = a.create_seq()
    a.append_slots(s0, 2)
    s1 = a.fork(s0)
    _, cow0 = a.append_slots(s0, 1)
    assert len(cow0) == 1
    _, cow1 = a.append_slots(s1, 1)       # s1 is now the only holder
    assert cow1 == []


def test_fragmentation_examples(golden):
    g = golden["velog_fragmentation"]
    assert accounting.contiguous_waste(g["reserved"], g["used"]) == g["expected_waste"]
    g = golden["studynote223_block_size"]
    assert accounting.paged_waste(g["used"], g["block_size"]) == g["expected_empty"]


def _capacity_pins(acc):
    """The capacity formula of [studynote 528] section IV (HBM = max-model-len
    x batch x KV bytes per token), pinned two ways that do not use its code."""
    # hand-worked: head_dim 128, 8 kv heads, bf16, one layer -> K row 256 B +
    # V row 256 B per head, 8 heads: 4,096 B per token; the page's
    # --max-model-len 8192 at a batch of 64: 8192 * 64 * 4096 B = 2 GiB
    assert acc.kv_bytes_per_token(1, 8, 128, 2) == 4096
    assert acc.capacity_bytes(8192, 64, acc.kv_bytes_per_token(1, 8, 128, 2)) == 2 << 30
    # 80 layers of that head shape: 320 KiB per token, 160 GiB for the same reservation
    assert acc.kv_bytes_per_token(80, 8, 128, 2) == 320 * 1024
    assert acc.capacity_bytes(8192, 64, acc.kv_bytes_per_token(80, 8, 128, 2)) == 160 << 30
    # against the size of real pools: a K pool and a V pool (numpy arrays of
    # the stored dtype) with exactly max_len * batch token slots per layer
    for dtype, b in (("bf16", 2), ("f32", 4)):
        for H, D, bs, max_len, batch, layers in ((8, 128, 16, 64, 3, 1), (2, 64, 8, 40, 5, 3)):
            nblk = max_len * batch // bs
            pools = [cache.new_pool(nblk, H, bs, D, dtype, 0) for _ in range(2 * layers)]
            assert sum(p.nbytes for p in pools) == \
                acc.capacity_bytes(max_len, batch, acc.kv_bytes_per_token(layers, H, D, b))


def test_capacity_formula_pins():
    _capacity_pins(accounting)


def test_planted_capacity_slips_are_caught(monkeypatch):
    real = accounting.kv_bytes_per_token
    # K+V counted once instead of twice
    monkeypatch.setattr(accounting, "kv_bytes_per_token", lambda L, H, D, b: real(L, H, D, b) // 2)
    with pytest.raises(AssertionError):
        _capacity_pins(accounting)
    monkeypatch.setattr(accounting, "kv_bytes_per_token", real)
    # the batch factor dropped
    monkeypatch.setattr(accounting, "capacity_bytes", lambda m, bt, k: m * k)
    with pytest.raises(AssertionError):
        _capacity_pins(accounting)


def test_stats_worked_example():
    # 10 tokens in 4-token blocks: 3 blocks, 2 empty slots in the last one
    a = BlockAllocator(8, 4)
    s = a.create_seq()
    a.append_slots(s, 10)
    st = a.stats()
    assert (st["used_blocks"], st["free_blocks"], st["logical_tokens"], st["stored_tokens"]) == (3, 5, 10, 10)
    assert 3 * 4 - st["stored_tokens"] == accounting.paged_waste(10, 4) == 2
    # a fork shares all three blocks: twice the logical tokens, the same slots
    c = a.fork(s)
    st = a.stats()
    assert (st["used_blocks"], st["shared_blocks"], st["logical_tokens"], st["stored_tokens"]) == (3, 3, 20, 10)
    # the child's next token copies the partial block: positions 8..10 of the
    # child in the copy, 8..9 of the parent in the original
    a.append_slots(c, 1)
    st = a.stats()
    assert (st["used_blocks"], st["shared_blocks"], st["logical_tokens"], st["stored_tokens"]) == (4, 2, 21, 13)
    assert (st["live_seqs"], st["hit_tokens"], st["evictions"], st["cached_blocks"]) == (2, 0, 0, 0)


def test_errors_leave_state_unchanged():
    a = BlockAllocator(3, 4)
    s = a.create_seq()
    a.append_slots(s, 8)                  # 2 blocks
    snap = (list(a.free), list(a.refcount), list(a.tables[s]), a.lengths[s])
    with pytest.raises(OutOfBlocks):
        a.append_slots(s, 5)              # needs 2 more, 1 free
    assert snap == (list(a.free), list(a.refcount), list(a.tables[s]), a.lengths[s])
    with pytest.raises(BadBlock):
        a.free_block(a.free[0])           # not allocated
    with pytest.raises(BadSequence):
        a.append_slots(99, 1)
    t = a.fork(s)
    a.free_seq(t)
    a.free_seq(s)
    assert sorted(a.free) == [0, 1, 2] and a.refcount == [0, 0, 0]


def _check_invariants(a, live_len):
    """Recompute everything from the tables: counts, free set, lengths, waste."""
    N, bs = a.num_blocks, a.block_size
    count = [0] * N
    for s, table in a.tables.items():
        for b in table:
            count[b] += 1
        L = a.lengths[s]
        assert L == live_len[s]
        assert len(table) == -(-L // bs)                    # ceil(L / bs) blocks
        assert len(table) * bs - L < bs or L == 0           # waste only in the last block
    assert count == a.refcount
    free = list(a.free)
    assert len(set(free)) == len(free)
    assert set(free) == {b for b in range(N) if count[b] == 0}
    assert len(free) + sum(1 for c in count if c > 0) == N
    # occupancy statistics, from the counts and the per-block reach of each holder
    st = a.stats()
    used = sum(1 for c in count if c > 0)
    assert (st["free_blocks"], st["used_blocks"], st["shared_blocks"], st["live_seqs"]) == \
        (len(free), used, sum(1 for c in count if c > 1), len(a.tables))
    assert st["logical_tokens"] == sum(live_len.values())
    reach = {}
    for s, table in a.tables.items():
        for i, b in enumerate(table):
            reach[b] = max(reach.get(b, 0), min(bs, a.lengths[s] - i * bs))
    assert st["stored_tokens"] == sum(reach.values())
    assert st["stored_tokens"] <= min(st["logical_tokens"], used * bs)
    if st["shared_blocks"] == 0:
        assert st["stored_tokens"] == st["logical_tokens"]
        assert used * bs - st["stored_tokens"] == sum(
            accounting.paged_waste(L, bs) for L in a.lengths.values())


@pytest.mark.parametrize("seed", range(12))
def test_random_ops_against_recomputed_state(seed):
    rnd = random.Random(seed)
    N, bs = rnd.choice([(6, 2), (9, 4), (16, 3), (12, 16)])
    a = BlockAllocator(N, bs, rnd.sample(range(N), N))
    live_len = {}
    for _ in range(1500):
        r = rnd.random()
        seqs = list(a.tables)
        if r < 0.15 or not seqs:
            s = a.create_seq()
            live_len[s] = 0
        elif r < 0.25:
            p = rnd.choice(seqs)
            c = a.fork(p)
            live_len[c] = live_len[p]
        elif r < 0.35:
            s = rnd.choice(seqs)
            a.free_seq(s)
            del live_len[s]
        elif r < 0.42:
            s = rnd.choice(seqs)
            if a.tables[s]:
                idx = rnd.randrange(len(a.tables[s]))
                before = a.tables[s][idx]
                pair = a.cow_block(s, idx) if a.num_free() else None
                if pair is not None:
                    assert pair[0] == before and a.tables[s][idx] == pair[1]
        else:
            s = rnd.choice(seqs)
            n = rnd.randint(1, 2 * bs)
            L = live_len[s]
            try:
                table_before = list(a.tables[s])
                slots, cow = a.append_slots(s, n)
            except OutOfBlocks:
                _check_invariants(a, live_len)
                continue
            assert len(cow) <= 1
            if cow:
                assert L % bs != 0 and cow[0][0] == table_before[-1]
            for i, slot in enumerate(slots):
                pos = L + i
                assert slot // bs == a.tables[s][pos // bs]
                assert slot % bs == pos % bs
            live_len[s] = L + n
            # freshly written slots belong to s alone
            for slot in slots:
                assert a.refcount[slot // bs] == 1
        _check_invariants(a, live_len)


def test_run_script_and_tables():
    a = BlockAllocator(10, 4, list(range(9, -1, -1)))
    res = run_script(a, [("create",), ("append", 0, 6), ("fork", 0), ("append", 1, 1),
                         ("create",), ("append", 2, 4)])
    assert res[0] == 0 and res[2] == 1 and res[4] == 2
    assert res[1] == ([36, 37, 38, 39, 32, 33], [])
    assert res[3] == ([30], [(8, 7)])      # block 8 was half full and shared
    tables, lens = a.block_tables([0, 1, 2], 3)
    assert tables == [[9, 8, -1], [9, 7, -1], [6, -1, -1]]
    assert lens == [6, 7, 4]
