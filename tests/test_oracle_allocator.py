"""Pins of the oracle's block manager.

* the block-mapping figure and the on-demand rule printed on the pages
  (golden fixture),
* prefix sharing arithmetic (stored once; page '生成一个字…', section
  'PagedAttention：把操作系统的老智慧搬进推理引擎'),
* a semantic model that knows nothing about blocks: every sequence is a plain
  Python list of token ids, fork copies the list.  Reading each sequence back
  through its table from a slot-addressed memory (with copy-on-write copies
  applied) must give exactly that list,
* accounting invariants after every operation on random op sequences, and
  the strong guarantee on pool exhaustion.
"""
import json
import os
import random

import numpy as np
import pytest

from oracle import BlockManager, OutOfBlocks, AllocatorError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_mapping_figure.json")
with open(GOLDEN, encoding="utf-8") as f:
    FIG = json.load(f)


def test_figure_mapping():
    bs = FIG["block_size"]
    phys = FIG["physical_blocks"]
    order = phys + [b for b in range(128) if b not in phys]
    bm = BlockManager(128, bs, free_order=order)
    s = bm.alloc()
    slots = []
    counts = {}
    for t in range(1, 49):
        sl, cw = bm.append(s, 1)
        assert cw == []
        slots.append(sl[0])
        counts[t] = len(bm.table(s))
    assert bm.table(s) == phys
    for tok, slot in FIG["token_to_slot"]:
        assert slots[tok - 1] == slot
    for tok, nblk in FIG["blocks_after_tokens"]:
        assert counts[tok] == nblk


def test_block_counts_of_tiny_workload():
    # lengths {5, 16, 17, 40} with 16-token blocks need 1, 1, 2, 3 blocks
    bm = BlockManager(64, 16)
    used = []
    for L in (5, 16, 17, 40):
        s = bm.alloc()
        bm.append(s, L)
        used.append(len(bm.table(s)))
    assert used == [1, 1, 2, 3]
    assert bm.num_free() == 64 - 7


def test_shared_prefix_stored_once():
    # 256 forks of a 2000-token prompt: 125 shared blocks plus each child's
    # private suffix blocks, not 256 * 125.
    bs = 16
    rng = np.random.default_rng(0)
    suffix = rng.integers(1, 513, size=256)
    nb = 125 + int(sum(-(-int(s) // bs) for s in suffix)) + 8
    bm = BlockManager(nb, bs)
    root = bm.alloc()
    bm.append(root, 2000)
    kids = [bm.fork(root) for _ in range(256)]
    bm.free(root)
    for blk in range(nb):
        pass
    prefix_blocks = bm.table(kids[0])
    assert all(bm.refcount(b) == 256 for b in prefix_blocks)
    for k, s in zip(kids, suffix):
        _, cows = bm.append(k, int(s))
        assert cows == []          # 2000 = 125 * 16: the last prefix block is full
    used = nb - bm.num_free()
    assert used == 125 + int(sum(-(-int(s) // bs) for s in suffix))


def test_cow_on_shared_partial_block():
    bm = BlockManager(8, 4, free_order=[5, 2, 7, 0, 1, 3, 4, 6])
    a = bm.alloc()
    assert bm.append(a, 6) == ([20, 21, 22, 23, 8, 9], [])
    b = bm.fork(a)
    assert bm.refcount(5) == 2 and bm.refcount(2) == 2
    # child writes into the shared partial block 2 -> copy to the next free (7)
    slots, cows = bm.append(b, 1)
    assert cows == [(2, 7)] and slots == [7 * 4 + 2]
    assert bm.table(b) == [5, 7] and bm.table(a) == [5, 2]
    assert bm.refcount(2) == 1 and bm.refcount(7) == 1
    # parent now owns block 2 alone and writes in place
    assert bm.append(a, 1) == ([2 * 4 + 2], [])
    # a full shared block is never copied: fill both to 8 then append
    bm.append(a, 1)
    bm.append(b, 1)
    c = bm.fork(a)
    slots, cows = bm.append(c, 1)
    assert cows == [] and bm.table(c)[:2] == bm.table(a)
    bm.free(a)
    bm.free(b)
    bm.free(c)
    assert bm.num_free() == 8
    assert all(bm.refcount(x) == 0 for x in range(8))


def test_fifo_order_and_release_order():
    bm = BlockManager(6, 2, free_order=[3, 1, 4, 0, 5, 2])
    a = bm.alloc()
    bm.append(a, 5)                  # takes 3, 1, 4
    assert bm.free_list() == [0, 5, 2]
    bm.free(a)                        # releases in table order
    assert bm.free_list() == [0, 5, 2, 3, 1, 4]


def test_oom_is_atomic():
    bm = BlockManager(4, 4)
    a = bm.alloc()
    bm.append(a, 10)                 # 3 blocks
    before = (bm.free_list(), bm.table(a), bm.length(a))
    with pytest.raises(OutOfBlocks):
        bm.append(a, 7)              # needs 2 more blocks, only 1 free
    assert (bm.free_list(), bm.table(a), bm.length(a)) == before
    b = bm.fork(a)
    c = bm.fork(a)
    # batch: a and b CoW (need 2 blocks), only 1 free -> nothing happens
    snap = (bm.free_list(), bm.table(a), bm.table(b), bm.table(c),
            [bm.refcount(i) for i in range(4)])
    with pytest.raises(OutOfBlocks):
        bm.append_batch([a, b, c])
    assert snap == (bm.free_list(), bm.table(a), bm.table(b), bm.table(c),
                    [bm.refcount(i) for i in range(4)])


def test_batch_cow_order_releases_last_holder():
    # two holders of one partial block: the first CoWs, the second writes in place
    bm = BlockManager(4, 4)
    a = bm.alloc()
    bm.append(a, 2)
    b = bm.fork(a)
    slots, cows = bm.append_batch([a, b])
    assert cows == [(0, 1)]
    assert bm.table(a) == [1] and bm.table(b) == [0]
    assert slots == [1 * 4 + 2, 0 * 4 + 2]


def test_errors():
    bm = BlockManager(4, 4)
    with pytest.raises(AllocatorError):
        bm.append(0, 1)
    s = bm.alloc()
    with pytest.raises(AllocatorError):
        bm.append(s, -1)
    bm.free(s)
    with pytest.raises(AllocatorError):
        bm.free(s)
    with pytest.raises(AllocatorError):
        bm.fork(s)
    with pytest.raises(AllocatorError):
        BlockManager(4, 4, free_order=[0, 1, 1, 2])
    t = bm.alloc()
    with pytest.raises(AllocatorError):
        bm.append_batch([t, t])


def _check_invariants(bm):
    nb = bm.num_blocks
    refs = [bm.refcount(b) for b in range(nb)]
    seqs = bm.sequences()
    # sum of reference counts = total (non-released) table entries
    assert sum(refs) == sum(sum(1 for b in bm.table(s) if b >= 0) for s in seqs)
    # free and referenced blocks partition the pool
    free = bm.free_list()
    assert len(set(free)) == len(free)
    assert set(free) == {b for b in range(nb) if refs[b] == 0}
    for s in seqs:
        assert len(bm.table(s)) == -(-bm.length(s) // bm.block_size)


def _random_ops(seed, nb, bs, steps):
    rng = random.Random(seed)
    order = list(range(nb))
    rng.shuffle(order)
    bm = BlockManager(nb, bs, free_order=order)
    memory = {}              # slot -> token id
    logical = {}             # seq -> list of token ids (the block-free model)
    gone = {}                # seq -> tokens before this index were released
    next_tok = 0
    for _ in range(steps):
        live = bm.sequences()
        op = rng.random()
        if op < 0.1 or not live:
            s = bm.alloc()
            logical[s] = []
            gone[s] = 0
        elif op < 0.22:
            p = rng.choice(live)
            c = bm.fork(p)
            logical[c] = list(logical[p])
            gone[c] = gone[p]
        elif op < 0.3:
            s = rng.choice(live)
            bm.free(s)
            del logical[s]
        elif op < 0.35:
            # window release: whole blocks before a token go back to the pool
            s = rng.choice(live)
            tok = rng.randint(0, bm.length(s))
            before = sum(1 for b in bm.table(s) if b >= 0)
            n = bm.release_before(s, tok)
            new_gone = max(gone[s], (tok // bs) * bs)
            assert n == before - sum(1 for b in bm.table(s) if b >= 0)
            assert n == (new_gone - gone[s]) // bs
            gone[s] = new_gone
        elif op < 0.5:
            batch = rng.sample(live, rng.randint(1, len(live)))
            try:
                slots, cows = bm.append_batch(batch)
            except OutOfBlocks:
                _check_invariants(bm)
                continue
            for src, dst in cows:
                for off in range(bs):
                    if src * bs + off in memory:
                        memory[dst * bs + off] = memory[src * bs + off]
            for s, slot in zip(batch, slots):
                memory[slot] = next_tok
                logical[s].append(next_tok)
                next_tok += 1
        else:
            s = rng.choice(live)
            n = rng.randint(0, 3 * bs)
            free_before = bm.free_list()
            try:
                slots, cows = bm.append(s, n)
            except OutOfBlocks:
                assert bm.free_list() == free_before
                _check_invariants(bm)
                continue
            assert len(cows) <= 1
            for src, dst in cows:
                for off in range(bs):
                    if src * bs + off in memory:
                        memory[dst * bs + off] = memory[src * bs + off]
            for slot in slots:
                # a written slot is never shared with another live sequence
                assert bm.refcount(slot // bs) == 1
                memory[slot] = next_tok
                logical[s].append(next_tok)
                next_tok += 1
        _check_invariants(bm)
        # read every sequence back through its table
        for s in bm.sequences():
            tab = bm.table(s)
            assert all(b < 0 for b in tab[:gone[s] // bs]) and all(b >= 0 for b in tab[gone[s] // bs:])
            got = [memory[tab[t // bs] * bs + t % bs] for t in range(gone[s], bm.length(s))]
            assert got == logical[s][gone[s]:], (seed, s)


@pytest.mark.parametrize("seed", range(40))
def test_random_ops_tiny_pools(seed):
    _random_ops(seed, nb=1 + seed % 8, bs=1 + seed % 4, steps=150)


@pytest.mark.parametrize("seed", range(4))
def test_random_ops_larger_pool(seed):
    _random_ops(100 + seed, nb=64, bs=16, steps=400)


def test_export_pads_with_minus_one():
    bm = BlockManager(8, 4, free_order=[7, 6, 5, 4, 3, 2, 1, 0])
    a, b = bm.alloc(), bm.alloc()
    bm.append(a, 5)
    bm.append(b, 1)
    tables, lens = bm.export([b, a], 3)
    assert tables.tolist() == [[5, -1, -1], [7, 6, -1]]
    assert lens.tolist() == [1, 5]
    with pytest.raises(AllocatorError):
        bm.export([a], 1)


def test_window_release_bounds_held_blocks():
    # page "生成一个字…", section "再往后：压 KV 的三条路线": with a sliding window
    # the cache a sequence holds is bounded by the window, not the context.
    # Decoding 1000 tokens with a 64-token window and releasing after every
    # step never holds more than ceil(64/16) + 1 blocks.
    bs, W = 16, 64
    bm = BlockManager(8, bs)
    s = bm.alloc()
    for n in range(1, 1001):
        bm.append(s, 1)
        bm.release_before(s, max(0, n + 1 - W))
        held = sum(1 for b in bm.table(s) if b >= 0)
        assert held <= -(-W // bs) + 1
        assert len(bm.table(s)) == -(-n // bs)
    # released entries keep their logical position: the next token's slot is
    # still table[n // bs] * bs + n % bs
    slots, _ = bm.append(s, 1)
    assert slots[0] == bm.table(s)[1000 // bs] * bs + 1000 % bs
    with pytest.raises(AllocatorError):
        bm.release_before(s, 1002)


def test_common_prefix_of_fork_families():
    # pages: a shared prefix is stored once and reference counted; forked
    # sequences hold the parent's blocks until they write into them.  The
    # common prefix is the run of leading blocks that are the same physical
    # blocks in every sequence and full in all of them.
    bs = 16
    bm = BlockManager(64, bs)
    root = bm.alloc()
    bm.append(root, 100)                       # 6 full blocks + 4 tokens in block 6
    kids = [bm.fork(root) for _ in range(5)]
    assert bm.common_prefix(kids) == 100 // bs == 6       # block 6 is shared but not full
    assert bm.common_prefix([root] + kids) == 6
    for k, n in zip(kids, (1, 2, 3, 1, 40)):
        _, cows = bm.append(k, n)
        assert len(cows) == 1                  # each copies the shared partial block 6
    assert bm.common_prefix(kids) == 6
    assert bm.common_prefix([kids[4]]) == (100 + 40) // bs  # one sequence: its full blocks
    # exact multiple: children take fresh blocks, the 6 full ones stay shared
    r2 = bm.alloc()
    bm.append(r2, 96)
    a, b = bm.fork(r2), bm.fork(r2)
    bm.append(a, 17)
    bm.append(b, 1)
    assert bm.common_prefix([a, b]) == 6
    # nested forks share more with each other than with the root
    c1, c2 = bm.fork(a), bm.fork(a)
    bm.append(c1, 5)
    bm.append(c2, 5)
    assert bm.common_prefix([c1, c2]) == (96 + 17) // bs == 7
    assert bm.common_prefix([r2, c1]) == 6
    # unrelated sequences share nothing; an empty batch has no prefix
    assert bm.common_prefix([root, r2]) == 0
    assert bm.common_prefix([]) == 0


def test_common_prefix_stops_at_released_blocks():
    bm = BlockManager(32, 16)
    root = bm.alloc()
    bm.append(root, 80)
    kids = [bm.fork(root) for _ in range(3)]
    assert bm.common_prefix(kids) == 5
    bm.release_before(kids[0], 40)             # kids[0] drops blocks 0 and 1 (entries -1)
    assert bm.common_prefix(kids) == 0
    assert bm.common_prefix(kids[1:]) == 5
    assert bm.common_prefix([kids[0]]) == 0
