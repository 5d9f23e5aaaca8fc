"""Block manager model (oracle; test infrastructure only).

What it models, from the pages:

* Page "生成一个字，为什么要背一整本账", section
  "PagedAttention：把操作系统的老智慧搬进推理引擎": each sequence's KV cache is
  cut into fixed-size blocks (16 tokens by default) that need not be adjacent
  in memory; a block table maps them; memory is taken on demand, so only the
  last block of a sequence can be partly empty.  Shared prefixes are stored
  once, counted by reference, and copied on write where branches diverge.
* Page "AI 陪读顶会论文（三）", section "PagedAttention 的破局哲学": the
  figure maps tokens 1-16 to logical block 0, 17-32 to block 1, 33-48 to
  block 2, each to an arbitrary physical block; innovation 2 takes the second
  block only when the 17th token arrives; innovation 3 shares prompt blocks
  between branches and copies on write at the fork.

Readings where the pages are silent (the C++ library follows the same ones):

* Tokens are 0-based: token n lives in logical block n // bs at offset
  n % bs, i.e. at slot ``table[n // bs] * bs + n % bs``.
* A block is taken exactly when a token with n % bs == 0 is appended.
* Free blocks form a FIFO queue initialised from ``free_order`` (ascending if
  absent): allocation pops the front, a block whose count drops to zero is
  pushed on the back.  Freed sequences release their blocks in table order.
* Copy-on-write is lazy: at the first append into a partly filled last block
  whose reference count exceeds one, a fresh block is popped, the pair
  (old, new) is reported for a whole-block copy, the old count drops by one
  and the table points at the new block.  A full shared block is never
  written again, so it is never copied.
* An append that cannot get every block it needs fails with no change to any
  state (strong guarantee); a batch append is all-or-nothing.
* Sequence ids count up from 0 and are never reused.
* Window release (page "生成一个字…", section "再往后：压 KV 的三条路线"): blocks
  wholly before a given token can be handed back; their table entries become
  -1 and keep their logical position.
"""
from collections import deque
import copy

import numpy as np


class AllocatorError(Exception):
    """Invalid call (unknown sequence, bad argument)."""


class OutOfBlocks(AllocatorError):
    """Not enough free blocks; nothing was changed."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocatorError("num_blocks and block_size must be positive")
        if free_order is None:
            order = list(range(num_blocks))
        else:
            order = [int(x) for x in free_order]
            if sorted(order) != list(range(num_blocks)):
                raise AllocatorError("free_order must be a permutation of 0..NB-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self._free = deque(order)
        self._ref = [0] * num_blocks
        self._tables = {}
        self._lens = {}
        self._next_id = 0

    # ---- queries -------------------------------------------------------
    def num_free(self) -> int:
        return len(self._free)

    def free_list(self):
        return list(self._free)

    def refcount(self, block: int) -> int:
        if not 0 <= block < self.num_blocks:
            raise AllocatorError("block id out of range")
        return self._ref[block]

    def table(self, seq: int):
        self._check(seq)
        return list(self._tables[seq])

    def length(self, seq: int) -> int:
        self._check(seq)
        return self._lens[seq]

    def sequences(self):
        return sorted(self._tables)

    def _check(self, seq):
        if seq not in self._tables:
            raise AllocatorError(f"unknown sequence {seq}")

    # ---- mutations -----------------------------------------------------
    def alloc(self) -> int:
        sid = self._next_id
        self._next_id += 1
        self._tables[sid] = []
        self._lens[sid] = 0
        return sid

    def _append_one_seq(self, seq, n_tokens):
        """Mutates state; raises OutOfBlocks possibly half-way (callers roll back)."""
        bs = self.block_size
        tab = self._tables[seq]
        start = self._lens[seq]
        slots, cows = [], []
        for pos in range(start, start + n_tokens):
            if pos % bs == 0:
                if not self._free:
                    raise OutOfBlocks("pool exhausted")
                blk = self._free.popleft()
                self._ref[blk] = 1
                tab.append(blk)
            elif pos == start and self._ref[tab[pos // bs]] > 1:
                if not self._free:
                    raise OutOfBlocks("pool exhausted")
                old = tab[pos // bs]
                new = self._free.popleft()
                self._ref[old] -= 1
                self._ref[new] = 1
                tab[pos // bs] = new
                cows.append((old, new))
            slots.append(tab[pos // bs] * bs + pos % bs)
        self._lens[seq] = start + n_tokens
        return slots, cows

    def _snapshot(self):
        return (deque(self._free), list(self._ref), copy.deepcopy(self._tables),
                dict(self._lens))

    def _restore(self, snap):
        self._free, self._ref, self._tables, self._lens = snap

    def append(self, seq: int, n_tokens: int):
        """Reserve slots for ``n_tokens`` new tokens of ``seq``.

        Returns (slots, cow_pairs): slot ids in token order and the list of
        (src, dst) whole-block copies the caller must perform before writing.
        """
        self._check(seq)
        if n_tokens < 0:
            raise AllocatorError("n_tokens must be >= 0")
        snap = self._snapshot()
        try:
            return self._append_one_seq(seq, n_tokens)
        except OutOfBlocks:
            self._restore(snap)
            raise

    def append_batch(self, seqs):
        """One new token for each sequence in ``seqs`` (distinct ids), in order,
        all-or-nothing.  Returns (slots, cow_pairs)."""
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise AllocatorError("duplicate sequence in batch")
        for s in seqs:
            self._check(s)
        snap = self._snapshot()
        slots, cows = [], []
        try:
            for s in seqs:
                sl, cw = self._append_one_seq(s, 1)
                slots += sl
                cows += cw
        except OutOfBlocks:
            self._restore(snap)
            raise
        return slots, cows

    def fork(self, parent: int) -> int:
        self._check(parent)
        child = self.alloc()
        self._tables[child] = list(self._tables[parent])
        self._lens[child] = self._lens[parent]
        for blk in self._tables[child]:
            if blk >= 0:
                self._ref[blk] += 1
        return child

    def free(self, seq: int):
        self._check(seq)
        for blk in self._tables[seq]:
            if blk < 0:
                continue
            self._ref[blk] -= 1
            if self._ref[blk] == 0:
                self._free.append(blk)
        del self._tables[seq]
        del self._lens[seq]

    def release_before(self, seq: int, token: int) -> int:
        """Give back every block of ``seq`` whose tokens all lie before
        ``token`` (page "生成一个字…", section "再往后：压 KV 的三条路线": with a
        sliding window only the last stretch of tokens is attended, so the
        cache a sequence holds is bounded by the window).  A released block's
        table entry becomes -1; logical positions, and so the slots of later
        tokens, do not move.  Released blocks go to the back of the free queue
        in table order once no other sequence holds them.  ``token`` may not
        exceed the sequence length.  Returns the number of entries released
        by this call."""
        self._check(seq)
        if not 0 <= token <= self._lens[seq]:
            raise AllocatorError("token must lie in [0, length]")
        tab = self._tables[seq]
        n = 0
        for i in range(token // self.block_size):
            blk = tab[i]
            if blk < 0:
                continue
            self._ref[blk] -= 1
            if self._ref[blk] == 0:
                self._free.append(blk)
            tab[i] = -1
            n += 1
        return n

    # ---- references held outside tables (prefix cache) -------------------
    def adopt(self, blocks, n_tokens: int) -> int:
        """A new sequence whose table is `blocks` (each gains a holder) and
        whose length is n_tokens, as a fork of a sequence holding exactly
        those blocks would be."""
        sid = self._next_id
        self._next_id += 1
        self._tables[sid] = [int(b) for b in blocks]
        self._lens[sid] = int(n_tokens)
        for b in self._tables[sid]:
            self._ref[b] += 1
        return sid

    def ref_block(self, blk: int):
        self._ref[blk] += 1

    def unref_block(self, blk: int):
        """One holder fewer; a block nobody holds goes to the back of the free queue."""
        self._ref[blk] -= 1
        if self._ref[blk] == 0:
            self._free.append(blk)

    # ---- shared prefix ----------------------------------------------------
    def common_prefix(self, seqs) -> int:
        """Number of leading logical blocks that every sequence in seqs holds
        as the very same physical blocks as the first one, counting only
        blocks that are full in all of them.  Forked sequences keep their
        parent's blocks until they write into them (page "生成一个字…", section
        "PagedAttention：…": a shared prefix is stored once and reference
        counted), so this is the part of the family's cache that is stored
        once."""
        seqs = [int(s) for s in seqs]
        for s in seqs:
            self._check(s)
        if not seqs:
            return 0
        first = self._tables[seqs[0]]
        k = 0
        while k < len(first) and first[k] >= 0:
            same = all(len(self._tables[s]) > k and self._tables[s][k] == first[k] for s in seqs)
            full = all((k + 1) * self.block_size <= self._lens[s] for s in seqs)
            if not (same and full):
                break
            k += 1
        return k

    # ---- dense export ----------------------------------------------------
    def export(self, seqs, max_blocks: int):
        """Dense int32 tables [n][max_blocks] padded with -1 and int32 lengths."""
        seqs = [int(s) for s in seqs]
        tables = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            self._check(s)
            tab = self._tables[s]
            if len(tab) > max_blocks:
                raise AllocatorError("table longer than max_blocks")
            tables[i, :len(tab)] = tab
            lens[i] = self._lens[s]
        return tables, lens
