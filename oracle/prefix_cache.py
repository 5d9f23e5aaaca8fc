"""Prefix cache model (oracle; test infrastructure only).

Page "第2章 KV Cache：模型内部的显存复用" (chapter summary and section 2.4): a
radix tree organises the prefixes of multi-turn conversations into a cache
that later requests hit.  Page "生成一个字，为什么要背一整本账", section
"PagedAttention：把操作系统的老智慧搬进推理引擎": shared blocks are stored
once, reference counted.

This model keeps no tree: it is the set of cached prefixes written out, one
entry per whole block.  Entry ``tokens[:k * bs]`` (a tuple) holds the block
with the k-th block of those tokens and the clock of the last call that
touched it.  Readings (the same as the library's):

* only whole blocks are cached or matched;
* the cache holds one reference on each block it caches; a match returns a
  new sequence holding the matched blocks (one more reference each);
* an insert adds only the prefixes not cached yet (the cache keeps the block
  it already has for known tokens);
* each match or insert is one clock tick and touches every entry on its path;
* eviction removes, one at a time, the least recently touched entry that is
  no prefix of another entry (a leaf) and whose block only the cache
  holds; destroying the cache removes every entry in the same order, whoever
  else holds the blocks.
"""


class PrefixCacheModel:
    def __init__(self, bm):
        self.bm = bm
        self.bs = bm.block_size
        self.entries = {}      # prefix tuple -> [block, last_use]
        self.clock = 0

    def _prefix(self, tokens, k):
        return tuple(int(t) for t in tokens[:k * self.bs])

    def match(self, tokens):
        """(new sequence id, matched tokens)."""
        k = 0
        while (k + 1) * self.bs <= len(tokens) and self._prefix(tokens, k + 1) in self.entries:
            k += 1
        blocks = [self.entries[self._prefix(tokens, j)][0] for j in range(1, k + 1)]
        seq = self.bm.adopt(blocks, k * self.bs)
        self.clock += 1
        for j in range(1, k + 1):
            self.entries[self._prefix(tokens, j)][1] = self.clock
        return seq, k * self.bs

    def insert(self, seq, tokens):
        table = self.bm.table(seq)
        n = min(len(tokens), self.bm.length(seq)) // self.bs
        n = min(n, len(table))
        for j in range(n):
            if table[j] < 0:
                n = j
                break
        self.clock += 1
        for j in range(1, n + 1):
            key = self._prefix(tokens, j)
            if key in self.entries:
                self.entries[key][1] = self.clock
            else:
                self.entries[key] = [table[j - 1], self.clock]
                self.bm.ref_block(table[j - 1])

    def _leaves(self):
        parents = {key[:-self.bs] for key in self.entries}
        return [key for key in self.entries if key not in parents]

    def _remove_oldest(self, only_unheld):
        cands = [k for k in self._leaves()
                 if not only_unheld or self.bm.refcount(self.entries[k][0]) == 1]
        if not cands:
            return False
        key = min(cands, key=lambda k: self.entries[k][1])
        blk = self.entries.pop(key)[0]
        self.bm.unref_block(blk)
        return True

    def evict(self, n_blocks):
        freed = 0
        while freed < n_blocks and self._remove_oldest(True):
            freed += 1
        return freed

    def destroy(self):
        while self._remove_oldest(False):
            pass

    def cached_blocks(self):
        return len(self.entries)
