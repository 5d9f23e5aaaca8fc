"""CPU oracle for paged KV-cache decode attention -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, obviously-correct reference that the HIP
library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``paged_kv_cache_406_amd``) never imports, calls or links anything here, and
nothing here imports the product path: the two share no code.  The only
module both sides use is ``workloads`` (seeded synthetic inputs, no method
arithmetic).

Pages the oracle follows (cited by title and section throughout):

* "生成一个字，为什么要背一整本账" -- KV byte formula (opening section),
  GQA (section "显存账本"), paging / on-demand blocks / prefix sharing with
  copy-on-write (section "PagedAttention：把操作系统的老智慧搬进推理引擎"),
  FP8 with per-channel scales and the 4K sliding window (section
  "再往后：压 KV 的三条路线").
* "AI 陪读顶会论文（三）：KV Cache 显存占用计算与 PagedAttention 原理拆解" --
  decode attention equation (section "为什么自回归解码…必须使用 KV Cache"),
  block mapping figure and the three innovations (section
  "PagedAttention 的破局哲学").
* "第2章 KV Cache：模型内部的显存复用" -- 7B at 32K/128K vs weights
  (section "拐点与结论"); the radix-tree prefix cache of multi-turn
  conversations (chapter summary, section 2.4).

Modules
-------
kv_bytes   KV byte formula.                                   pinned
allocator  block manager: FIFO free list, tables, refcounts,
           on-demand append, fork, copy-on-write, free.       pinned
e4m3       OCP FP8 E4M3 decode table and RNE-saturating encoder. pinned
pool       bit-exact pool model: append (copy / FP8 quantise),
           whole-block copy.                                  pinned
attention  gather + fp64 textbook decode attention (GQA,
           window, FP8 dequant) and the split / log-sum-exp
           merge identity.                                     pinned
prefix_cache  cached whole-block prefixes of token sequences,
           LRU leaf eviction (the pages' radix-tree cache as a
           plain set of prefixes).                             pinned

Every function is pinned by tests under ``tests/`` marked ``not gpu``; no
function here is "parity unpinned".
"""

from .kv_bytes import kv_cache_bytes
from .e4m3 import e4m3_decode_table, e4m3_encode, E4M3_MAX
from .allocator import BlockManager, AllocatorError, OutOfBlocks
from .pool import PoolModel, bits_to_f64
from .attention import (decode_attention, gather_kv, partial_attention,
                        lse_merge, decode_attention_split)
from .prefix_cache import PrefixCacheModel

__all__ = [
    "kv_cache_bytes", "e4m3_decode_table", "e4m3_encode", "E4M3_MAX",
    "BlockManager", "AllocatorError", "OutOfBlocks", "PoolModel",
    "bits_to_f64", "decode_attention", "gather_kv", "partial_attention",
    "lse_merge", "decode_attention_split", "PrefixCacheModel",
]
