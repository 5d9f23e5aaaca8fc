"""Builds oracle-side state (block manager + bit-exact pool) from a workload.

Test helper: uses only ``oracle`` and ``workloads``.
"""
import numpy as np

import workloads as wl
from oracle import BlockManager, PoolModel


def fp8_channel_scales(w, d):
    """Per-(layer, KV head, channel) scales from the absmax of the drawn
    source-dtype cache of every sequence (K and V separately)."""
    ks, vs = [], []
    for b, L in enumerate(d.lengths):
        kb, vb = wl.kv_tokens_bits(w, (1, b), int(L))
        ks.append(wl.bits_as_f32(kb, w.src_dtype))
        vs.append(wl.bits_as_f32(vb, w.src_dtype))
    k_scale, k_inv = wl.fp8_scales(wl.channel_absmax(ks, w.num_kv_heads, w.head_dim))
    v_scale, v_inv = wl.fp8_scales(wl.channel_absmax(vs, w.num_kv_heads, w.head_dim))
    shape = (w.num_layers, w.num_kv_heads, w.head_dim)
    rep = lambda a: np.broadcast_to(a, shape).copy()
    return rep(k_scale), rep(v_scale), rep(k_inv), rep(v_inv)


class OracleState:
    def __init__(self, w, d, free_order=None, scales=None, layer=0):
        self.w, self.d, self.layer = w, d, layer
        order = d.free_order if free_order is None else free_order
        self.bm = BlockManager(d.num_blocks, w.block_size, order)
        kw = {}
        if w.kv_dtype == "fp8":
            if scales is None:
                scales = fp8_channel_scales(w, d)
            self.k_scale, self.v_scale, self.k_inv, self.v_inv = scales
            kw = dict(k_scale=self.k_scale, v_scale=self.v_scale,
                      k_inv_scale=self.k_inv, v_inv_scale=self.v_inv)
        self.pool = PoolModel(w.num_layers, d.num_blocks, w.num_kv_heads, w.block_size,
                              w.head_dim, w.kv_dtype, **kw)
        self.seqs = []
        self.slots = []
        for b, L in enumerate(d.lengths):
            s = self.bm.alloc()
            slots, cows = self.bm.append(s, int(L))
            assert not cows
            kb, vb = wl.kv_tokens_bits(w, (1, b), int(L))
            self.pool.append(layer, kb, vb, w.src_dtype, slots)
            self.seqs.append(s)
            self.slots.append(np.asarray(slots, dtype=np.int64))

    def max_blocks(self):
        return max(1, max(-(-int(L) // self.w.block_size) for L in self.d.lengths))

    def export(self, max_blocks=None):
        return self.bm.export(self.seqs, max_blocks or self.max_blocks())
