"""GPU parity on pools of several layers.

The byte formula counts layers (page "生成一个字，为什么要背一整本账", opening
section: 2 x layers x KV heads x head_dim x tokens x bytes), and a pool holds
every layer's blocks under one block table: a sequence's block p holds its
tokens in every layer.  These cases give each layer its own K/V values and,
for FP8, its own per-channel scales, then

* append every sequence's tokens into every layer,
* fork each sequence and append one token to the branch and to the parent
  (page "AI 陪读顶会论文（三）", section "PagedAttention 的破局哲学",
  innovation 3: a shared partial last block is copied, in every layer,
  before the first write into it),
* compare the tables and every layer's pool bytes bit for bit with the
  oracle, and decode every layer against the oracle.
"""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_406_amd as P
import workloads as wl
from oracle import BlockManager, PoolModel, decode_attention
from gpu_state import to_dev, out_to_f64, from_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-3, "f16": 2e-3, "bf16": 2e-3, "fp8": 3e-2}

CASES = {
    "bf16_gqa8_l3": wl.scaled(wl.WORKLOADS["c3"], batch=6, num_q_heads=16, num_kv_heads=2,
                              lengths_kind="fixed", lengths_args=(1, 17, 40, 95, 300, 33), num_layers=3),
    "fp8_gqa8_l3": wl.scaled(wl.WORKLOADS["c5_fp8"], batch=4, num_q_heads=16, num_kv_heads=2,
                             lengths_kind="fixed", lengths_args=(700, 37, 64, 1), pool_blocks=0,
                             num_layers=3),
    "f16_mha_bs32_l2": wl.scaled(wl.WORKLOADS["c2"], batch=4, num_q_heads=4, num_kv_heads=4, block_size=32,
                                 lengths_kind="fixed", lengths_args=(5, 32, 33, 150), num_layers=2),
}
_STATES = {}


def _logical(w, nb, t, which):
    """Device pool bytes of K or V as logical [layers][NB][Hkv][bs][D] bit patterns."""
    eb = wl.ELEM_BYTES[w.kv_dtype]
    npd = {4: np.uint32, 2: np.uint16, 1: np.uint8}[eb]
    L, H, BS, D = w.num_layers, w.num_kv_heads, w.block_size, w.head_dim
    a = from_dev(t, npd)
    if which == "k":
        x = 16 // eb
        return a.reshape(L, nb, H, D // x, BS, x).transpose(0, 1, 2, 4, 3, 5).reshape(L, nb, H, BS, D)
    vt = min(BS, {"f32": 16, "f16": 32, "bf16": 32, "fp8": 64}[w.kv_dtype])
    return a.reshape(L, nb, H, BS // vt, D, vt).transpose(0, 1, 2, 3, 5, 4).reshape(L, nb, H, BS, D)


class MultiLayerState:
    def __init__(self, w):
        self.w = w
        d = wl.draw(w, extra_blocks=2 * w.batch)
        self.d = d
        NL = w.num_layers
        kv = {(b, l): wl.kv_tokens_bits(w, wl.kv_stream(b, l), int(n))
              for b, n in enumerate(d.lengths) for l in range(NL)}
        # one new token per branch and per parent, in every layer
        new_child = {l: wl.kv_tokens_bits(w, (6, l, 0), w.batch) for l in range(NL)}
        new_parent = {l: wl.kv_tokens_bits(w, (6, l, 1), w.batch) for l in range(NL)}
        sc = {}
        if w.kv_dtype == "fp8":
            per = {"k": [], "v": []}
            for l in range(NL):
                for which, idx in (("k", 0), ("v", 1)):
                    vals = [wl.bits_as_f32(kv[(b, l)][idx], w.src_dtype) for b in range(w.batch)]
                    vals += [wl.bits_as_f32(new_child[l][idx], w.src_dtype),
                             wl.bits_as_f32(new_parent[l][idx], w.src_dtype)]
                    per[which].append(wl.fp8_scales(wl.channel_absmax(vals, w.num_kv_heads, w.head_dim)))
            sc = dict(k_scale=np.stack([s for s, _ in per["k"]]), k_inv_scale=np.stack([i for _, i in per["k"]]),
                      v_scale=np.stack([s for s, _ in per["v"]]), v_inv_scale=np.stack([i for _, i in per["v"]]))
            # the scales really differ between layers
            assert not np.array_equal(sc["k_scale"][0], sc["k_scale"][1])
        self.pool = P.TorchKVPool(NL, w.num_kv_heads, w.head_dim, w.block_size, d.num_blocks, w.kv_dtype,
                                  free_order=d.free_order, **sc)
        self.pool.k_cache.fill_(0xFF)
        self.pool.v_cache.fill_(0xFF)
        self.bm = BlockManager(d.num_blocks, w.block_size, d.free_order)
        self.opool = PoolModel(NL, d.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, w.kv_dtype, **sc)
        h = self.pool.handle
        self.seqs = []
        for b, n in enumerate(d.lengths):
            s, o = P.block_table_alloc(h), self.bm.alloc()
            assert s == o
            self.seqs.append(s)
            self._append(s, int(n), [kv[(b, l)] for l in range(NL)])
        # a branch of every sequence; the branch writes first (copy-on-write of a
        # shared partial last block, every layer), then the parent (in place)
        self.children = [P.block_table_fork(h, s) for s in self.seqs]
        assert self.children == [self.bm.fork(s) for s in self.seqs]
        self.n_cow = 0
        for b, c in enumerate(self.children):
            self.n_cow += self._append(c, 1, [tuple(x[b:b + 1] for x in new_child[l]) for l in range(NL)])
        for b, s in enumerate(self.seqs):
            assert self._append(s, 1, [tuple(x[b:b + 1] for x in new_parent[l]) for l in range(NL)]) == 0
        torch.cuda.synchronize()

    def _append(self, s, n, kv_layers):
        """n tokens into sequence s, kv_layers[l] = (k, v) bits of layer l;
        returns the number of copy-on-write pairs."""
        h = self.pool.handle
        slots, cows = P.block_table_append(h, s, n)
        oslots, ocows = self.bm.append(s, n)
        assert slots.tolist() == oslots and cows == ocows
        if cows:
            P.kv_pool_copy_blocks(h, torch.tensor(cows, dtype=torch.int32).cuda(), len(cows))
            self.opool.copy_blocks(ocows)
        sd = torch.from_numpy(slots).cuda()
        for l, (kb, vb) in enumerate(kv_layers):
            P.paged_kv_append(h, l, to_dev(kb), to_dev(vb), self.w.src_dtype, sd, n)
            self.opool.append(l, kb, vb, self.w.src_dtype, oslots)
        return len(cows)

    def all_seqs(self):
        return self.seqs + self.children

    def export(self):
        seqs = self.all_seqs()
        mb = max(len(self.bm.table(s)) for s in seqs)
        t, ln = P.block_table_export(self.pool.handle, seqs, mb)
        ot, ol = self.bm.export(seqs, mb)
        assert np.array_equal(t, ot) and np.array_equal(ln, ol)
        return ot, ol

    def close(self):
        self.pool.close()


def _state(name):
    if name not in _STATES:
        _STATES[name] = MultiLayerState(CASES[name])
    return _STATES[name]


@pytest.mark.parametrize("name", list(CASES))
def test_every_layer_pool_bits_exact(name):
    st = _state(name)
    w, d = st.w, st.d
    assert st.n_cow > 0
    st.export()
    written = st.opool.written
    assert all(written[l].any() for l in range(w.num_layers))
    for which, arr in (("k", st.opool.k), ("v", st.opool.v)):
        dev = _logical(w, d.num_blocks, st.pool.k_cache if which == "k" else st.pool.v_cache, which)
        for l in range(w.num_layers):
            blk, off = np.nonzero(written[l])
            got = dev[l, blk, :, off]
            want = arr[l, blk, :, off]
            assert np.array_equal(got, want), (name, which, l)
    # every layer's slots were written, and the layers hold different bytes
    assert all(np.array_equal(written[0], written[l]) for l in range(w.num_layers))
    blk, off = np.nonzero(written[0])
    assert not np.array_equal(st.opool.k[0, blk, :, off], st.opool.k[1, blk, :, off])


@pytest.mark.parametrize("splits", [1, 0, 3])
@pytest.mark.parametrize("name", list(CASES))
def test_decode_every_layer(name, splits):
    st = _state(name)
    w = st.w
    tables, lens = st.export()
    B = len(lens)
    scale = 1.0 / math.sqrt(w.head_dim)
    for layer in range(w.num_layers):
        q = wl.q_bits(w, batch=B, stream=(2, layer))
        ref = decode_attention(st.opool, layer, q, w.q_dtype, tables, lens, scale)
        out = torch.full((B, w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        qd = to_dev(q)
        td = torch.from_numpy(np.ascontiguousarray(tables, dtype=np.int32)).cuda()
        ld = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).cuda()
        a = P.make_decode_args(layer, B, w.num_q_heads, tables.shape[1], qd, w.q_dtype, td, ld, scale, out, "f32",
                               num_splits=splits)
        nbytes = P.paged_attention_workspace_size(st.pool.handle, a)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        a.workspace, a.workspace_bytes = ws.data_ptr(), nbytes
        P.paged_attention_decode(st.pool.handle, a)
        torch.cuda.synchronize()
        got = out_to_f64(out, "f32")
        assert np.isfinite(got).all()
        err = np.abs(got - ref).max()
        assert err <= TOL[w.kv_dtype], (name, layer, splits, err)


@pytest.mark.parametrize("name", list(CASES))
def test_shared_prefix_every_layer(name):
    """The longest sequence and its branch share their full leading blocks;
    the shared-prefix decode (those blocks read once for both rows) of every
    layer matches the oracle: the prefix pass's block addresses and FP8
    scales are those of the layer asked for."""
    st = _state(name)
    w = st.w
    h = st.pool.handle
    b = int(np.argmax(st.d.lengths))
    pair = [st.seqs[b], st.children[b]]
    mb = max(len(st.bm.table(s)) for s in pair)
    tables, lens = P.block_table_export(h, pair, mb)
    ot, ol = st.bm.export(pair, mb)
    assert np.array_equal(tables, ot) and np.array_equal(lens, ol)
    k = P.block_table_common_prefix(h, pair)
    assert k == st.bm.common_prefix(pair) and k >= 1
    scale = 1.0 / math.sqrt(w.head_dim)
    for layer in range(w.num_layers):
        q = wl.q_bits(w, batch=2, stream=(7, layer))
        ref = decode_attention(st.opool, layer, q, w.q_dtype, ot, ol, scale)
        out = torch.full((2, w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        td = torch.from_numpy(np.ascontiguousarray(tables, dtype=np.int32)).cuda()
        ld = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).cuda()
        qd = to_dev(q)
        a = P.make_decode_args(layer, 2, w.num_q_heads, mb, qd, w.q_dtype, td, ld, scale, out, "f32",
                               shared_prefix_blocks=k)
        nbytes = P.paged_attention_workspace_size(h, a)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        a.workspace, a.workspace_bytes = ws.data_ptr(), nbytes
        P.paged_attention_decode(h, a)
        torch.cuda.synchronize()
        got = out_to_f64(out, "f32")
        assert np.isfinite(got).all()
        err = np.abs(got - ref).max()
        assert err <= TOL[w.kv_dtype], (name, layer, k, err)


@pytest.mark.parametrize("name", list(CASES))
def test_fused_step_in_first_layer(name):
    """One decode step of a model of several layers over device-resident
    tables and lengths.  Layer 0's call fuses the append: it stores layer 0's
    token and writes each row's table entry and length, once for the step.
    Every later layer stores its own token with paged_kv_append and decodes
    the L + 1 tokens.  Every layer's output matches the oracle's append then
    decode, and the tables and lengths advance by one token, not one per
    layer."""
    w = CASES[name]
    st = MultiLayerState(w)    # a fresh pool: the step changes it
    try:
        h = st.pool.handle
        seqs = st.all_seqs()
        B = len(seqs)
        mb = max(len(st.bm.table(s)) for s in seqs) + 1
        t0, l0 = P.block_table_export(h, seqs, mb)
        d_tables, d_lens = torch.from_numpy(t0).cuda(), torch.from_numpy(l0).cuda()
        slots, cows = P.block_table_append_batch(h, seqs)
        oslots, ocows = st.bm.append_batch(seqs)
        assert slots.tolist() == oslots
        assert len(cows) == 0 and len(ocows) == 0   # every row's last block is its own
        d_slots = torch.from_numpy(np.asarray(slots, dtype=np.int64)).cuda()
        ot, ol = st.bm.export(seqs, mb)
        scale = 1.0 / math.sqrt(w.head_dim)
        for layer in range(w.num_layers):
            kb, vb = wl.kv_tokens_bits(w, (8, layer), B)
            q = wl.q_bits(w, batch=B, stream=(9, layer))
            kw = {}
            if layer == 0:
                kw = dict(new_k=to_dev(kb), new_v=to_dev(vb), new_dtype=w.src_dtype, new_slots=d_slots)
            else:
                P.paged_kv_append(h, layer, to_dev(kb), to_dev(vb), w.src_dtype, d_slots, B)
            out = torch.full((B, w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
            a = P.make_decode_args(layer, B, w.num_q_heads, mb, to_dev(q), w.q_dtype, d_tables, d_lens, scale, out,
                                   "f32", **kw)
            nbytes = P.paged_attention_workspace_size(h, a)
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
            a.workspace, a.workspace_bytes = ws.data_ptr(), nbytes
            P.paged_attention_decode(h, a)
            torch.cuda.synchronize()
            st.opool.append(layer, kb, vb, w.src_dtype, oslots)
            ref = decode_attention(st.opool, layer, q, w.q_dtype, ot, ol, scale)
            got = out_to_f64(out, "f32")
            assert np.isfinite(got).all()
            err = np.abs(got - ref).max()
            assert err <= TOL[w.kv_dtype], (name, layer, err)
            # one token further after layer 0's call, and no further after the others
            assert np.array_equal(d_tables.cpu().numpy(), ot) and np.array_equal(d_lens.cpu().numpy(), ol), layer
    finally:
        st.close()
