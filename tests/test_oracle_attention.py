"""Pins of the oracle's decode attention.

* brute force: scalar loops with math.fsum over the *unpaged* logical K/V the
  appends were made from (page 'AI 陪读顶会论文（三）', section
  '为什么自回归解码…必须使用 KV Cache', the attention equation);
* library: torch scaled_dot_product_attention on contiguous float64 CPU
  tensors, GQA by repeat_interleave;
* closed forms: L = 1 gives v_0; q = 0 gives the mean of V; equal keys give
  the mean of V; window 1 gives v_{L-1}; window >= L equals no window;
* paging invariance: another physical placement gives bitwise-equal output;
* fork identity: a forked sequence decodes bitwise-equal to its parent, and
  after copy-on-write the parent's bytes are unchanged;
* split / log-sum-exp merge over any partition equals the unsplit result.
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import (decode_attention, decode_attention_split, partial_attention,
                    lse_merge, bits_to_f64, BlockManager, PoolModel)
from oracle_state import OracleState


def _logical_f64(w, b, L):
    kb, vb = wl.kv_tokens_bits(w, (1, b), L)
    return (wl.bits_as_f32(kb, w.src_dtype).astype(np.float64),
            wl.bits_as_f32(vb, w.src_dtype).astype(np.float64))


def _brute(q, K, V, scale, lo=0):
    """q [D]; K, V [L][D] python-float loops."""
    L, D = len(K), len(q)
    s = [scale * math.fsum(q[d] * K[j][d] for d in range(D)) for j in range(lo, L)]
    m = max(s)
    p = [math.exp(x - m) for x in s]
    den = math.fsum(p)
    return [math.fsum(p[j] * V[lo + j][d] for j in range(len(p))) / den for d in range(D)]


TINY = [
    wl.WORKLOADS["c1"],
    wl.scaled(wl.WORKLOADS["c1"], name="t_g1", num_q_heads=2, num_kv_heads=2, head_dim=8,
              block_size=4, lengths_args=(1, 4, 5, 13), pool_blocks=16),
    wl.scaled(wl.WORKLOADS["c3"], name="t_bf16", batch=3, num_q_heads=8, num_kv_heads=2,
              head_dim=16, block_size=4, lengths_kind="fixed", lengths_args=(7, 1, 9),
              pool_blocks=12),
    wl.scaled(wl.WORKLOADS["c2"], name="t_f16", batch=2, num_q_heads=3, num_kv_heads=1,
              head_dim=8, block_size=2, lengths_kind="fixed", lengths_args=(5, 3),
              pool_blocks=9),
]


@pytest.mark.parametrize("w", TINY, ids=lambda w: w.name)
@pytest.mark.parametrize("window", [0, 3])
def test_brute_force(w, window):
    d = wl.draw(w)
    st = OracleState(w, d)
    tables, lens = st.export()
    q = wl.q_bits(w)
    scale = 1.0 / math.sqrt(w.head_dim)
    out = decode_attention(st.pool, 0, q, w.q_dtype, tables, lens, scale, window)
    qf = wl.bits_as_f32(q, w.q_dtype).astype(np.float64)
    G = w.group
    for b, L in enumerate(d.lengths):
        K, V = _logical_f64(w, b, int(L))
        lo = max(0, int(L) - window) if window else 0
        for h in range(w.num_q_heads):
            ref = _brute(qf[b, h].tolist(), K[:, h // G].tolist(), V[:, h // G].tolist(), scale, lo)
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["c1", "c3_small", "c2_small"])
def test_matches_torch_sdpa(name):
    if name == "c1":
        w = wl.WORKLOADS["c1"]
    elif name == "c3_small":
        w = wl.scaled(wl.WORKLOADS["c3"], batch=6, lengths_args=(60.0, 0.8, 1, 300))
    else:
        w = wl.scaled(wl.WORKLOADS["c2"], batch=3, num_q_heads=4, num_kv_heads=4,
                      lengths_args=(1, 200), block_size=32)
    d = wl.draw(w)
    st = OracleState(w, d)
    tables, lens = st.export()
    q = wl.q_bits(w)
    scale = 1.0 / math.sqrt(w.head_dim)
    out = decode_attention(st.pool, 0, q, w.q_dtype, tables, lens, scale)
    qf = torch.from_numpy(wl.bits_as_f32(q, w.q_dtype).astype(np.float64))
    for b, L in enumerate(d.lengths):
        K, V = _logical_f64(w, b, int(L))
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(w.group, dim=0)
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(w.group, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qf[b][:, None, :], Kt, Vt, scale=scale)[:, 0, :].numpy()
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def _single_seq_pool(K, V, bs, order=None, dtype="f32"):
    L, D = K.shape
    nb = -(-L // bs) + 2
    bm = BlockManager(nb, bs, order)
    s = bm.alloc()
    slots, _ = bm.append(s, L)
    pool = PoolModel(1, nb, 1, bs, D, dtype)
    kb = K.astype(np.float32).view(np.uint32)[:, None, :]
    vb = V.astype(np.float32).view(np.uint32)[:, None, :]
    pool.append(0, kb, vb, "f32", slots)
    tables, lens = bm.export([s], -(-L // bs))
    return pool, tables, lens


def test_closed_forms():
    rng = np.random.default_rng(11)
    D, bs = 8, 4
    K = rng.standard_normal((10, D)).astype(np.float32)
    V = rng.standard_normal((10, D)).astype(np.float32)
    pool, tables, lens = _single_seq_pool(K, V, bs)
    q = rng.standard_normal((1, 1, D)).astype(np.float32).view(np.uint32)
    run = lambda qq, ll, win=0: decode_attention(pool, 0, qq, "f32", tables, np.array([ll]), 0.3, win)[0, 0]
    # one token: the output is its value vector
    assert np.array_equal(run(q, 1), V[0].astype(np.float64))
    # zero query: uniform weights -> mean of V
    q0 = np.zeros((1, 1, D), np.float32).view(np.uint32)
    np.testing.assert_allclose(run(q0, 10), V.astype(np.float64).mean(0), atol=1e-15)
    # window of one key: the newest value vector
    assert np.array_equal(run(q, 10, 1), V[9].astype(np.float64))
    # window covering everything equals no window
    assert np.array_equal(run(q, 10, 10), run(q, 10))
    assert np.array_equal(run(q, 10, 50), run(q, 10))
    # empty context -> zeros
    assert np.array_equal(run(q, 0), np.zeros(D))
    # all keys equal -> mean of V
    Ke = np.repeat(K[:1], 10, axis=0)
    pool2, t2, l2 = _single_seq_pool(Ke, V, bs)
    out = decode_attention(pool2, 0, q, "f32", t2, l2, 0.3)[0, 0]
    np.testing.assert_allclose(out, V.astype(np.float64).mean(0), atol=1e-15)


def test_gqa_equals_mha_with_repeated_kv():
    w = wl.scaled(wl.WORKLOADS["c1"], lengths_args=(3, 9, 17, 33))
    d = wl.draw(w)
    st = OracleState(w, d)
    tables, lens = st.export()
    q = wl.q_bits(w)
    out = decode_attention(st.pool, 0, q, "f32", tables, lens, 0.125)
    # MHA pool: every KV head duplicated G times, in the order h // G
    G = w.group
    mha = PoolModel(1, d.num_blocks, w.num_q_heads, w.block_size, w.head_dim, "f32")
    mha.k[:] = np.repeat(st.pool.k, G, axis=2)
    mha.v[:] = np.repeat(st.pool.v, G, axis=2)
    out2 = decode_attention(mha, 0, q, "f32", tables, lens, 0.125)
    assert np.array_equal(out, out2)


def test_permutation_invariance_bitwise():
    w = wl.scaled(wl.WORKLOADS["c3"], batch=5, num_q_heads=8, num_kv_heads=2, head_dim=32,
                  lengths_args=(40.0, 0.8, 1, 200))
    d = wl.draw(w)
    q = wl.q_bits(w)
    outs = []
    for seed in range(3):
        order = np.random.default_rng(seed).permutation(d.num_blocks)
        st = OracleState(w, d, free_order=order)
        tables, lens = st.export()
        outs.append(decode_attention(st.pool, 0, q, "bf16", tables, lens, 0.17))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    # and a direct permutation of a built pool + table
    st = OracleState(w, d)
    tables, lens = st.export()
    perm = np.random.default_rng(9).permutation(d.num_blocks)
    moved = PoolModel(1, d.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, "bf16")
    moved.k[:, perm] = st.pool.k
    moved.v[:, perm] = st.pool.v
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    a = decode_attention(st.pool, 0, q, "bf16", tables, lens, 0.17)
    b = decode_attention(moved, 0, q, "bf16", t2, lens, 0.17)
    assert np.array_equal(a, b)


def test_fork_identity_and_cow_preserves_parent():
    w = wl.scaled(wl.WORKLOADS["c3"], batch=1, num_q_heads=4, num_kv_heads=2, head_dim=16,
                  block_size=4, lengths_kind="fixed", lengths_args=(10,), pool_blocks=16)
    d = wl.draw(w)
    st = OracleState(w, d)
    parent = st.seqs[0]
    child = st.bm.fork(parent)
    q = wl.q_bits(w)
    t, l = st.bm.export([parent, child], 4)
    o = decode_attention(st.pool, 0, np.concatenate([q, q]), "bf16", t, l, 0.25)
    assert np.array_equal(o[0], o[1])
    parent_bits = st.pool.k[0, st.bm.table(parent)].copy()
    # both append the same token: the first CoWs, the second writes in place
    kb, vb, _ = wl.step_tokens_bits(w, 0, batch=1)
    slots, cows = st.bm.append_batch([child, parent])
    assert len(cows) == 1
    st.pool.copy_blocks(cows)
    st.pool.append(0, np.concatenate([kb, kb]), np.concatenate([vb, vb]), "bf16", slots)
    # parent's original blocks (before its own in-place write) are untouched
    assert np.array_equal(st.pool.k[0, st.bm.table(parent)[:2]], parent_bits[:2])
    t, l = st.bm.export([parent, child], 4)
    o = decode_attention(st.pool, 0, np.concatenate([q, q]), "bf16", t, l, 0.25)
    assert np.array_equal(o[0], o[1])


def test_lse_merge_identity():
    w = wl.scaled(wl.WORKLOADS["c3"], batch=4, num_q_heads=8, num_kv_heads=2, head_dim=16,
                  lengths_args=(100.0, 0.8, 1, 400))
    d = wl.draw(w)
    st = OracleState(w, d)
    tables, lens = st.export()
    q = wl.q_bits(w)
    ref = decode_attention(st.pool, 0, q, "bf16", tables, lens, 0.25)
    bs = w.block_size
    for cuts in (lambda L: range(bs, L, bs),                    # every block
                 lambda L: [],                                  # one split
                 lambda L: sorted({1, L // 3, L // 2} - {0, L}),  # ragged cuts
                 lambda L: range(1, L)):                        # every token
        got = decode_attention_split(st.pool, 0, q, "bf16", tables, lens, 0.25, cuts)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    # with a window as well
    ref_w = decode_attention(st.pool, 0, q, "bf16", tables, lens, 0.25, window=37)
    got_w = decode_attention_split(st.pool, 0, q, "bf16", tables, lens, 0.25,
                                   lambda L: range(bs, L, bs), window=37)
    np.testing.assert_allclose(got_w, ref_w, rtol=0, atol=1e-12)


def test_partial_and_merge_edge_cases():
    D = 4
    o, m, l = partial_attention(np.ones(D), np.zeros((0, D)), np.zeros((0, D)), 1.0)
    assert m == -np.inf and l == 0.0 and not o.any()
    K = np.eye(D)
    V = np.arange(16.0).reshape(4, 4)
    whole = lse_merge([partial_attention(np.ones(D), K, V, 2.0)])
    parts = [partial_attention(np.ones(D), K[:1], V[:1], 2.0),
             partial_attention(np.ones(D), K[1:1], V[1:1], 2.0),   # empty piece
             partial_attention(np.ones(D), K[1:], V[1:], 2.0)]
    np.testing.assert_allclose(lse_merge(parts), whole, atol=1e-15)
    np.testing.assert_allclose(whole, V.mean(0), atol=1e-15)


def test_fp8_decode_uses_codes_times_scale():
    w = wl.scaled(wl.WORKLOADS["c5_fp8"], batch=2, lengths_kind="fixed", lengths_args=(19, 40),
                  pool_blocks=8, num_q_heads=4, num_kv_heads=2, head_dim=16)
    d = wl.draw(w)
    st = OracleState(w, d)
    tables, lens = st.export()
    q = wl.q_bits(w)
    out = decode_attention(st.pool, 0, q, "bf16", tables, lens, 0.25)
    # rebuild K, V from the codes and scales by hand and run the brute force
    from oracle.e4m3 import e4m3_to_f64
    qf = wl.bits_as_f32(q, "bf16").astype(np.float64)
    for b, L in enumerate(d.lengths):
        blocks = tables[b][: -(-int(L) // w.block_size)]
        for h in range(w.num_q_heads):
            g = h // w.group
            K = e4m3_to_f64(st.pool.k[0, blocks, g]).reshape(-1, w.head_dim)[:L] * st.k_scale[0, g]
            V = e4m3_to_f64(st.pool.v[0, blocks, g]).reshape(-1, w.head_dim)[:L] * st.v_scale[0, g]
            ref = _brute(qf[b, h].tolist(), K.tolist(), V.tolist(), 0.25)
            np.testing.assert_allclose(out[b, h], ref, atol=1e-12)
    # FP8 result stays close to the bf16 result it quantises (reported, not a parity bar)
    wb = wl.scaled(w, kv_dtype="bf16")
    stb = OracleState(wb, d)
    ob = decode_attention(stb.pool, 0, q, "bf16", tables, lens, 0.25)
    assert np.abs(out - ob).max() < 0.15


@pytest.mark.parametrize("window", [1, 16, 17, 24])
def test_window_reads_only_the_window(window):
    # page "生成一个字…", section "再往后：压 KV 的三条路线": the query attends the
    # last stretch only, so releasing every block wholly before it (table
    # entries -1) leaves the result bitwise unchanged
    w = wl.WORKLOADS["c1"]
    d = wl.draw(w)
    st = OracleState(w, d)
    q = wl.q_bits(w)
    tables, lens = st.export()
    scale = 1.0 / math.sqrt(w.head_dim)
    before = decode_attention(st.pool, 0, q, w.q_dtype, tables, lens, scale, window)
    for s, L in zip(st.seqs, lens):
        st.bm.release_before(s, max(0, int(L) - window))
    t2, l2 = st.export()
    assert (t2 == -1).sum() > (tables == -1).sum()
    after = decode_attention(st.pool, 0, q, w.q_dtype, t2, l2, scale, window)
    assert np.array_equal(before, after)
    # without the window the released blocks are needed: the gather refuses
    with pytest.raises(ValueError):
        decode_attention(st.pool, 0, q, w.q_dtype, t2, l2, scale, 0)
