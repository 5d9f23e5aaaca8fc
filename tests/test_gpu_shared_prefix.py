"""GPU parity of the shared-prefix decode (shared_prefix_blocks > 0).

Families of sequences forked from one root (a shared prefix stored once,
then private suffixes; copy-on-write of the prefix's partial last block) are
built through the C ABI and mirrored in the oracle's block manager.  The
number of shared blocks comes from block_table_common_prefix (checked against
the oracle), and the decode that reads those blocks once for the whole batch
is compared with the oracle's plain attention on every row, for several split
counts, and with the ordinary decode of the same state.
"""
import math

import numpy as np
import pytest

import paged_kv_cache_406_amd as P
import workloads as wl
from test_gpu_full_size import FullState, TOL

pytestmark = pytest.mark.gpu

C4 = wl.WORKLOADS["c4"]
CASES = {
    "bf16_g4": wl.scaled(C4, batch=12, prefix_len=100, lengths_args=(0, 70)),
    "bf16_g4_tiny_suffix": wl.scaled(C4, batch=9, prefix_len=37, lengths_args=(0, 3)),
    "bf16_g4_prefix_only": wl.scaled(C4, batch=5, prefix_len=96, lengths_args=(0, 0)),
    "bf16_many_rows": wl.scaled(C4, batch=41, num_q_heads=8, num_kv_heads=2, prefix_len=64,
                                lengths_args=(1, 30)),
    "f16_mha": wl.scaled(wl.WORKLOADS["c2"], batch=9, num_q_heads=4, num_kv_heads=4, lengths_kind="prefix",
                         prefix_len=130, lengths_args=(1, 90)),
    "fp8_g8": wl.scaled(wl.WORKLOADS["c5_fp8"], batch=6, num_q_heads=16, num_kv_heads=2, lengths_kind="prefix",
                        prefix_len=150, lengths_args=(0, 100), pool_blocks=0),
    "bf16_bs32": wl.scaled(C4, batch=7, prefix_len=200, lengths_args=(1, 60), block_size=32),
    "bf16_bs128_d64": wl.scaled(C4, batch=5, head_dim=64, block_size=128, prefix_len=300,
                                lengths_args=(0, 200)),
    "f32_d64": wl.scaled(wl.WORKLOADS["c1"], batch=6, lengths_kind="prefix", prefix_len=40,
                         lengths_args=(0, 30), pool_blocks=0),
}


def _family(name, extra=0):
    w = CASES[name]
    d = wl.draw(w, extra_blocks=extra + 4)
    st = FullState(w, d)
    return w, d, st


@pytest.mark.parametrize("name", sorted(CASES))
def test_shared_prefix_decode_parity(name):
    w, d, st = _family(name)
    try:
        k = P.block_table_common_prefix(st.pool.handle, st.seqs)
        assert k == st.bm.common_prefix(st.oseqs) == w.prefix_len // w.block_size
        q = wl.q_bits(w)
        plain, ot, ol = st.decode(st.seqs, st.oseqs, q)
        ref = st.reference(q, ot, ol)
        st.check(plain, ref)
        for splits in (0, 1, 7):
            got, _, _ = st.decode(st.seqs, st.oseqs, q, shared=k, splits=splits)
            st.check(got, ref)
            assert np.abs(got - plain).max() <= 2 * TOL[w.kv_dtype], splits
        # a shorter shared run than the common one is as valid
        if k > 1:
            got, _, _ = st.decode(st.seqs, st.oseqs, q, shared=k // 2)
            st.check(got, ref)
    finally:
        st.close()


@pytest.mark.parametrize("scale_mult", [-1.0, 0.0])
@pytest.mark.parametrize("name", ["bf16_g4", "f16_mha", "fp8_g8", "f32_d64"])
def test_shared_prefix_negative_and_zero_scale(name, scale_mult):
    """The prefix pass works with the scale's magnitude and moves its sign
    into the queries; a negative scale (softmax of the negated scores) and a
    zero one (uniform weights) still give the oracle's attention."""
    w, d, st = _family(name)
    try:
        k = P.block_table_common_prefix(st.pool.handle, st.seqs)
        assert k > 0
        q = wl.q_bits(w)
        scale = scale_mult / math.sqrt(w.head_dim)
        got, ot, ol = st.decode(st.seqs, st.oseqs, q, shared=k, scale=scale)
        st.check(got, st.reference(q, ot, ol, scale=scale))
    finally:
        st.close()


def _reference_skipping(st, q, tables, lens):
    """The decode's result when table entries outside the pool are empty
    blocks whose tokens are skipped (the decode's documented reading of such
    entries): per row, KV head and query head, the oracle's partial over the
    attended tokens of each real block, joined by the oracle's log-sum-exp
    merge."""
    from oracle.attention import lse_merge, partial_attention
    from oracle.pool import bits_to_f64
    w, pool, bs = st.w, st.opool, st.w.block_size
    qf = bits_to_f64(q, w.q_dtype)
    B, Hq, D = qf.shape
    G = Hq // w.num_kv_heads
    scale = 1.0 / math.sqrt(w.head_dim)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(lens[b])
        for g in range(w.num_kv_heads):
            parts = {h: [] for h in range(g * G, (g + 1) * G)}
            for j in range(-(-L // bs)):
                blk = int(tables[b, j])
                if blk < 0 or blk >= pool.num_blocks:
                    continue
                n = min(bs, L - j * bs)
                K = pool.values("k", 0, [blk], g)[:n]
                V = pool.values("v", 0, [blk], g)[:n]
                for h in parts:
                    parts[h].append(partial_attention(qf[b, h], K, V, scale))
            for h, pr in parts.items():
                if pr:
                    out[b, h] = lse_merge(pr)
    return out


@pytest.mark.parametrize("name", ["bf16_g4", "fp8_g8", "bf16_bs128_d64"])
def test_shared_prefix_short_rows_and_empty_blocks(name):
    # Rows that end inside the shared run (at a sub-tile edge, inside a
    # sub-tile, near its start, at 0), and entries of the shared run that are
    # not real blocks (the same in every row, as the contract asks), which
    # make the prefix pass mask sub-tiles before the end of its chunk.
    w, d, st = _family(name)
    try:
        k = P.block_table_common_prefix(st.pool.handle, st.seqs)
        kT = k * w.block_size
        q = wl.q_bits(w)

        def short(tables, lens):
            for r, L in zip(range(1, len(lens), 2), (kT - 5, 32, 3, 0, kT - 1)):
                lens[r] = max(0, min(L, kT))
            return tables, lens

        for splits in (0, 7):
            got, ot, ol = st.decode(st.seqs, st.oseqs, q, shared=k, splits=splits, edit=short)
            assert (ol < kT).any()
            st.check(got, st.reference(q, ot, ol))

        def holes(tables, lens):
            for j in sorted({1, k // 2, k - 1}):
                tables[:, j] = -1
            return tables, lens

        got, ot, ol = st.decode(st.seqs, st.oseqs, q, shared=k, edit=holes)
        ref = _reference_skipping(st, q, ot, ol)
        st.check(got, ref)
        # the ordinary decode reads the same entries the same way
        plain, _, _ = st.decode(st.seqs, st.oseqs, q, edit=holes)
        st.check(plain, ref)
    finally:
        st.close()


def test_shared_prefix_after_branch_step():
    # fork a branch per sequence, append one token to each (copy-on-write of
    # the shared partial last blocks), decode the branches reading their
    # common prefix once
    import torch
    from gpu_state import to_dev
    w, d, st = _family("bf16_g4", extra=2 * CASES["bf16_g4"].batch)
    h = st.pool.handle
    try:
        branches = P.block_table_fork_batch(h, st.seqs).tolist()
        obranches = [st.bm.fork(o) for o in st.oseqs]
        assert branches == obranches
        slots, cows = P.block_table_append_batch(h, branches)
        oslots, ocows = st.bm.append_batch(obranches)
        assert slots.tolist() == oslots and [tuple(c) for c in cows.tolist()] == ocows
        if len(ocows):
            P.kv_pool_copy_blocks(h, torch.from_numpy(np.ascontiguousarray(cows)).cuda(), len(cows))
            st.opool.copy_blocks(ocows)
        kb, vb, qb = wl.step_tokens_bits(w, 0)
        P.paged_kv_append(h, 0, to_dev(kb), to_dev(vb), w.src_dtype, torch.from_numpy(slots).cuda(), w.batch)
        st.opool.append(0, kb, vb, w.src_dtype, oslots)
        k = P.block_table_common_prefix(h, branches)
        assert k == st.bm.common_prefix(obranches) == w.prefix_len // w.block_size
        got, ot, ol = st.decode(branches, obranches, qb, shared=k)
        st.check(got, st.reference(qb, ot, ol))
    finally:
        st.close()


def test_shared_prefix_argument_checks():
    w, d, st = _family("bf16_g4")
    try:
        import torch
        B = w.batch
        q = torch.zeros((B, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
        out = torch.zeros((B, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        t = torch.zeros((B, 20), dtype=torch.int32, device="cuda")
        ln = torch.zeros(B, dtype=torch.int32, device="cuda")
        a = P.make_decode_args(0, B, w.num_q_heads, 20, q, "bf16", t, ln, 0.1, out, shared_prefix_blocks=21)
        with pytest.raises(P.PagedKVError):
            P.paged_attention_workspace_size(st.pool.handle, a)
        a = P.make_decode_args(0, B, w.num_q_heads, 20, q, "bf16", t, ln, 0.1, out, sliding_window=8,
                               shared_prefix_blocks=2)
        with pytest.raises(P.PagedKVError):
            P.paged_attention_workspace_size(st.pool.handle, a)
        a = P.make_decode_args(0, B, w.num_q_heads, 20, q, "bf16", t, ln, 0.1, out, num_splits=1,
                               shared_prefix_blocks=2)
        assert P.paged_attention_workspace_size(st.pool.handle, a) > 0
    finally:
        st.close()
