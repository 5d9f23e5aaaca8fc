"""paged_attention_decode_static (for callers that cannot allocate device
memory) against paged_attention_decode with a caller-owned workspace.

Both run the same kernels on the same arguments, so their outputs must be
identical bit for bit; both are also held to the oracle at the usual bar
(2e-3 max-abs, bf16 KV).  Two calls in a row, the second with a smaller
input, then a shared-prefix call (the workspace then also holds the prefix
partials) and fused-append steps (bf16 and FP8 pools); a call needing more
than the static workspace, and a call that brings its own workspace, are
refused on the host before any launch.
"""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_406_amd as P
import workloads as wl
from oracle import decode_attention
from oracle_state import OracleState
from gpu_state import GpuState, to_dev, out_to_f64
from test_gpu_full_size import FullState

pytestmark = pytest.mark.gpu

C3 = wl.WORKLOADS["c3"]
BIG = wl.scaled(C3, batch=24, num_q_heads=32, num_kv_heads=4, lengths_args=(300.0, 0.8, 1, 1500))
SMALL = wl.scaled(C3, batch=5, num_q_heads=16, num_kv_heads=2, lengths_args=(60.0, 0.8, 1, 400))
PREFIX = wl.scaled(wl.WORKLOADS["c4"], batch=12, prefix_len=100, lengths_args=(0, 70))


def _args(w, tables, lens, q, out, splits=0, shared=0):
    qd = to_dev(q)
    td = torch.from_numpy(np.ascontiguousarray(tables, dtype=np.int32)).cuda()
    ld = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).cuda()
    return P.make_decode_args(0, len(lens), w.num_q_heads, tables.shape[1], qd, w.q_dtype, td, ld,
                              1.0 / math.sqrt(w.head_dim), out, "f32", num_splits=splits,
                              shared_prefix_blocks=shared)


def _both(pool, w, tables, lens, q, splits=0, shared=0):
    """(output with a caller-owned workspace, output with the static one)."""
    B = len(lens)
    outs = []
    for static in (False, True):
        out = torch.full((B, w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        a = _args(w, tables, lens, q, out, splits, shared)
        if static:
            P.paged_attention_decode_static(pool.handle, a)
        else:
            nbytes = P.paged_attention_workspace_size(pool.handle, a)
            assert 0 < nbytes <= P.PKV_STATIC_WORKSPACE_BYTES
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            a.workspace, a.workspace_bytes = ws.data_ptr(), nbytes
            a._refs = a._refs + (ws,)
            P.paged_attention_decode(pool.handle, a)
        torch.cuda.synchronize()
        outs.append(out_to_f64(out, "f32"))
    return outs


@pytest.mark.parametrize("w", [BIG, SMALL], ids=["first_call_larger", "second_call_smaller"])
def test_static_workspace_decode_matches(w):
    d = wl.draw(w)
    ost = OracleState(w, d)
    gst = GpuState(w, d)
    try:
        tables, lens = ost.export()
        q = wl.q_bits(w)
        ref = decode_attention(ost.pool, 0, q, w.q_dtype, tables, lens, 1.0 / math.sqrt(w.head_dim))
        for splits in (0, 5):
            with_ws, static = _both(gst.pool, w, tables, lens, q, splits)
            assert np.array_equal(static, with_ws), (w.batch, splits)
            assert np.abs(static - ref).max() <= 2e-3
    finally:
        gst.close()


def test_static_workspace_shared_prefix_decode_matches():
    w = PREFIX
    d = wl.draw(w, extra_blocks=4)
    st = FullState(w, d)
    try:
        k = P.block_table_common_prefix(st.pool.handle, st.seqs)
        assert k == w.prefix_len // w.block_size
        mb = max(len(st.bm.table(o)) for o in st.oseqs)
        tables, lens = P.block_table_export(st.pool.handle, st.seqs, mb)
        otables, olens = st.bm.export(st.oseqs, mb)
        assert np.array_equal(tables, otables) and np.array_equal(lens, olens)
        q = wl.q_bits(w)
        with_ws, static = _both(st.pool, w, tables, lens, q, shared=k)
        assert np.array_equal(static, with_ws)
        st.check(static, st.reference(q, otables, olens))
    finally:
        st.close()


@pytest.mark.parametrize("name", ["gqa8_bf16", "gqa8_fp8"])
def test_static_workspace_fused_append_matches(name):
    # the fused append through both entry points, on two identical states:
    # outputs, device tables and lengths, and both pools bit for bit, over
    # two consecutive steps
    from test_gpu_fused_append import CASES, FusedState, TOL
    w = CASES[name]
    d = wl.draw(w, extra_blocks=w.batch * 2)
    a, b = FusedState(w, d), FusedState(w, d)
    try:
        for t in range(2):
            got_ws, ref = a.step(t, 0)
            got_static, _ = b.step(t, 0, static=True)
            assert np.array_equal(got_static, got_ws), (name, t)
            assert np.abs(got_static - ref).max() <= TOL[w.kv_dtype]
            assert torch.equal(a.d_tables, b.d_tables) and torch.equal(a.d_lens, b.d_lens)
            assert torch.equal(a.pool.k_cache, b.pool.k_cache) and torch.equal(a.pool.v_cache, b.pool.v_cache)
    finally:
        a.close()
        b.close()


def test_static_workspace_refusals_on_the_host():
    w = wl.scaled(C3, batch=2, num_q_heads=16, num_kv_heads=1, lengths_kind="fixed", lengths_args=(40, 3))
    d = wl.draw(w)
    gst = GpuState(w, d)
    try:
        tables, lens = gst.export()
        q = wl.q_bits(w)
        out = torch.zeros((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        # 16384 ranges x 2 slots x 16 heads x 128 dims x 4 bytes = 256 MiB of partials
        a = _args(w, tables, lens, q, out, splits=16384)
        assert P.paged_attention_workspace_size(gst.pool.handle, a) > P.PKV_STATIC_WORKSPACE_BYTES
        with pytest.raises(P.PagedKVError) as e:
            P.paged_attention_decode_static(gst.pool.handle, a)
        assert e.value.status == P.PKV_E_UNSUPPORTED and "static workspace" in str(e.value)
        # a caller-owned workspace is refused: this call uses the static one
        ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
        a = _args(w, tables, lens, q, out, splits=0)
        a.workspace, a.workspace_bytes = ws.data_ptr(), 1 << 20
        with pytest.raises(P.PagedKVError) as e:
            P.paged_attention_decode_static(gst.pool.handle, a)
        assert e.value.status == P.PKV_E_INVAL
        torch.cuda.synchronize()
        assert (out == 0).all()          # nothing was launched
    finally:
        gst.close()
