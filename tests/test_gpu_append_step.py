"""paged_kv_append_step: one token per row with the rows' device-resident
tables and lengths updated in the same kernel.  After every few steps the
device tables and lengths must equal the host block manager's export bit for
bit, the appended K/V must equal the oracle pool's, and the decode over the
device metadata must match the oracle.  Slots come alternately from a
page-locked host buffer and from device memory; one case forks every
sequence first so that each step copies the shared partial blocks."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_406_amd as P
import workloads as wl
from oracle import decode_attention
from oracle_state import OracleState, fp8_channel_scales
from gpu_state import GpuState, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-3, "f16": 2e-3, "bf16": 2e-3, "fp8": 3e-2}
CASES = {
    "gqa8_bf16": wl.scaled(wl.WORKLOADS["c3"], batch=10, num_q_heads=16, num_kv_heads=2,
                           lengths_args=(60.0, 0.8, 1, 400)),
    "mha_f16_bs32": wl.scaled(wl.WORKLOADS["c2"], batch=5, num_q_heads=2, num_kv_heads=2,
                              lengths_args=(1, 300), block_size=32),
    "gqa8_fp8": wl.scaled(wl.WORKLOADS["c5_fp8"], batch=3, num_q_heads=16, num_kv_heads=2,
                          lengths_kind="uniform", lengths_args=(1, 500), pool_blocks=0),
}
STEPS = 40


def _run(name, fork):
    w = CASES[name]
    d = wl.draw(w, extra_blocks=4 * w.batch * (STEPS // w.block_size + 2))
    scales = fp8_channel_scales(w, d) if w.kv_dtype == "fp8" else None
    ost = OracleState(w, d, scales=scales)
    gst = GpuState(w, d, scales=scales)
    h = gst.pool.handle
    try:
        seqs, oseqs = gst.seqs, ost.seqs
        if fork:
            seqs = P.block_table_fork_batch(h, seqs).tolist()
            oseqs = [ost.bm.fork(o) for o in oseqs]
            assert seqs == oseqs
        B = w.batch
        mb = max(len(ost.bm.table(o)) for o in oseqs) + STEPS // w.block_size + 2
        tables, lens = P.block_table_export(h, seqs, mb)
        td, ld = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
        pinned = torch.empty(B, dtype=torch.int64, pin_memory=True)
        n_cow = 0
        for step in range(STEPS):
            slots, cows = P.block_table_append_batch(h, seqs)
            oslots, ocows = ost.bm.append_batch(oseqs)
            assert slots.tolist() == oslots and [tuple(c) for c in cows.tolist()] == ocows
            if len(cows):
                n_cow += len(cows)
                P.kv_pool_copy_blocks(h, torch.from_numpy(np.ascontiguousarray(cows)).cuda(), len(cows))
                ost.pool.copy_blocks(ocows)
            kb, vb, _ = wl.step_tokens_bits(w, step)
            if step % 2 == 0:
                torch.cuda.synchronize()          # the previous step's kernel has read the buffer
                pinned.numpy()[:] = slots
                src = pinned
            else:
                src = torch.from_numpy(slots).cuda()
            P.paged_kv_append_step(h, 0, to_dev(kb), to_dev(vb), w.src_dtype, src, B, td, ld, mb)
            ost.pool.append(0, kb, vb, w.src_dtype, oslots)
            if step % 8 == 7:
                torch.cuda.synchronize()
                ht, hl = P.block_table_export(h, seqs, mb)
                assert np.array_equal(td.cpu().numpy(), ht), step
                assert np.array_equal(ld.cpu().numpy(), hl), step
        torch.cuda.synchronize()
        if fork:
            # each shared partly filled last block is copied once, at its first append
            assert n_cow == sum(1 for L in d.lengths if int(L) % w.block_size)
        # appended K/V bits equal the oracle pool's
        k, v = gst.pool_logical()
        ht, hl = P.block_table_export(h, seqs, mb)
        bs = w.block_size
        for r in range(B):
            for pos in range(int(hl[r]) - STEPS, int(hl[r])):
                blk, off = ht[r][pos // bs], pos % bs
                assert np.array_equal(k[0, blk, :, off], ost.pool.k[0][blk, :, off]), (r, pos)
                assert np.array_equal(v[0, blk, :, off], ost.pool.v[0][blk, :, off]), (r, pos)
        # decode over the device metadata
        _, _, qb = wl.step_tokens_bits(w, STEPS)
        out = torch.full((B, w.num_q_heads, w.head_dim), -7.0, dtype=torch.float32, device="cuda")
        scale = 1.0 / math.sqrt(w.head_dim)
        a = P.make_decode_args(0, B, w.num_q_heads, mb, to_dev(qb), w.q_dtype, td, ld, scale, out)
        nbytes = P.paged_attention_workspace_size(h, a)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        a.workspace, a.workspace_bytes = ws.data_ptr(), nbytes
        P.paged_attention_decode(h, a)
        torch.cuda.synchronize()
        ot, ol = ost.bm.export(oseqs, mb)
        ref = decode_attention(ost.pool, 0, qb, w.q_dtype, ot, ol, scale, 0)
        assert np.abs(out.cpu().numpy().astype(np.float64) - ref).max() <= TOL[w.kv_dtype]
    finally:
        gst.close()


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_step_keeps_device_tables_exact(name):
    _run(name, fork=False)


def test_append_step_with_copy_on_write():
    _run("gqa8_bf16", fork=True)


def test_append_step_argument_checks():
    w = CASES["gqa8_bf16"]
    d = wl.draw(w)
    gst = GpuState(w, d)
    try:
        h = gst.pool.handle
        k = torch.zeros((2, w.num_kv_heads, w.head_dim), dtype=torch.int16, device="cuda")
        t = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
        ln = torch.zeros(2, dtype=torch.int32, device="cuda")
        pageable = np.zeros(2, dtype=np.int64)
        with pytest.raises(P.PagedKVError):     # slots neither device nor page-locked memory
            P.paged_kv_append_step(h, 0, k, k, w.src_dtype, pageable.ctypes.data, 2, t, ln, 4)
        with pytest.raises(P.PagedKVError):
            P.paged_kv_append_step(h, 0, k, k, w.src_dtype, torch.zeros(2, dtype=torch.int64, device="cuda"),
                                   2, t, ln, 0)
        torch.cuda.synchronize()
    finally:
        gst.close()
