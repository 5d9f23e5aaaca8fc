"""Paged decode-attention benchmark on one MI355X.

One step is one pass of the whole decode hot path over one batch:
  1. host: reserve one slot per sequence (block_table_append_batch: on-demand
     blocks, copy-on-write of shared partial blocks),
  2. paged_attention_decode with the fused append: the range-split decode of
     the cached tokens, whose last workgroups store the new tokens into their
     slots (FP8 pools: the merge stores them), then the log-sum-exp merge,
     which folds in the new token and writes the row's table entry and
     length (device-resident tables; the slots are read from the page-locked
     buffer the host wrote them to).  Forked families, whose tables change
     every step, first export and upload the step's metadata and copy the
     copy-on-write blocks.  --unfused runs paged_kv_append_step (or
     paged_kv_append) before a plain decode instead.
Inputs (the cache and every step's q, k, v) are resident in HBM before the
timed region starts.  Several independently placed copies of the cache are
rotated so the working set is several times the 256 MB Infinity Cache.

Prints one JSON line.  ``value`` is KV GB/s over the whole step (algorithmic
bytes of the decode / step time).  ``roofline`` is the dominant kernel
(decode_append_kernel, or decode_kernel for FP8 and unfused runs) alone: its
algorithmic bytes (everything the decode must move except the output, which
the merge writes, plus the new tokens it stores) over its own launch
duration, recorded by the kernel's start and end events on the launch
stream; ``roofline.call_*`` and ``decode_ms`` / ``decode_GBps`` are the whole
call (decode + merge, with the append's bytes).  With a shared prefix the three kernels of
the call are one unit and ``roofline`` is the call.  With the default
workload (c3), ``targets`` holds the same figures for the 128K-context
workloads (bf16 and FP8 KV), measured by shorter runs in the same process.
``cpu_baseline`` is the CPU oracle timed on a bounded sample of the same
workload.

    python bench.py [--steps K] [--warmup W] [--workload c3] [--targets c5,c5_fp8]
"""
import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "paged decode attention: KV GB/s achieved and % of HBM peak; seq·heads/s"
HBM_PEAK_GBS = 8000.0
WORKLOAD_NAMES = {
    "c2": "llama2-7b-mha-decode-layer (B=64, 32/32 heads, d=128, fp16 KV, block 16)",
    "c2_bs32": "llama2-7b-mha-decode-layer (B=64, 32/32 heads, d=128, fp16 KV, block 32)",
    "c2_bs128": "llama2-7b-mha-decode-layer (B=64, 32/32 heads, d=128, fp16 KV, block 128)",
    "c3": "llama2-70b-gqa-decode-layer (B=128, 64/8 heads, d=128, bf16 KV, block 16, lognormal lengths)",
    "c4": "prefix-shared-decode (B=256 forks of a 2000-token prefix + private suffix U[1,512], 32/8 heads, "
          "d=128, bf16 KV, block 16; each step forks a branch per sequence, appends with copy-on-write, "
          "decodes the branches)",
    "c5": "long-context-128k-decode (B=4, L=131072, 64/8 heads, d=128, bf16 KV, block 16)",
    "c5_fp8": "long-context-128k-decode-fp8 (B=4, L=131072, 64/8 heads, d=128, FP8-E4M3 KV, block 16)",
    "c5w": "long-context-128k-window-4096 (B=4, L=131072, 64/8 heads, d=128, bf16 KV, block 16)",
}


# HBM bytes per launch of the dominant kernel (decode_append_kernel, or
# decode_kernel for FP8; read + write), from rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE runs scaled by what the same counters read for a
# plain 1 GiB device copy (FETCH x 2.0, WRITE x 1.0).  Each entry holds for the
# kernel source it was measured on (kernels_sha()); for any other source the
# figure is not reported.
MEASURED_TRAFFIC = {
    "c3": (511.0e6, "f2f9a337c66b7863"),
    "c2": (1985.8e6, "f2f9a337c66b7863"),
    "c2_bs128": (2047.5e6, "f2f9a337c66b7863"),
    "c5": (2155.3e6, "f2f9a337c66b7863"),
    "c5_fp8": (1080.5e6, "f2f9a337c66b7863"),
    "c5w": (72.1e6, "f2f9a337c66b7863"),
    "c4": (373.6e6, "f2f9a337c66b7863"),   # the whole call: prefix, suffix and merge kernels
}


def kernels_sha():
    """sha256 prefix of the device source the decode is built from (kernels.hip
    and the headers beside it)."""
    import hashlib
    csrc = os.path.join(ROOT, "paged_kv_cache_406_amd", "csrc")
    h = hashlib.sha256()
    for name in ["kernels.hip"] + sorted(f for f in os.listdir(csrc) if f.endswith(".h")):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


class HipEvent:
    """A timing event created with flags torch does not expose, through the
    HIP runtime the process already holds (torch's: found in the process's
    mapped libraries, so that no second runtime is loaded).

    hipEventDisableSystemFence: the kernel that records the event does not
    end with a system-scope fence (cache write-back and invalidation), which
    the HIP documentation recommends for timing; the host still learns that
    the work before the event has finished."""

    DISABLE_SYSTEM_FENCE = 0x20000000
    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64.so" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded")
            hip = ctypes.CDLL(path)
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self, flags=DISABLE_SYSTEM_FENCE):
        import ctypes
        self._ct = ctypes
        self.handle = ctypes.c_void_p()
        rc = self._runtime().hipEventCreateWithFlags(ctypes.byref(self.handle), flags)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    @property
    def address(self):
        return self.handle.value

    def synchronize(self):
        rc = self._runtime().hipEventSynchronize(self.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventSynchronize failed ({rc})")

    def elapsed_time(self, end):
        ms = self._ct.c_float()
        rc = self._runtime().hipEventElapsedTime(self._ct.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.handle:
            self._hip.hipEventDestroy(self.handle)


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def unique_kv_bytes(w, lengths):
    """KV bytes of the distinct tokens one decode of the prefix-shared workload
    reads: the shared prefix once, every private suffix once."""
    eb = wl.ELEM_BYTES[w.kv_dtype]
    per_tok = w.num_kv_heads * 2 * w.head_dim * eb
    return (w.prefix_len + sum(int(L) - w.prefix_len for L in lengths)) * per_tok


def out_bytes(w, lengths):
    """The fp32 output of one decode call (written by merge_kernel for split
    sequences)."""
    return len(lengths) * w.num_q_heads * w.head_dim * 4


def decode_bytes(w, lengths):
    """Algorithmic bytes of one decode call: KV of every attended token, q,
    the fp32 output, the block-table entries read, the context lengths and
    (FP8) the per-channel scales."""
    eb = wl.ELEM_BYTES[w.kv_dtype]
    qb = wl.ELEM_BYTES[w.q_dtype]
    bs = w.block_size
    kv = tables = 0
    for L in lengths:
        L = int(L)
        lo = max(0, L - w.window) if w.window else 0
        kv += (L - lo) * w.num_kv_heads * 2 * w.head_dim * eb
        tables += (-(-L // bs) - lo // bs) * 4 if L > lo else 0
    B = len(lengths)
    total = kv + B * w.num_q_heads * w.head_dim * (qb + 4) + tables + B * 4
    if w.kv_dtype == "fp8":
        total += 2 * w.num_kv_heads * w.head_dim * 4
    return total, kv


def new_token_bytes(w, batch):
    """The new tokens of a fused call: each row's K and V read in the source
    dtype and written into the pool."""
    return batch * w.num_kv_heads * w.head_dim * 2 * (wl.ELEM_BYTES[w.src_dtype] + wl.ELEM_BYTES[w.kv_dtype])


def append_bytes(w, batch):
    """Algorithmic bytes of a fused call's append: the new tokens, each row's
    slot read (8 B), its length read and written and its table entry written
    (12 B)."""
    return new_token_bytes(w, batch) + batch * (8 + 12)


class Replica:
    """One independently placed copy of the workload's cache."""

    def __init__(self, P, torch, w, d, order, kv_cache, max_blocks, scales):
        self.P, self.torch, self.w = P, torch, w
        self.pool = P.TorchKVPool(w.num_layers, w.num_kv_heads, w.head_dim, w.block_size,
                                  d.num_blocks, w.kv_dtype, free_order=order, **scales)
        h = self.pool.handle
        self.seqs = []
        if w.lengths_kind == "prefix":
            # one root holds the shared prefix; every sequence is a fork of it
            # (refcount B on the prefix blocks) with its own suffix
            root = P.block_table_alloc(h)
            slots, _ = P.block_table_append(h, root, w.prefix_len)
            kd, vd = kv_cache["prefix"]
            P.paged_kv_append(h, 0, kd, vd, w.src_dtype, torch.from_numpy(slots).cuda(), w.prefix_len)
            self.seqs = P.block_table_fork_batch(h, [root] * len(d.lengths)).tolist()
            P.block_table_free(h, root)
            for b, s in enumerate(self.seqs):
                n = int(d.suffix[b])
                slots, cows = P.block_table_append(h, s, n)
                if cows:
                    pairs = torch.tensor(cows, dtype=torch.int32).cuda()
                    P.kv_pool_copy_blocks(h, pairs, len(cows))
                kd, vd = kv_cache[b]
                P.paged_kv_append(h, 0, kd, vd, w.src_dtype, torch.from_numpy(slots).cuda(), n)
        else:
            for b, L in enumerate(d.lengths):
                s = P.block_table_alloc(h)
                slots, _ = P.block_table_append(h, s, int(L))
                kd, vd = kv_cache[b]
                P.paged_kv_append(h, 0, kd, vd, w.src_dtype, torch.from_numpy(slots).cuda(), int(L))
                self.seqs.append(s)
        self.seq_arr = np.asarray(self.seqs, dtype=np.int32)
        B = len(self.seqs)
        self.max_blocks = max_blocks
        # device metadata block: slots (int64 [B]), copy pairs (int32 [B][2]),
        # tables (int32 [B][max_blocks]), lens (int32 [B])
        self.n_meta = 2 * B + 2 * B + B * max_blocks + B
        self.meta = torch.empty(self.n_meta, dtype=torch.int32, device="cuda")
        self.d_slots = self.meta[: 2 * B].view(torch.int64)
        self.d_cows = self.meta[2 * B: 4 * B]
        self.d_tables = self.meta[4 * B: 4 * B + B * max_blocks]
        self.d_lens = self.meta[4 * B + B * max_blocks:]
        self.lengths = np.array([int(x) for x in d.lengths], dtype=np.int64)


def build_state(args, P, torch):
    w = wl.WORKLOADS[args.workload]
    steps_total = args.steps + args.warmup
    # headroom: every sequence may take one new block per block_size steps
    extra = w.batch * (-(-steps_total // w.block_size) + 1)
    if w.lengths_kind == "prefix":
        extra = 2 * w.batch      # each step's branches take one block each, freed at its end
    d = wl.draw(w, extra_blocks=extra)
    bytes0, kv0 = decode_bytes(w, d.lengths)
    if w.lengths_kind == "prefix":
        kv0 = unique_kv_bytes(w, d.lengths)
    reps = args.replicas or max(1, math.ceil(2 * 2 ** 30 / kv0))
    log(f"workload {w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim} "
        f"bs={w.block_size} kv={w.kv_dtype} pool={d.num_blocks} blocks, KV bytes/call={kv0/1e9:.3f} GB, "
        f"replicas={reps}")
    t0 = time.time()
    kv_cache = {}
    absmax_k = np.zeros((w.num_kv_heads, w.head_dim), np.float32)
    absmax_v = np.zeros((w.num_kv_heads, w.head_dim), np.float32)
    streams = [(b, (1, b), int(L)) for b, L in enumerate(d.lengths)]
    if w.lengths_kind == "prefix":
        streams = [("prefix", (3,), w.prefix_len)] + [(b, (1, b), int(n)) for b, n in enumerate(d.suffix)]
    # the streams are drawn in parallel (NumPy releases the interpreter lock
    # in the draws and conversions); results are used in stream order
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        drawn = list(ex.map(lambda s: wl.kv_tokens_bits(w, s[1], s[2]), streams))
    for (b, stream_id, L), (kb, vb) in zip(streams, drawn):
        if w.kv_dtype == "fp8":
            absmax_k = np.maximum(absmax_k, np.abs(wl.bits_as_f32(kb, w.src_dtype)).max(axis=0))
            absmax_v = np.maximum(absmax_v, np.abs(wl.bits_as_f32(vb, w.src_dtype)).max(axis=0))
        tdt = np.int16 if kb.dtype == np.uint16 else np.int32
        kv_cache[b] = (torch.from_numpy(kb.view(tdt)).cuda(), torch.from_numpy(vb.view(tdt)).cuda())
    del drawn
    scales = {}
    if w.kv_dtype == "fp8":
        ks, _ = wl.fp8_scales(absmax_k)
        vs, _ = wl.fp8_scales(absmax_v)
        scales = dict(k_scale=ks[None], v_scale=vs[None])
    log(f"generated K/V in {time.time() - t0:.1f}s")
    max_len = int(max(d.lengths)) + steps_total + 1
    max_blocks = -(-max_len // w.block_size) + 1
    reps_list = []
    for r in range(reps):
        order = np.random.default_rng([w.seed, 5, r]).permutation(d.num_blocks).astype(np.int32)
        reps_list.append(Replica(P, torch, w, d, order, kv_cache, max_blocks, scales))
    torch.cuda.synchronize()
    del kv_cache
    log(f"built {reps} replicas in {time.time() - t0:.1f}s")
    # per-step new tokens and queries, resident on the device
    steps = []
    for t in range(steps_total):
        kb, vb, qb = wl.step_tokens_bits(w, t)
        tdt = np.int16 if kb.dtype == np.uint16 else np.int32
        qdt = np.int16 if qb.dtype == np.uint16 else np.int32
        steps.append((torch.from_numpy(kb.view(tdt)).cuda(), torch.from_numpy(vb.view(tdt)).cuda(),
                      torch.from_numpy(qb.view(qdt)).cuda()))
    host_scales = None
    if w.kv_dtype == "fp8":
        host_scales = (scales["k_scale"], scales["v_scale"])
    return w, d, reps_list, steps, host_scales


def run(args):
    import torch
    import paged_kv_cache_406_amd as P

    torch.cuda.set_device(0)
    w, d, reps, steps, scales = build_state(args, P, torch)
    B = w.batch
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    out = torch.empty((B, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(w.head_dim)
    # shared-prefix decode for forked families: the prefix's full blocks
    shared0 = 0
    if w.lengths_kind == "prefix" and not args.no_shared_prefix:
        shared0 = w.prefix_len // w.block_size
    # the decode call appends the step's token itself (fused append) unless
    # --unfused asks for the separate append kernel
    fused = not args.unfused
    fuse_kw = lambda t, slots: (dict(new_k=steps[t][0], new_v=steps[t][1], new_dtype=w.src_dtype,
                                     new_slots=slots) if fused else {})
    args0 = P.make_decode_args(0, B, w.num_q_heads, reps[0].max_blocks, steps[0][2], w.q_dtype,
                               reps[0].d_tables, reps[0].d_lens, scale, out, "f32",
                               sliding_window=w.window, num_splits=args.splits, shared_prefix_blocks=shared0,
                               **fuse_kw(0, reps[0].d_slots))
    ws_bytes = P.paged_attention_workspace_size(reps[0].pool.handle, args0)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    # pinned staging ring for the per-step metadata; a buffer is rewritten only
    # once the upload that last read it has run
    RING = 16   # two sampling periods: the host waits on a step at least 8 behind
    ring = []
    for _ in range(RING):
        buf = torch.empty(reps[0].n_meta, dtype=torch.int32, pin_memory=True)
        buf.numpy().fill(0)     # touched once here, not first inside a timed step
        ring.append((buf, buf.numpy()))
    mb = reps[0].max_blocks
    meta_bytes = reps[0].n_meta * 4
    prefix = w.lengths_kind == "prefix"
    n_total = args.warmup + args.steps

    def unique_or_logical(lens_list):
        logical = float(np.mean([decode_bytes(w, L)[0] for L in lens_list]))
        if not prefix:
            return logical, logical
        # HBM bound on the distinct bytes: the shared prefix is one set of blocks
        # (its repeated reads are served by the caches); the other terms as usual
        kv_logical = float(np.mean([decode_bytes(w, L)[1] for L in lens_list]))
        uniq = logical - kv_logical + float(np.mean([unique_kv_bytes(w, L) for L in lens_list]))
        return logical, uniq

    resident = not prefix and not args.full_metadata
    # per-step decode arguments and timing events, made before the timed loop;
    # with the fused append a resident batch's slots are read from the
    # page-locked staging buffer, otherwise from the uploaded metadata
    dec_args = []
    for t in range(n_total):
        rep = reps[t % len(reps)]
        slots_src = ring[t % RING][0] if resident else rep.d_slots
        dec_args.append(P.make_decode_args(0, B, w.num_q_heads, mb, steps[t][2], w.q_dtype, rep.d_tables,
                                           rep.d_lens, scale, out, "f32", sliding_window=w.window,
                                           num_splits=args.splits, workspace=ws, workspace_bytes=ws_bytes,
                                           shared_prefix_blocks=shared0, **fuse_kw(t, slots_src)))
    # Every TIME_EVERY-th step's decode is timed by its own kernels (attention
    # start/end, merge start/end), with events that skip the system-scope
    # fence (see HipEvent); an event still costs a little, so only a sample
    # of steps carries them.  The last event of a sampled step also tells the
    # host that the kernels up to that step have finished reading the
    # page-locked staging buffers (staging ring reuse).  The first timed step
    # is not sampled (unless it is the only one): a call with events costs
    # the host tens of microseconds more, the first one over a hundred, and
    # at the start of the timed region the device would wait for them.
    TIME_EVERY = 8
    PHASE = (args.warmup + 1) % TIME_EVERY
    sample_steps = set(range(PHASE, n_total, TIME_EVERY))
    if not any(t >= args.warmup for t in sample_steps):
        sample_steps.add(args.warmup)
    sampled = {t: [HipEvent() for _ in range(4)] for t in sorted(sample_steps)}
    torch.cuda.synchronize()
    n_kernels = {}
    step_lens = {}
    # A steady batch keeps its tables resident on the device: one full export
    # and upload here, then each step's call (or paged_kv_append_step, unfused)
    # updates them with its token.  The forked branches of the prefix workload
    # change every step and are exported and uploaded every step.
    if resident:
        buf, npb = ring[0]
        for rep in reps:
            P.block_table_export(rep.pool.handle, rep.seq_arr, mb, tables_out=npb[4 * B: 4 * B + B * mb].reshape(B, mb),
                                 lens_out=npb[4 * B + B * mb:])
            P.kv_metadata_upload(rep.meta, buf, meta_bytes, sptr)
            torch.cuda.synchronize()

    def step(t, record):
        rep = reps[t % len(reps)]
        h = rep.pool.handle
        buf, npb = ring[t % RING]
        if t >= RING:
            # the oldest sampled step at or after t - RING: its end implies that
            # step t - RING's upload (the last reader of this buffer) has run,
            # and the host may stay several steps ahead of the device
            f = (t - RING) + (PHASE - (t - RING)) % TIME_EVERY
            sampled[f][3 if n_kernels[f] == 2 else 1].synchronize()
        slots_np = npb[: 2 * B].view(np.int64)
        cows_np = npb[2 * B: 4 * B].reshape(B, 2)
        tables_np = npb[4 * B: 4 * B + B * mb].reshape(B, mb)
        lens_np = npb[4 * B + B * mb:]
        if prefix:
            # a sampling branch per sequence: fork, append (copy-on-write of the
            # shared partial last block), decode, free
            seqs = P.block_table_fork_batch(h, rep.seq_arr)
        else:
            seqs = rep.seq_arr
            rep.lengths += 1
        _, cows = P.block_table_append_batch(h, seqs, slots_out=slots_np, cow_out=cows_np)
        kd, vd, _ = steps[t]
        if resident:
            if len(cows):
                raise RuntimeError("copy-on-write in a batch without forks")
            if not fused:
                # new K/V and the rows' tables and lengths in one kernel; the
                # slots are read from the page-locked buffer
                P.paged_kv_append_step(h, 0, kd, vd, w.src_dtype, buf, B, rep.d_tables, rep.d_lens, mb, sptr)
        else:
            P.block_table_export(h, seqs, mb, tables_out=tables_np, lens_out=lens_np)
            if fused:
                lens_np -= 1        # the cached tokens before the step's token, which the call adds
        if shared0:
            # the blocks the batch holds in common, read once by the decode
            k = P.block_table_common_prefix(h, seqs)
            if k != shared0:
                raise RuntimeError(f"common prefix {k} blocks, expected {shared0}")
            dec_args[t].shared_prefix_blocks = k
        if not resident:
            P.kv_metadata_upload(rep.meta, buf, meta_bytes, sptr)
            if len(cows):
                P.kv_pool_copy_blocks(h, rep.d_cows, len(cows), sptr)
            if not fused:
                P.paged_kv_append(h, 0, kd, vd, w.src_dtype, rep.d_slots, B, sptr)
        if t in sampled:
            n_kernels[t] = P.paged_attention_decode_timed(h, dec_args[t], [e.address for e in sampled[t]], sptr)
        else:
            P.paged_attention_decode(h, dec_args[t], sptr)
        if record:
            step_lens[t] = rep.lengths + 1 if prefix else rep.lengths.copy()
        if prefix:
            # host bookkeeping only: stream order keeps this step's kernels ahead
            # of any later reuse of the freed blocks
            P.block_table_free_batch(h, seqs)

    # no garbage-collector pass inside the timed loop: a full pass over this
    # process's objects takes tens of milliseconds.  Collected before the
    # warm-up, whose steps then bring the host's caches back.
    gc.collect()
    gc.freeze()
    gc.disable()
    log(f"warmup {args.warmup} steps")
    for t in range(args.warmup):
        step(t, False)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for t in range(args.warmup, args.warmup + args.steps):
        step(t, True)
    t_stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    # context: the same decodes back to back with two events around the
    # batch (no per-call events), each replica at its final state
    last_t = {}
    for t in range(args.warmup, args.warmup + args.steps):
        last_t[t % len(reps)] = t
    order = [last_t[r] for r in sorted(last_t)]
    n_b2b = max(len(order), 20)
    # plain decodes of the final state (a fused call would append again)
    b2b_args = {t: P.make_decode_args(0, B, w.num_q_heads, mb, steps[t][2], w.q_dtype, reps[t % len(reps)].d_tables,
                                      reps[t % len(reps)].d_lens, scale, out, "f32", sliding_window=w.window,
                                      num_splits=args.splits, workspace=ws, workspace_bytes=ws_bytes,
                                      shared_prefix_blocks=dec_args[t].shared_prefix_blocks)
                for t in order}
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for k in range(n_b2b):
        t = order[k % len(order)]
        P.paged_attention_decode(reps[t % len(reps)].pool.handle, b2b_args[t], sptr)
    b1.record(stream)
    torch.cuda.synchronize()
    b2b_ms = b0.elapsed_time(b1) / n_b2b
    if resident:
        # the resident tables must still equal the host block manager's
        for rep in reps:
            ht, hl = P.block_table_export(rep.pool.handle, rep.seq_arr, mb)
            dt = rep.d_tables.view(B, mb).cpu().numpy()
            dl = rep.d_lens.cpu().numpy()
            if not (np.array_equal(dt, ht) and np.array_equal(dl, hl)):
                raise RuntimeError("device-resident block tables differ from the host block manager")
    b2b_bytes = float(np.mean([unique_or_logical([step_lens[order[k % len(order)]]])[1] for k in range(n_b2b)]))
    gc.enable()
    gc.unfreeze()
    timed = [t for t in range(args.warmup, args.warmup + args.steps) if t in sampled]
    dec_ms = []      # the call: every kernel's duration
    kern_ms = []     # decode_kernel (with a shared prefix: prefix_kernel start to decode_kernel end)
    for t in timed:
        e = sampled[t]
        k0 = e[0].elapsed_time(e[1])
        ms = k0
        if n_kernels[t] == 2:
            ms += e[2].elapsed_time(e[3])
        dec_ms.append(ms)
        kern_ms.append(k0)
    step_ms = t_start.elapsed_time(t_stop) / args.steps
    all_lens = [step_lens[t] for t in range(args.warmup, args.warmup + args.steps)]
    avg_dec_ms = float(np.mean(dec_ms))

    logical_bytes, avg_bytes = unique_or_logical(all_lens)          # the whole timed region
    s_logical, s_bytes = unique_or_logical([step_lens[t] for t in timed])   # the sampled decodes
    log(f"step {step_ms:.4f} ms (host wall {1e3 * wall / args.steps:.4f} ms), decode kernels {avg_dec_ms:.4f} ms "
        f"(min {min(dec_ms):.4f}, max {max(dec_ms):.4f}, {len(dec_ms)} sampled steps; first kernel "
        f"{float(np.mean(kern_ms)):.4f} ms), back to back {b2b_ms:.4f} ms")
    value = avg_bytes / (step_ms * 1e-3) / 1e9
    traffic = args.traffic * 1e9 if args.traffic else None
    if traffic is None and w.name in MEASURED_TRAFFIC and MEASURED_TRAFFIC[w.name][1] == kernels_sha():
        traffic = MEASURED_TRAFFIC[w.name][0]
    traffic_source = None
    if args.traffic:
        traffic_source = "given on the command line (--traffic)"
    elif traffic is not None:
        traffic_source = (f"stored calibration, not read in this run: rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE "
                          f"of this kernel source (kernels_sha {kernels_sha()}) scaled by a plain 1 GiB copy")
    # the call's bytes: the decode's, and with a fused append the new tokens'
    call_bytes = s_bytes + (append_bytes(w, B) if fused else 0)
    achieved = call_bytes / (avg_dec_ms * 1e-3) / 1e9
    avg_kern_ms = float(np.mean(kern_ms))
    # with a fused append into a pool other than FP8 the first kernel is
    # decode_append_kernel, which also stores the new tokens (K and V read and
    # written, the slot read and copied for the merge)
    tail_append = fused and w.kv_dtype != "fp8"
    decode_name = "decode_append_kernel" if tail_append else "decode_kernel"
    if prefix:
        # prefix, suffix and merge kernels work as one: the roofline is the call
        r_kernel, r_ms, r_bytes = (f"paged_attention_decode (prefix_kernel + {decode_name} + merge_kernel)",
                                   avg_dec_ms, call_bytes)
    else:
        s_out = float(np.mean([out_bytes(w, step_lens[t]) for t in timed]))
        # decode_append_kernel: the new tokens, each slot read and copied
        tail = new_token_bytes(w, B) + 16 * B if tail_append else 0
        r_kernel, r_ms, r_bytes = decode_name, avg_kern_ms, s_bytes - s_out + tail
    r_achieved = r_bytes / (r_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES.get(w.name, w.name),
            "batch": B, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "kv_dtype": w.kv_dtype,
            "mean_context": float(np.mean(d.lengths)), "sliding_window": w.window,
            "num_splits": args.splits, "replicas": len(reps), "shared_prefix_blocks": shared0,
            "metadata": ("device-resident tables" if resident else "tables exported and uploaded every step"),
            "append": ("fused: the decode call appends the step's token, its table entry and length" if fused
                       else "separate append kernel before the decode"),
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_heads_per_s": round(B * w.num_q_heads / (step_ms * 1e-3), 1),
        "decode_ms": round(avg_dec_ms, 5),
        "decode_GBps": round(achieved, 2),
        "decode_seq_heads_per_s": round(B * w.num_q_heads / (avg_dec_ms * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(r_achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r_achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_source": traffic_source,
            "kernel": r_kernel,
            "launch_ms": round(r_ms, 5),
            "algorithmic_bytes": round(r_bytes),
            # the whole paged_attention_decode call (every kernel it launches,
            # all its algorithmic bytes), beside the dominant kernel alone
            "call_ms": round(avg_dec_ms, 5),
            "call_achieved": round(achieved, 2),
            "call_frac": round(achieved / HBM_PEAK_GBS, 4),
        },
        "decode_timing": f"kernel durations recorded by the kernels themselves (hipExtLaunchKernelGGL "
                         f"start and end events, created with hipEventDisableSystemFence) on {len(dec_ms)} "
                         f"of the {args.steps} timed steps; decode_ms sums the call's kernels",
        "decode_back_to_back_ms": round(b2b_ms, 5),
        "decode_back_to_back_GBps": round(b2b_bytes / (b2b_ms * 1e-3) / 1e9, 2),
        "cpu_baseline": None,
    }
    if prefix:
        res["logical_decode_GBps"] = round(s_logical / (avg_dec_ms * 1e-3) / 1e9, 2)
        res["bytes_basis"] = "unique (shared prefix counted once)"
    return res, w, d, scales


def _oracle_sample(w, d, n, scales):
    """Oracle state (block manager + bit-exact pool) for the first n sequences
    of the workload, built the way the GPU state is (prefix workloads: one
    root holding the prefix, forked, plus each sequence's private suffix)."""
    from oracle import BlockManager, PoolModel
    bs = w.block_size
    if w.lengths_kind == "prefix":
        nb = -(-w.prefix_len // bs) + sum(-(-int(x) // bs) + 1 for x in d.suffix[:n])
    else:
        nb = sum(-(-int(L) // bs) for L in d.lengths[:n])
    bm = BlockManager(nb, bs)
    kw = {}
    if w.kv_dtype == "fp8":
        ks, vs = scales
        kw = dict(k_scale=ks, v_scale=vs, k_inv_scale=(np.float32(1) / ks).astype(np.float32),
                  v_inv_scale=(np.float32(1) / vs).astype(np.float32))
    pool = PoolModel(1, nb, w.num_kv_heads, bs, w.head_dim, w.kv_dtype, **kw)
    seqs = []
    if w.lengths_kind == "prefix":
        root = bm.alloc()
        slots, _ = bm.append(root, w.prefix_len)
        kb, vb = wl.kv_tokens_bits(w, (3,), w.prefix_len)
        pool.append(0, kb, vb, w.src_dtype, slots)
        for b in range(n):
            s = bm.fork(root)
            slots, cows = bm.append(s, int(d.suffix[b]))
            pool.copy_blocks(cows)
            kb, vb = wl.kv_tokens_bits(w, (1, b), int(d.suffix[b]))
            pool.append(0, kb, vb, w.src_dtype, slots)
            seqs.append(s)
    else:
        for b, L in enumerate(d.lengths[:n]):
            s = bm.alloc()
            slots, _ = bm.append(s, int(L))
            kb, vb = wl.kv_tokens_bits(w, (1, b), int(L))
            pool.append(0, kb, vb, w.src_dtype, slots)
            seqs.append(s)
    tables, lens = bm.export(seqs, max(len(bm.table(x)) for x in seqs))
    return pool, tables, lens


def cpu_baseline(w, d, budget_s, scales=None):
    """The oracle, as it stands, timed on a bounded sample of the same
    workload: the first n sequences (n grown until one decode takes a sizeable
    share of the budget, or the whole batch), decoded repeatedly for at least a
    few seconds.  State building is outside the timed region."""
    import threadpoolctl
    from oracle import decode_attention
    B = len(d.lengths)
    scale = 1.0 / math.sqrt(w.head_dim)
    q_all = wl.q_bits(w)
    n = 1
    while True:
        pool, tables, lens = _oracle_sample(w, d, n, scales)
        t0 = time.perf_counter()
        decode_attention(pool, 0, q_all[:n], w.q_dtype, tables, lens, scale, w.window)
        one = time.perf_counter() - t0
        if one >= budget_s / 4 or n >= B:
            break
        n = min(B, max(n + 1, int(n * (budget_s / 4) / max(one, 1e-6))))
    reps = max(1, int(min(budget_s, max(3.0, one)) / max(one, 1e-9)))
    t0 = time.perf_counter()
    for _ in range(reps):
        decode_attention(pool, 0, q_all[:n], w.q_dtype, tables, lens, scale, w.window)
    elapsed = (time.perf_counter() - t0) / reps
    if w.lengths_kind == "prefix":
        total, kv = decode_bytes(w, lens)
        nbytes = total - kv + unique_kv_bytes(w, lens)
    else:
        nbytes, _ = decode_bytes(w, lens)
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    return {
        "value": round(nbytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"first {n} of {B} sequences of the same workload (its cache, tables and q); one decode "
                  f"call takes {elapsed:.2f} s, averaged over {reps} calls (float64 NumPy gather + textbook "
                  f"attention)",
        "seq_heads_per_s": round(n * w.num_q_heads / elapsed, 2),
        "host_cpus": len(os.sched_getaffinity(0)),
        "host_cpu_count": os.cpu_count(),
        "cpu_model": _cpu_model(),
        "blas": [f"{i.get('internal_api', '?')} {i.get('num_threads', '?')} threads" for i in info],
    }


def _cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def read_probe(nbytes, reps):
    """Achievable HBM read rate on this device: pkv_hbm_read_probe over a
    buffer of nbytes (several times the 256 MB Infinity Cache), timed with
    events around each call on one stream; the median in GB/s."""
    import torch
    import paged_kv_cache_406_amd as P
    buf = torch.full((nbytes // 4,), 1.0, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    P.pkv_hbm_read_probe(buf, nbytes, sink, stream=s.cuda_stream)   # warm-up
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(s)
        P.pkv_hbm_read_probe(buf, nbytes, sink, stream=s.cuda_stream)
        b.record(s)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def copy_probe(nbytes, reps):
    """A plain device-to-device copy of known size, run under rocprofv3 --pmc
    so that FETCH_SIZE / WRITE_SIZE can be calibrated against bytes moved."""
    import torch
    torch.cuda.set_device(0)
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--splits", type=int, default=0, help="num_splits passed to decode (0 = automatic)")
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--full-metadata", action="store_true",
                    help="export and upload every step's tables instead of keeping them resident")
    ap.add_argument("--unfused", action="store_true",
                    help="append the step's token with its own kernel before the decode call")
    ap.add_argument("--no-shared-prefix", action="store_true",
                    help="decode forked families without reading their common prefix once")
    ap.add_argument("--traffic", type=float, default=None,
                    help="HBM bytes per decode_kernel launch from rocprofv3 counters (GB)")
    ap.add_argument("--targets", default="c5,c5_fp8",
                    help="with the default c3 workload, also measure these workloads (comma list; '' for none)")
    ap.add_argument("--target-steps", type=int, default=24)
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    ap.add_argument("--read-probe", type=int, default=0,
                    help="only run the streaming HBM read probe over this many bytes")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe(args.copy_probe, 5)
        return
    if args.read_probe:
        print(json.dumps({"read_probe_bytes": args.read_probe,
                          "GBps": round(read_probe(args.read_probe, 20), 1)}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the decode path runs on a single MI355X; "
              "multi-GPU runs are not part of this benchmark", file=sys.stderr)
        sys.exit(2)
    res, w, d, scales = run(args)
    # the other configurations the 70 % target is stated on (128K context,
    # bf16 and FP8 KV), measured in the same process with the same timing:
    # a shorter run of each, decode kernel and whole call
    if args.targets and args.workload == "c3":
        res["targets"] = {}
        for name in [x for x in args.targets.split(",") if x]:
            sub = argparse.Namespace(**vars(args))
            sub.workload, sub.steps, sub.warmup, sub.replicas = name, args.target_steps, 3, 0
            r, _, _, _ = run(sub)
            res["targets"][name] = {
                "workload": r["config"]["workload"], "steps": r["steps"], "ms_per_step": r["ms_per_step"],
                "value_GBps": r["value"], "decode_kernel_ms": r["roofline"]["launch_ms"],
                "decode_kernel_bytes": r["roofline"]["algorithmic_bytes"],
                "decode_kernel_GBps": r["roofline"]["achieved"], "decode_kernel_frac": r["roofline"]["frac"],
                "call_ms": r["roofline"]["call_ms"], "call_GBps": r["roofline"]["call_achieved"],
                "call_frac": r["roofline"]["call_frac"], "seq_heads_per_s": r["decode_seq_heads_per_s"],
                "traffic": r["roofline"]["traffic"], "traffic_source": r["roofline"]["traffic_source"],
            }
            res["targets"][name]["kernel"] = r["roofline"]["kernel"]
            log(f"{name}: {r['roofline']['kernel']} {r['roofline']['launch_ms']:.4f} ms, frac {r['roofline']['frac']:.3f}; "
                f"call {r['roofline']['call_ms']:.4f} ms, frac {r['roofline']['call_frac']:.3f}")
    # context for the roofline: what a plain streaming read of 2 GiB reaches
    # on this device (pkv_hbm_read_probe, median of 10 calls)
    res["hbm_read_probe_GBps"] = round(read_probe(1 << 31, 10), 1)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(w, d, args.cpu_budget, scales)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
