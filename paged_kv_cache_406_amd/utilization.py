"""KV-cache memory utilisation: paged blocks against contiguous max-length
reservation, on seeded synthetic request traces (host only).

What it measures, from the pages:

* Page "生成一个字，为什么要背一整本账", section
  "PagedAttention：把操作系统的老智慧搬进推理引擎": systems that store each
  request's KV contiguously reserve room for the longest possible output, and
  only a fifth to two fifths of what they reserve holds real data.  The waste
  has three sources: the reservation for tokens not yet (or never) generated,
  the unused tail of a reservation, and free space split into pieces too
  small for the next contiguous reservation.  Paged storage takes fixed-size
  blocks on demand, so the waste shrinks to part of each request's last block.
  The same section: larger blocks lose more to that last block on workloads of
  short sequences.
* Page "AI 陪读顶会论文（三）", section on KV allocation waste: the
  contiguous scheme pre-allocates the maximum output length; requests that
  start and end at different times fragment the free space.

Model (the pages give no simulator; these are the plainest readings):

* A trace is a list of requests (prompt tokens, output tokens), all arriving
  at step 0 and admitted in order, first come first served.  At every step
  each running request appends one token (the prompt is appended in full at
  admission); a request finishes once its output is complete and its memory
  is released at the end of that step.
* Contiguous: admission reserves prompt + max_output slots as one run of a
  memory of `capacity` slots (first fit).  A request that does not fit waits;
  no later request is admitted before it (FCFS).
* Paged: admission needs the blocks of prompt + 1 token; each later token may
  take one more block (taken through the library's block manager,
  block_table_append).  A running request that cannot get its next block is
  not modelled: the trace is admitted only while the pool has blocks for
  every running request to finish (the reservation a scheduler would keep).
  This keeps both schemes free of preemption, so the difference is only in
  how memory is held.
* Utilisation at a step = tokens stored / slots held; it is averaged over
  steps weighted by slots held (i.e. total stored token-steps over total held
  slot-steps).

Everything is integer arithmetic on seeded draws; run as
``python -m paged_kv_cache_406_amd.utilization`` for the report.
"""
from __future__ import annotations

import json
from dataclasses import dataclass

import numpy as np


@dataclass
class Request:
    prompt: int
    output: int


@dataclass
class Result:
    scheme: str
    steps: int = 0
    token_steps: int = 0          # sum over steps of tokens stored
    held_steps: int = 0           # sum over steps of slots held (reserved or allocated)
    reserved_unfilled_steps: int = 0  # contiguous: slots reserved for tokens not yet generated
    tail_steps: int = 0           # slots that no token of the request will ever fill
    max_running: int = 0
    mean_running: float = 0.0
    blocked_steps: int = 0        # steps where the head of the queue waited although
    #                               enough slots were free in total (external fragmentation)

    @property
    def utilisation(self) -> float:
        return self.token_steps / self.held_steps if self.held_steps else 0.0

    def as_dict(self):
        d = {k: v for k, v in self.__dict__.items()}
        d["utilisation"] = round(self.utilisation, 4)
        d["mean_running"] = round(self.mean_running, 2)
        return d


# ---------------------------------------------------------------------------
# traces (seeded stand-ins for the conversation / short-instruction workloads
# the pages mention; no dataset item is reproduced)
# ---------------------------------------------------------------------------
def trace(kind: str, n: int, seed: int) -> list[Request]:
    """kind: 'conversation' (lognormal prompts around 800 tokens, outputs
    around 250), 'short' (short instructions: prompts around 40, outputs
    around 60), or 'uniform' (prompt and output uniform in [16, 1024])."""
    rng = np.random.default_rng([seed, 7])
    if kind == "conversation":
        p = np.clip(np.rint(np.exp(rng.normal(np.log(800.0), 0.8, n))), 16, 4096)
        o = np.clip(np.rint(np.exp(rng.normal(np.log(250.0), 0.7, n))), 1, 2048)
    elif kind == "short":
        p = np.clip(np.rint(np.exp(rng.normal(np.log(40.0), 0.6, n))), 4, 512)
        o = np.clip(np.rint(np.exp(rng.normal(np.log(60.0), 0.7, n))), 1, 512)
    elif kind == "uniform":
        p = rng.integers(16, 1024, n, endpoint=True)
        o = rng.integers(16, 1024, n, endpoint=True)
    else:
        raise ValueError(kind)
    return [Request(int(a), int(b)) for a, b in zip(p, o)]


# ---------------------------------------------------------------------------
# contiguous max-length reservation
# ---------------------------------------------------------------------------
class FirstFit:
    """Free runs of a linear memory of `capacity` slots, first-fit."""

    def __init__(self, capacity: int):
        self.capacity = capacity
        self.free = [(0, capacity)]          # sorted (start, length)

    def alloc(self, n: int):
        for k, (s, ln) in enumerate(self.free):
            if ln >= n:
                if ln == n:
                    self.free.pop(k)
                else:
                    self.free[k] = (s + n, ln - n)
                return s
        return None

    def release(self, start: int, n: int):
        self.free.append((start, n))
        self.free.sort()
        merged = []
        for s, ln in self.free:
            if merged and merged[-1][0] + merged[-1][1] == s:
                merged[-1] = (merged[-1][0], merged[-1][1] + ln)
            else:
                merged.append((s, ln))
        self.free = merged

    def total_free(self) -> int:
        return sum(ln for _, ln in self.free)


def run_contiguous(reqs: list[Request], capacity: int, max_output: int) -> Result:
    """Each admitted request holds prompt + max_output contiguous slots until it
    finishes.  Its output never exceeds max_output (longer outputs are cut)."""
    res = Result("contiguous")
    mem = FirstFit(capacity)
    queue = list(range(len(reqs)))
    running = {}        # id -> (start, reserved, stored, remaining outputs)
    running_sum = 0
    while queue or running:
        # admit in order while the head fits
        while queue:
            r = reqs[queue[0]]
            need = r.prompt + max_output
            if need > capacity:
                raise ValueError("a request larger than the whole memory")
            start = mem.alloc(need)
            if start is None:
                if mem.total_free() >= need:
                    res.blocked_steps += 1
                break
            running[queue.pop(0)] = [start, need, r.prompt, min(r.output, max_output)]
        # one decode step
        res.steps += 1
        running_sum += len(running)
        res.max_running = max(res.max_running, len(running))
        done = []
        for rid, st in running.items():
            st[2] += 1
            st[3] -= 1
            final = reqs[rid].prompt + min(reqs[rid].output, max_output)
            res.token_steps += st[2]
            res.held_steps += st[1]
            res.tail_steps += st[1] - final
            res.reserved_unfilled_steps += final - st[2]
            if st[3] == 0:
                done.append(rid)
        for rid in done:
            start, reserved, _, _ = running.pop(rid)
            mem.release(start, reserved)
    res.mean_running = running_sum / res.steps if res.steps else 0.0
    return res


# ---------------------------------------------------------------------------
# paged allocation through the library's block manager
# ---------------------------------------------------------------------------
def run_paged(reqs: list[Request], capacity: int, block_size: int, max_output: int, lib=None) -> Result:
    """The same trace on a pool of capacity // block_size blocks, taken on demand
    by the block manager (block_table_alloc / append / free).  A request is
    admitted when the free blocks cover every running request's remaining
    growth plus this request's whole length (no preemption is ever needed).
    `lib`: the binding module (default: this package's)."""
    if lib is None:
        from . import _binding as lib  # noqa: PLC0415
    nb = capacity // block_size
    desc = lib.make_desc(1, 1, 16, block_size, nb, "f16")
    pool = lib.kv_pool_create(desc)
    res = Result(f"paged bs={block_size}")
    try:
        blocks = lambda n: -(-n // block_size)  # noqa: E731
        queue = list(range(len(reqs)))
        running = {}      # id -> [seq, stored, remaining, final]
        committed = 0     # blocks the running requests will hold at their end
        running_sum = 0
        while queue or running:
            while queue:
                r = reqs[queue[0]]
                final = r.prompt + min(r.output, max_output)
                if blocks(final) > nb:
                    raise ValueError("a request larger than the whole pool")
                if committed + blocks(final) > nb:
                    break
                rid = queue.pop(0)
                seq = lib.block_table_alloc(pool)
                lib.block_table_append(pool, seq, r.prompt)
                running[rid] = [seq, r.prompt, min(r.output, max_output), final]
                committed += blocks(final)
            res.steps += 1
            running_sum += len(running)
            res.max_running = max(res.max_running, len(running))
            if running:
                ids = list(running)
                lib.block_table_append_batch(pool, [running[i][0] for i in ids])
            held = nb - lib.kv_pool_num_free(pool)
            done = []
            for rid, st in running.items():
                st[1] += 1
                st[2] -= 1
                res.token_steps += st[1]
                res.tail_steps += blocks(st[1]) * block_size - st[1]
                if st[2] == 0:
                    done.append(rid)
            res.held_steps += held * block_size
            for rid in done:
                seq, _, _, final = running.pop(rid)
                lib.block_table_free(pool, seq)
                committed -= blocks(final)
        res.mean_running = running_sum / res.steps if res.steps else 0.0
    finally:
        lib.kv_pool_destroy(pool)
    return res


def last_block_waste(lengths, block_size: int) -> float:
    """Share of allocated slots that the last, partly filled block of each
    sequence leaves empty: sum(ceil(L / bs) * bs - L) / sum(ceil(L / bs) * bs)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    alloc = (-(-lengths // block_size)) * block_size
    return float((alloc - lengths).sum() / alloc.sum()) if alloc.sum() else 0.0


def report(n: int = 400, seed: int = 4066, capacity: int = 1 << 17, max_output: int = 2048) -> dict:
    out = {"requests": n, "seed": seed, "capacity_slots": capacity, "max_output": max_output, "traces": {}}
    for kind in ("conversation", "short", "uniform"):
        reqs = trace(kind, n, seed)
        c = run_contiguous(reqs, capacity, max_output)
        rows = {"contiguous": c.as_dict()}
        for bs in (16, 64, 256):
            rows[f"paged_bs{bs}"] = run_paged(reqs, capacity, bs, max_output).as_dict()
        final = [r.prompt + min(r.output, max_output) for r in reqs]
        rows["last_block_waste_of_final_lengths"] = {
            str(bs): round(last_block_waste(final, bs), 4) for bs in (8, 16, 32, 64, 128, 256)}
        out["traces"][kind] = rows
    return out


if __name__ == "__main__":
    print(json.dumps(report(), indent=1))
