"""Seeded synthetic inputs for paged decode attention.

This module is shared by the tests, the bench and the oracle-side checks.  It
holds NO step of the method: it only draws numbers (context lengths, the
order in which free blocks are handed out, K/V/q values) and stores them in
the dtype each workload names.  Every draw comes from ``numpy.random.
default_rng`` with a fixed seed and a fixed order, so two processes that ask
for the same workload get identical bits.

The workloads are shaped after the models and situations the pages discuss;
no dataset item is used.

* ``c1`` tiny: 1 layer, 4 sequences of lengths {5, 16, 17, 40}, 4 query / 2
  KV heads, head_dim 64, block 16, 64 physical blocks, fp32, N(0,1).
* ``c2`` Llama-2-7B-shaped MHA layer (32 layers / 32 heads / head_dim 128 on
  page "生成一个字，为什么要背一整本账", opening section): 32/32 heads,
  fp16, batch 64, lengths uniform in [128, 4096], values N(0,1)*0.5, blocks
  16 / 32 / 128.
* ``c3`` Llama-2-70B-shaped GQA layer (64 query / 8 KV heads, same page,
  section "显存账本"): bf16, batch 128, lengths lognormal with median 800 and
  sigma 0.8 clipped to [16, 4096], N(0,1).
* ``c4`` shared system prompt (same page, section "PagedAttention：…"): 256
  sequences forked from one 2000-token prefix, private suffixes uniform in
  [1, 512], 32/8 heads, bf16.
* ``c5`` long context (Llama 3 70B at 128K, same page, section "显存账本"):
  batch 4, 131072 tokens each, 64/8 heads, bf16 and an FP8 variant with
  per-channel fp32 scales (absmax / 448), plus a 4096-token sliding window.

Draw order per workload: lengths, then the free-block permutation, from
``default_rng(seed)``; K/V of sequence b from ``default_rng([seed, 1, b])``
(so values depend only on logical coordinates, never on placement); q from
``default_rng([seed, 2])``; the shared prefix of c4 from
``default_rng([seed, 3])``; the token appended at decode step t from
``default_rng([seed, 4, t])``.  A pool of several layers holds different
values in each: sequence b's K/V in layer l > 0 come from
``default_rng([seed, 5, l, b])`` (layer 0 keeps ``[seed, 1, b]``).
"""
from dataclasses import dataclass, field, replace
import math

import numpy as np

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
SOURCE_DTYPE = {"f32": "f32", "f16": "f16", "bf16": "bf16", "fp8": "bf16"}
FP8_MAX = 448.0


# ---------------------------------------------------------------------------
# storage conversions of drawn float32 values (input preparation only)
# ---------------------------------------------------------------------------
def f32_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round drawn float32 values to the storage dtype (nearest-even) and
    return the raw bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.view(np.uint32).copy()
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return rounded.astype(np.uint16)
    raise ValueError(f"not a source dtype: {dtype}")


def bits_as_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen 32/16-bit storage patterns to float32 (exact)."""
    if dtype == "f32":
        return bits.view(np.float32)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# workload descriptions
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str            # pool dtype: f32 / f16 / bf16 / fp8
    q_dtype: str             # f32 / f16 / bf16
    value_std: float
    lengths_kind: str        # fixed / uniform / lognormal / prefix / const
    lengths_args: tuple
    num_layers: int = 1
    pool_blocks: int = 0     # 0 -> ceil(1.25 * blocks needed)
    window: int = 0
    prefix_len: int = 0      # c4 only

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    @property
    def src_dtype(self):
        return SOURCE_DTYPE[self.kv_dtype]


WORKLOADS = {
    "c1": Workload("c1", 4061, 4, 4, 2, 64, 16, "f32", "f32", 1.0, "fixed",
                   (5, 16, 17, 40), pool_blocks=64),
    "c2": Workload("c2", 4062, 64, 32, 32, 128, 16, "f16", "f16", 0.5, "uniform",
                   (128, 4096)),
    "c3": Workload("c3", 4063, 128, 64, 8, 128, 16, "bf16", "bf16", 1.0, "lognormal",
                   (800.0, 0.8, 16, 4096)),
    "c4": Workload("c4", 4064, 256, 32, 8, 128, 16, "bf16", "bf16", 1.0, "prefix",
                   (1, 512), prefix_len=2000),
    "c5": Workload("c5", 4065, 4, 64, 8, 128, 16, "bf16", "bf16", 1.0, "const",
                   (131072,), pool_blocks=40960),
}
WORKLOADS["c5_fp8"] = replace(WORKLOADS["c5"], name="c5_fp8", kv_dtype="fp8")
WORKLOADS["c5w"] = replace(WORKLOADS["c5"], name="c5w", window=4096)
WORKLOADS["c2_bs32"] = replace(WORKLOADS["c2"], name="c2_bs32", block_size=32)
WORKLOADS["c2_bs128"] = replace(WORKLOADS["c2"], name="c2_bs128", block_size=128)


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields changed (smaller test shapes)."""
    return replace(w, **changes)


@dataclass
class Draw:
    """Host-side draw of one workload: lengths, free order, pool size."""
    workload: Workload
    lengths: np.ndarray          # int64 [B]: tokens in cache incl. the new one
    suffix: np.ndarray = None    # c4: private suffix lengths
    free_order: np.ndarray = None
    num_blocks: int = 0


def _blocks(n, bs):
    return -(-int(n) // bs)


def draw(w: Workload, extra_blocks: int = 0) -> Draw:
    """Lengths, free-block permutation and pool size of a workload."""
    rng = np.random.default_rng(w.seed)
    suffix = None
    if w.lengths_kind == "fixed":
        lengths = np.array(w.lengths_args, dtype=np.int64)
        assert len(lengths) == w.batch
    elif w.lengths_kind == "uniform":
        a, b = w.lengths_args
        lengths = rng.integers(a, b, size=w.batch, endpoint=True).astype(np.int64)
    elif w.lengths_kind == "lognormal":
        med, sigma, lo, hi = w.lengths_args
        raw = np.exp(rng.normal(math.log(med), sigma, size=w.batch))
        lengths = np.clip(np.rint(raw), lo, hi).astype(np.int64)
    elif w.lengths_kind == "prefix":
        a, b = w.lengths_args
        suffix = rng.integers(a, b, size=w.batch, endpoint=True).astype(np.int64)
        lengths = suffix + w.prefix_len
    elif w.lengths_kind == "const":
        lengths = np.full(w.batch, w.lengths_args[0], dtype=np.int64)
    else:
        raise ValueError(w.lengths_kind)
    bs = w.block_size
    if w.lengths_kind == "prefix":
        # the prefix's full blocks are stored once, each sequence owns the rest
        shared = w.prefix_len // bs
        need = shared + sum(_blocks(L, bs) - shared for L in lengths)
    else:
        need = sum(_blocks(L, bs) for L in lengths)
    nb = w.pool_blocks or int(math.ceil(1.25 * need))
    nb += extra_blocks
    order = rng.permutation(nb).astype(np.int32)
    return Draw(w, lengths, suffix, order, nb)


def kv_tokens(w: Workload, stream, n_tokens: int, start: int = 0):
    """K and V float32 values [n][Hkv][D] of tokens start..start+n-1 of a
    stream (``stream`` is the tuple appended to the seed: (1, b) for sequence
    b, (3,) for the c4 prefix).  Values depend only on the stream and the
    token index."""
    rng = np.random.default_rng([w.seed, *stream])
    shape = (start + n_tokens, w.num_kv_heads, w.head_dim)
    k = rng.standard_normal(shape, dtype=np.float32) * np.float32(w.value_std)
    v = rng.standard_normal(shape, dtype=np.float32) * np.float32(w.value_std)
    return k[start:], v[start:]


def kv_stream(b: int, layer: int = 0):
    """Stream id of sequence b's K/V in one layer of the pool."""
    return (1, b) if layer == 0 else (5, layer, b)


def kv_tokens_bits(w: Workload, stream, n_tokens: int, start: int = 0):
    """Same as ``kv_tokens`` rounded to the source dtype, as bit patterns."""
    k, v = kv_tokens(w, stream, n_tokens, start)
    return f32_to_bits(k, w.src_dtype), f32_to_bits(v, w.src_dtype)


def q_bits(w: Workload, batch: int = None, stream=(2,)):
    """q bit patterns [B][Hq][D] in the workload's q dtype."""
    rng = np.random.default_rng([w.seed, *stream])
    B = w.batch if batch is None else batch
    q = rng.standard_normal((B, w.num_q_heads, w.head_dim), dtype=np.float32)
    return f32_to_bits(q * np.float32(w.value_std), w.q_dtype)


def step_tokens_bits(w: Workload, step: int, batch: int = None):
    """New-token k, v [B][Hkv][D] and q [B][Hq][D] bit patterns for decode step t."""
    B = w.batch if batch is None else batch
    rng = np.random.default_rng([w.seed, 4, step])
    kshape = (B, w.num_kv_heads, w.head_dim)
    k = rng.standard_normal(kshape, dtype=np.float32) * np.float32(w.value_std)
    v = rng.standard_normal(kshape, dtype=np.float32) * np.float32(w.value_std)
    q = rng.standard_normal((B, w.num_q_heads, w.head_dim), dtype=np.float32)
    q = q * np.float32(w.value_std)
    return (f32_to_bits(k, w.src_dtype), f32_to_bits(v, w.src_dtype),
            f32_to_bits(q, w.q_dtype))


def fp8_scales(absmax: np.ndarray):
    """Per-channel scale (absmax / 448, fp32) and its fp32 reciprocal; a
    channel that is all zero gets scale 1."""
    a = np.asarray(absmax, dtype=np.float64)
    scale = np.where(a > 0, a / FP8_MAX, 1.0).astype(np.float32)
    inv = (np.float32(1.0) / scale).astype(np.float32)
    return scale, inv


def channel_absmax(values_list, num_kv_heads, head_dim):
    """Absmax per (KV head, channel) over a list of [n][Hkv][D] arrays."""
    m = np.zeros((num_kv_heads, head_dim), dtype=np.float32)
    for arr in values_list:
        if len(arr):
            m = np.maximum(m, np.abs(arr).max(axis=0))
    return m
