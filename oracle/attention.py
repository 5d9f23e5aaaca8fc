"""Decode attention over a paged KV cache (oracle; test infrastructure only).

Page "AI 陪读顶会论文（三）", section "为什么自回归解码…必须使用 KV Cache": the
token being generated at position t attends with
softmax(q_t K_{1:t}^T / sqrt(d)) V_{1:t}, where K and V hold every cached
token including the new one (appended first).  Paging only changes where the
bytes live (page "生成一个字，为什么要背一整本账", section
"PagedAttention：把操作系统的老智慧搬进推理引擎"), so the result is plain
attention over the logically contiguous cache: gather the blocks through the
table, cut to L tokens, run the textbook formula in float64.

Other readings used here:

* GQA (page "生成一个字…", section "显存账本"): query heads are grouped,
  consecutive heads sharing one KV head: head h reads KV head h // G with
  G = Hq / Hkv.
* d in sqrt(d) is the head dimension; the scale is passed in explicitly.
* Sliding window (page "生成一个字…", section "再往后：压 KV 的三条路线"):
  with window W > 0 the query attends keys max(0, L - W) .. L - 1, i.e. W keys
  including itself; W >= L means no restriction.
* L = 0 (or nothing to attend) gives an all-zero output.

The split form (``partial_attention`` + ``lse_merge``) states the same
quantity as a combination of per-range partial results: for each key range
the unnormalised output o = sum_j exp(s_j - m) v_j, the range max m and the
range sum l = sum_j exp(s_j - m); the ranges combine by rescaling each to the
overall max.  It is the definition of the softmax written over a partition of
the keys, so it equals the unsplit result up to rounding.
"""
import numpy as np

from .pool import bits_to_f64


def _textbook(qh, K, V, scale):
    s = scale * (K @ qh)
    m = s.max()
    p = np.exp(s - m)
    return (p @ V) / p.sum()


def _key_range(L, window):
    lo = max(0, L - window) if window and window > 0 else 0
    return lo, L


def gather_kv(pool, layer, table, L, kv_head, lo=0):
    """Contiguous float64 K, V [L - lo][D] of tokens lo .. L-1 of one sequence
    and KV head.  Only the blocks holding those tokens are read (a sliding
    window may have released the earlier ones)."""
    bs = pool.block_size
    first, nblk = lo // bs, -(-L // bs)
    blocks = list(table[first:nblk])
    if len(blocks) < nblk - first or any(b < 0 or b >= pool.num_blocks for b in blocks):
        raise ValueError("block table does not cover the attended tokens")
    skip = lo - first * bs
    K = pool.values("k", layer, blocks, kv_head)[skip:L - first * bs]
    V = pool.values("v", layer, blocks, kv_head)[skip:L - first * bs]
    return K, V


def decode_attention(pool, layer, q, q_dtype, tables, lens, scale, window=0):
    """float64 [B][Hq][D] decode output.

    q: bit patterns [B][Hq][D] of ``q_dtype`` ('f32', 'f16', 'bf16');
    tables: [B][max_blocks] physical ids; lens: [B] context lengths including
    the new token.
    """
    qf = bits_to_f64(q, q_dtype)
    B, Hq, D = qf.shape
    Hkv = pool.num_kv_heads
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        lo, hi = _key_range(L, window)
        if hi - lo <= 0:
            continue
        for g in range(Hkv):
            K, V = gather_kv(pool, layer, tables[b], hi, g, lo)
            for h in range(g * G, (g + 1) * G):
                out[b, h] = _textbook(qf[b, h], K, V, scale)
    return out


def partial_attention(qh, K, V, scale):
    """(o_unnormalised [D], m, l) over one key range; empty range -> (0, -inf, 0)."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), -np.inf, 0.0
    s = scale * (K @ qh)
    m = s.max()
    p = np.exp(s - m)
    return p @ V, m, p.sum()


def lse_merge(parts):
    """Combine partials [(o, m, l), ...] into the normalised output."""
    ms = np.array([m for _, m, _ in parts], dtype=np.float64)
    if len(parts) == 0 or np.all(np.isneginf(ms)):
        return np.zeros_like(parts[0][0]) if parts else None
    M = ms.max()
    w = np.exp(ms - M)
    num = sum(wi * o for wi, (o, _, _) in zip(w, parts))
    den = sum(wi * l for wi, (_, _, l) in zip(w, parts))
    return num / den


def decode_attention_split(pool, layer, q, q_dtype, tables, lens, scale,
                           boundaries_fn, window=0):
    """Same quantity as ``decode_attention`` computed as partials over key
    ranges and merged.  ``boundaries_fn(L_eff)`` returns the cut points
    (ascending, within (0, L_eff)) of the attended key range."""
    qf = bits_to_f64(q, q_dtype)
    B, Hq, D = qf.shape
    Hkv = pool.num_kv_heads
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        lo, hi = _key_range(L, window)
        if hi - lo <= 0:
            continue
        cuts = [0] + list(boundaries_fn(hi - lo)) + [hi - lo]
        for g in range(Hkv):
            K, V = gather_kv(pool, layer, tables[b], hi, g, lo)
            for h in range(g * G, (g + 1) * G):
                parts = [partial_attention(qf[b, h], K[a:e], V[a:e], scale)
                         for a, e in zip(cuts[:-1], cuts[1:])]
                out[b, h] = lse_merge(parts)
    return out
