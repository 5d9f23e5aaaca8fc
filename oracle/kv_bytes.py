"""KV-cache byte formula (oracle; test infrastructure only).

Page "生成一个字，为什么要背一整本账", opening section: the cache holds one K
and one V vector per layer, per KV head, per token and per sequence, so its
size is 2 x layers x KV heads x head_dim x sequence length x batch x bytes per
element; the factor 2 is the K/V pair.

The page "AI 陪读顶会论文（三）", section "核心账本", prints the same formula
with a second, unexplained factor of 2; its own worked example (80 layers,
d_model 8192, 4096 tokens, batch 16, 2 bytes -> 171,798,691,840 bytes) uses a
single factor, so the single-factor form is the one implemented here.
"""


def kv_cache_bytes(num_layers: int, num_kv_heads: int, head_dim: int,
                   seq_len: int, batch: int, dtype_bytes: int) -> int:
    """Bytes of K plus V for ``batch`` sequences of ``seq_len`` tokens."""
    for v in (num_layers, num_kv_heads, head_dim, seq_len, batch, dtype_bytes):
        if int(v) != v or v < 0:
            raise ValueError("all arguments must be non-negative integers")
    return 2 * num_layers * num_kv_heads * head_dim * seq_len * batch * dtype_bytes
