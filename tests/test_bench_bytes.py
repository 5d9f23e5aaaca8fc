"""Byte accounting of bench.py, the denominators of every GB/s it reports.

Pinned to the per-call KV bytes of the 128K and window workloads (4 sequences
of 131072 tokens, 8 KV heads, head_dim 128: 2 GiB at bf16, 1 GiB at FP8, the
4096-token window 64 MiB), to the oracle's KV-cache formula, and, for small
cases, to counts done by hand (K and V of each attended token, q, the fp32
output, the block-table entries of the attended blocks, the lengths, the FP8
scales).
"""
import bench
import workloads as wl
from oracle.kv_bytes import kv_cache_bytes


def test_128k_kv_bytes_match_the_cache_formula():
    for name, eb in (("c5", 2), ("c5_fp8", 1)):
        w = wl.WORKLOADS[name]
        total, kv = bench.decode_bytes(w, [131072] * 4)
        assert kv == kv_cache_bytes(1, 8, 128, 131072, 4, eb)
        assert kv == (2 ** 31 if eb == 2 else 2 ** 30)
        B, Hq, D = 4, 64, 128
        tables = B * (131072 // 16) * 4
        scales = 2 * 8 * D * 4 if eb == 1 else 0
        assert total == kv + B * Hq * D * (2 + 4) + tables + B * 4 + scales


def test_window_reads_only_the_window():
    w = wl.WORKLOADS["c5w"]
    total, kv = bench.decode_bytes(w, [131072] * 4)
    assert kv == kv_cache_bytes(1, 8, 128, 4096, 4, 2) == 2 ** 26
    # 256 table entries per sequence: the window's blocks only
    assert total - kv == 4 * 64 * 128 * (2 + 4) + 4 * 256 * 4 + 4 * 4


def test_small_case_by_hand():
    w = wl.scaled(wl.WORKLOADS["c3"], batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64)   # bf16, block 16
    total, kv = bench.decode_bytes(w, [5, 17])
    assert kv == (5 + 17) * 2 * 2 * 64 * 2            # tokens x KV heads x (K, V) x D x 2 bytes
    assert total == kv + 2 * 4 * 64 * (2 + 4) + (1 + 2) * 4 + 2 * 4


def test_window_with_a_partial_first_block():
    # window 10 over L = 37 at block 16: keys 27..36, blocks 1 and 2
    w = wl.scaled(wl.WORKLOADS["c3"], batch=1, num_q_heads=4, num_kv_heads=2, head_dim=64, window=10)
    total, kv = bench.decode_bytes(w, [37])
    assert kv == 10 * 2 * 2 * 64 * 2
    assert total - kv == 4 * 64 * (2 + 4) + 2 * 4 + 4


def test_shared_prefix_counts_the_prefix_once():
    w = wl.WORKLOADS["c4"]
    lengths = [2000 + 7, 2000 + 1, 2000 + 512]
    assert bench.unique_kv_bytes(w, lengths) == kv_cache_bytes(1, 8, 128, 2000 + 7 + 1 + 512, 1, 2)


def test_fused_append_bytes():
    w = wl.WORKLOADS["c3"]
    src, kv = wl.ELEM_BYTES[w.src_dtype], wl.ELEM_BYTES[w.kv_dtype]
    assert bench.new_token_bytes(w, 128) == 128 * 8 * 128 * 2 * (src + kv)
    assert bench.append_bytes(w, 128) == bench.new_token_bytes(w, 128) + 128 * (8 + 12)
    w8 = wl.WORKLOADS["c5_fp8"]
    assert wl.ELEM_BYTES[w8.kv_dtype] == 1
    assert bench.new_token_bytes(w8, 4) == 4 * 8 * 128 * 2 * (wl.ELEM_BYTES[w8.src_dtype] + 1)


def test_more_than_one_gpu_is_refused():
    """The bench measures one GPU: --gpus 2 (or a torchrun world of two) exits
    with a message, before anything touches a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *argv], capture_output=True, text=True,
                           timeout=120, env={**os.environ, **env}, cwd=root)
        assert r.returncode != 0
        assert "one GPU" in r.stderr + r.stdout
