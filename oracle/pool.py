"""Bit-exact pool model (oracle; test infrastructure only).

The physical pool is a set of fixed-size blocks scattered through device
memory (page "生成一个字，为什么要背一整本账", section
"PagedAttention：把操作系统的老智慧搬进推理引擎"; page "AI 陪读顶会论文（三）",
section "PagedAttention 的破局哲学", innovation 1).  This model keeps, per
layer, the raw bit patterns of K and V in the *logical* shape
[num_blocks][kv_heads][block_size][head_dim]; it knows nothing about the
memory layout the HIP library uses.

* append: the new token's k and v go to their slot (page "AI 陪读顶会论文（三）",
  section "为什么自回归解码…必须使用 KV Cache": only the new token's k_t, v_t
  are computed and appended).  When the pool dtype equals the source dtype the
  bits are copied; for an FP8 pool the value is taken to fp32, multiplied in
  fp32 by the per-channel inverse scale (page "生成一个字…", section
  "再往后：压 KV 的三条路线": per-channel calibrated scaling), and encoded to
  E4M3 with round-to-nearest-even and saturation.
* copy_blocks: a copy-on-write copies a whole block, K and V, in every layer.
"""
import numpy as np

from .e4m3 import e4m3_encode, e4m3_to_f64

DTYPES = ("f32", "f16", "bf16", "fp8")
BITS_DTYPE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


def bits_to_f64(bits, dtype: str) -> np.ndarray:
    """Exact value of stored bit patterns as float64 (FP8 unscaled)."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "fp8":
        return e4m3_to_f64(bits)
    raise ValueError(f"unknown dtype {dtype}")


def bits_to_f32(bits, dtype: str) -> np.ndarray:
    """Exact value of 32/16-bit source patterns as float32."""
    if dtype == "fp8":
        raise ValueError("fp8 is not a source dtype")
    return bits_to_f64(bits, dtype).astype(np.float32)


class PoolModel:
    def __init__(self, num_layers, num_blocks, num_kv_heads, block_size, head_dim,
                 kv_dtype, k_inv_scale=None, v_inv_scale=None, k_scale=None,
                 v_scale=None):
        if kv_dtype not in DTYPES:
            raise ValueError(kv_dtype)
        self.num_layers, self.num_blocks = num_layers, num_blocks
        self.num_kv_heads, self.block_size, self.head_dim = num_kv_heads, block_size, head_dim
        self.kv_dtype = kv_dtype
        shape = (num_layers, num_blocks, num_kv_heads, block_size, head_dim)
        self.k = np.zeros(shape, dtype=BITS_DTYPE[kv_dtype])
        self.v = np.zeros(shape, dtype=BITS_DTYPE[kv_dtype])
        self.written = np.zeros((num_layers, num_blocks, block_size), dtype=bool)
        if kv_dtype == "fp8":
            sshape = (num_layers, num_kv_heads, head_dim)
            for name, arr in (("k_inv_scale", k_inv_scale), ("v_inv_scale", v_inv_scale),
                              ("k_scale", k_scale), ("v_scale", v_scale)):
                if arr is None or np.shape(arr) != sshape:
                    raise ValueError(f"{name} of shape {sshape} is required for fp8")
            self.k_inv_scale = np.asarray(k_inv_scale, dtype=np.float32)
            self.v_inv_scale = np.asarray(v_inv_scale, dtype=np.float32)
            self.k_scale = np.asarray(k_scale, dtype=np.float32)
            self.v_scale = np.asarray(v_scale, dtype=np.float32)

    def _encode(self, bits, src_dtype, inv_scale_layer):
        if self.kv_dtype == src_dtype:
            return np.asarray(bits, dtype=BITS_DTYPE[src_dtype])
        if self.kv_dtype != "fp8":
            raise ValueError("only same-dtype copy or quantisation to fp8")
        x = bits_to_f32(bits, src_dtype)                       # [n][Hkv][D]
        y = (x * inv_scale_layer[None, :, :]).astype(np.float32)  # one fp32 multiply
        return e4m3_encode(y)

    def append(self, layer, k_bits, v_bits, src_dtype, slots):
        """Write tokens [n][Hkv][D] (bit patterns of ``src_dtype``) at ``slots``;
        negative slots are skipped."""
        slots = np.asarray(slots, dtype=np.int64)
        kq = self._encode(k_bits, src_dtype,
                          self.k_inv_scale[layer] if self.kv_dtype == "fp8" else None)
        vq = self._encode(v_bits, src_dtype,
                          self.v_inv_scale[layer] if self.kv_dtype == "fp8" else None)
        bs = self.block_size
        for i, s in enumerate(slots):
            if s < 0:
                continue
            blk, off = divmod(int(s), bs)
            self.k[layer, blk, :, off, :] = kq[i]
            self.v[layer, blk, :, off, :] = vq[i]
            self.written[layer, blk, off] = True

    def copy_blocks(self, pairs):
        for src, dst in pairs:
            self.k[:, dst] = self.k[:, src]
            self.v[:, dst] = self.v[:, src]
            self.written[:, dst] = self.written[:, src]

    def values(self, which, layer, blocks, head):
        """float64 [len(blocks)*bs][D] of K or V for one KV head, dequantised
        (FP8 codes times the per-channel scale, product exact in fp64)."""
        arr = self.k if which == "k" else self.v
        bits = arr[layer, np.asarray(blocks, dtype=np.int64), head]   # [nb][bs][D]
        vals = bits_to_f64(bits, self.kv_dtype).reshape(-1, self.head_dim)
        if self.kv_dtype == "fp8":
            sc = (self.k_scale if which == "k" else self.v_scale)[layer, head]
            vals = vals * sc.astype(np.float64)[None, :]
        return vals
