"""Device buffers of a pool allocated with torch (memory plumbing only)."""
import numpy as np

from . import _binding as B


class TorchKVPool:
    """Allocates the K/V buffers (and FP8 scales) of one pool with torch and
    creates the library pool over them.  ``handle`` is what the C entry
    points take.  Scales are host arrays [num_layers][num_kv_heads][head_dim]
    (fp32); the inverse scales default to their fp32 reciprocals."""

    def __init__(self, num_layers, num_kv_heads, head_dim, block_size, num_blocks, kv_dtype,
                 device="cuda", free_order=None, k_scale=None, v_scale=None,
                 k_inv_scale=None, v_inv_scale=None):
        import torch
        self.num_layers, self.num_kv_heads, self.head_dim = num_layers, num_kv_heads, head_dim
        self.block_size, self.num_blocks = block_size, num_blocks
        self.kv_dtype = B.DTYPE_CODE.get(kv_dtype, kv_dtype)
        if self.kv_dtype == B.PKV_FP8_E4M3:
            # the kernels index every scale array as [num_layers][num_kv_heads][head_dim]
            want = (num_layers, num_kv_heads, head_dim)
            for name, arr in (("k_scale", k_scale), ("v_scale", v_scale),
                              ("k_inv_scale", k_inv_scale), ("v_inv_scale", v_inv_scale)):
                if arr is None and name.endswith("inv_scale"):
                    continue
                if arr is None:
                    raise ValueError("FP8 pools need k_scale and v_scale")
                if np.shape(arr) != want:
                    raise ValueError(f"{name} must have shape {want} (num_layers, num_kv_heads, head_dim), "
                                     f"got {np.shape(arr)}")
        probe = B.make_desc(num_layers, num_kv_heads, head_dim, block_size, num_blocks, self.kv_dtype)
        self.cache_bytes = B.kv_pool_cache_bytes(probe)
        self.k_cache = torch.empty(self.cache_bytes, dtype=torch.uint8, device=device)
        self.v_cache = torch.empty(self.cache_bytes, dtype=torch.uint8, device=device)
        self.scales = {}
        if self.kv_dtype == B.PKV_FP8_E4M3:
            k_scale = np.asarray(k_scale, dtype=np.float32)
            v_scale = np.asarray(v_scale, dtype=np.float32)
            if k_inv_scale is None:
                k_inv_scale = (np.float32(1.0) / k_scale).astype(np.float32)
            if v_inv_scale is None:
                v_inv_scale = (np.float32(1.0) / v_scale).astype(np.float32)
            for name, arr in (("k_scale", k_scale), ("v_scale", v_scale),
                              ("k_inv_scale", k_inv_scale), ("v_inv_scale", v_inv_scale)):
                self.scales[name] = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
        self.desc = B.make_desc(num_layers, num_kv_heads, head_dim, block_size, num_blocks, self.kv_dtype,
                                self.k_cache, self.v_cache, free_order=free_order, **self.scales)
        self.handle = B.kv_pool_create(self.desc)

    def close(self):
        if getattr(self, "handle", None):
            B.kv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
