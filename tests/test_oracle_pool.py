"""Pins of the oracle's pool model: FP8 quantise-on-write and bit copies.

Page "生成一个字，为什么要背一整本账", section "再往后：压 KV 的三条路线":
K/V may be stored in FP8 with per-channel calibrated scales.  The reading
used on both sides: a channel is (layer, KV head, head_dim element), kept
separately for K and V; the stored code is the E4M3 round-to-nearest-even,
saturating encoding of the fp32 product x * inv_scale, one IEEE fp32
multiply.

The expected codes here come from torch's own float8_e4m3fn cast of a torch
fp32 product (an implementation that shares nothing with the oracle's
table-search encoder), from the format definition for the special values,
and from hand-built double-rounding cases that only a single fp32 multiply
followed by one rounding gets right.
"""
import numpy as np
import pytest
import torch

from oracle import PoolModel

L, NB, HKV, BS, D = 3, 7, 3, 4, 8


def _torch_f32(bits, src):
    """fp32 value of source bit patterns, decoded by torch (not the oracle)."""
    if src == "f32":
        return torch.from_numpy(np.asarray(bits, np.uint32).view(np.int32)).view(torch.float32)
    t = torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16))
    return t.view(torch.bfloat16 if src == "bf16" else torch.float16).to(torch.float32)


def _src_bits(x_f32, src):
    """Round fp32 values to the source dtype with torch and return the bits."""
    t = torch.from_numpy(np.asarray(x_f32, np.float32))
    if src == "f32":
        return t.view(torch.int32).numpy().view(np.uint32)
    dt = torch.bfloat16 if src == "bf16" else torch.float16
    return t.to(dt).view(torch.int16).numpy().view(np.uint16)


def _scales(rng):
    # distinct per (layer, head, channel): a wrong layer, head or channel
    # index, or a transposed scale array, changes the codes
    scale = (rng.uniform(0.01, 0.4, (L, HKV, D)) * (1 + np.arange(L))[:, None, None]).astype(np.float32)
    inv = (np.float32(1.0) / scale).astype(np.float32)
    return scale, inv


def _fp8_pool(rng):
    ks, kinv = _scales(rng)
    vs, vinv = _scales(rng)
    pool = PoolModel(L, NB, HKV, BS, D, "fp8", k_inv_scale=kinv, v_inv_scale=vinv,
                     k_scale=ks, v_scale=vs)
    return pool, kinv, vinv


@pytest.mark.parametrize("src", ["bf16", "f16", "f32"])
def test_fp8_append_codes_match_torch_cast(src):
    rng = np.random.default_rng(11)
    pool, kinv, vinv = _fp8_pool(rng)
    n = 9
    slots = rng.permutation(NB * BS)[:n]
    for layer in range(L):
        # magnitudes chosen so every product lies below torch's overflow
        # threshold (464), where its cast and the pages' saturating encoder agree
        k = (rng.standard_normal((n, HKV, D)) * 0.3 * rng.uniform(0.05, 1.0, (n, 1, 1))).astype(np.float32)
        v = (rng.standard_normal((n, HKV, D)) * 0.3).astype(np.float32)
        kb, vb = _src_bits(k, src), _src_bits(v, src)
        pool.append(layer, kb, vb, src, slots)
        for bits, inv, arr in ((kb, kinv, pool.k), (vb, vinv, pool.v)):
            y = _torch_f32(bits, src) * torch.from_numpy(inv[layer])[None]
            assert float(y.abs().max()) < 464.0
            want = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            for i, s in enumerate(slots):
                blk, off = divmod(int(s), BS)
                assert np.array_equal(arr[layer, blk, :, off, :], want[i]), (layer, i)
    # every layer was written with its own scales; none was left untouched
    assert pool.written.sum() == L * n


def test_fp8_append_special_values():
    # format definition (OCP E4M3): largest finite 448 = 0x7E, no infinities,
    # NaN = S.1111.111, signed zero kept; the encoder saturates
    pool = PoolModel(2, 2, 1, 2, 8, "fp8", k_inv_scale=np.ones((2, 1, 8), np.float32),
                     v_inv_scale=np.full((2, 1, 8), 2.0, np.float32),
                     k_scale=np.ones((2, 1, 8), np.float32),
                     v_scale=np.full((2, 1, 8), 0.5, np.float32))
    x = np.array([1000.0, -1000.0, np.inf, -np.inf, np.nan, -0.0, 0.0, 448.0], np.float32)
    bits = _src_bits(x, "bf16")[None, None, :]          # [1][1][8]
    pool.append(1, bits, bits, "bf16", [3])
    assert list(pool.k[1, 1, 0, 1]) == [0x7E, 0xFE, 0x7E, 0xFE, 0x7F, 0x80, 0x00, 0x7E]
    # V: inv scale 2 -> 448 * 2 saturates too; the rest as for K
    assert list(pool.v[1, 1, 0, 1]) == [0x7E, 0xFE, 0x7E, 0xFE, 0x7F, 0x80, 0x00, 0x7E]
    assert not pool.written[0].any()


def _double_rounding_cases():
    """(x, inv, code) with bf16 x and fp32 inv whose exact product lies just off
    an E4M3 midpoint while its fp32 rounding lands on the midpoint, so ties to
    even decides.  A bf16 x (8 significant bits) times an fp32 inv (24 bits) is
    exact in fp64, which is how the exact product is known here."""
    cases = []
    # midpoint 1.0625 of 1.0 (0x38, even) and 1.125 (0x39): exact above it
    # rounds to 0x39 once, but the fp32 product is the tie -> 0x38.
    # midpoint 1.1875 of 1.125 (0x39) and 1.25 (0x3A, even): exact below it
    # rounds to 0x39 once, but the fp32 product is the tie -> 0x3A.
    for mid, want, side in ((1.0625, 0x38, 1), (1.1875, 0x3A, -1)):
        for k in range(1, 128):
            x = np.float32(1 + k / 128)
            c = np.float32(mid / float(x))
            for d in range(-3, 4):
                inv = c
                for _ in range(abs(d)):
                    inv = np.nextafter(inv, np.float32(np.inf * np.sign(d)))
                exact = float(x) * float(inv)
                if float(x * inv) == mid and (exact - mid) * side > 0:
                    cases.append((float(x), float(inv), want))
    return cases


def test_fp8_append_rounds_the_fp32_product_once():
    cases = _double_rounding_cases()
    assert len(cases) >= 20
    D1 = 8
    for x, inv, want in cases:
        invs = np.full((1, 1, D1), inv, np.float32)
        pool = PoolModel(1, 1, 1, 1, D1, "fp8", k_inv_scale=invs, v_inv_scale=invs,
                         k_scale=1 / invs, v_scale=1 / invs)
        bits = _src_bits(np.full(D1, x, np.float32), "bf16")[None, None, :]
        pool.append(0, bits, bits, "bf16", [0])
        assert (pool.k[0, 0, 0, 0] == want).all(), (x, inv)
        assert (pool.v[0, 0, 0, 0] == want).all(), (x, inv)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_same_dtype_append_copies_bits(dt):
    # a pool in the source dtype stores the source bits unchanged, in the
    # right layer, block, head and offset
    rng = np.random.default_rng(5)
    pool = PoolModel(L, NB, HKV, BS, D, dt)
    n = 6
    slots = rng.permutation(NB * BS)[:n]
    x = rng.standard_normal((L, n, HKV, D)).astype(np.float32)
    for layer in range(L):
        b = _src_bits(x[layer], dt)
        pool.append(layer, b, b ^ 1, dt, slots)
        for i, s in enumerate(slots):
            blk, off = divmod(int(s), BS)
            assert np.array_equal(pool.k[layer, blk, :, off], b[i])
            assert np.array_equal(pool.v[layer, blk, :, off], b[i] ^ 1)


def test_copy_blocks_copies_every_layer():
    rng = np.random.default_rng(6)
    pool = PoolModel(L, NB, HKV, BS, D, "bf16")
    slots = np.arange(BS)                                      # fill block 0
    for layer in range(L):
        b = _src_bits(rng.standard_normal((BS, HKV, D)).astype(np.float32), "bf16")
        pool.append(layer, b, b, "bf16", slots)
    before = pool.k.copy()
    pool.copy_blocks([(0, 5)])
    for layer in range(L):
        assert np.array_equal(pool.k[layer, 5], before[layer, 0])
        assert np.array_equal(pool.v[layer, 5], pool.v[layer, 0])
    assert np.array_equal(pool.k[:, 0], before[:, 0])          # source unchanged
    assert pool.written[:, 5].all()
