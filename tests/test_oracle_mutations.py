"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each case swaps one oracle function for a plausibly wrong variant -- a wrong
index, a dropped term, an off-by-one -- runs the pin tests that should catch
it, and asserts that at least one of them fails.  Nothing here touches the
HIP library.
"""
import numpy as np
import pytest

import oracle
import oracle.allocator as alloc_mod
import oracle.attention as att_mod
import oracle.e4m3 as e4m3_mod
import oracle.pool as pool_mod
import test_oracle_allocator as TA
import test_oracle_attention as TT
import test_oracle_e4m3 as TE
import test_oracle_pool as TP


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _attention_pins():
    return [lambda: TT.test_brute_force(w, win) for w in TT.TINY for win in (0, 3)] + \
           [TT.test_closed_forms, TT.test_gqa_equals_mha_with_repeated_kv,
            lambda: TT.test_matches_torch_sdpa("c1")]


def _any_fails(pins):
    return any(_fails(p) for p in pins)


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    orig = att_mod.decode_attention

    def mutated(pool, layer, q, q_dtype, tables, lens, scale, window=0):
        # uses KV head h % Hkv instead of h // G
        B, Hq, _ = q.shape
        Hkv = pool.num_kv_heads
        G = Hq // Hkv
        perm = np.array([(h % Hkv) * G + h // Hkv for h in range(Hq)])
        out = orig(pool, layer, q[:, perm], q_dtype, tables, lens, scale, window)
        inv = np.argsort(perm)
        return out[:, inv]
    monkeypatch.setattr(TT, "decode_attention", mutated)
    assert _any_fails(_attention_pins())


def test_dropped_new_token_is_caught(monkeypatch):
    orig = att_mod.decode_attention
    monkeypatch.setattr(TT, "decode_attention",
                        lambda pool, layer, q, qd, t, lens, sc, window=0:
                        orig(pool, layer, q, qd, t, np.maximum(np.asarray(lens) - 1, 0), sc, window))
    assert _any_fails(_attention_pins())


def test_missing_scale_is_caught(monkeypatch):
    orig = att_mod.decode_attention
    monkeypatch.setattr(TT, "decode_attention",
                        lambda pool, layer, q, qd, t, lens, sc, window=0:
                        orig(pool, layer, q, qd, t, lens, 1.0, window))
    assert _any_fails(_attention_pins())


def test_window_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(att_mod, "_key_range",
                        lambda L, window: ((max(0, L - window + 1) if window else 0), L))
    assert _any_fails(_attention_pins())


def test_merge_without_rescaling_l_is_caught(monkeypatch):
    def bad_merge(parts):
        ms = np.array([m for _, m, _ in parts])
        M = ms.max()
        w = np.exp(ms - M)
        return sum(wi * o for wi, (o, _, _) in zip(w, parts)) / sum(l for _, _, l in parts)
    monkeypatch.setattr(att_mod, "lse_merge", bad_merge)
    monkeypatch.setattr(TT, "lse_merge", bad_merge)
    assert _fails(TT.test_lse_merge_identity) or _fails(TT.test_partial_and_merge_edge_cases)


def test_allocator_without_cow_is_caught(monkeypatch):
    orig = alloc_mod.BlockManager._append_one_seq

    def no_cow(self, seq, n):
        # pretend every block is private: write into shared blocks in place
        saved = list(self._ref)
        self._ref = [min(r, 1) for r in self._ref]
        try:
            return orig(self, seq, n)
        finally:
            self._ref = [max(a, b) if a > 1 else b for a, b in zip(saved, self._ref)]
    monkeypatch.setattr(alloc_mod.BlockManager, "_append_one_seq", no_cow)
    pins = [lambda s=s: TA.test_random_ops_tiny_pools(s) for s in range(10)] + \
           [TA.test_cow_on_shared_partial_block]
    assert _any_fails(pins)


def test_allocator_eager_block_is_caught(monkeypatch):
    # take the next block as soon as the current one fills, instead of when
    # the first token that needs it arrives
    orig = alloc_mod.BlockManager._append_one_seq

    def eager(self, seq, n_tokens):
        slots, cows = orig(self, seq, n_tokens)
        bs = self.block_size
        tab = self._tables[seq]
        if self._lens[seq] % bs == 0 and self._free and len(tab) * bs == self._lens[seq]:
            blk = self._free.popleft()
            self._ref[blk] = 1
            tab.append(blk)
        return slots, cows
    monkeypatch.setattr(alloc_mod.BlockManager, "_append_one_seq", eager)
    assert _fails(TA.test_figure_mapping) or _fails(TA.test_block_counts_of_tiny_workload)


def test_e4m3_ties_away_from_zero_is_caught(monkeypatch):
    orig = e4m3_mod.e4m3_encode

    def away(x):
        a = np.asarray(x, dtype=np.float64)
        c = orig(a)
        t = e4m3_mod._TABLE
        bumped = np.where(np.abs(a) > np.abs(t[c]), c + 1, c).astype(np.uint8)
        return np.where(np.isnan(a) | (np.abs(a) >= 448), c, bumped).astype(np.uint8)
    monkeypatch.setattr(TE, "e4m3_encode", away)
    assert _fails(TE.test_ties_go_to_even_mantissa) or _fails(TE.test_matches_torch_float8_in_range)


def test_e4m3_wrong_bias_is_caught(monkeypatch):
    monkeypatch.setattr(e4m3_mod, "_EXP_BIAS", 8)
    monkeypatch.setattr(TE, "e4m3_decode_table", e4m3_mod.e4m3_decode_table)
    assert _fails(TE.test_special_values_from_format_definition)


def test_release_one_block_too_many_is_caught(monkeypatch):
    # release the block that contains `token` as well (off by one)
    def too_many(self, seq, token):
        self._check(seq)
        tab = self._tables[seq]
        n = 0
        for i in range(min(len(tab), token // self.block_size + 1)):
            blk = tab[i]
            if blk < 0:
                continue
            self._ref[blk] -= 1
            if self._ref[blk] == 0:
                self._free.append(blk)
            tab[i] = -1
            n += 1
        return n
    monkeypatch.setattr(alloc_mod.BlockManager, "release_before", too_many)
    pins = [lambda s=s: TA.test_random_ops_tiny_pools(s) for s in range(20)] + \
           [TA.test_window_release_bounds_held_blocks]
    assert _any_fails(pins)


def test_release_without_freeing_is_caught(monkeypatch):
    # mark entries released but never give the blocks back
    def leak(self, seq, token):
        tab = self._tables[seq]
        n = 0
        for i in range(token // self.block_size):
            if tab[i] >= 0:
                tab[i] = -1
                n += 1
        return n
    monkeypatch.setattr(alloc_mod.BlockManager, "release_before", leak)
    pins = [lambda s=s: TA.test_random_ops_tiny_pools(s) for s in range(20)] + \
           [TA.test_window_release_bounds_held_blocks]
    assert _any_fails(pins)


def _fp8_pool_pins():
    return [lambda s=s: TP.test_fp8_append_codes_match_torch_cast(s) for s in ("bf16", "f16", "f32")] + \
           [TP.test_fp8_append_special_values, TP.test_fp8_append_rounds_the_fp32_product_once]


def test_pool_fp8_round_toward_zero_is_caught(monkeypatch):
    orig = e4m3_mod.e4m3_encode

    def rtz(x):
        # truncate the magnitude to the code at or below it
        a = np.asarray(x, dtype=np.float64)
        c = orig(a)
        t = e4m3_mod._TABLE
        over = np.isfinite(a) & (np.abs(t[c]) > np.abs(a)) & ((c & 0x7F) != 0)
        return np.where(over, c - 1, c).astype(np.uint8)
    monkeypatch.setattr(pool_mod, "e4m3_encode", rtz)
    assert _any_fails(_fp8_pool_pins())


def test_pool_fp8_fp64_multiply_is_caught(monkeypatch):
    def encode64(self, bits, src_dtype, inv_scale_layer):
        if self.kv_dtype == src_dtype:
            return np.asarray(bits, dtype=pool_mod.BITS_DTYPE[src_dtype])
        x = pool_mod.bits_to_f64(bits, src_dtype)
        return e4m3_mod.e4m3_encode(x * inv_scale_layer.astype(np.float64)[None])
    monkeypatch.setattr(pool_mod.PoolModel, "_encode", encode64)
    assert _any_fails(_fp8_pool_pins())


def test_pool_fp8_layer_zero_scales_is_caught(monkeypatch):
    # quantise every layer with layer 0's inverse scales
    orig = pool_mod.PoolModel.append

    def first_layer_scales(self, layer, k_bits, v_bits, src_dtype, slots):
        if self.kv_dtype != "fp8":
            return orig(self, layer, k_bits, v_bits, src_dtype, slots)
        saved = self.k_inv_scale, self.v_inv_scale
        self.k_inv_scale = np.broadcast_to(saved[0][:1], saved[0].shape)
        self.v_inv_scale = np.broadcast_to(saved[1][:1], saved[1].shape)
        try:
            return orig(self, layer, k_bits, v_bits, src_dtype, slots)
        finally:
            self.k_inv_scale, self.v_inv_scale = saved
    monkeypatch.setattr(pool_mod.PoolModel, "append", first_layer_scales)
    assert _any_fails(_fp8_pool_pins())
