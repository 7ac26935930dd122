"""The pins catch planted mistakes (CPU only).

Each case plants one plausible mistake in a copy of an oracle routine --
a transposed layout index, a dropped scale, a wrong GQA head map, an off-by-one
causal boundary, a skipped copy-on-write -- and checks that the matching pin
in test_oracle_pins / test_alloc_model now fails.  The mistakes live only in
this file and only on the CPU.
"""

import numpy as np
import pytest

import oracle.attention as attention
import oracle.cache as cache
from oracle.alloc_model import AllocModel
from tests import test_alloc_model as tam
from tests import test_oracle_pins as pins


def _expect_failure(fn, *args, **kw):
    with pytest.raises(AssertionError):
        fn(*args, **kw)


def test_transposed_key_layout_is_caught(monkeypatch):
    def bad_read_key_page(k_cache, block, head):
        return k_cache[block, head].reshape(k_cache.shape[3], -1)  # chunks not moved behind tokens
    monkeypatch.setattr(attention, "read_key_page", bad_read_key_page)
    _expect_failure(pins.test_decode_matches_torch_sdpa, "bf16")


def test_wrong_offset_in_gather_is_caught(monkeypatch):
    def bad_read_value_page(v_cache, block, head):
        return np.roll(v_cache[block, head].T, 1, axis=0)
    monkeypatch.setattr(attention, "read_value_page", bad_read_value_page)
    _expect_failure(pins.test_decode_matches_torch_sdpa, "f32")


def test_page_reader_off_by_one_is_caught(monkeypatch):
    def bad(k_cache, block, head):
        page = k_cache[block, head]
        return np.roll(page.transpose(1, 0, 2).reshape(page.shape[1], -1), -1, axis=0)
    monkeypatch.setattr(cache, "read_key_page", bad)
    _expect_failure(pins.test_page_readers_match_row_readers)


def test_prefill_rows_mask_off_by_one_is_caught(monkeypatch):
    def bad_prefill_rows(q, k_cache, v_cache, block_tables, qsl, lens, scale, dtype):
        q64 = cache.to_f64(q, dtype)
        Tq, H, D = q64.shape
        group = H // k_cache.shape[1]
        out = np.zeros((Tq, H, D))
        for s in range(len(lens)):
            r0, r1 = int(qsl[s]), int(qsl[s + 1])
            n_q, L = r1 - r0, int(lens[s])
            pos = L - n_q + np.arange(n_q)
            masked = np.arange(L)[None, :] >= pos[:, None]  # mistake: hides the query's own key
            for h in range(H):
                K, V = attention.gather_kv(k_cache, v_cache, block_tables[s], L, h // group, dtype)
                S = float(scale) * (q64[r0:r1, h] @ K.T)
                S[masked] = -np.inf
                P = np.exp(S - S.max(axis=1, keepdims=True))
                out[r0:r1, h] = np.nan_to_num(P / P.sum(axis=1, keepdims=True)) @ V
        return out
    monkeypatch.setattr(attention, "prefill_rows", bad_prefill_rows)
    _expect_failure(pins.test_prefill_rows_matches_row_by_row)


def test_dropped_scale_is_caught(monkeypatch):
    orig = attention.softmax_weights
    monkeypatch.setattr(attention, "softmax_weights", lambda q, K, scale: orig(q, K, 1.0))
    _expect_failure(pins.test_decode_matches_torch_sdpa, "f32")


def test_wrong_max_sign_is_caught(monkeypatch):
    def bad(q, K, scale):
        s = float(scale) * (K @ q)
        e = np.exp(-(s - s.max()))
        return e / e.sum()
    monkeypatch.setattr(attention, "softmax_weights", bad)
    _expect_failure(pins.test_decode_matches_torch_sdpa, "f32")


def test_wrong_gqa_head_map_is_caught(monkeypatch):
    orig = attention.gather_kv

    def bad_gather(k_cache, v_cache, bt, L, kv_head, dtype):
        # serve the other KV head: h % KVH instead of h // group
        return orig(k_cache, v_cache, bt, L, (kv_head + 1) % k_cache.shape[1], dtype)
    monkeypatch.setattr(attention, "gather_kv", bad_gather)
    _expect_failure(pins.test_decode_matches_torch_sdpa, "bf16")


def test_wrong_head_map_in_decode_weights_is_caught(monkeypatch):
    orig = attention.gather_kv

    def bad_weights(q, k_cache, v_cache, bt, L, head, group, scale, dtype):
        # query head h read against kv head h % KVH instead of h // group
        K, _ = orig(k_cache, v_cache, bt, L, head % k_cache.shape[1], dtype)
        return attention.softmax_weights(cache.to_f64(q, dtype), K, scale)
    monkeypatch.setattr(attention, "decode_weights", bad_weights)
    _expect_failure(pins.test_softmax_weights_sum_to_one)


def test_causal_off_by_one_is_caught(monkeypatch):
    orig = attention.attend

    def bad_attend(q, K, V, scale):
        return orig(q, K[:-1] if K.shape[0] > 1 else K, V[:-1] if V.shape[0] > 1 else V, scale)
    monkeypatch.setattr(attention, "attend", bad_attend)
    _expect_failure(pins.test_prefill_matches_torch_sdpa, [0, 0])


def test_transposed_value_write_is_caught(monkeypatch):
    def bad_write(key, value, k_cache, v_cache, slot_mapping):
        bs, x = k_cache.shape[3], k_cache.shape[4]
        for i, slot in enumerate(slot_mapping):
            if slot < 0:
                continue
            b, o = int(slot) // bs, int(slot) % bs
            for g in range(key.shape[1]):
                k_cache[b, g, :, o, :] = key[i, g].reshape(-1, x)
                v_cache[b, g, :, o] = value[i, g][::-1]
    monkeypatch.setattr(cache, "reshape_and_cache", bad_write)
    _expect_failure(pins.test_cache_layout_offsets, "bf16")


def test_skipped_copy_on_write_is_caught(monkeypatch):
    def bad_append(self, seq, n):
        bs = self.block_size
        table = self.tables[seq]
        L = self.lens[seq]
        grow = -(-(L + n) // bs) - len(table)
        if grow > len(self.free):
            return -2, [], []
        for _ in range(grow):
            b = self.free.pop()
            self.refcount[b] = 1
            table.append(b)
        self.lens[seq] = L + n
        return 0, [table[p // bs] * bs + p % bs for p in range(L, L + n)], []
    monkeypatch.setattr(AllocModel, "append", bad_append)
    _expect_failure(tam.test_random_operations_keep_sharing_semantics, 0, 40, 16)


def test_fork_without_refcount_is_caught(monkeypatch):
    def bad_fork(self, parent, child):
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        return 0
    monkeypatch.setattr(AllocModel, "fork", bad_fork)
    _expect_failure(tam.test_random_operations_keep_sharing_semantics, 1, 40, 16)


def test_wrong_merge_weight_is_caught(monkeypatch):
    def bad_partitioned(q_row, K, V, scale, partition):
        outs = []
        for a in range(0, K.shape[0], partition):
            outs.append(attention.attend(q_row, K[a:a + partition], V[a:a + partition], scale))
        return np.mean(outs, 0)  # forgets the l_p * exp(m_p - M) weights
    monkeypatch.setattr(attention, "decode_partitioned", bad_partitioned)
    _expect_failure(pins.test_partition_merge_equals_one_pass, 3)


# ---------------------------------------------------------------- prefix caching
from tests import test_prefix_cache as tpc


def test_most_recent_first_eviction_is_caught(monkeypatch):
    def bad_kept(self):
        ks = [b for b in self.cached if self.refcount[b] == 0]
        return sorted(ks, key=lambda b: (-self.last_use[b], -self.cached[b].depth, b))
    monkeypatch.setattr(AllocModel, "_kept", bad_kept)
    _expect_failure(tpc.test_worked_scenario_match_keep_and_evict)


def test_matching_the_whole_prompt_is_caught(monkeypatch):
    def bad_new_cached(self, seq, prompt):
        # a copy of AllocModel.new_cached that may match every full block,
        # leaving no prompt token to compute
        if seq in self.tables:
            return -4, 0
        self.clock += 1
        bs = self.block_size
        prompt = [int(t) for t in prompt]
        node, table = self.root, []
        for i in range(len(prompt) // bs):
            key = tuple(prompt[i * bs:(i + 1) * bs])
            if key not in node.children:
                break
            node = node.children[key]
            self.refcount[node.block] += 1
            self.last_use[node.block] = self.clock
            table.append(node.block)
        n_hit = len(table) * bs
        self.tables[seq], self.lens[seq] = table, n_hit
        self.tokens[seq], self.walk[seq] = prompt[:n_hit], node
        self.hit_tokens += n_hit
        self.query_tokens += len(prompt)
        return 0, n_hit
    monkeypatch.setattr(AllocModel, "new_cached", bad_new_cached)
    _expect_failure(tpc.test_worked_scenario_match_keep_and_evict)


def test_freeing_kept_blocks_is_caught(monkeypatch):
    def bad_release(self, b):
        self.free.append(b)
    monkeypatch.setattr(AllocModel, "_release", bad_release)
    _expect_failure(tpc.test_worked_scenario_match_keep_and_evict)


def test_registering_partial_blocks_is_caught(monkeypatch):
    orig = AllocModel._register

    def bad_register(self, seq, first, last):
        # also enter the partially filled tail block
        L = self.lens[seq]
        return orig(self, seq, first, -(-L // self.block_size) if L % self.block_size else last)
    monkeypatch.setattr(AllocModel, "_register", bad_register)
    _expect_failure(tpc.test_worked_scenario_match_keep_and_evict)
