"""Pins of the oracle against things other than itself (CPU only).

* the worked block-table example printed on the deep-dive page;
* hand-worked offsets of the documented cache layout;
* torch's scaled_dot_product_attention in float64 (an independent library
  routine) on contiguous K/V assembled straight from the random draws, never
  through a block table;
* closed forms (one token returns V exactly; equal keys or a zero query give
  the mean of V; a dominant key returns its value);
* invariants (softmax weights sum to 1; any permutation of physical blocks
  gives bit-identical results; shared-prefix sequences equal unshared copies;
  a prefill row equals decode at the matching context; the partition merge
  equals the one-pass result).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, cache, run
from oracle.alloc_model import OK, AllocModel
from synth import Spec, decode_script, prefill_script, shared_prefix_script

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def logical_tokens(script):
    """Per-sequence K/V by logical position, straight from the draws: new ->
    empty, append -> extend, fork -> copy of the parent.  No allocator, no
    block table, no cache layout is involved."""
    toks = {}
    for op in script.ops():
        if op.kind == "new":
            toks[op.seq] = ([], [])
        elif op.kind == "fork":
            toks[op.seq] = (list(toks[op.parent][0]), list(toks[op.parent][1]))
        else:
            k, v = script.kv(op)
            toks[op.seq][0].extend(k)
            toks[op.seq][1].extend(v)
    d = script.spec.dtype
    return {s: (cache.to_f64(np.array(k), d), cache.to_f64(np.array(v), d)) for s, (k, v) in toks.items()}


def sdpa(q, k, v, scale, causal_offset=None):
    """torch SDPA in float64: q [H, n, D], k/v [KVH, L, D]."""
    qt = torch.from_numpy(q)[None]
    kt = torch.from_numpy(k)[None]
    vt = torch.from_numpy(v)[None]
    mask = None
    if causal_offset is not None:
        n, L = q.shape[1], k.shape[1]
        mask = (torch.arange(L)[None, :] <= (causal_offset + torch.arange(n))[:, None])
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=True)
    return out[0].numpy()


# ---------------------------------------------------------------- golden
def test_worked_block_table_example():
    g = json.load(open(os.path.join(GOLDEN, "worked_block_tables.json")))
    bs = g["block_size"]
    head = g["free_order_head"]
    order = head + [b for b in range(64) if b not in head]
    m = AllocModel(64, bs, order)
    slots = {}
    for s in g["sequences"]:
        assert m.new(s["seq"]) == OK
        rc, sl, pairs = m.append(s["seq"], s["tokens"])
        assert rc == OK and pairs == []
        slots[s["seq"]] = sl
        assert len(m.block_table(s["seq"])) == s["num_blocks"] == math.ceil(s["tokens"] / bs)
        assert m.block_table(s["seq"]) == s["block_table"]
    for e in g["slots"]:
        assert slots[e["seq"]][e["position"]] == e["slot"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cache_layout_offsets(dtype):
    g = json.load(open(os.path.join(GOLDEN, "cache_layout_small.json")))[dtype]
    assert cache.chunk_elems(dtype) == g["X"]
    nb, kvh, d, bs = g["num_blocks"], g["num_kv_heads"], g["head_dim"], g["block_size"]
    for e in g["entries"]:
        kc, vc = cache.empty_cache(nb, kvh, d, bs, dtype, poison=0)
        key = np.zeros((1, kvh, d), cache.storage_dtype(dtype))
        val = np.zeros((1, kvh, d), cache.storage_dtype(dtype))
        key[0, e["head"], e["dim"]] = 7
        val[0, e["head"], e["dim"]] = 9
        cache.reshape_and_cache(key, val, kc, vc, np.array([e["block"] * bs + e["offset"]]))
        assert np.flatnonzero(kc.reshape(-1)).tolist() == [e["k_flat"]]
        assert np.flatnonzero(vc.reshape(-1)).tolist() == [e["v_flat"]]


def test_negative_slot_is_skipped_and_poison_kept():
    kc, vc = cache.empty_cache(4, 2, 16, 4, "bf16")
    k = np.arange(3 * 2 * 16, dtype=np.uint16).reshape(3, 2, 16)
    cache.reshape_and_cache(k, k + 1, kc, vc, np.array([5, -1, 14]))
    touched = np.zeros((4, 4), bool)
    touched[1, 1] = touched[3, 2] = True
    for b in range(4):
        for o in range(4):
            for g in range(2):
                kr = cache.read_key(kc, b, g, o)
                if touched[b, o]:
                    src = 0 if (b, o) == (1, 1) else 2
                    assert np.array_equal(kr, k[src, g])
                    assert np.array_equal(cache.read_value(vc, b, g, o), k[src, g] + 1)
                else:
                    assert np.all(kr == 0xFFFF)


# ---------------------------------------------------------------- library routine
def _decode_vs_sdpa(spec, lens, seed):
    sc = decode_script(spec, lens, seed)
    st = run.build(sc)
    q = sc.q()
    out = run.step_output(st, sc, q)
    toks = logical_tokens(sc)
    q64 = cache.to_f64(q, spec.dtype)
    for i, s in enumerate(sc.batch):
        K, V = toks[s]
        assert K.shape[0] == lens[i]
        ref = sdpa(q64[i][:, None, :], K.transpose(1, 0, 2), V.transpose(1, 0, 2), spec.scale)[:, 0]
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_matches_torch_sdpa(dtype):
    spec = Spec("t", "decode", 6, 2, 16, 4, dtype)
    _decode_vs_sdpa(spec, [1, 2, 5, 13, 16, 17], seed=11)


def test_decode_mha_head_dim_128_matches_torch_sdpa():
    spec = Spec("t", "decode", 2, 2, 128, 16, "bf16")
    _decode_vs_sdpa(spec, [33, 70], seed=12)


@pytest.mark.parametrize("cached", [[0, 0], [0, 20, 9]])
def test_prefill_matches_torch_sdpa(cached):
    spec = Spec("t", "prefill", 4, 2, 16, 4, "bf16")
    chunk = 7
    sc = prefill_script(spec, cached, chunk, seed=13)
    st = run.build(sc)
    q = sc.q()
    out = run.step_output(st, sc, q)
    toks = logical_tokens(sc)
    q64 = cache.to_f64(q, "bf16")
    for i, s in enumerate(sc.batch):
        K, V = toks[s]
        qs = q64[i * chunk:(i + 1) * chunk].transpose(1, 0, 2)
        if cached[i] == 0:
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qs)[None], torch.from_numpy(K.transpose(1, 0, 2))[None],
                torch.from_numpy(V.transpose(1, 0, 2))[None], is_causal=True, scale=spec.scale,
                enable_gqa=True)[0].numpy()
        else:
            ref = sdpa(qs, K.transpose(1, 0, 2), V.transpose(1, 0, 2), spec.scale,
                       causal_offset=cached[i])
        np.testing.assert_allclose(out[i * chunk:(i + 1) * chunk], ref.transpose(1, 0, 2),
                                   rtol=1e-12, atol=1e-13)


def test_shared_prefix_decode_matches_torch_sdpa():
    spec = Spec("t", "decode", 2, 2, 16, 4, "bf16")
    sc = shared_prefix_script(spec, prompts=2, samples=3, prefix=6, suffix_lens=[1, 3, 5, 2, 4, 9],
                              seed=14)
    st = run.build(sc)
    assert st.cow_pairs, "a 6-token prefix leaves a partial shared block, so CoW must fire"
    q = sc.q()
    out = run.step_output(st, sc, q)
    toks = logical_tokens(sc)
    q64 = cache.to_f64(q, "bf16")
    for i, s in enumerate(sc.batch):
        K, V = toks[s]
        ref = sdpa(q64[i][:, None, :], K.transpose(1, 0, 2), V.transpose(1, 0, 2), spec.scale)[:, 0]
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- closed forms
def _one_seq_cache(K, V, bs=4, order=None, dtype="f32"):
    L, D = K.shape
    nb = max(1, -(-L // bs))
    order = list(range(nb)) if order is None else order
    m = AllocModel(nb, bs, order)
    m.new(0)
    rc, slots, _ = m.append(0, L)
    assert rc == OK
    kc, vc = cache.empty_cache(nb, 1, D, bs, dtype)
    cache.reshape_and_cache(K[:, None, :].astype(np.float32), V[:, None, :].astype(np.float32), kc, vc,
                            np.array(slots))
    return kc, vc, np.array(m.padded_tables([0], nb), np.int32)


def test_single_token_returns_v_exactly():
    g = np.random.default_rng(0)
    K = g.standard_normal((1, 8)).astype(np.float32)
    V = g.standard_normal((1, 8)).astype(np.float32)
    kc, vc, bt = _one_seq_cache(K, V)
    q = g.standard_normal((1, 1, 8)).astype(np.float32)
    out = attention.decode(q, kc, vc, bt, np.array([1]), 0.3, "f32")
    assert np.array_equal(out[0, 0], V[0].astype(np.float64))


def test_equal_keys_and_zero_query_give_mean_of_v():
    g = np.random.default_rng(1)
    V = g.standard_normal((11, 8)).astype(np.float32)
    K = np.repeat(g.standard_normal((1, 8)).astype(np.float32), 11, 0)
    kc, vc, bt = _one_seq_cache(K, V)
    q = g.standard_normal((1, 1, 8)).astype(np.float32)
    mean = V.astype(np.float64).mean(0)
    np.testing.assert_allclose(attention.decode(q, kc, vc, bt, np.array([11]), 0.7, "f32")[0, 0],
                               mean, rtol=0, atol=1e-14)
    K2 = g.standard_normal((11, 8)).astype(np.float32)
    kc, vc, bt = _one_seq_cache(K2, V)
    np.testing.assert_allclose(attention.decode(np.zeros_like(q), kc, vc, bt, np.array([11]), 0.7,
                                                "f32")[0, 0], mean, rtol=0, atol=1e-14)


def test_dominant_key_returns_its_value():
    g = np.random.default_rng(2)
    V = g.standard_normal((9, 8)).astype(np.float32)
    K = np.zeros((9, 8), np.float32)
    K[6, 0] = 1.0
    q = np.zeros((1, 1, 8), np.float32)
    q[0, 0, 0] = 1.0
    kc, vc, bt = _one_seq_cache(K, V)
    out = attention.decode(q, kc, vc, bt, np.array([9]), 1000.0, "f32")[0, 0]
    np.testing.assert_allclose(out, V[6].astype(np.float64), rtol=0, atol=1e-300 + 1e-12)


def test_empty_context_gives_zero_row():
    kc, vc = cache.empty_cache(2, 1, 8, 4, "f32")
    out = attention.decode(np.ones((1, 1, 8), np.float32), kc, vc, np.array([[-1, -1]], np.int32),
                           np.array([0]), 0.5, "f32")
    assert np.array_equal(out, np.zeros((1, 1, 8)))


# ---------------------------------------------------------------- invariants
def test_softmax_weights_sum_to_one():
    spec = Spec("t", "decode", 4, 2, 16, 4, "bf16")
    sc = decode_script(spec, [3, 40, 17], seed=5)
    st = run.build(sc)
    q = sc.q()
    tables, lens = run.batch_tables(st, sc)
    ref = attention.decode(q, st.k_cache, st.v_cache, tables, lens, spec.scale, "bf16")
    for i in range(3):
        for h in range(4):
            p = attention.decode_weights(q[i, h], st.k_cache, st.v_cache, tables[i], lens[i], h, 2,
                                         spec.scale, "bf16")
            assert p.shape == (lens[i],) and np.all(p > 0)
            assert abs(p.sum() - 1.0) <= 1e-12
            # the weights' head map: applied to the values of kv head h // 2
            # (heads 0, 1 -> 0; 2, 3 -> 1) they give decode's row, which the
            # SDPA pins fix independently
            _, V = attention.gather_kv(st.k_cache, st.v_cache, tables[i], lens[i], h // 2, "bf16")
            np.testing.assert_allclose(p @ V, ref[i, h], rtol=0, atol=1e-12)


def test_physical_block_permutation_is_bit_invariant():
    spec = Spec("t", "decode", 4, 2, 16, 4, "bf16")
    lens = [7, 29, 16, 1]
    sc = decode_script(spec, lens, seed=6)
    outs, tables = [], []
    for perm_seed in (0, 1, 2):
        sc.free_order = np.random.default_rng(perm_seed).permutation(sc.num_blocks).astype(np.int32)
        st = run.build(sc)
        outs.append(run.step_output(st, sc, sc.q()))
        tables.append(run.batch_tables(st, sc)[0])
    assert not np.array_equal(tables[0], tables[1]), "placements must differ"
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_shared_prefix_equals_unshared_copies():
    spec = Spec("t", "decode", 2, 2, 16, 4, "bf16")
    suffix = [2, 5, 1, 8]
    shared = shared_prefix_script(spec, prompts=1, samples=4, prefix=9, suffix_lens=suffix, seed=7)
    st = run.build(shared)
    out_shared = run.step_output(st, shared, shared.q())
    # Unshared: each sample is its own sequence holding a private copy of the
    # prefix tokens followed by its suffix tokens.
    toks = logical_tokens(shared)
    for i, s in enumerate(shared.batch):
        K, V = toks[s]
        m = AllocModel(64, 4, np.random.default_rng(i).permutation(64))
        m.new(0)
        rc, slots, _ = m.append(0, len(K))
        kc, vc = cache.empty_cache(64, 2, 16, 4, "bf16")
        # rebuild the stored bf16 bit patterns from the float64 values (exact)
        kb = (K.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        vb = (V.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        cache.reshape_and_cache(kb, vb, kc, vc, np.array(slots))
        bt = np.array(m.padded_tables([0], 16), np.int32)
        out = attention.decode(shared.q()[i:i + 1], kc, vc, bt, np.array([len(K)]), spec.scale, "bf16")
        assert np.array_equal(out[0], out_shared[i])


def test_prefill_row_equals_decode_at_matching_context():
    spec = Spec("t", "prefill", 2, 1, 16, 4, "bf16")
    cached, chunk = [5, 12], 6
    sc = prefill_script(spec, cached, chunk, seed=8)
    st = run.build(sc)
    q = sc.q()
    out = run.step_output(st, sc, q)
    tables, lens = run.batch_tables(st, sc)
    for s in range(2):
        for i in range(chunk):
            r = s * chunk + i
            dec = attention.decode(q[r:r + 1], st.k_cache, st.v_cache, tables[s:s + 1],
                                   np.array([cached[s] + i + 1]), spec.scale, "bf16")
            np.testing.assert_allclose(out[r], dec[0], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("partition", [1, 3, 16, 100])
def test_partition_merge_equals_one_pass(partition):
    g = np.random.default_rng(9)
    for L in (1, 5, 16, 17, 64):
        K = g.standard_normal((L, 8)) * 3
        V = g.standard_normal((L, 8))
        q = g.standard_normal(8)
        a = attention.attend(q, K, V, 0.9)
        b = attention.decode_partitioned(q, K, V, 0.9, partition)
        np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-14)


# ------------------------------------------------ page readers, matrix-form prefill
def test_page_readers_match_row_readers():
    """read_key_page / read_value_page row o is the row read_key / read_value
    return for offset o (pinned to the hand-worked layout by the golden test)."""
    g = np.random.default_rng(11)
    for dtype, x in (("bf16", 8), ("f32", 4)):
        kc, vc = cache.empty_cache(3, 2, 16, 8, dtype)
        raw = g.integers(0, 1 << 15, size=kc.size).astype(kc.dtype if dtype == "bf16" else np.float32)
        kc[...] = raw.reshape(kc.shape)
        vc[...] = g.integers(0, 1 << 15, size=vc.size).astype(vc.dtype).reshape(vc.shape)
        for b in range(3):
            for h in range(2):
                kp, vp = cache.read_key_page(kc, b, h), cache.read_value_page(vc, b, h)
                assert kp.shape == (8, 16) and vp.shape == (8, 16)
                for o in range(8):
                    assert np.array_equal(kp[o], cache.read_key(kc, b, h, o))
                    assert np.array_equal(vp[o], cache.read_value(vc, b, h, o))


def test_prefill_rows_matches_row_by_row():
    """The matrix form over every row equals the per-row oracle (pinned to
    SDPA) to 1e-12, for ragged chunks and grouped heads."""
    spec = Spec("t", "prefill", 4, 2, 16, 4, "bf16")
    sc = prefill_script(spec, [0, 5, 13], 7, seed=31)
    st = run.build(sc)
    tables, lens = run.batch_tables(st, sc)
    q = sc.q()
    qsl = np.concatenate([[0], np.cumsum(sc.query_lens)]).astype(np.int32)
    ref = attention.prefill(q, st.k_cache, st.v_cache, tables, qsl, lens, spec.scale, "bf16")
    got = attention.prefill_rows(q, st.k_cache, st.v_cache, tables, qsl, lens, spec.scale, "bf16")
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
