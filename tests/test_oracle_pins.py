"""Pins of the oracle against what the pages and the mathematics fix (CPU only).

Each test ties the paged C oracle to something other than itself: the pages'
worked examples (tests/golden/), brute-force dense attention written out in
numpy, closed forms, and invariances the pages state in prose.
"""
import dataclasses
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def q64(wl):
    return W.to_f64(W.q_host(wl), wl.dtype)


def dense_rows(wl, s):
    """Brute-force dense attention for sequence s on its contiguous K/V."""
    a, b = wl.query_start_loc[s], wl.query_start_loc[s + 1]
    k = W.to_f64(W.seq_kv_host(wl, s, "k"), wl.dtype)
    v = W.to_f64(W.seq_kv_host(wl, s, "v"), wl.dtype)
    return oracle.dense_attention(q64(wl)[a:b], k, v, int(wl.context_lens[s]), wl.scale)


def run_attention(wl, pool, q=None, tables=None):
    q = W.q_host(wl) if q is None else q
    bt = wl.block_tables if tables is None else tables
    return oracle.attention(q, pool, bt, wl.query_start_loc, wl.seq_lens, wl.context_lens, wl.scale, wl.dtype)


# --- block arithmetic ---------------------------------------------------------
@pytest.mark.parametrize("cfg,expected", [(1, 16384), (2, 16384), (3, 65536), (4, 65536), (5, 65536)])
def test_block_bytes_formula_and_pool_stride(cfg, expected):
    g = gold("block_arithmetic.json")
    wl = W.config_workload(cfg)
    formula = 2 * g["block_size"] * wl.num_kv_heads * wl.head_size * wl.elem_bytes
    assert formula == expected == wl.block_bytes
    if wl.dtype == "bf16":
        assert wl.elem_bytes == g["bf16_bytes"]
    pool = W.pool_host(W.sub_workload(wl, [0]))
    assert pool.strides[0] == expected  # one physical block is exactly that many bytes


def test_seventeen_tokens_take_two_blocks():
    g = gold("block_arithmetic.json")["ceil_example"]
    wl = W.config_workload(1)
    s = list(wl.seq_lens).index(g["tokens"])
    assert wl.blocks_used(s) == g["blocks"]
    out, pool = oracle.run_workload(wl)
    # The oracle reads exactly ceil(17/16) = 2 table entries for that sequence:
    bt = wl.block_tables.copy()
    bt[s, g["blocks"]:] = -1
    assert np.array_equal(run_attention(wl, pool, tables=bt), out)
    bt[s, g["blocks"] - 1] = -1
    with pytest.raises(oracle.OracleError):
        run_attention(wl, pool, tables=bt)


# --- KV write and gather through a block table -------------------------------------
def test_ngrok_block_table_places_tokens_in_order():
    g = gold("ngrok_block_table.json")
    table, bs = g["block_table"], g["block_size"]
    L, Hkv, D, NB = len(table) * bs, 2, 8, 10
    rs = np.random.default_rng(0)
    k = rs.standard_normal((L, Hkv, D)).astype(np.float32)
    v = rs.standard_normal((L, Hkv, D)).astype(np.float32)
    pool = np.full((NB, 2, bs, Hkv, D), np.nan, np.float32)
    slots = np.array([table[j // bs] * bs + j % bs for j in range(L)], np.int64)
    assert slots[17] == 5 * 16 + 1
    oracle.reshape_and_cache(k, v, pool, slots, "f32")
    for j in range(L):
        assert np.array_equal(pool[table[j // bs], 0, j % bs], k[j])
        assert np.array_equal(pool[table[j // bs], 1, j % bs], v[j])
    untouched = [b for b in range(NB) if b not in table]
    assert np.isnan(pool[untouched]).all()
    for h in range(Hkv):
        assert np.array_equal(oracle.gather(pool, np.array(table), L, h, "k", "f32"), k[:, h].astype(np.float64))
        assert np.array_equal(oracle.gather(pool, np.array(table), L, h, "v", "f32"), v[:, h].astype(np.float64))


@pytest.mark.parametrize("cfg", [1, 2])
def test_gather_equals_contiguous_generator_rows(cfg):
    wl = W.config_workload(cfg)
    _, pool = oracle.run_workload(wl)
    for s in range(wl.num_seqs):
        L = int(wl.seq_lens[s])
        ks = W.to_f64(W.seq_kv_host(wl, s, "k"), wl.dtype)
        vs = W.to_f64(W.seq_kv_host(wl, s, "v"), wl.dtype)
        for h in range(wl.num_kv_heads):
            assert np.array_equal(oracle.gather(pool, wl.block_tables[s], L, h, "k", wl.dtype), ks[:, h])
            assert np.array_equal(oracle.gather(pool, wl.block_tables[s], L, h, "v", wl.dtype), vs[:, h])


@pytest.mark.parametrize("cfg", [1, 2])
def test_write_touches_only_its_slots(cfg):
    wl = W.config_workload(cfg)
    before = W.pool_host(wl)
    k, v = W.new_kv_host(wl)
    after = before.copy()
    oracle.reshape_and_cache(k, v, after, wl.slot_mapping, wl.dtype)
    touched = np.zeros((wl.num_blocks, W.BLOCK_SIZE), bool)
    for t, slot in enumerate(wl.slot_mapping):
        b, r = divmod(int(slot), W.BLOCK_SIZE)
        touched[b, r] = True
        assert after[b, 0, r].tobytes() == k[t].tobytes()
        assert after[b, 1, r].tobytes() == v[t].tobytes()
    keep = ~touched  # [block, row]; pool axes are [block, kv, row, ...]
    assert after.transpose(0, 2, 1, 3, 4)[keep].tobytes() == before.transpose(0, 2, 1, 3, 4)[keep].tobytes()


def test_write_errors_and_skip():
    Hkv, D, NB = 1, 4, 2
    k = np.ones((3, Hkv, D), np.float32)
    pool = np.zeros((NB, 2, 16, Hkv, D), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.reshape_and_cache(k, k, pool, np.array([0, 5, 5]), "f32")  # duplicate slot
    with pytest.raises(oracle.OracleError):
        oracle.reshape_and_cache(k, k, pool, np.array([0, 1, 32]), "f32")  # past the pool
    oracle.reshape_and_cache(k, k, pool, np.array([-1, 3, -7]), "f32")  # negative = skip
    assert pool[0, :, 3].sum() == 2 * D and pool.sum() == 2 * D


def test_metadata_errors():
    wl = W.config_workload(1)
    out, pool = oracle.run_workload(wl)
    q = W.q_host(wl)
    bad = wl.seq_lens.copy()
    bad[2] += 1  # seq_lens != context_lens + query_len
    with pytest.raises(oracle.OracleError):
        oracle.attention(q, pool, wl.block_tables, wl.query_start_loc, bad, wl.context_lens, wl.scale, wl.dtype)
    bt = wl.block_tables.copy()
    bt[3, 0] = wl.num_blocks  # block id past the pool
    with pytest.raises(oracle.OracleError):
        run_attention(wl, pool, tables=bt)


# --- softmax attention vs brute force ----------------------------------------------
def random_mix(seed):
    rs = np.random.default_rng(seed)
    S = int(rs.integers(1, 9))
    ctx, ql = [], []
    for _ in range(S):
        if rs.random() < 0.5:
            ctx.append(int(rs.integers(0, 70)))
            ql.append(1)
        else:
            ctx.append(int(rs.integers(0, 50)))
            ql.append(int(rs.integers(2, 21)))
    Hq, Hkv = [(4, 2), (4, 4), (8, 2), (6, 3)][seed % 4]
    D = [16, 64, 32][seed % 3]
    dtype = "f32" if seed % 2 == 0 else "bf16"
    return W.build_workload(f"mix{seed}", dtype, Hq, Hkv, D, ctx, ql, seed=1000 + seed)


@pytest.mark.parametrize("seed", range(8))
def test_oracle_matches_dense_bruteforce(seed):
    wl = random_mix(seed)
    out, _ = oracle.run_workload(wl)
    for s in range(wl.num_seqs):
        a, b = wl.query_start_loc[s], wl.query_start_loc[s + 1]
        np.testing.assert_allclose(out[a:b], dense_rows(wl, s), rtol=0, atol=1e-12)


def test_dense_mask_is_causal_with_offset():
    m = oracle.visibility_mask(3, 2, 5)
    assert m.tolist() == [[True, True, True, True, False], [True, True, True, True, True]]


# --- closed forms ------------------------------------------------------------------
def test_single_key_returns_its_value_exactly():
    wl = W.config_workload(1)
    s = list(wl.seq_lens).index(1)  # empty cache: the new token is the only key
    out, _ = oracle.run_workload(wl)
    _, v = W.new_kv_host(wl)
    t = wl.query_start_loc[s]
    G = wl.num_q_heads // wl.num_kv_heads
    for h in range(wl.num_q_heads):
        assert np.array_equal(out[t, h], v[t, h // G].astype(np.float64))


def test_zero_query_gives_mean_of_values():
    wl = W.config_workload(1)
    _, pool = oracle.run_workload(wl)
    q = np.zeros_like(W.q_host(wl))
    out = run_attention(wl, pool, q=q)
    G = wl.num_q_heads // wl.num_kv_heads
    for s in range(wl.num_seqs):
        vs = W.to_f64(W.seq_kv_host(wl, s, "v"), wl.dtype)
        for h in range(wl.num_q_heads):
            np.testing.assert_allclose(out[wl.query_start_loc[s], h], vs[:, h // G].mean(axis=0), rtol=0, atol=1e-15)


def test_constant_values_come_back_unchanged():
    wl = W.config_workload(1)
    _, pool = oracle.run_workload(wl)
    const = np.linspace(-1, 1, wl.head_size).astype(np.float32)
    pool[:, 1] = const  # every value row of every block
    out = run_attention(wl, pool)
    np.testing.assert_allclose(out, np.broadcast_to(const.astype(np.float64), out.shape), rtol=0, atol=1e-15)


# --- invariances stated by the pages -----------------------------------------------
def single_sequence_pool(num_tokens, Hq=4, Hkv=2, D=32, dtype="f32", seed=7):
    """One sequence's values (identity 0) and a 2-block placement."""
    wl = W.build_workload("one", dtype, Hq, Hkv, D, [0], [num_tokens], seed=seed, num_blocks=8)
    return wl


def test_chunked_prefill_equals_whole_prefill():
    g = gold("chunked_prefill_example.json")
    n = g["prompt_tokens"]
    assert sum(g["chunk_tokens"]) == n
    whole = single_sequence_pool(n)
    out_whole, _ = oracle.run_workload(whole)
    # the same sequence processed chunk by chunk through one persistent pool
    pool = W.pool_host(whole)  # nothing cached yet: all canary
    kall, vall = W.new_kv_host(whole)
    qall = W.q_host(whole)
    done, rows = 0, []
    for c in g["chunk_tokens"]:
        step = dataclasses.replace(
            whole, seq_lens=np.array([done + c], np.int32), context_lens=np.array([done], np.int32),
            query_start_loc=np.array([0, c], np.int32), slot_mapping=whole.slot_mapping[done:done + c],
            q_ident=whole.q_ident[done:done + c])
        oracle.reshape_and_cache(kall[done:done + c], vall[done:done + c], pool, step.slot_mapping, step.dtype)
        rows.append(run_attention(step, pool, q=qall[done:done + c]))
        done += c
    assert np.array_equal(np.concatenate(rows), out_whole)


def test_decode_equals_last_row_of_a_chunk():
    chunk = W.build_workload("chunk", "bf16", 4, 2, 64, [30], [11], seed=11)
    dec = dataclasses.replace(W.build_workload("dec", "bf16", 4, 2, 64, [40], [1], seed=11),
                              q_ident=chunk.q_ident[-1:])
    out_c, _ = oracle.run_workload(chunk)
    out_d, _ = oracle.run_workload(dec)
    assert np.array_equal(out_d[0], out_c[-1])


def test_gqa_equals_mha_with_repeated_kv_heads():
    wl = random_mix(3)  # 6 query heads over 3 KV heads
    G = wl.num_q_heads // wl.num_kv_heads
    out, pool = oracle.run_workload(wl)
    mha_pool = np.ascontiguousarray(np.repeat(pool, G, axis=3))
    out_mha = oracle.attention(W.q_host(wl), mha_pool, wl.block_tables, wl.query_start_loc, wl.seq_lens,
                               wl.context_lens, wl.scale, wl.dtype)
    assert np.array_equal(out, out_mha)


@pytest.mark.parametrize("seed", [0, 1, 5])
def test_physical_block_permutation_changes_nothing(seed):
    wl = random_mix(seed)
    out, _ = oracle.run_workload(wl)
    pi = np.random.default_rng(seed + 99).permutation(wl.num_blocks)
    pool = W.pool_host(wl)
    pool_p = np.empty_like(pool)
    pool_p[pi] = pool
    wl_p = W.with_block_tables(wl, pi[wl.block_tables], wl.num_blocks, int(pi[wl.canary_block]))
    assert np.array_equal(wl_p.slot_mapping, pi[wl.slot_mapping // 16] * 16 + wl.slot_mapping % 16)
    out_p, _ = oracle.run_workload(wl_p, pool=pool_p)
    assert np.array_equal(out, out_p)


def test_shared_prefix_blocks_equal_private_copies():
    gd = gold("shared_prefix_blocks.json")
    bs = gd["block_size"]
    # req A: 2 blocks [42, 7]; req B: shared block 42 then a private block 3
    base = W.build_workload("shared", "bf16", 4, 2, 64, [bs + 9, bs + 4], [1, 1], seed=21,
                            shared_prefix_tokens=bs, num_blocks=64)
    tables = np.array([gd["req_a"], gd["req_b_prefix"] + [3]])
    shared = W.with_block_tables(base, tables, 64, 63)
    out_s, _ = oracle.run_workload(shared)
    for s in range(2):
        np.testing.assert_allclose(out_s[s:s + 1], dense_rows(shared, s), rtol=0, atol=1e-12)
    # private copies: B reads its own copy (#43) of the prefix block
    private = W.with_block_tables(base, np.array([gd["req_a"], [43, 3]]), 64, 63)
    pool = W.pool_host(shared)
    pool[43] = pool[42]
    out_p, _ = oracle.run_workload(private, pool=pool)
    assert np.array_equal(out_s, out_p)


def test_shared_prefix_config_equals_private_copies():
    wl = W.sub_workload(W.config_workload(5), [0, 1, 2])
    n_sh = int(wl.shared_len[0]) // 16
    out_s, pool_s = oracle.run_workload(wl)
    # give sequences 1 and 2 private copies of the shared prefix blocks
    extra = wl.num_blocks
    NB = extra + 2 * n_sh + 1
    tables = np.full((3, wl.max_blocks), NB - 1, np.int64)
    tables[:, : wl.max_blocks] = wl.block_tables
    pool = np.empty((NB,) + W.pool_host(wl).shape[1:], W.np_dtype(wl.dtype))
    pool[...] = W.canary_np(wl.dtype)
    pool[: wl.num_blocks] = W.pool_host(wl)
    for i, s in enumerate([1, 2]):
        ids = np.arange(extra + i * n_sh, extra + (i + 1) * n_sh)
        pool[ids] = pool[wl.block_tables[s, :n_sh]]
        tables[s, :n_sh] = ids
    priv = W.with_block_tables(wl, tables, NB, NB - 1)
    out_p, _ = oracle.run_workload(priv, pool=pool)
    assert np.array_equal(out_s, out_p)


def test_mixed_batch_rows_equal_each_sequence_alone():
    g = gold("mixed_batch_example.json")
    d_len = g["token_budget"] - g["decodes"] - g["left_after_d"]
    assert d_len == 6 and g["e_prompt"] > g["left_after_d"]
    ctx = [20, 33, 47, 0]
    ql = [1] * g["decodes"] + [d_len]
    wl = W.build_workload("budget16", "f32", 4, 2, 64, ctx, ql, seed=31)
    assert wl.num_tokens == g["decodes"] + d_len <= g["token_budget"]
    out, _ = oracle.run_workload(wl)
    for s in range(wl.num_seqs):
        alone = W.sub_workload(wl, [s])
        out_alone, _ = oracle.run_workload(alone)
        a, b = wl.query_start_loc[s], wl.query_start_loc[s + 1]
        assert np.array_equal(out[a:b], out_alone)
        np.testing.assert_allclose(out[a:b], dense_rows(wl, s), rtol=0, atol=1e-12)
