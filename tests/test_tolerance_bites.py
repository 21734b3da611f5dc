"""The parity bounds catch plausible kernel mistakes (CPU only).

Each probe plants one mistake in what the oracle is given -- never in the GPU
path -- and shows that the comparison rules the GPU parity tests use
(tests/parity.py) reject the result, while the oracle's own output rounded the
way a correct bf16 kernel rounds passes them.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import bf16_round_f64, within


def q64(wl):
    return W.to_f64(W.q_host(wl), wl.dtype)


def seq_dense(wl, s, keep=None):
    """Dense attention of sequence s over its keys, optionally only the rows in `keep`."""
    a, b = wl.query_start_loc[s], wl.query_start_loc[s + 1]
    k = W.to_f64(W.seq_kv_host(wl, s, "k"), wl.dtype)
    v = W.to_f64(W.seq_kv_host(wl, s, "v"), wl.dtype)
    if keep is not None:
        k, v = k[keep], v[keep]
    n = b - a
    return oracle.dense_attention(q64(wl)[a:b], k, v, k.shape[0] - n, wl.scale)


@pytest.fixture(scope="module")
def long_ctx():
    """One 32k-token decode sequence shaped like the 70B long-context layer."""
    wl = W.sub_workload(W.config_workload(4), [0])
    ref, _ = oracle.run_workload(wl)
    return wl, ref


@pytest.fixture(scope="module")
def short_ctx():
    wl = W.config_workload(2)
    ref, _ = oracle.run_workload(wl)
    return wl, ref


def test_correct_bf16_rounding_passes(long_ctx, short_ctx):
    for wl, ref in (long_ctx, short_ctx):
        ok, e = within(bf16_round_f64(ref), ref, "bf16")
        assert ok, e
        assert e["rel"] < 0.5 * 3e-2  # margin below the bound


def test_all_zero_output_fails_at_32k(long_ctx):
    wl, ref = long_ctx
    ok, e = within(np.zeros_like(ref), ref, "bf16")
    assert e["mean_abs"] <= 1e-2  # the absolute mean bound alone would be blind here ...
    assert not ok  # ... the rms-relative bound is not


def test_skipping_last_partition_fails(long_ctx):
    wl, ref = long_ctx
    L = int(wl.seq_lens[0])
    keep = np.r_[0 : L - 1 - 512, L - 1]  # drop the 512 keys before the new token
    ok, e = within(bf16_round_f64(seq_dense(wl, 0, keep)), ref, "bf16")
    assert not ok, e


def test_skipping_first_partition_fails(long_ctx):
    wl, ref = long_ctx
    L = int(wl.seq_lens[0])
    ok, e = within(bf16_round_f64(seq_dense(wl, 0, np.arange(512, L))), ref, "bf16")
    assert not ok, e


@pytest.mark.parametrize("cfg", [1, 2])
def test_excluding_the_diagonal_fails(cfg):
    wl = W.config_workload(cfg)
    ref, _ = oracle.run_workload(wl)
    rows = []
    for s in range(wl.num_seqs):
        L = int(wl.seq_lens[s])
        with np.errstate(invalid="ignore"):
            rows.append(seq_dense(wl, s, np.arange(L - 1)) if L > 1 else np.full((1,) + ref.shape[1:], np.nan))
    ok, e = within(np.concatenate(rows), ref, wl.dtype)
    assert not ok, e


def test_chunk_off_by_one_mask_fails():
    wl = W.build_workload("chunk", "bf16", 8, 2, 64, [100, 0], [64, 48], seed=5)
    ref, _ = oracle.run_workload(wl)
    # query i sees keys j < C + i (its own key missing): shift K/V by one row
    rows = []
    for s in range(wl.num_seqs):
        a, b = wl.query_start_loc[s], wl.query_start_loc[s + 1]
        C = int(wl.context_lens[s])
        k = W.to_f64(W.seq_kv_host(wl, s, "k"), wl.dtype)
        v = W.to_f64(W.seq_kv_host(wl, s, "v"), wl.dtype)
        out = np.empty((b - a,) + ref.shape[1:])
        for i in range(b - a):
            kk, vv = k[: C + i], v[: C + i]
            if kk.shape[0] == 0:
                out[i] = np.nan
                continue
            out[i] = oracle.dense_attention(q64(wl)[a + i : a + i + 1], kk, vv, kk.shape[0] - 1, wl.scale)[0]
        rows.append(out)
    ok, e = within(bf16_round_f64(np.concatenate(rows)), ref, "bf16")
    assert not ok, e


@pytest.mark.parametrize("cfg", [1, 2])
def test_interleaved_head_mapping_fails(cfg):
    base = W.config_workload(cfg)
    wl = W.sub_workload(base, range(base.num_seqs))  # same values, a pool of the referenced blocks only
    ref, pool = oracle.run_workload(wl)
    Hq, Hkv = wl.num_q_heads, wl.num_kv_heads
    mha = np.ascontiguousarray(pool[:, :, :, [h % Hkv for h in range(Hq)]])  # h % Hkv instead of h // G
    out = oracle.attention(W.q_host(wl), mha, wl.block_tables, wl.query_start_loc, wl.seq_lens, wl.context_lens,
                           wl.scale, wl.dtype)
    ok, e = within(out, ref, wl.dtype)
    assert not ok, e


@pytest.mark.parametrize("cfg", [1, 2])
def test_ignoring_slot_row_in_write_fails(cfg):
    wl = W.config_workload(cfg)
    ref, _ = oracle.run_workload(wl)
    bad = W.with_block_tables(wl, wl.block_tables, wl.num_blocks, wl.canary_block)
    bad.slot_mapping = (wl.slot_mapping // 16) * 16  # every new row written to row 0 of its block
    with np.errstate(invalid="ignore"):
        out, _ = oracle.run_workload(bad)
    ok, e = within(out, ref, wl.dtype)
    assert not ok, e


@pytest.mark.parametrize("cfg", [1, 2])
def test_unpermuted_block_reads_fail(cfg):
    wl = W.config_workload(cfg)
    ref, pool = oracle.run_workload(wl)
    ident = np.tile(np.arange(wl.max_blocks, dtype=np.int32), (wl.num_seqs, 1)) % wl.num_blocks
    with np.errstate(invalid="ignore"):
        out = oracle.attention(W.q_host(wl), pool, ident, wl.query_start_loc, wl.seq_lens, wl.context_lens,
                               wl.scale, wl.dtype)
    ok, e = within(out, ref, wl.dtype)
    assert not ok, e


def test_wrong_scale_fails(short_ctx):
    wl, ref = short_ctx
    _, pool = oracle.run_workload(wl)
    out = oracle.attention(W.q_host(wl), pool, wl.block_tables, wl.query_start_loc, wl.seq_lens, wl.context_lens,
                           1.0, wl.dtype)
    ok, e = within(bf16_round_f64(out), ref, "bf16")
    assert not ok, e
