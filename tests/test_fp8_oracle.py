"""Oracle of the 8-bit (OCP FP8 E4M3) KV pool, on the CPU.

The oracle decodes codes from the format's definition and encodes by a plain
nearest-value search over the finite codes. Pins:
- decoding equals torch's float8_e4m3fn widening for all 256 codes, and the
  format's closed forms (448, 2^-6, 2^-9, 1.0, NaN);
- encoding equals torch's float8_e4m3fn rounding (nearest, ties to even) for
  magnitudes below 464, on random values, every exact code value, and every
  midpoint between neighbouring codes; at and above 464 the oracle saturates
  to +-448 where torch gives NaN (the reading taken: the cache keeps the
  largest finite value);
- quantize divides by the scale in fp32 before rounding;
- the fp8 KV write stores exactly the quantized codes at the slots and leaves
  every other byte alone;
- attention over an fp8 pool equals the dense brute force on the decoded,
  scaled K/V.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.dense import dense_attention


def torch_encode(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_library_and_closed_forms():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all() and nan.sum() == 2
    assert (ours[~nan] == ref[~nan]).all()
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9 and ours[0x38] == 1.0 and ours[0x00] == 0.0


def test_encode_matches_library_below_saturation():
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.fp8_decode(finite)
    pos = np.unique(vals[vals >= 0])
    mids = (pos[1:] + pos[:-1]) / 2  # exact in fp32 (few significant bits)
    rs = np.random.default_rng(0)
    rnd = np.concatenate([rs.normal(0, 1, 20000) * 10.0 ** rs.integers(-4, 3, 20000),
                          rs.uniform(-463.9, 463.9, 20000)])
    x = np.concatenate([vals, mids, -mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20), rnd]).astype(np.float32)
    x = x[np.abs(x) < 464]
    assert (oracle.fp8_quantize(x, "f32", 1.0) == torch_encode(x)).all()
    # every finite code is its own value's code
    assert (oracle.fp8_quantize(vals.astype(np.float32), "f32", 1.0) == finite).all()


def test_saturation_nan_and_sign():
    x = np.array([464.0, 479.0, 480.0, 1e30, np.inf, -464.0, -np.inf, np.nan, -0.0, -1e-6], np.float32)
    got = oracle.fp8_quantize(x, "f32", 1.0)
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x80, 0x80]


def test_quantize_divides_in_fp32():
    x = np.array([3.0, -7.25, 0.3, 100.0], np.float32)
    for scale in (0.1, 0.0625, 1.7):
        q = (x / np.float32(scale)).astype(np.float32)  # one IEEE fp32 division each
        assert (oracle.fp8_quantize(x, "f32", scale) == torch_encode(np.clip(q, -463, 463))).all()
    # bf16 input: widened exactly first
    b = W.rng.f32_to_bf16_bits(x)
    assert (oracle.fp8_quantize(b, "bf16", 0.1) == oracle.fp8_quantize(W.rng.bf16_bits_to_f32(b), "f32", 0.1)).all()


def test_fp8_write_stores_codes_at_slots_only():
    rs = np.random.default_rng(1)
    NB, Hkv, D, T = 6, 2, 16, 5
    pool = np.full((NB, 2, 16, Hkv, D), 0x7F, np.uint8)
    k = W.rng.f32_to_bf16_bits(rs.normal(0, 1, (T, Hkv, D)).astype(np.float32))
    v = W.rng.f32_to_bf16_bits(rs.normal(0, 1, (T, Hkv, D)).astype(np.float32))
    slots = np.array([0, 17, -1, 95, 40], np.int64)
    before = pool.copy()
    oracle.reshape_and_cache_fp8(k, v, pool, slots, "bf16", 0.05, 0.125)
    touched = np.zeros(pool.shape, bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        b, r = divmod(int(s), 16)
        assert (pool[b, 0, r] == oracle.fp8_quantize(k[t], "bf16", 0.05)).all()
        assert (pool[b, 1, r] == oracle.fp8_quantize(v[t], "bf16", 0.125)).all()
        touched[b, :, r] = True
    assert (pool[~touched] == before[~touched]).all()


def test_fp8_attention_equals_dense_on_decoded_kv():
    rs = np.random.default_rng(2)
    Hq, Hkv, D, NB = 4, 2, 32, 16
    k_scale, v_scale = 0.03, 0.0625
    lens = [(1, 0), (1, 20), (5, 9), (12, 30)]  # (new tokens, cached)
    pool = rs.integers(0, 0x7F, (NB, 2, 16, Hkv, D)).astype(np.uint8)  # NaN codes excluded
    pool |= (rs.integers(0, 2, pool.shape) * 0x80).astype(np.uint8)
    perm = rs.permutation(NB)
    tables, qsl, sl, cl, used = [], [0], [], [], 0
    for n, C in lens:
        L = n + C
        nb = -(-L // 16)
        tables.append(list(perm[used:used + nb]) + [0] * (4 - nb))
        used += nb
        qsl.append(qsl[-1] + n)
        sl.append(L)
        cl.append(C)
    T = qsl[-1]
    q = W.rng.f32_to_bf16_bits(rs.normal(0, 1, (T, Hq, D)).astype(np.float32))
    scale = float(np.float32(1 / np.sqrt(D)))
    got = oracle.attention_fp8(q, pool, np.array(tables), np.array(qsl), np.array(sl), np.array(cl), scale, "bf16",
                               k_scale, v_scale)
    for s, (n, C) in enumerate(lens):
        L = n + C
        rows = [(tables[s][j // 16], j % 16) for j in range(L)]
        kk = np.stack([oracle.fp8_decode(pool[b, 0, r]) for b, r in rows]) * np.float64(np.float32(k_scale))
        vv = np.stack([oracle.fp8_decode(pool[b, 1, r]) for b, r in rows]) * np.float64(np.float32(v_scale))
        qq = W.to_f64(q[qsl[s]:qsl[s + 1]], "bf16")
        ref = dense_attention(qq, kk, vv, C, scale)
        assert np.abs(got[qsl[s]:qsl[s + 1]] - ref).max() < 1e-12
