"""Counter-based random values for the synthetic paged-attention inputs.

This module holds no part of the attention method. It only turns
(stream, identity, position, element) coordinates into reproducible values, so
that the host side (numpy) and the device side (torch, any device) produce the
same bits without sharing state.

Generator: SplitMix64 as published by Steele, Lea and Flood ("Fast splittable
pseudorandom number generators", OOPSLA 2014), used in counter form: the n-th
output of a stream with key ``s`` is ``mix64(s + (n + 1) * GAMMA)`` modulo
2**64, where ``mix64`` is the finaliser with the shifts 30/27/31 and the two
odd multipliers below (the constants of the public splitmix64 reference).

Values: each 64-bit output is cut into four 16-bit fields; field ``u`` selects
``NORMAL_F32[u] = Phi^-1((u + 0.5) / 65536)``, the standard-normal quantile at
the centre of the u-th of 65536 equal-probability bins. The result is a
discretised N(0, 1) sample (|x| <= 4.33). ``NORMAL_BF16`` is the same table
rounded to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX_M1 = 0xBF58476D1CE4E5B9
MIX_M2 = 0x94D049BB133111EB
# Odd multiplier that spreads identities (sequence ids) across the key space.
IDENT_MUL = 0xD1B54A32D192ED03


def mix64_int(z: int) -> int:
    """SplitMix64 finaliser on a Python int (exact modulo 2**64)."""
    z &= MASK64
    z ^= z >> 30
    z = (z * MIX_M1) & MASK64
    z ^= z >> 27
    z = (z * MIX_M2) & MASK64
    return z ^ (z >> 31)


def _mul64(a, b):
    return np.multiply(a, b, dtype=np.uint64)


def _add64(a, b):
    return np.add(a, b, dtype=np.uint64)


def mix64_np(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wrap-around multiply)."""
    z = np.asarray(z, dtype=np.uint64)
    z = z ^ (z >> np.uint64(30))
    z = _mul64(z, np.uint64(MIX_M1))
    z = z ^ (z >> np.uint64(27))
    z = _mul64(z, np.uint64(MIX_M2))
    return z ^ (z >> np.uint64(31))


def _s64(x: int) -> int:
    x &= MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


def mix64_torch(z):
    """SplitMix64 finaliser on an int64 torch tensor holding uint64 bit patterns.

    torch has no unsigned 64-bit arithmetic, so logical right shifts are an
    arithmetic shift followed by a mask, and multiplies wrap in two's
    complement (the same bits as unsigned wrap-around).
    """
    z = z ^ ((z >> 30) & ((1 << 34) - 1))
    z = z * _s64(MIX_M1)
    z = z ^ ((z >> 27) & ((1 << 37) - 1))
    z = z * _s64(MIX_M2)
    z = z ^ ((z >> 31) & ((1 << 33) - 1))
    return z


def stream_key(seed: int, stream: int) -> int:
    """Key of one named stream (q, new-and-cached K, V) of one workload seed."""
    return mix64_int((seed * GAMMA) ^ (stream << 56) ^ 0x5EED)


def _normal_table_f32() -> np.ndarray:
    from scipy.special import ndtri

    u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return ndtri(u).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs must be finite (the table and the canaries are handled apart).
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return b.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


NORMAL_F32 = _normal_table_f32()
NORMAL_BF16 = f32_to_bf16_bits(NORMAL_F32)

# 8-bit (OCP FP8 E4M3) pool contents, drawn as codes from the same 16-bit
# fields, shaped like N(0, 1): bit 15 is the sign, bits 8..10 the mantissa,
# and the low byte picks the exponent field with about the probability that
# |N(0, 1)| falls in that power-of-two band ([2, 4): 12/256, [1, 2): 70/256,
# [1/2, 1): 77/256, ... down to the subnormals). Built from bit fields and a
# fixed table of thresholds, with no rounding arithmetic.
_FP8_EXP_THRESHOLDS = np.array([12, 82, 159, 204, 229, 242, 249, 253, 256])  # exponent fields 8, 7, ..., 0


def _fp8_codes() -> np.ndarray:
    u = np.arange(65536)
    e = 8 - np.searchsorted(_FP8_EXP_THRESHOLDS, u & 0xFF, side="right")
    return (((u >> 8) & 0x80) | (e << 3) | ((u >> 8) & 7)).astype(np.uint8)


FP8_CODES = _fp8_codes()
# A heavier-tailed alternative: the low byte picks one of the 56 codes 0x18 ..
# 0x4F (magnitudes 1/16 .. 3.75) with equal probability, bit 15 the sign. It
# puts far more mass near the top of the range than N(0, 1) does, which makes
# softmax rows spikier; kept to track the bf16 rounding margin on such rows.
FP8_CODES_BAND = (((np.arange(65536) >> 8) & 0x80) | (0x18 + (np.arange(65536) & 0xFF) % 56)).astype(np.uint8)
CANARY_FP8 = 0x7F

# NaN canaries for pool memory that a correct kernel never reads.
CANARY_F32_BITS = 0x7FC00000
CANARY_BF16_BITS = 0x7FC0


def row_keys_np(key: int, ident: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Per-row keys for rows addressed by (identity, position)."""
    ident = np.asarray(ident, dtype=np.uint64)
    pos = np.asarray(pos, dtype=np.uint64)
    z = _add64(_mul64(ident, np.uint64(IDENT_MUL)), _mul64(_add64(pos, np.uint64(1)), np.uint64(GAMMA)))
    return mix64_np(_add64(z, np.uint64(key)))


def row_fields_np(rkeys: np.ndarray, width: int) -> np.ndarray:
    """16-bit table indices [nrows, width] for rows with keys ``rkeys``.

    Element e of a row is bits 16*(e % 4) .. 16*(e % 4) + 15 of word e // 4.
    """
    assert width % 4 == 0
    w = _mul64(np.arange(1, width // 4 + 1, dtype=np.uint64), np.uint64(GAMMA))
    z = mix64_np(_add64(rkeys.reshape(-1, 1).astype(np.uint64), w.reshape(1, -1)))
    # Little-endian uint16 view: field f of a word is its bits 16f .. 16f + 15.
    return np.ascontiguousarray(z).astype("<u8", copy=False).view("<u2").reshape(rkeys.size, width)


def row_keys_torch(key: int, ident, pos):
    """Torch twin of ``row_keys_np`` (int64 tensors on any device)."""
    import torch

    ident = ident.to(torch.int64)
    pos = pos.to(torch.int64)
    z = _s64(key) + ident * _s64(IDENT_MUL) + (pos + 1) * _s64(GAMMA)
    return mix64_torch(z)


def row_fields_torch(rkeys, width: int):
    """Torch twin of ``row_fields_np``."""
    import torch

    assert width % 4 == 0
    w = torch.arange(1, width // 4 + 1, dtype=torch.int64, device=rkeys.device)
    z = mix64_torch(rkeys.reshape(-1, 1) + w.reshape(1, -1) * _s64(GAMMA)).contiguous()
    # Same field order as the numpy twin: little-endian 16-bit view of each word.
    return (z.view(torch.int16).to(torch.int32) & 0xFFFF).reshape(rkeys.numel(), width)
