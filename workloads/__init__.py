"""Seeded synthetic workloads for paged attention over a block-paged KV cache.

Test and benchmark infrastructure shared by the GPU path's callers and by the
oracle. It holds none of the attention arithmetic: it decides sequence lengths,
which physical blocks each sequence owns, where the new tokens go
(``slot_mapping``) and what the q/k/v values are.

Shapes follow the pages' statement of the problem:
- KV pool ``[num_blocks, 2, 16, num_kv_heads, head_size]``; one block holds 16
  tokens' K and V ("Inside vLLM", page 2, "LLM Engine constructor": block bytes
  are 2 * block_size * num_kv_heads * head_size * dtype bytes; ngrok, "Serving
  models at scale with vLLM", section "PagedAttention").
- Per-sequence block tables listing physical blocks in order (ngrok,
  "PagedAttention": Req 2 -> blocks 2, 5, 8).
- A flat ``slot_mapping`` for the new tokens ("Inside vLLM", "Run forward
  pass", step "Prepare inputs"), read as ``block_table[pos // 16] * 16 +
  pos % 16``: the pages' worked example of it is a missing figure.
- One flattened super-sequence with ``query_start_loc`` ("Inside vLLM", "Run
  forward pass", step "Forward pass").

Values: every K/V row is addressed by (identity, position); a sequence's
private rows use its own identity, rows of a shared prefix use one common
identity. New tokens are generated from the same definition as cached ones, so
after the KV write the pool holds exactly ``seq_kv(s)`` at every position.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional, Sequence

import numpy as np

from . import rng as _rng

BLOCK_SIZE = 16
SHARED_IDENT = 1 << 40  # identity of rows in a shared prefix
STREAM_Q, STREAM_K, STREAM_V = 1, 2, 3
DTYPE_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str  # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    num_blocks: int
    seq_lens: np.ndarray  # int32 [S]
    context_lens: np.ndarray  # int32 [S]
    query_start_loc: np.ndarray  # int32 [S + 1]
    block_tables: np.ndarray  # int32 [S, MB]
    slot_mapping: np.ndarray  # int64 [T]
    seq_ident: np.ndarray  # int64 [S]: identity of each sequence's private rows
    shared_len: np.ndarray  # int32 [S]: positions below this use SHARED_IDENT
    q_ident: np.ndarray  # int64 [T]: identity of each query row
    scale: float
    seed: int
    canary_block: int  # an unreferenced block; unused table entries point at it
    block_size: int = BLOCK_SIZE
    # 8-bit pool: kv_dtype "fp8" (OCP E4M3 codes, a cached element reads back as
    # value(code) * k_scale or * v_scale); "" = the pool holds `dtype`
    kv_dtype: str = ""
    k_scale: float = 1.0
    v_scale: float = 1.0
    # 8-bit pool contents: "normal" (codes shaped like N(0, 1)) or "band"
    # (uniform over the magnitudes 1/16 .. 3.75, heavier-tailed)
    fp8_codes: str = "normal"

    @property
    def pool_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def kv_elem_bytes(self) -> int:
        return DTYPE_BYTES[self.pool_dtype]

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int32)

    @property
    def elem_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]

    @property
    def block_bytes(self) -> int:
        return 2 * self.block_size * self.num_kv_heads * self.head_size * self.kv_elem_bytes

    def blocks_used(self, s: int) -> int:
        return -(-int(self.seq_lens[s]) // self.block_size)

    def referenced_blocks(self) -> np.ndarray:
        ids = [self.block_tables[s, : self.blocks_used(s)] for s in range(self.num_seqs)]
        return np.unique(np.concatenate(ids)) if ids else np.zeros(0, np.int32)

    def decode_mask(self) -> np.ndarray:
        return self.query_lens == 1

    # --- algorithmic work (what the method must move or compute) ---------
    def kv_read_bytes(self, seqs: Optional[np.ndarray] = None) -> int:
        """K and V bytes attention must read: every key of every sequence once."""
        L = self.seq_lens.astype(np.int64) if seqs is None else self.seq_lens[seqs].astype(np.int64)
        return int(L.sum()) * 2 * self.num_kv_heads * self.head_size * self.kv_elem_bytes

    def decode_bytes(self) -> int:
        """Decode roofline bytes: KV read + block-table reads + q read + out write."""
        m = self.decode_mask()
        L = self.seq_lens[m].astype(np.int64)
        kv = int(L.sum()) * 2 * self.num_kv_heads * self.head_size * self.kv_elem_bytes
        tables = int((-(-L // self.block_size)).sum()) * 4
        qo = 2 * int(m.sum()) * self.num_q_heads * self.head_size * self.elem_bytes
        return kv + tables + qo

    def prefill_flops(self) -> int:
        """Causal-exact FLOPs of the sequences with more than one query token."""
        total = 0
        for s in np.nonzero(~self.decode_mask())[0]:
            c, n = int(self.context_lens[s]), int(self.query_lens[s])
            keys = n * c + n * (n + 1) // 2  # sum over i of (c + i + 1)
            total += keys
        return 4 * self.head_size * self.num_q_heads * total

    def write_bytes(self) -> int:
        """KV-write bytes: read k and v rows, write them into the pool."""
        n = int((self.slot_mapping >= 0).sum())
        return 2 * n * self.num_kv_heads * self.head_size * (self.elem_bytes + self.kv_elem_bytes)


def _draw_rng(cfg_id: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0x5EED, cfg_id, stream])))


def build_workload(
    name: str,
    dtype: str,
    num_q_heads: int,
    num_kv_heads: int,
    head_size: int,
    context_lens: Sequence[int],
    query_lens: Sequence[int],
    *,
    seed: int,
    num_blocks: Optional[int] = None,
    shared_prefix_tokens: int = 0,
    max_blocks: Optional[int] = None,
    pool_slack: float = 1.25,
) -> Workload:
    """Assign blocks and slots for sequences with the given (context, query) lengths.

    Logical blocks are taken in sequence order from a seeded random permutation
    of the pool. With ``shared_prefix_tokens`` (a multiple of 16), every
    sequence's first blocks are the same physical blocks; new tokens never land
    in a shared block (each sequence's context must cover the prefix).
    """
    C = np.asarray(context_lens, dtype=np.int64)
    n = np.asarray(query_lens, dtype=np.int64)
    assert C.shape == n.shape and C.ndim == 1
    assert (n >= 1).all() and (C >= 0).all()
    assert num_q_heads % num_kv_heads == 0
    S = C.shape[0]
    L = C + n
    nblk = -(-L // BLOCK_SIZE)
    assert shared_prefix_tokens % BLOCK_SIZE == 0
    n_shared = shared_prefix_tokens // BLOCK_SIZE
    if n_shared:
        assert (C >= shared_prefix_tokens).all(), "new tokens must not land in shared blocks"
    referenced = n_shared + int((nblk - n_shared).sum())
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_slack * referenced))
    num_blocks = max(int(num_blocks), referenced + 1)
    MB = int(max_blocks) if max_blocks is not None else int(nblk.max())
    assert MB >= int(nblk.max())

    r = _draw_rng(seed, 1)
    if num_blocks <= (1 << 23):
        ids = r.permutation(num_blocks)[: referenced + 1]
    else:
        ids = r.choice(num_blocks, size=referenced + 1, replace=False)
    ids = ids.astype(np.int64)
    canary = int(ids[-1])
    tables = np.full((S, MB), canary, dtype=np.int64)
    shared_ids = ids[:n_shared]
    cursor = n_shared
    for s in range(S):
        tables[s, :n_shared] = shared_ids
        k = int(nblk[s]) - n_shared
        tables[s, n_shared : n_shared + k] = ids[cursor : cursor + k]
        cursor += k

    qsl = np.zeros(S + 1, dtype=np.int64)
    qsl[1:] = np.cumsum(n)
    T = int(qsl[-1])
    seq_of_tok = np.repeat(np.arange(S), n)
    pos = C[seq_of_tok] + (np.arange(T) - qsl[seq_of_tok])
    slots = tables[seq_of_tok, pos // BLOCK_SIZE] * BLOCK_SIZE + pos % BLOCK_SIZE

    return Workload(
        name=name,
        dtype=dtype,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_size=head_size,
        num_blocks=num_blocks,
        seq_lens=L.astype(np.int32),
        context_lens=C.astype(np.int32),
        query_start_loc=qsl.astype(np.int32),
        block_tables=tables.astype(np.int32),
        slot_mapping=slots.astype(np.int64),
        seq_ident=np.arange(S, dtype=np.int64),
        shared_len=np.full(S, shared_prefix_tokens, dtype=np.int32),
        q_ident=np.arange(T, dtype=np.int64),
        scale=float(np.float32(1.0 / math.sqrt(head_size))),
        seed=seed,
        canary_block=canary,
    )


# --- the five model-shaped single-layer steps --------------------------------
CONFIG_NAMES = {
    1: "tiny_decode_f32",
    2: "tinyllama_1.1b_decode_bf16",
    3: "llama3_8b_mixed_prefill_decode_bf16",
    4: "llama3_70b_32k_decode_bf16",
    5: "prefix_shared_decode_bf16",
    6: "llama3_8b_spec_verify_bf16",
    7: "llama3_70b_32k_decode_fp8kv",
    8: "llama3_8b_mixed_prefill_decode_fp8kv",
    9: "llama3_8b_long_prompt_last_chunk_bf16",
}

DEFAULT_HBM_BYTES = 288 * (1 << 30)


def config_workload(cfg: int, *, hbm_bytes: Optional[int] = None) -> Workload:
    """The benchmark/parity workloads (decode lengths include the new token).

    1-5 are the path's configurations; 6 is speculative-decode verification
    (short multi-token queries over long contexts); 7 and 8 are the 70B 32k
    decode and the 8B mixed step over an 8-bit (fp8) KV pool (the 70B pool
    again ~60% of HBM, in 32 KiB blocks); 9 is the last 512-token chunk of a
    32,512-token prompt with Llama-3-8B heads (a few long prefill items)."""
    name = CONFIG_NAMES[cfg]
    if cfg == 7:
        hbm = DEFAULT_HBM_BYTES if hbm_bytes is None else int(hbm_bytes)
        return with_fp8_pool(config_workload(4, hbm_bytes=2 * hbm))
    if cfg == 8:
        return with_fp8_pool(config_workload(3))
    r = _draw_rng(cfg, 0)
    if cfg == 1:
        L = np.array([1, 17, 50, 100])
        return build_workload(name, "f32", 4, 2, 64, L - 1, np.ones(4, np.int64), seed=cfg, num_blocks=64)
    if cfg == 2:
        L = r.integers(128, 2048, size=64, endpoint=True)
        return build_workload(name, "bf16", 32, 4, 64, L - 1, np.ones(64, np.int64), seed=cfg,
                              num_blocks=16384, max_blocks=2048 // BLOCK_SIZE)
    if cfg == 3:
        Ld = r.integers(256, 8192, size=4096, endpoint=True)
        Cp = r.integers(0, 4096, size=8, endpoint=True)
        ctx = np.concatenate([Ld - 1, Cp])
        q = np.concatenate([np.ones(4096, np.int64), np.full(8, 512, np.int64)])
        return build_workload(name, "bf16", 32, 8, 128, ctx, q, seed=cfg, max_blocks=8192 // BLOCK_SIZE)
    if cfg == 4:
        hbm = DEFAULT_HBM_BYTES if hbm_bytes is None else int(hbm_bytes)
        nb = int(0.6 * hbm) // (2 * BLOCK_SIZE * 8 * 128 * 2)
        L = np.full(32, 32768)
        return build_workload(name, "bf16", 64, 8, 128, L - 1, np.ones(32, np.int64), seed=cfg, num_blocks=nb)
    if cfg == 5:
        p = r.integers(0, 512, size=256, endpoint=True)
        L = 2048 + p + 1
        return build_workload(name, "bf16", 32, 8, 128, L - 1, np.ones(256, np.int64), seed=cfg,
                              shared_prefix_tokens=2048, max_blocks=128 + -(-513 // BLOCK_SIZE))
    if cfg == 6:
        # speculative-decode verification: 3 draft tokens + 1 per sequence
        # (n = 4 new tokens), long cached contexts, Llama-3-8B heads
        C = r.integers(1024, 8192, size=256, endpoint=True)
        return build_workload(name, "bf16", 32, 8, 128, C, np.full(256, 4, np.int64), seed=cfg,
                              max_blocks=(8192 + 4) // BLOCK_SIZE + 1)
    if cfg == 9:
        return build_workload(name, "bf16", 32, 8, 128, np.array([32000]), np.array([512]), seed=cfg)
    raise ValueError(f"unknown config {cfg}")


# --- values -------------------------------------------------------------------
def _table_np(dtype: str) -> np.ndarray:
    if dtype == "fp8band":
        return _rng.FP8_CODES_BAND
    if dtype == "fp8":
        return _rng.FP8_CODES
    return _rng.NORMAL_F32 if dtype == "f32" else _rng.NORMAL_BF16


def canary_np(dtype: str):
    if dtype == "fp8":
        return np.uint8(_rng.CANARY_FP8)
    if dtype == "f32":
        return np.array([_rng.CANARY_F32_BITS], np.uint32).view(np.float32)[0]
    return np.uint16(_rng.CANARY_BF16_BITS)


def np_dtype(dtype: str):
    """Host element type: float32, uint16 bit patterns for bfloat16, uint8 codes for fp8."""
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dtype]


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of host elements to float64."""
    if dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    return _rng.bf16_bits_to_f32(x).astype(np.float64)


def _rows_np(key: int, ident, pos, width: int, dtype: str) -> np.ndarray:
    rk = _rng.row_keys_np(key, ident, pos)
    return _table_np(dtype)[_rng.row_fields_np(rk, width)]


def kv_ident(wl: Workload, s: int, pos: np.ndarray) -> np.ndarray:
    return np.where(pos < wl.shared_len[s], SHARED_IDENT, wl.seq_ident[s]).astype(np.int64)


def q_host(wl: Workload) -> np.ndarray:
    """Queries [T, Hq, D] (host element type)."""
    key = _rng.stream_key(wl.seed, STREAM_Q)
    T, W = wl.num_tokens, wl.num_q_heads * wl.head_size
    v = _rows_np(key, wl.q_ident, np.zeros(T, np.int64), W, wl.dtype)
    return v.reshape(T, wl.num_q_heads, wl.head_size)


def seq_kv_host(wl: Workload, s: int, which: str, upto: Optional[int] = None) -> np.ndarray:
    """Contiguous K or V rows [L, Hkv, D] of sequence s (never via a block table)."""
    L = int(wl.seq_lens[s]) if upto is None else int(upto)
    key = _rng.stream_key(wl.seed, STREAM_K if which == "k" else STREAM_V)
    pos = np.arange(L, dtype=np.int64)
    W = wl.num_kv_heads * wl.head_size
    return _rows_np(key, kv_ident(wl, s, pos), pos, W, wl.dtype).reshape(L, wl.num_kv_heads, wl.head_size)


def _new_token_coords(wl: Workload):
    n = wl.query_lens.astype(np.int64)
    seq_of_tok = np.repeat(np.arange(wl.num_seqs), n)
    pos = wl.context_lens[seq_of_tok].astype(np.int64) + (np.arange(wl.num_tokens) - wl.query_start_loc[seq_of_tok])
    ident = np.where(pos < wl.shared_len[seq_of_tok], SHARED_IDENT, wl.seq_ident[seq_of_tok]).astype(np.int64)
    return ident, pos


def new_kv_host(wl: Workload):
    """K and V rows [T, Hkv, D] of the new tokens (positions context_len + i)."""
    ident, pos = _new_token_coords(wl)
    W = wl.num_kv_heads * wl.head_size
    shape = (wl.num_tokens, wl.num_kv_heads, wl.head_size)
    k = _rows_np(_rng.stream_key(wl.seed, STREAM_K), ident, pos, W, wl.dtype).reshape(shape)
    v = _rows_np(_rng.stream_key(wl.seed, STREAM_V), ident, pos, W, wl.dtype).reshape(shape)
    return k, v


def prior_blocks(wl: Workload):
    """Pool blocks that hold cached (prior-context) rows, one entry per physical block.

    Returns (phys, ident, first_pos, limit): block ``phys`` holds positions
    first_pos .. first_pos + 15 of rows with identity ``ident``; only positions
    below ``limit`` are cached context, the rest of the block is canary.
    """
    phys, ident, first, limit = [], [], [], []
    seen_shared = False
    for s in range(wl.num_seqs):
        C = int(wl.context_lens[s])
        nb = -(-C // BLOCK_SIZE)
        sh = int(wl.shared_len[s]) // BLOCK_SIZE
        lo = 0
        if sh:
            if not seen_shared:
                phys.append(wl.block_tables[s, :sh])
                ident.append(np.full(sh, SHARED_IDENT))
                first.append(np.arange(sh) * BLOCK_SIZE)
                limit.append(np.full(sh, int(wl.shared_len[s])))
                seen_shared = True
            lo = sh
        if nb > lo:
            b = np.arange(lo, nb)
            phys.append(wl.block_tables[s, lo:nb])
            ident.append(np.full(nb - lo, wl.seq_ident[s]))
            first.append(b * BLOCK_SIZE)
            limit.append(np.full(nb - lo, C))
    if not phys:
        z = np.zeros(0, np.int64)
        return z, z, z, z
    cat = lambda xs: np.concatenate(xs).astype(np.int64)
    return cat(phys), cat(ident), cat(first), cat(limit)


def _context_table(wl: Workload) -> str:
    """The value table of a workload's cached context."""
    return "fp8band" if wl.pool_dtype == "fp8" and wl.fp8_codes == "band" else wl.pool_dtype


def pool_host(wl: Workload) -> np.ndarray:
    """Host pool [NB, 2, 16, Hkv, D] before the KV write: cached rows placed, canaries elsewhere."""
    Hkv, D, pd = wl.num_kv_heads, wl.head_size, wl.pool_dtype
    pool = np.empty((wl.num_blocks, 2, BLOCK_SIZE, Hkv, D), dtype=np_dtype(pd))
    pool[...] = canary_np(pd)
    phys, ident, first, limit = prior_blocks(wl)
    if phys.size == 0:
        return pool
    r = np.arange(BLOCK_SIZE)
    pos = (first[:, None] + r[None, :]).reshape(-1)
    idn = np.repeat(ident, BLOCK_SIZE)
    valid = (pos < np.repeat(limit, BLOCK_SIZE)).reshape(-1, BLOCK_SIZE)
    for kv, stream in ((0, STREAM_K), (1, STREAM_V)):
        vals = _rows_np(_rng.stream_key(wl.seed, stream), idn, pos, Hkv * D, _context_table(wl))
        vals = vals.reshape(-1, BLOCK_SIZE, Hkv, D)
        vals[~valid] = canary_np(pd)
        pool[phys, kv] = vals
    return pool


def sub_workload(wl: Workload, seqs: Sequence[int]) -> Workload:
    """The sequences ``seqs`` alone, with a compact pool.

    Identities are kept, so values are unchanged; physical blocks are relabelled
    in order of first use (plus one canary block).
    """
    seqs = np.asarray(seqs, dtype=np.int64)
    n = wl.query_lens[seqs].astype(np.int64)
    used = [wl.block_tables[s, : wl.blocks_used(s)] for s in seqs]
    uniq, order = [], {}
    for u in used:
        for b in u.tolist():
            if b not in order:
                order[b] = len(uniq)
                uniq.append(b)
    canary = len(uniq)
    MB = max(wl.blocks_used(s) for s in seqs)
    tables = np.full((len(seqs), MB), canary, np.int64)
    for i, u in enumerate(used):
        tables[i, : len(u)] = [order[b] for b in u.tolist()]
    qsl = np.zeros(len(seqs) + 1, np.int64)
    qsl[1:] = np.cumsum(n)
    q_ident = np.concatenate([wl.q_ident[wl.query_start_loc[s] : wl.query_start_loc[s + 1]] for s in seqs])
    C = wl.context_lens[seqs].astype(np.int64)
    T = int(qsl[-1])
    seq_of_tok = np.repeat(np.arange(len(seqs)), n)
    pos = C[seq_of_tok] + (np.arange(T) - qsl[seq_of_tok])
    slots = tables[seq_of_tok, pos // BLOCK_SIZE] * BLOCK_SIZE + pos % BLOCK_SIZE
    return dataclasses.replace(
        wl,
        name=wl.name + f"[{len(seqs)} seqs]",
        num_blocks=canary + 1,
        seq_lens=wl.seq_lens[seqs].copy(),
        context_lens=wl.context_lens[seqs].copy(),
        query_start_loc=qsl.astype(np.int32),
        block_tables=tables.astype(np.int32),
        slot_mapping=slots.astype(np.int64),
        seq_ident=wl.seq_ident[seqs].copy(),
        shared_len=wl.shared_len[seqs].copy(),
        q_ident=q_ident.astype(np.int64),
        canary_block=canary,
    )


def with_block_tables(wl: Workload, tables, num_blocks: int, canary_block: int) -> Workload:
    """Same sequences and values, placed through the given literal block tables."""
    tables = np.asarray(tables, dtype=np.int64)
    assert tables.shape[0] == wl.num_seqs
    n = wl.query_lens.astype(np.int64)
    C = wl.context_lens.astype(np.int64)
    T = wl.num_tokens
    seq_of_tok = np.repeat(np.arange(wl.num_seqs), n)
    pos = C[seq_of_tok] + (np.arange(T) - wl.query_start_loc[seq_of_tok])
    slots = tables[seq_of_tok, pos // BLOCK_SIZE] * BLOCK_SIZE + pos % BLOCK_SIZE
    return dataclasses.replace(wl, num_blocks=int(num_blocks), block_tables=tables.astype(np.int32),
                               slot_mapping=slots.astype(np.int64), canary_block=int(canary_block))


# --- device materialisation (torch; any device) -----------------------------
def _table_torch(dtype: str, device):
    import torch

    if dtype == "fp8band":
        return torch.from_numpy(_rng.FP8_CODES_BAND.copy()).to(device)
    if dtype == "fp8":
        return torch.from_numpy(_rng.FP8_CODES.copy()).to(device)
    if dtype == "f32":
        return torch.from_numpy(_rng.NORMAL_F32.copy()).to(device)
    return torch.from_numpy(_rng.NORMAL_BF16.view(np.int16).copy()).to(device).view(torch.bfloat16)


def torch_dtype(dtype: str):
    import torch

    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[dtype]


def _rows_torch(key, ident, pos, width, table):
    rk = _rng.row_keys_torch(key, ident, pos)
    return table[_rng.row_fields_torch(rk, width)]


def q_device(wl: Workload, device):
    import torch

    table = _table_torch(wl.dtype, device)
    key = _rng.stream_key(wl.seed, STREAM_Q)
    ident = torch.from_numpy(wl.q_ident).to(device)
    v = _rows_torch(key, ident, torch.zeros_like(ident), wl.num_q_heads * wl.head_size, table)
    return v.reshape(wl.num_tokens, wl.num_q_heads, wl.head_size).contiguous()


def new_kv_device(wl: Workload, device):
    import torch

    table = _table_torch(wl.dtype, device)
    ident, pos = _new_token_coords(wl)
    ident = torch.from_numpy(ident).to(device)
    pos = torch.from_numpy(pos).to(device)
    W = wl.num_kv_heads * wl.head_size
    shape = (wl.num_tokens, wl.num_kv_heads, wl.head_size)
    k = _rows_torch(_rng.stream_key(wl.seed, STREAM_K), ident, pos, W, table).reshape(shape).contiguous()
    v = _rows_torch(_rng.stream_key(wl.seed, STREAM_V), ident, pos, W, table).reshape(shape).contiguous()
    return k, v


def canary_torch(dtype: str, device):
    import torch

    if dtype == "fp8":
        return torch.tensor([_rng.CANARY_FP8], dtype=torch.uint8).to(device)
    if dtype == "f32":
        return torch.tensor([_rng.CANARY_F32_BITS], dtype=torch.int32).view(torch.float32).to(device)
    return torch.tensor([_rng.CANARY_BF16_BITS], dtype=torch.int16).view(torch.bfloat16).to(device)


def pool_device(wl: Workload, device, *, blocks_per_chunk: int = 8192):
    """Device pool [NB, 2, 16, Hkv, D] before the KV write (same bits as ``pool_host``)."""
    import torch

    Hkv, D, pd = wl.num_kv_heads, wl.head_size, wl.pool_dtype
    # an 8-bit pool is filled through a uint8 view (integer indexing) and returned as float8_e4m3fn
    pool = torch.empty((wl.num_blocks, 2, BLOCK_SIZE, Hkv, D), dtype=torch.uint8 if pd == "fp8" else torch_dtype(pd),
                       device=device)
    can = canary_torch(pd, device)
    fill_canary(pool, pd)
    phys, ident, first, limit = prior_blocks(wl)
    table = _table_torch(_context_table(wl), device)
    keys = (_rng.stream_key(wl.seed, STREAM_K), _rng.stream_key(wl.seed, STREAM_V))
    r = torch.arange(BLOCK_SIZE, device=device, dtype=torch.int64)
    for a in range(0, phys.size, blocks_per_chunk):
        b = min(phys.size, a + blocks_per_chunk)
        ph = torch.from_numpy(phys[a:b]).to(device)
        pos = (torch.from_numpy(first[a:b]).to(device)[:, None] + r[None, :]).reshape(-1)
        idn = torch.from_numpy(ident[a:b]).to(device).repeat_interleave(BLOCK_SIZE)
        lim = torch.from_numpy(limit[a:b]).to(device).repeat_interleave(BLOCK_SIZE)
        invalid = (pos >= lim).reshape(-1, BLOCK_SIZE)
        for kv in (0, 1):
            vals = _rows_torch(keys[kv], idn, pos, Hkv * D, table).reshape(-1, BLOCK_SIZE, Hkv, D)
            vals[invalid] = can
            pool[ph, kv] = vals
    return pool.view(torch.float8_e4m3fn) if pd == "fp8" else pool


def fill_canary(t, dtype: str):
    """Fill a tensor with the NaN canary bit pattern (exact bits, in place)."""
    import torch

    if dtype == "fp8":
        t.view(torch.uint8).fill_(_rng.CANARY_FP8)
    elif dtype == "f32":
        t.view(torch.int32).fill_(_rng.CANARY_F32_BITS)
    else:
        t.view(torch.int16).fill_(_rng.CANARY_BF16_BITS)
    return t


# ---------------------------------------------------------------------------
# Token-stream inputs for multi-step runs (a request's tokens arrive and are
# computed over several steps). A position's rows depend on every token id
# up to and including it, as a model's K/V do, so requests that share a
# token prefix share those rows exactly, which is what lets one request's
# cached blocks serve another.


def prefix_idents(tokens) -> np.ndarray:
    """Identity of each position of a token sequence: a 62-bit chained digest
    (BLAKE2b) of the token ids up to and including it."""
    out = np.empty(len(tokens), np.int64)
    prev = b"\0" * 8
    for i, t in enumerate(tokens):
        prev = hashlib.blake2b(prev + int(t).to_bytes(4, "little", signed=True), digest_size=8).digest()
        out[i] = int.from_bytes(prev, "little") >> 2
    return out


def token_rows(seed: int, stream: int, idents, positions, heads: int, head_size: int, dtype: str) -> np.ndarray:
    """Rows [n, heads, head_size] (host element type) addressed by (identity, position)."""
    key = _rng.stream_key(seed, stream)
    rows = _rows_np(key, np.asarray(idents, np.int64), np.asarray(positions, np.int64), heads * head_size, dtype)
    return rows.reshape(-1, heads, head_size)


def with_fp8_pool(wl: Workload, k_scale: float = 1.0, v_scale: float = 1.0, codes: str = "normal") -> Workload:
    """The same workload over an 8-bit pool: q, k, v and out keep ``dtype`` (bf16);
    cached context is drawn as E4M3 codes (``codes``: "normal" or the heavier-
    tailed "band"); new tokens are quantized by the KV write."""
    assert wl.dtype == "bf16", "8-bit pools are read by the bf16 compute path"
    assert codes in ("normal", "band")
    return dataclasses.replace(wl, name=wl.name.replace("_bf16", "") + "_fp8kv", kv_dtype="fp8",
                               k_scale=float(np.float32(k_scale)), v_scale=float(np.float32(v_scale)),
                               fp8_codes=codes)
