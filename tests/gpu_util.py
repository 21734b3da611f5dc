"""Helpers for the GPU parity tests: put a workload on the device, run the
library through its C ABI, bring results back as numpy."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W


def device_case(wl, device="cuda"):
    """All inputs of one step on the device (pool before the KV write)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    q = W.q_device(wl, device)
    k, v = W.new_kv_device(wl, device)
    pool = W.pool_device(wl, device)
    return {
        "q": q, "k": k, "v": v, "pool": pool,
        "slot_mapping": t(wl.slot_mapping), "block_tables": t(wl.block_tables),
        "query_start_loc": t(wl.query_start_loc), "seq_lens": t(wl.seq_lens), "context_lens": t(wl.context_lens),
    }


def run_step(pa, wl, c, out=None, workspace=None):
    """pa_step: KV write then attention, through the C ABI."""
    pool = c["pool"]
    return pa.step(c["q"], c["k"], c["v"], pool[:, 0], pool[:, 1], c["slot_mapping"], c["block_tables"],
                   c["query_start_loc"], c["seq_lens"], c["context_lens"], wl.scale, out=out, workspace=workspace)


def to_f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def raw_bytes(x: torch.Tensor) -> np.ndarray:
    """The tensor's bytes, flattened (uint8)."""
    x = x.detach().contiguous()
    if x.dtype == torch.bfloat16:
        x = x.view(torch.int16)
    return x.cpu().numpy().reshape(-1).view(np.uint8)


def sample_seqs(wl, k: int, seed: int = 0):
    """A sample of sequences that always holds the longest and shortest of each kind."""
    rs = np.random.default_rng(seed)
    pick = set()
    dec = np.nonzero(wl.decode_mask())[0]
    pre = np.nonzero(~wl.decode_mask())[0]
    for group in (dec, pre):
        if group.size:
            L = wl.seq_lens[group]
            pick.update([int(group[np.argmax(L)]), int(group[np.argmin(L)])])
    rest = np.setdiff1d(np.arange(wl.num_seqs), sorted(pick))
    extra = rs.choice(rest, size=min(k, rest.size), replace=False) if rest.size else []
    return sorted(pick.union(int(x) for x in extra))


def rows_of(wl, seqs):
    return np.concatenate([np.arange(wl.query_start_loc[s], wl.query_start_loc[s + 1]) for s in seqs])
