"""Plain model of the KV block manager -- TEST INFRASTRUCTURE ONLY.

A slow, obviously correct restatement of what the pages say the KV-cache
manager does, used to check the library's C++ manager decision by decision
(which blocks, which hits, which reference counts). It shares no code with
the library.

- Free block queue: a Python list; allocation takes from the front, a block
  whose last reference goes away is appended at the back ("Inside vLLM:
  Anatomy of a High-Throughput LLM Inference System", section "Scheduler",
  allocate_slots and the free_block_queue; section "Engine loop").
- allocate_slots: ceil((computed + new) / block_size) blocks in all; if the
  queue is too short nothing changes (same section).
- Prefix caching: a block's hash depends on every token before it and on its
  own ("Inside vLLM", section "Prefix caching"; "Serving models at scale with
  vLLM", section "Prefix caching"). The model keys its cache on that whole
  token prefix itself (plus the cache salt), which is what the hash chain
  stands for, so it needs no hash function. Hits pin the block (reference
  count + 1; a free block leaves the queue); recycling a free block forgets
  its prefix. Freed blocks are recycled least recently freed first.
- Readings where the pages are silent (the same as the library's): hits stop
  one block short of the whole prompt; a request frees its blocks last block
  first; hits are taken when the request is added.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


class NoBlocks(Exception):
    """The free queue holds fewer blocks than the request needs."""


class BlockModel:
    def __init__(self, num_blocks: int, block_size: int, prefix_caching: bool = True):
        self.bs = block_size
        self.caching = prefix_caching
        self.free_queue: List[int] = list(range(num_blocks))
        self.ref = [0] * num_blocks
        self.key_of: Dict[int, Tuple] = {}  # cached block -> its prefix key
        self.block_of: Dict[Tuple, int] = {}  # prefix key -> cached block
        self.reqs: Dict[int, dict] = {}

    def _key(self, req: dict, i: int) -> Tuple:
        """Identity of the request's block i: salt and every token up to its end."""
        return (req["salt"], tuple(req["tokens"][: (i + 1) * self.bs]))

    def add_request(self, rid: int, prompt: Sequence[int], salt: int = 0) -> int:
        assert rid not in self.reqs and len(prompt) >= 1
        req = {"tokens": list(prompt), "salt": salt, "computed": 0, "blocks": [], "hashed": 0}
        if self.caching:
            for i in range((len(prompt) - 1) // self.bs):
                b = self.block_of.get(self._key(req, i))
                if b is None:
                    break
                req["blocks"].append(b)
            for b in req["blocks"]:
                if self.ref[b] == 0:
                    self.free_queue.remove(b)
                self.ref[b] += 1
            req["hashed"] = len(req["blocks"])
            req["computed"] = len(req["blocks"]) * self.bs
        self.reqs[rid] = req
        return req["computed"]

    def append_tokens(self, rid: int, tokens: Sequence[int]):
        self.reqs[rid]["tokens"].extend(tokens)

    def allocate_slots(self, rid: int, n_new: int):
        req = self.reqs[rid]
        assert req["computed"] + n_new <= len(req["tokens"])
        need = -(-(req["computed"] + n_new) // self.bs) - len(req["blocks"])
        if need <= 0:
            return
        if need > len(self.free_queue):
            raise NoBlocks(rid)
        for _ in range(need):
            b = self.free_queue.pop(0)
            if b in self.key_of:  # recycled: its cached prefix is forgotten
                del self.block_of[self.key_of.pop(b)]
            self.ref[b] = 1
            req["blocks"].append(b)

    def commit(self, rid: int, n_new: int):
        req = self.reqs[rid]
        req["computed"] += n_new
        assert req["computed"] <= min(len(req["tokens"]), len(req["blocks"]) * self.bs)
        if not self.caching:
            return
        while (req["hashed"] + 1) * self.bs <= req["computed"]:
            i = req["hashed"]
            req["hashed"] += 1
            b, key = req["blocks"][i], self._key(req, i)
            if b in self.key_of or key in self.block_of:
                continue
            self.key_of[b] = key
            self.block_of[key] = b

    def free(self, rid: int):
        req = self.reqs.pop(rid)
        for b in reversed(req["blocks"]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free_queue.append(b)

    def step_inputs(self, rids: Sequence[int], n_new: Sequence[int], max_blocks: int) -> dict:
        qsl, seq_lens, ctx, tables, slots = [0], [], [], [], []
        for rid, n in zip(rids, n_new):
            req = self.reqs[rid]
            C = req["computed"]
            seq_lens.append(C + n)
            ctx.append(C)
            tables.append(req["blocks"] + [0] * (max_blocks - len(req["blocks"])))
            slots += [req["blocks"][p // self.bs] * self.bs + p % self.bs for p in range(C, C + n)]
            qsl.append(len(slots))
        return {"query_start_loc": qsl, "seq_lens": seq_lens, "context_lens": ctx, "block_tables": tables,
                "slot_mapping": slots}

    def num_free(self) -> int:
        return len(self.free_queue)

    def is_cached(self, b: int) -> bool:
        return b in self.key_of

    def request_blocks(self, rid: int) -> Tuple[List[int], int]:
        req = self.reqs[rid]
        return list(req["blocks"]), req["computed"]

    def cached_block(self, salt: int, tokens: Sequence[int]) -> Optional[int]:
        return self.block_of.get((salt, tuple(tokens)))
