"""Automatic prefix caching over the block bookkeeping, plain and slow --
TEST INFRASTRUCTURE ONLY.

What the pages fix ("vLLM 与 PagedAttention" section 四 "Prefix Caching：复用
system prompt 的 KV"; section 二 "PagedAttention 的解法": requests with the same
prefix point at the same physical blocks; "指南", "Copy-on-Write：Prefix
Caching 的基础"):

* the first request to prefill a prompt leaves its KV in a cache kept in
  least-recently-used order;
* a later request whose prompt starts the same way reuses that KV and
  prefills only the rest (the pages' customer-service example: a 1500-token
  system prompt and an 8-token question);
* the reuse is read-only sharing of physical blocks, copied on write.

Readings where the pages are silent (the library follows the same ones):

* the unit of caching is a full block: block i of a request is known by its
  whole token prefix, tokens[0 : (i + 1) * block_size] -- the same tokens
  after a different prefix are a different block; a partly filled block is
  never cached;
* a new request reuses the longest run of cached blocks that its prompt
  starts with, but always leaves at least one prompt token to compute (the
  caller needs that token's output), so at most (n - 1) // block_size blocks;
* a block becomes a cache entry as soon as the request that fills it has all
  its tokens (the caller writes their KV before the next request looks the
  prompt up); if that prefix is already cached in another block, the new
  block stays private;
* a cached block that no request holds is still cached but can be taken:
  an allocation takes a free block if there is one (lowest index first),
  else the cached block released longest ago (ties: lowest index), which
  leaves the cache;
* a request's blocks are released last block first, so that the head of a
  prefix outlives its tail in the cache;
* only requests whose every token was given (``add_cached`` /
  ``append_tokens``) put blocks in the cache.

The model keys the cache by the token prefix itself (a tuple), so a lookup
is exact by construction.
"""
from __future__ import annotations

from .blocks import BlockManagerModel, NoBlocks


class PrefixCacheModel(BlockManagerModel):
    """BlockManagerModel with an index of cached GPU blocks by token prefix."""

    def __init__(self, num_gpu_blocks: int, num_cpu_blocks: int, block_size: int):
        super().__init__(num_gpu_blocks, num_cpu_blocks, block_size)
        self.cache: dict[tuple, int] = {}        # token prefix through a full block -> block
        self.key_of: dict[int, tuple] = {}       # cached block -> its prefix
        self.released: dict[int, int] = {}       # cached block -> clock when its last holder let go
        self.clock = 0
        self.tokens: dict[int, list | None] = {}   # every token of a request, or None if not all known
        self.registered: dict[int, int] = {}       # blocks of a request already offered to the cache

    # -- the GPU pool with cached blocks --------------------------------------
    def free_blocks(self, pool: str = "gpu") -> list[int]:
        return [b for b, r in enumerate(self.ref[pool]) if r == 0 and not (pool == "gpu" and b in self.key_of)]

    def evictable(self) -> list[int]:
        return [b for b in self.key_of if self.ref["gpu"][b] == 0]

    def _available(self, pool: str) -> int:
        return len(self.free_blocks(pool)) + (len(self.evictable()) if pool == "gpu" else 0)

    def _take(self, pool: str) -> int:
        if pool == "gpu" and not self.free_blocks("gpu") and self.evictable():
            b = min(self.evictable(), key=lambda x: (self.released[x], x))
            del self.cache[self.key_of.pop(b)]
            del self.released[b]
        return super()._take(pool)

    def _drop(self, pool: str, b: int) -> None:
        super()._drop(pool, b)
        if pool == "gpu" and self.ref["gpu"][b] == 0 and b in self.key_of:
            self.clock += 1
            self.released[b] = self.clock

    def _hold(self, b: int) -> None:
        self.ref["gpu"][b] += 1

    # -- requests ---------------------------------------------------------------
    def add(self, sid: int) -> None:
        super().add(sid)
        self.tokens[sid], self.registered[sid] = [], 0

    def add_cached(self, sid: int, prompt) -> int:
        """A new request for `prompt`: its table starts with the cached blocks the
        prompt begins with.  Returns the tokens already there (a multiple of
        block_size, less than len(prompt) unless the prompt is empty)."""
        prompt = list(prompt)
        super().add(sid)
        bs, table = self.bs, self.tables[sid]
        for i in range(max(0, (len(prompt) - 1) // bs)):
            b = self.cache.get(tuple(prompt[: (i + 1) * bs]))
            if b is None:
                break
            self._hold(b)
            table.append(b)
        self.lens[sid] = len(table) * bs
        self.tokens[sid] = prompt[: self.lens[sid]]
        self.registered[sid] = len(table)
        return self.lens[sid]

    def _register(self, sid: int) -> None:
        toks, bs, table = self.tokens[sid], self.bs, self.tables[sid]
        if toks is None:
            return
        for j in range(self.registered[sid], len(toks) // bs):
            key = tuple(toks[: (j + 1) * bs])
            if key not in self.cache and table[j] not in self.key_of:
                self.cache[key] = table[j]
                self.key_of[table[j]] = key
        self.registered[sid] = max(self.registered[sid], len(toks) // bs)

    def append(self, sid: int, n: int):
        out = super().append(sid, n)
        if n > 0:
            self.tokens[sid] = None              # tokens unknown from here on
        return out

    def append_tokens(self, sid: int, new_tokens):
        new_tokens = list(new_tokens)
        slots, copies = super().append(sid, len(new_tokens))
        if self.tokens[sid] is not None:
            self.tokens[sid] += new_tokens
            self._register(sid)
        return slots, copies

    def fork(self, parent: int, child: int) -> None:
        super().fork(parent, child)
        t = self.tokens[parent]
        self.tokens[child] = None if t is None else list(t)
        self.registered[child] = self.registered[parent]

    def free(self, sid: int) -> None:
        super().free(sid)
        del self.tokens[sid], self.registered[sid]

    def swap_in(self, sid: int):
        pairs = super().swap_in(sid)
        # fresh GPU copies: the full blocks among them are not offered to the cache
        self.registered[sid] = len(self.tables[sid]) if self.tokens[sid] is None else \
            len(self.tokens[sid]) // self.bs
        return pairs

    def cache_stats(self) -> tuple[int, int]:
        """(cached blocks, cached blocks no request holds)."""
        return len(self.key_of), len(self.evictable())


__all__ = ["PrefixCacheModel", "NoBlocks"]
