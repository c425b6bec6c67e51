"""Block bookkeeping and block copies, plain and slow -- TEST INFRASTRUCTURE ONLY.

What the pages fix ("vLLM 与 PagedAttention", section 二 "PagedAttention 的解
法"; "vLLM让大模型推理快10倍？..." section "PagedAttention怎么解决？"; "指南",
"Copy-on-Write：Prefix Caching 的基础"; "4. vLLM初识" 4.3):

* the KV history of a request lives in fixed-size blocks of one shared pool,
  reached through the request's own table (logical block -> physical block);
* a block is taken from the pool only when the request's last block is full
  (no reservation ahead of need); a request of n tokens holds ceil(n / bs);
* requests with the same prefix point at the same physical blocks and read
  them shared; a request that writes into a shared block first copies it
  (copy on write), so the others keep the old contents;
* under memory pressure a request's KV moves to CPU memory and comes back
  later.

Readings where the pages are silent (the library follows the same ones):
* a free block is taken lowest index first, so that every run is
  reproducible; a finished request's blocks return to the pool when no other
  request holds them;
* swapping out copies every block of the request to a CPU block (a block that
  other requests still hold stays on the GPU for them); swapping in gives the
  request fresh GPU blocks, no longer shared;
* an operation that would need more free blocks than there are does nothing
  and reports it.

``BlockManagerModel`` is the bookkeeping; ``copy_blocks`` / ``swap_blocks``
are the data movement the bookkeeping asks for, on numpy pools
``[num_blocks, ...]``.
"""
from __future__ import annotations

import numpy as np


class NoBlocks(Exception):
    """Not enough free blocks for the operation (nothing was changed)."""


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs) -> None:
    """For each (src, dst): block dst of both pools takes the contents block src
    had before the call.  A pair with an index outside the pool is skipped."""
    swap_blocks(k_cache, v_cache, k_cache.copy(), v_cache.copy(), pairs)


def swap_blocks(dst_k: np.ndarray, dst_v: np.ndarray, src_k: np.ndarray, src_v: np.ndarray, pairs) -> None:
    """For each (src, dst): block dst of the destination pools takes block src
    of the source pools (a pair with an index outside either pool is skipped)."""
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if 0 <= src < src_k.shape[0] and 0 <= dst < dst_k.shape[0]:
            dst_k[dst] = src_k[src]
            dst_v[dst] = src_v[src]


class BlockManagerModel:
    """Tables, reference counts and free blocks of a GPU and a CPU pool."""

    def __init__(self, num_gpu_blocks: int, num_cpu_blocks: int, block_size: int):
        self.bs = block_size
        self.ref = {"gpu": [0] * num_gpu_blocks, "cpu": [0] * num_cpu_blocks}
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.where: dict[int, str] = {}            # "gpu" or "cpu"

    # -- the pools ----------------------------------------------------------
    def free_blocks(self, pool: str = "gpu") -> list[int]:
        return [b for b, r in enumerate(self.ref[pool]) if r == 0]

    def _take(self, pool: str) -> int:
        free = self.free_blocks(pool)
        if not free:
            raise NoBlocks(pool)
        b = min(free)
        self.ref[pool][b] = 1
        return b

    def _drop(self, pool: str, b: int) -> None:
        self.ref[pool][b] -= 1
        assert self.ref[pool][b] >= 0

    def _available(self, pool: str) -> int:
        """Blocks an allocation can take."""
        return len(self.free_blocks(pool))

    # -- requests -----------------------------------------------------------
    def add(self, sid: int) -> None:
        assert sid not in self.tables
        self.tables[sid], self.lens[sid], self.where[sid] = [], 0, "gpu"

    def fork(self, parent: int, child: int) -> None:
        """child reads parent's blocks, shared."""
        assert self.where[parent] == "gpu" and child not in self.tables
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        self.where[child] = "gpu"
        for b in self.tables[child]:
            self.ref["gpu"][b] += 1

    def blocks_needed(self, sid: int, n: int) -> int:
        """Free GPU blocks an append of n tokens takes (new blocks + one copy)."""
        t0, bs, table = self.lens[sid], self.bs, self.tables[sid]
        new = -(-(t0 + n) // bs) - len(table)
        cow = 1 if n > 0 and t0 % bs != 0 and self.ref["gpu"][table[t0 // bs]] > 1 else 0
        return new + cow

    def append(self, sid: int, n: int):
        """Grow a request by n tokens: (slot of each new token, copies (src, dst))."""
        assert self.where[sid] == "gpu"
        if self.blocks_needed(sid, n) > self._available("gpu"):
            raise NoBlocks("gpu")
        table, bs = self.tables[sid], self.bs
        slots, copies = [], []
        for t in range(self.lens[sid], self.lens[sid] + n):
            j = t // bs
            if j == len(table):                      # the last block is full: take one
                table.append(self._take("gpu"))
            elif self.ref["gpu"][table[j]] > 1:      # writing into a shared block: copy it first
                new = self._take("gpu")
                copies.append((table[j], new))
                self._drop("gpu", table[j])
                table[j] = new
            slots.append(table[j] * bs + t % bs)
        self.lens[sid] += n
        return slots, copies

    def free(self, sid: int) -> None:
        """Drop a request; its blocks are released last block first."""
        pool = self.where.pop(sid)
        for b in reversed(self.tables.pop(sid)):
            self._drop(pool, b)
        del self.lens[sid]

    def swap_out(self, sid: int):
        """Move a request to CPU blocks: (gpu block, cpu block) pairs to copy."""
        assert self.where[sid] == "gpu"
        table = self.tables[sid]
        if len(table) > self._available("cpu"):
            raise NoBlocks("cpu")
        pairs = [(b, self._take("cpu")) for b in table]
        for b in reversed(table):                   # GPU blocks released last block first
            self._drop("gpu", b)
        table[:] = [c for _, c in pairs]
        self.where[sid] = "cpu"
        return pairs

    def swap_in(self, sid: int):
        """Move a request back to fresh GPU blocks: (cpu block, gpu block) pairs."""
        assert self.where[sid] == "cpu"
        table = self.tables[sid]
        if len(table) > self._available("gpu"):
            raise NoBlocks("gpu")
        pairs = []
        for j, c in enumerate(table):
            b = self._take("gpu")
            pairs.append((c, b))
            self._drop("cpu", c)
            table[j] = b
        self.where[sid] = "gpu"
        return pairs

    def block_tables(self, sids, max_blocks: int):
        """Dense int32 [len(sids), max_blocks] tables (-1 past the end) and int32 lengths."""
        tables = np.full((len(sids), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(sids), dtype=np.int32)
        for i, s in enumerate(sids):
            assert self.where[s] == "gpu" and len(self.tables[s]) <= max_blocks
            tables[i, :len(self.tables[s])] = self.tables[s]
            lens[i] = self.lens[s]
        return tables, lens
