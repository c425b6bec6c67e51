"""Seeded synthetic inputs for paged decode attention and the KV append.

This module only draws inputs: random q/K/V, block tables, context lengths,
slot mappings and pools.  It holds none of the attention arithmetic, and both
the GPU path and the CPU oracle receive exactly the arrays it returns.

Workload shapes follow the pages' workloads (see the workload docstrings):
block size 16 by default with 8/16/32 as the alternatives, Llama-2-7B-shaped
heads (32 heads x 128), a Llama-2-70B-shaped grouped-query layer (64 query
heads over 8 KV heads), a 20 % short / 80 % long request mix, and a ~1500
token shared system prompt.  The pages name no public benchmark or dataset
for this path; these generators stand in for their workloads.

Storage convention: f32 -> numpy.float32, f16 -> numpy.float16, bf16 ->
numpy.uint16 holding bfloat16 bit patterns (numpy has no bfloat16).  Caches
are returned in the pages' layout [num_blocks, block_size, num_kv_heads,
head_dim] ("block, token, head, dim").
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
NAN_BITS = {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}


def blocks_needed(tokens: int, block_size: int) -> int:
    """Blocks a request of `tokens` tokens occupies (a partly filled last block counts)."""
    return -(-int(tokens) // int(block_size))


def kv_bytes(context_lens, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K plus V bytes one decode call must read: sum_s ctx_s * Hkv * 2 * D * es."""
    return int(np.sum(np.asarray(context_lens, dtype=np.int64))) * num_kv_heads * 2 * head_dim * elem_bytes


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """KV cache bytes per token of a whole model: 2 (K and V) * L * H * D * es."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


def to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 draws to the storage type (nearest, ties to even)."""
    if dtype == "f32":
        return x32.astype(np.float32, copy=False)
    if dtype == "f16":
        return x32.astype(np.float16)
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    return ((u + (0x7FFF + ((u >> 16) & 1))) >> 16).astype(np.uint16)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    q: np.ndarray                 # [S, Hq, D]
    k_cache: np.ndarray           # [NB, bs, Hkv, D]  (slots of the appended tokens poisoned when poison=True)
    v_cache: np.ndarray
    block_tables: np.ndarray      # [S, MB] int32, -1 past each sequence's last block
    context_lens: np.ndarray      # [S] int32, appended token included
    scale: float                  # an fp32 value
    partition_tokens: int         # split-K partition the workload is specified with (0 = library's choice)
    new_k: Optional[np.ndarray] = None         # [T, Hkv, D] tokens appended this step
    new_v: Optional[np.ndarray] = None
    slot_mapping: Optional[np.ndarray] = None  # [T] int64
    description: str = ""
    shared_prefix_blocks: int = 0              # leading blocks every table shares (0: blocks are private)

    @property
    def num_seqs(self): return self.q.shape[0]
    @property
    def num_q_heads(self): return self.q.shape[1]
    @property
    def head_dim(self): return self.q.shape[2]
    @property
    def num_blocks(self): return self.k_cache.shape[0]
    @property
    def block_size(self): return self.k_cache.shape[1]
    @property
    def num_kv_heads(self): return self.k_cache.shape[2]
    @property
    def max_blocks_per_seq(self): return self.block_tables.shape[1]
    @property
    def elem_bytes(self): return ELEM_BYTES[self.dtype]

    def kv_bytes(self) -> int:
        return kv_bytes(self.context_lens, self.num_kv_heads, self.head_dim, self.elem_bytes)


def _scatter_tables(rng, nblk_per_seq, MB, NB, shared_prefix=None):
    """Block tables with distinct physical blocks drawn from one permutation of the pool.

    shared_prefix: list of physical blocks every table starts with (they are
    drawn first from the same permutation).
    """
    S = len(nblk_per_seq)
    perm = rng.permutation(NB).astype(np.int32)
    tables = np.full((S, MB), -1, dtype=np.int32)
    pos = 0
    prefix = []
    if shared_prefix:
        prefix = list(perm[:shared_prefix])
        pos = shared_prefix
    for s, n in enumerate(nblk_per_seq):
        row = list(prefix[: min(len(prefix), n)])
        take = n - len(row)
        row.extend(perm[pos:pos + take])
        pos += take
        tables[s, :n] = row
    assert pos <= NB
    return tables


def _fill_pool(rng, NB, bs, Hkv, D, dtype, tables, ctx, poison):
    """Pool of N(0,1) values; with poison, every slot no table maps below ctx is NaN."""
    k = to_storage(rng.standard_normal((NB, bs, Hkv, D), dtype=np.float32), dtype)
    v = to_storage(rng.standard_normal((NB, bs, Hkv, D), dtype=np.float32), dtype)
    if poison:
        live = np.zeros((NB, bs), dtype=bool)
        for s in range(tables.shape[0]):
            L = int(ctx[s])
            n = blocks_needed(L, bs)
            if n == 0:
                continue
            blocks = tables[s, :n]
            live[blocks[:-1], :] = True
            tail = L - (n - 1) * bs
            live[blocks[-1], :tail] = True
        k[~live] = NAN_BITS[dtype]
        v[~live] = NAN_BITS[dtype]
    return k, v


def _take_appended(k, v, tables, ctx, bs, poison, dtype, rows=None):
    """Move each listed sequence's last token out of the pool into new_k/new_v.

    The slot goes back to NaN (poison) so only the append can make it valid.
    """
    S = tables.shape[0]
    rows = range(S) if rows is None else rows
    slots, nk, nv = [], [], []
    for s in rows:
        t = int(ctx[s]) - 1
        b = int(tables[s, t // bs])
        off = t % bs
        slots.append(b * bs + off)
        nk.append(k[b, off].copy())
        nv.append(v[b, off].copy())
        if poison:
            k[b, off] = NAN_BITS[dtype]
            v[b, off] = NAN_BITS[dtype]
    return np.stack(nk), np.stack(nv), np.array(slots, dtype=np.int64)


def _pool_size(needed: int) -> int:
    """Needed blocks plus 10 % free blocks."""
    return needed + max(1, int(math.ceil(0.10 * needed)))


def _finish(name, dtype, rng, q_shape, ctx, bs, Hkv, D, MB, poison, append, scale, partition_tokens,
            description, NB=None, shared_prefix_blocks=None):
    ctx = np.asarray(ctx, dtype=np.int32)
    nblk = [blocks_needed(c, bs) for c in ctx]
    if shared_prefix_blocks:
        needed = shared_prefix_blocks + sum(n - shared_prefix_blocks for n in nblk)
    else:
        needed = sum(nblk)
    NB = NB if NB is not None else _pool_size(needed)
    tables = _scatter_tables(rng, nblk, MB, NB, shared_prefix=shared_prefix_blocks)
    q = to_storage(rng.standard_normal(q_shape, dtype=np.float32), dtype)
    k, v = _fill_pool(rng, NB, bs, Hkv, D, dtype, tables, ctx, poison)
    w = Workload(name=name, dtype=dtype, q=q, k_cache=k, v_cache=v, block_tables=tables,
                 context_lens=ctx, scale=float(np.float32(scale)), partition_tokens=partition_tokens,
                 description=description, shared_prefix_blocks=int(shared_prefix_blocks or 0))
    if append:
        w.new_k, w.new_v, w.slot_mapping = _take_appended(k, v, tables, ctx, bs, poison, dtype)
    return w


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def tiny_f32(seed: int = 1, poison: bool = True, append: bool = True) -> Workload:
    """3 sequences, 2 heads (MHA), head_dim 32, block size 16, context {1, 17, 40},
    fp32, a pool of 8 physical blocks, tables from a seeded permutation of the pool."""
    rng = np.random.default_rng(seed)
    return _finish("tiny_f32", "f32", rng, (3, 2, 32), [1, 17, 40], 16, 2, 32, 3, poison, append,
                   1.0 / math.sqrt(32), 0, "3 seqs x 2 heads x 32, fp32, bs 16, ctx {1,17,40}, pool 8",
                   NB=8)


def llama7b(seed: int = 2, poison: bool = True, append: bool = True, num_seqs: int = 64,
            max_ctx: int = 2048, block_size: int = 16) -> Workload:
    """Llama-2-7B-shaped single-layer decode: 32 q heads = 32 kv heads x 128, fp16,
    block size 16, context uniform in [1, 2048], pool = needed + 10 %, plus the
    append of one token per sequence."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1, max_ctx + 1, size=num_seqs)
    MB = blocks_needed(max_ctx, block_size)
    return _finish("llama7b", "f16", rng, (num_seqs, 32, 128), ctx, block_size, 32, 128, MB, poison,
                   append, 1.0 / math.sqrt(128), 0,
                   f"{num_seqs} seqs, 32x128 MHA, fp16, bs {block_size}, ctx U[1,{max_ctx}]")


def mixed_batch(block_size: int = 16, seed: int = 3, poison: bool = True, append: bool = True,
                num_seqs: int = 256) -> Workload:
    """Continuous-batching step: 20 % short requests (prompt 64 + U[1,50] generated),
    80 % long (prompt 512 + U[1,300] generated), shuffled; Llama-2-7B heads, fp16.
    The context lengths do not depend on block_size (same seed -> same lengths)."""
    rng = np.random.default_rng(seed)
    n_short = int(round(0.2 * num_seqs))
    short = 64 + rng.integers(1, 51, size=n_short)
    long_ = 512 + rng.integers(1, 301, size=num_seqs - n_short)
    ctx = np.concatenate([short, long_])
    rng.shuffle(ctx)
    MB = blocks_needed(512 + 300, block_size)
    return _finish(f"mixed_bs{block_size}", "f16", rng, (num_seqs, 32, 128), ctx, block_size, 32, 128,
                   MB, poison, append, 1.0 / math.sqrt(128), 0,
                   f"{num_seqs} seqs, 20% short / 80% long, 32x128 fp16, bs {block_size}")


def shared_prefix(seed: int = 4, poison: bool = True, append: bool = True, num_seqs: int = 128) -> Workload:
    """Copy-on-write shared prefix: every table starts with the same 94 physical blocks
    (a 1504-token system prompt at block size 16), then 1-13 private blocks
    (8-200 private tokens); 32x128 heads, fp16."""
    rng = np.random.default_rng(seed)
    bs, prefix_blocks = 16, 94
    priv = rng.integers(8, 201, size=num_seqs)
    ctx = prefix_blocks * bs + priv
    MB = prefix_blocks + blocks_needed(200, bs)
    return _finish("shared_prefix", "f16", rng, (num_seqs, 32, 128), ctx, bs, 32, 128, MB, poison, append,
                   1.0 / math.sqrt(128), 0,
                   f"{num_seqs} seqs, 94 shared prefix blocks + 8..200 private tokens, 32x128 fp16, bs 16",
                   shared_prefix_blocks=prefix_blocks)


def llama70b_gqa(seed: int = 5, poison: bool = True, append: bool = True, num_seqs: int = 32,
                 min_ctx: int = 2048, max_ctx: int = 8192) -> Workload:
    """Llama-2-70B-shaped grouped-query long context: 64 q heads over 8 kv heads x 128,
    bf16, block size 16, context uniform in [2048, 8192], split-K partitions of 512
    tokens."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(min_ctx, max_ctx + 1, size=num_seqs)
    MB = blocks_needed(max_ctx, 16)
    return _finish("llama70b_gqa", "bf16", rng, (num_seqs, 64, 128), ctx, 16, 8, 128, MB, poison, append,
                   1.0 / math.sqrt(128), 512,
                   f"{num_seqs} seqs, 64 q / 8 kv heads x 128, bf16, bs 16, ctx U[{min_ctx},{max_ctx}]")


def llama70b_tp8(seed: int = 5, poison: bool = True, append: bool = True, num_seqs: int = 32,
                 min_ctx: int = 2048, max_ctx: int = 8192) -> Workload:
    """One GPU's share of the Llama-2-70B-shaped workload when its heads are split over
    8 GPUs: 8 q heads over 1 kv head x 128, bf16, block size 16, the same context
    lengths (same seed, U[2048, 8192])."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(min_ctx, max_ctx + 1, size=num_seqs)
    MB = blocks_needed(max_ctx, 16)
    return _finish("llama70b_tp8", "bf16", rng, (num_seqs, 8, 128), ctx, 16, 1, 128, MB, poison, append,
                   1.0 / math.sqrt(128), 512,
                   f"{num_seqs} seqs, 8 q / 1 kv head x 128 (one of 8 head shards), bf16, bs 16, "
                   f"ctx U[{min_ctx},{max_ctx}]")


def custom(name: str, dtype: str, ctxs, num_q_heads: int, num_kv_heads: int, head_dim: int,
           block_size: int, seed: int = 0, poison: bool = True, append: bool = False,
           free_fraction: float = 0.10, table_pad: int = 0, scale: Optional[float] = None,
           partition_tokens: int = 0, shared_prefix_blocks: int = 0) -> Workload:
    """Any shape, for edge cases: explicit context lengths, optional extra table columns; with
    shared_prefix_blocks every table starts with the same blocks (as far as its own blocks go)."""
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctxs, dtype=np.int32)
    nblk = [blocks_needed(c, block_size) for c in ctx]
    MB = max(max(nblk) if len(nblk) else 1, 1) + table_pad
    needed = sum(nblk)
    NB = max(1, needed + int(math.ceil(free_fraction * needed)))
    if append:
        assert np.all(ctx >= 1)
    w = _finish(name, dtype, rng, (len(ctx), num_q_heads, head_dim), ctx, block_size, num_kv_heads,
                head_dim, MB, poison, append,
                scale if scale is not None else 1.0 / math.sqrt(head_dim), partition_tokens,
                f"custom {name}", NB=NB, shared_prefix_blocks=shared_prefix_blocks or None)
    return w


WORKLOADS = {
    "tiny_f32": tiny_f32,
    "llama7b": llama7b,
    "mixed_bs8": lambda **kw: mixed_batch(block_size=8, **kw),
    "mixed_bs16": lambda **kw: mixed_batch(block_size=16, **kw),
    "mixed_bs32": lambda **kw: mixed_batch(block_size=32, **kw),
    "shared_prefix": shared_prefix,
    "llama70b_gqa": llama70b_gqa,
    "llama70b_tp8": llama70b_tp8,
}
