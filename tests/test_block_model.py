"""Pins of the block-bookkeeping oracle (oracle/blocks.py), CPU only.

Against what the pages fix -- blocks taken only when the last one is full, a
request of n tokens holding ceil(n / bs) blocks ([VB] sketch: 50 tokens at 16
per page -> 4 pages; 512 -> 32), shared prefixes read shared and copied on
write ([VP] 二, [VG] Copy-on-Write), swapping out and back ([VI] 4.3) -- and by
brute force: random operation sequences drive a pool of token ids through the
model's slots, copies and swaps, and every live request must read back
exactly the tokens written to it.
"""
import random

import numpy as np
import pytest

from oracle.blocks import BlockManagerModel, NoBlocks, copy_blocks, swap_blocks


def test_blocks_taken_only_when_the_last_is_full():
    m = BlockManagerModel(64, 0, 16)
    m.add(0)
    taken_at = []
    for t in range(50):
        before = len(m.tables[0])
        slots, copies = m.append(0, 1)
        assert copies == []
        if len(m.tables[0]) != before:
            taken_at.append(t)
        assert slots == [m.tables[0][t // 16] * 16 + t % 16]
    assert taken_at == [0, 16, 32, 48]
    assert len(m.tables[0]) == 4                   # ceil(50 / 16)
    m.add(1)
    m.append(1, 512)
    assert len(m.tables[1]) == 32                  # 512 / 16


def test_fresh_blocks_lowest_first_and_returned_on_free():
    m = BlockManagerModel(8, 0, 4)
    m.add(0)
    m.add(1)
    m.append(0, 6)            # blocks 0, 1
    m.append(1, 4)            # block 2
    assert m.tables == {0: [0, 1], 1: [2]}
    m.free(0)
    assert m.free_blocks() == [0, 1, 3, 4, 5, 6, 7]
    m.add(2)
    m.append(2, 5)            # reuses 0, then 1
    assert m.tables[2] == [0, 1]


def test_fork_shares_and_copy_on_write():
    m = BlockManagerModel(16, 0, 4)
    m.add(0)
    m.append(0, 6)                                 # blocks [0, 1], block 1 half full
    m.fork(0, 1)
    assert m.tables[1] == [0, 1] and m.ref["gpu"][:2] == [2, 2]
    # the child writes into the shared half-full block: one copy, to a fresh block
    slots, copies = m.append(1, 1)
    assert copies == [(1, 2)]
    assert m.tables[1] == [0, 2] and m.tables[0] == [0, 1]
    assert slots == [2 * 4 + 2]
    assert m.ref["gpu"][:3] == [2, 1, 1]
    # the parent's block 1 is no longer shared: it writes in place
    slots, copies = m.append(0, 1)
    assert copies == [] and slots == [1 * 4 + 2]
    # sharing whole blocks only: appending at a block boundary takes a new block, no copy
    m.add(2)
    m.append(2, 8)                                 # blocks 3, 4, both full
    m.fork(2, 3)
    slots, copies = m.append(3, 1)
    assert copies == [] and m.tables[3] == [3, 4, 5] and m.tables[2] == [3, 4]


def test_no_blocks_changes_nothing():
    m = BlockManagerModel(3, 1, 4)
    m.add(0)
    m.append(0, 12)
    before = (dict(m.tables), dict(m.lens), list(m.ref["gpu"]))
    with pytest.raises(NoBlocks):
        m.append(0, 1)
    assert (m.tables, m.lens, m.ref["gpu"]) == (before[0], before[1], before[2])
    with pytest.raises(NoBlocks):
        m.swap_out(0)                              # 3 blocks, 1 CPU block
    assert m.where[0] == "gpu" and m.ref["cpu"] == [0]


def test_copy_blocks_reads_the_state_before_the_call():
    k = np.arange(5 * 3, dtype=np.float32).reshape(5, 3)
    v = -k
    copy_blocks(k, v, [(0, 1), (1, 2), (7, 3), (3, -1)])
    # block 2 takes the old block 1, not the new one; pairs off the pool are skipped
    assert k[1].tolist() == [0, 1, 2] and k[2].tolist() == [3, 4, 5] and k[3].tolist() == [9, 10, 11]
    assert (v == -k).all()


def test_swap_blocks_between_pools():
    gk = np.zeros((4, 2), np.float16)
    gv = np.zeros((4, 2), np.float16)
    ck = np.arange(6, dtype=np.float16).reshape(3, 2)
    cv = ck + 100
    swap_blocks(gk, gv, ck, cv, [(2, 0), (0, 3), (5, 1)])
    assert gk.tolist() == [[4, 5], [0, 0], [0, 0], [0, 1]]
    assert gv.tolist() == [[104, 105], [0, 0], [0, 0], [100, 101]]


def _check_invariants(m: BlockManagerModel):
    counts = {"gpu": [0] * len(m.ref["gpu"]), "cpu": [0] * len(m.ref["cpu"])}
    for s, table in m.tables.items():
        assert len(table) == -(-m.lens[s] // m.bs)
        for b in table:
            counts[m.where[s]][b] += 1
    assert counts == m.ref


@pytest.mark.parametrize("seed", range(12))
def test_random_operations_keep_every_request_readable(seed):
    rng = random.Random(seed)
    bs = rng.choice([2, 4, 8, 16])
    NG, NC = rng.randint(6, 40), rng.randint(0, 30)
    m = BlockManagerModel(NG, NC, bs)
    gpu = np.full((NG, bs), -1, np.int64)          # the pools hold token ids
    cpu = np.full((max(NC, 1), bs), -1, np.int64)
    history: dict[int, list[int]] = {}
    next_sid, next_tok = 0, 0
    for _ in range(300):
        live = list(m.tables)
        on_gpu = [s for s in live if m.where[s] == "gpu"]
        op = rng.choice(["add", "append", "append", "append", "fork", "free", "swap_out", "swap_in"])
        try:
            if op == "add" or not live:
                m.add(next_sid)
                history[next_sid] = []
                next_sid += 1
            elif op == "append" and on_gpu:
                s = rng.choice(on_gpu)
                n = rng.randint(1, 3 * bs)
                slots, copies = m.append(s, n)
                copy_blocks(gpu, gpu.copy(), copies)
                for slot in slots:
                    gpu[slot // bs, slot % bs] = next_tok
                    history[s].append(next_tok)
                    next_tok += 1
            elif op == "fork" and on_gpu:
                p = rng.choice(on_gpu)
                m.fork(p, next_sid)
                history[next_sid] = list(history[p])
                next_sid += 1
            elif op == "free":
                s = rng.choice(live)
                m.free(s)
                del history[s]
            elif op == "swap_out" and on_gpu:
                s = rng.choice(on_gpu)
                pairs = m.swap_out(s)
                swap_blocks(cpu, cpu.copy(), gpu, gpu, pairs)
            elif op == "swap_in":
                on_cpu = [s for s in live if m.where[s] == "cpu"]
                if on_cpu:
                    s = rng.choice(on_cpu)
                    pairs = m.swap_in(s)
                    swap_blocks(gpu, gpu.copy(), cpu, cpu, pairs)
        except NoBlocks:
            pass
        _check_invariants(m)
        for s, toks in history.items():
            pool = gpu if m.where[s] == "gpu" else cpu
            got = [int(pool[m.tables[s][t // bs], t % bs]) for t in range(m.lens[s])]
            assert got == toks, (seed, s)
