"""Pins of the prefix-cache model (oracle/prefix_cache.py) against what the
pages state and what follows from the definitions, CPU only.

* The pages' example ("vLLM 与 PagedAttention" section 四): a 1500-token system
  prompt shared by requests with short questions -- a later request computes
  only what is not in whole cached blocks, a saving within or above the 80-95 %
  the pages quote.
* A block is known by its whole prefix: the same tokens after another prefix
  are not reused.
* At least one prompt token is always left to compute.
* Least-recently-released eviction, worked out by hand on a 4-block pool.
* Invariants over random operations: a cached block always holds the prefix
  its key names, reference counts equal table entries, and every block is
  free, cached and unheld, or held.
"""
import random

import pytest

from oracle.blocks import NoBlocks
from oracle.prefix_cache import PrefixCacheModel


def test_pages_example_system_prompt_reuse():
    bs = 16
    m = PrefixCacheModel(400, 0, bs)
    rng = random.Random(5)
    system = [rng.randrange(32000) for _ in range(1500)]
    q1 = [rng.randrange(32000) for _ in range(8)]
    q2 = [rng.randrange(32000) for _ in range(8)]
    assert m.add_cached(1, system + q1) == 0            # the first request computes everything
    m.append_tokens(1, system + q1)
    hit = m.add_cached(2, system + q2)
    assert hit == (1500 // bs) * bs == 1488             # whole blocks of the shared prompt
    saved = hit / len(system + q2)
    assert saved >= 0.80                                # the pages: 80-95 % of the prefill saved
    # the shared blocks are the first request's blocks, read by both
    assert m.tables[2] == m.tables[1][:1500 // bs]
    assert all(m.ref["gpu"][b] == 2 for b in m.tables[2])


def test_same_block_after_another_prefix_is_not_reused():
    m = PrefixCacheModel(16, 0, 4)
    m.add_cached(1, [])
    m.append_tokens(1, [1, 2, 3, 4, 5, 6, 7, 8, 9])
    # block 1 of request 1 holds 5..8 after 1..4; here 5..8 come after 9..12
    assert m.add_cached(2, [9, 10, 11, 12, 5, 6, 7, 8, 0]) == 0
    # the same first block is reused, the second too when its prefix matches
    assert m.add_cached(3, [1, 2, 3, 4, 5, 6, 7, 8, 0]) == 8
    assert m.add_cached(4, [1, 2, 3, 4, 6, 6, 7, 8, 0]) == 4


def test_one_prompt_token_is_always_left():
    m = PrefixCacheModel(16, 0, 4)
    m.add_cached(1, [])
    m.append_tokens(1, list(range(8)))
    assert m.add_cached(2, list(range(8))) == 4         # 2 full blocks cached, 1 reused
    assert m.add_cached(3, list(range(9))) == 8
    assert m.add_cached(4, []) == 0 and m.add_cached(5, [0]) == 0


def test_least_recently_released_is_evicted_first():
    m = PrefixCacheModel(4, 0, 2)
    assert m.add_cached(1, [1, 2, 3, 4, 5]) == 0
    m.append_tokens(1, [1, 2, 3, 4, 5])
    assert m.tables[1] == [0, 1, 2] and m.cache_stats() == (2, 0)
    m.free(1)                                           # released last first: 2 (free), 1, then 0
    assert m.free_blocks() == [2, 3] and sorted(m.evictable()) == [0, 1]
    assert m.add_cached(2, [1, 2, 3, 4, 9]) == 4 and m.tables[2] == [0, 1]
    m.append_tokens(2, [9])
    assert m.tables[2] == [0, 1, 2]
    m.add(3)
    with pytest.raises(NoBlocks):                       # 1 free block, none evictable
        m.append_tokens(3, [7, 7, 7, 7, 7])
    assert m.tables[3] == [] and m.lens[3] == 0
    m.free(2)                                           # 2 freed; 1 released before 0
    m.append_tokens(3, [7, 7, 7, 7, 7])                 # free 2, 3, then the older of 0 and 1: 1
    assert m.tables[3] == [2, 3, 1]
    assert m.add_cached(4, [1, 2, 3, 4, 5]) == 2        # [1, 2] still cached, [1, 2, 3, 4] evicted
    assert m.tables[4] == [0]


def _check_invariants(m: PrefixCacheModel):
    held = [0] * len(m.ref["gpu"])
    for sid, table in m.tables.items():
        if m.where[sid] != "gpu":
            continue
        for b in table:
            held[b] += 1
        toks = m.tokens[sid]
        if toks is not None:
            for j, b in enumerate(table[: len(toks) // m.bs]):
                if b in m.key_of:
                    assert m.key_of[b] == tuple(toks[: (j + 1) * m.bs])
    assert held == m.ref["gpu"]
    free, evict = set(m.free_blocks()), set(m.evictable())
    used = {b for b, r in enumerate(m.ref["gpu"]) if r > 0}
    assert not (free & evict) and not (free & used) and not (evict & used)
    assert free | evict | used == set(range(len(m.ref["gpu"])))
    assert all(m.cache[k] == b for b, k in m.key_of.items()) and len(m.cache) == len(m.key_of)


@pytest.mark.parametrize("seed", range(8))
def test_invariants_hold_over_random_operations(seed):
    rng = random.Random(seed)
    bs = rng.choice([2, 4, 8])
    m = PrefixCacheModel(rng.randint(8, 48), rng.randint(0, 24), bs)
    prefixes = [[rng.randrange(6) for _ in range(rng.randint(0, 5 * bs))] for _ in range(3)]
    sid = 0
    for _ in range(300):
        live = list(m.tables)
        gpu = [s for s in live if m.where[s] == "gpu"]
        op = rng.choice(["add_cached", "append_tokens", "append_tokens", "free", "fork", "append", "swap"])
        try:
            if op == "add_cached" or not gpu:
                prompt = rng.choice(prefixes) + [rng.randrange(6) for _ in range(rng.randint(0, 2 * bs))]
                hit = m.add_cached(sid, prompt)
                sid += 1
                assert hit % bs == 0 and (hit < len(prompt) or hit == 0)
                m.append_tokens(sid - 1, prompt[hit:])
            elif op == "append_tokens":
                m.append_tokens(rng.choice(gpu), [rng.randrange(6) for _ in range(rng.randint(0, bs + 1))])
            elif op == "append":
                m.append(rng.choice(gpu), rng.randint(0, 2))
            elif op == "fork":
                sid += 1
                m.fork(rng.choice(gpu), sid - 1)
            elif op == "free":
                m.free(rng.choice(live))
            elif op == "swap":
                s = rng.choice(live)
                m.swap_out(s) if m.where[s] == "gpu" else m.swap_in(s)
        except NoBlocks:
            pass
        _check_invariants(m)
