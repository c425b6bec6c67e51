"""The host block manager's prefix cache (pa_bm_add_cached, pa_bm_append_tokens,
pa_bm_cache_stats; C++) against the prefix-cache model (oracle/prefix_cache.py),
CPU only: random sequences of requests sharing a few prompts -- hits, appends,
forks, frees, swaps, plain appends and running out of blocks -- must give the
same hits, slots, copies, swap pairs, tables, reference counts, free and
cached blocks; failed calls change nothing."""
import random

import pytest

from oracle.blocks import NoBlocks
from oracle.prefix_cache import PrefixCacheModel
from paged_kv_cache_405_amd import binding as B


def _same_state(bm: B.BlockManager, m: PrefixCacheModel):
    assert bm.num_free(B.POOL_GPU) == m._available("gpu")
    assert bm.num_free(B.POOL_CPU) == m._available("cpu")
    assert bm.cache_stats() == m.cache_stats()
    for pool, name in ((B.POOL_GPU, "gpu"), (B.POOL_CPU, "cpu")):
        assert [bm.ref_count(pool, b) for b in range(len(m.ref[name]))] == m.ref[name]
    for s in m.tables:
        assert bm.info(s) == (m.lens[s], len(m.tables[s]), m.where[s] == "gpu")
    on_gpu = [s for s in m.tables if m.where[s] == "gpu"]
    if on_gpu:
        mb = max(1, max(len(m.tables[s]) for s in on_gpu))
        got_t, got_l = bm.block_tables(on_gpu, mb)
        want_t, want_l = m.block_tables(on_gpu, mb)
        assert (got_t == want_t).all() and (got_l == want_l).all()


def _both(native, model):
    try:
        want = model()
    except NoBlocks:
        with pytest.raises(B.PaError) as e:
            native()
        assert e.value.status == B.PA_ERR_NO_BLOCKS
        return None
    return native(), want


@pytest.mark.parametrize("seed", range(12))
def test_matches_the_model_on_random_operations(seed):
    rng = random.Random(700 + seed)
    bs = rng.choice([1, 2, 4, 16])
    NG, NC = rng.randint(6, 64), rng.randint(0, 32)
    bm, m = B.BlockManager(NG, NC, bs), PrefixCacheModel(NG, NC, bs)
    vocab = rng.choice([2, 5, 1000])
    prompts = [[rng.randrange(vocab) for _ in range(rng.randint(0, 6 * bs))] for _ in range(4)]
    sid = 0
    for _ in range(350):
        live = list(m.tables)
        gpu = [s for s in live if m.where[s] == "gpu"]
        cpu = [s for s in live if m.where[s] == "cpu"]
        op = rng.choice(["new", "new", "append_tokens", "append_tokens", "append", "fork", "free", "free",
                         "swap_out", "swap_in"])
        if op == "new" or not gpu:
            prompt = rng.choice(prompts) + [rng.randrange(vocab) for _ in range(rng.randint(0, 2 * bs))]
            hit = m.add_cached(sid, prompt)
            assert bm.add_cached(sid, prompt) == hit
            rest = prompt[hit:]
            r = _both(lambda: bm.append_tokens(sid, rest), lambda: m.append_tokens(sid, rest))
            if r:
                assert r[0][0] == r[1][0] and r[0][1] == [tuple(c) for c in r[1][1]]
            sid += 1
        elif op == "append_tokens":
            s = rng.choice(gpu)
            toks = [rng.randrange(vocab) for _ in range(rng.randint(0, 2 * bs + 1))]
            r = _both(lambda: bm.append_tokens(s, toks), lambda: m.append_tokens(s, toks))
            if r:
                assert r[0][0] == r[1][0] and r[0][1] == [tuple(c) for c in r[1][1]]
        elif op == "append":
            s, n = rng.choice(gpu), rng.randint(0, 2)
            r = _both(lambda: bm.append(s, n), lambda: m.append(s, n))
            if r:
                assert r[0][0] == r[1][0] and r[0][1] == [tuple(c) for c in r[1][1]]
        elif op == "fork":
            p = rng.choice(gpu)
            bm.fork(p, sid)
            m.fork(p, sid)
            sid += 1
        elif op == "free":
            s = rng.choice(live)
            bm.free(s)
            m.free(s)
        elif op == "swap_out" and gpu:
            s = rng.choice(gpu)
            r = _both(lambda: bm.swap_out(s), lambda: m.swap_out(s))
            if r:
                assert r[0] == [tuple(p) for p in r[1]]
        elif op == "swap_in" and cpu:
            s = rng.choice(cpu)
            r = _both(lambda: bm.swap_in(s), lambda: m.swap_in(s))
            if r:
                assert r[0] == [tuple(p) for p in r[1]]
        _same_state(bm, m)
    bm.close()


def test_pages_example_through_the_library():
    # a 1500-token system prompt and two 8-token questions (block size 16)
    rng = random.Random(3)
    system = [rng.randrange(32000) for _ in range(1500)]
    bm = B.BlockManager(256, 0, 16)
    assert bm.add_cached(1, system + [1] * 8) == 0
    bm.append_tokens(1, system + [1] * 8)
    assert bm.cache_stats() == (94, 0)                  # 1508 tokens: 94 full blocks
    assert bm.add_cached(2, system + [2] * 8) == 1488   # 93 blocks of the system prompt
    t, _ = bm.block_tables([1, 2], 95)
    assert (t[1, :93] == t[0, :93]).all()
    bm.free(1)
    bm.free(2)
    assert bm.cache_stats() == (94, 94) and bm.num_free() == 256
    bm.close()


def test_argument_errors():
    bm = B.BlockManager(8, 0, 4)
    L = B.lib()
    import ctypes
    hit = ctypes.c_int32(0)
    toks = (ctypes.c_int32 * 4)(1, 2, 3, 4)
    assert L.pa_bm_add_cached(bm._h, 1, None, 3, ctypes.byref(hit)) == B.PA_ERR_INVALID_ARG
    assert L.pa_bm_add_cached(bm._h, 1, toks, -1, ctypes.byref(hit)) == B.PA_ERR_INVALID_ARG
    assert L.pa_bm_add_cached(bm._h, 1, toks, 4, None) == B.PA_ERR_INVALID_ARG
    assert L.pa_bm_add_cached(None, 1, toks, 4, ctypes.byref(hit)) == B.PA_ERR_INVALID_ARG
    bm.add(7)
    assert L.pa_bm_add_cached(bm._h, 7, toks, 4, ctypes.byref(hit)) == B.PA_ERR_INVALID_ARG   # id taken
    n = ctypes.c_int32(0)
    slots = (ctypes.c_int64 * 4)()
    assert L.pa_bm_append_tokens(bm._h, 7, None, 2, slots, None, 0, ctypes.byref(n)) == B.PA_ERR_INVALID_ARG
    assert L.pa_bm_append_tokens(bm._h, 9, toks, 2, slots, None, 0, ctypes.byref(n)) == B.PA_ERR_INVALID_ARG
    c, e = ctypes.c_int32(0), ctypes.c_int32(0)
    assert L.pa_bm_cache_stats(bm._h, None, ctypes.byref(e)) == B.PA_ERR_INVALID_ARG
    assert L.pa_bm_cache_stats(bm._h, ctypes.byref(c), ctypes.byref(e)) == B.PA_OK
    assert bm.info(7) == (0, 0, True)
    bm.close()
