"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on
the same seeded inputs, element by element.

Bounds (written here, from the benchmark spec's tolerance): fp16/bf16 max-abs <= 2e-3
and relative L2 <= 1e-3, fp32 1e-5 for both, against the oracle rounded to the
output type (nearest even); the comparison against the unrounded oracle is
logged too.  Free blocks, tail slots and the appended tokens' slots hold NaN
before the append, so a read of anything the definition does not read shows
up as a non-finite result.
"""
import math

import numpy as np
import pytest
import torch

from paged_kv_cache_405_amd import binding as B
from paged_kv_cache_405_amd import workloads as W
from tests.pa_harness import assert_close, compare, gpu_step, log, oracle_step, upload

pytestmark = pytest.mark.gpu

WORKLOADS = ["tiny_f32", "llama7b", "mixed_bs8", "mixed_bs16", "mixed_bs32", "shared_prefix", "llama70b_gqa",
             "llama70b_tp8"]


@pytest.fixture(scope="module")
def cache():
    return {}


def _workload(cache, name):
    if name not in cache:
        cache[name] = W.WORKLOADS[name]()
    return cache[name]


@pytest.mark.parametrize("name", WORKLOADS)
def test_workload_parity_default(cache, name):
    """Each workload at full size: append one token per sequence, then decode
    with the library's own partition choice (the configuration the benchmark times)."""
    w = _workload(cache, name)
    log(f"[gpu] {name}: {w.description}")
    g = upload(w)
    out = gpu_step(w, g, partition_tokens=w.partition_tokens)
    torch.cuda.synchronize()
    ref = oracle_step(w)
    assert_close(compare(out, ref, w.dtype), w.dtype, f"{name} pt={w.partition_tokens}")


@pytest.mark.parametrize("name", ["tiny_f32", "llama7b", "mixed_bs8", "llama70b_gqa"])
@pytest.mark.parametrize("pt", [0, -1, -2, 16, 256, 512, 1024])
def test_partitions(cache, name, pt):
    w = _workload(cache, name)
    if pt > 0 and pt % w.block_size:
        pytest.skip("partition not a multiple of the block size")
    log(f"[gpu] {name} partition {pt}")
    g = upload(w)
    out = gpu_step(w, g, partition_tokens=pt)
    torch.cuda.synchronize()
    assert_close(compare(out, oracle_step(w), w.dtype), w.dtype, f"{name} pt={pt}")


@pytest.mark.parametrize("name", ["tiny_f32", "llama7b", "llama70b_gqa"])
def test_layouts_agree_bit_for_bit(cache, name):
    """The two cache layouts change addresses only: same lanes, same order, same bits."""
    w = _workload(cache, name)
    log(f"[gpu] {name} layouts")
    outs = []
    for layout in (B.PA_LAYOUT_BHTD, B.PA_LAYOUT_BTHD):
        g = upload(w, layout)
        outs.append(gpu_step(w, g, partition_tokens=w.partition_tokens))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    assert_close(compare(outs[1], oracle_step(w), w.dtype), w.dtype, f"{name} BTHD layout")


def _shapes():
    cases = []
    for dtype in ("f32", "f16", "bf16"):
        for D in (32, 64, 128, 256):
            for bs in (8, 16, 32):
                cases.append((dtype, D, bs, 4, 2))
    for Hq, Hkv in ((4, 4), (6, 2), (6, 3), (16, 4), (16, 2), (32, 2), (10, 5)):
        cases.append(("bf16", 128, 16, Hq, Hkv))
    return cases


@pytest.mark.parametrize("dtype,D,bs,Hq,Hkv", _shapes())
def test_shapes_ragged(dtype, D, bs, Hq, Hkv):
    """Every supported head_dim x block_size x element type, grouped-query ratios
    1..16, ragged lengths around block and partition edges, split and single pass."""
    ctxs = [1, bs - 1, bs, bs + 1, 2 * bs, 3 * bs + 5, 97, 300, 513, 1000]
    w = W.custom(f"ragged_{dtype}_{D}_{bs}_{Hq}x{Hkv}", dtype, ctxs, Hq, Hkv, D, bs,
                 seed=D * 7 + bs + Hq, append=True, table_pad=3)
    log(f"[gpu] {w.name}")
    g = upload(w)
    for pt in (-1, 0, -2, 4 * bs, 256):
        out = gpu_step(w, g, partition_tokens=pt, append=(pt == -1))
        torch.cuda.synchronize()
        assert_close(compare(out, oracle_step(w), dtype), dtype, f"{w.name} pt={pt}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_context_zero_and_one(dtype):
    """ctx = 0 gives a zero row; ctx = 1 gives V[0] bit for bit."""
    w = W.custom(f"edge_{dtype}", dtype, [0, 1, 0, 1, 33], 4, 2, 128, 16, seed=5, append=False)
    log(f"[gpu] {w.name}")
    g = upload(w)
    for pt in (-1, 0, -2, 16):
        out = gpu_step(w, g, partition_tokens=pt, append=False)
        torch.cuda.synchronize()
        got = out.cpu()
        assert torch.all(got[0] == 0) and torch.all(got[2] == 0)
        for s in (1, 3):
            b = int(w.block_tables[s, 0])
            for h in range(4):
                vrow = torch.from_numpy(np.ascontiguousarray(w.v_cache[b, 0, h // 2]).view(
                    np.int16 if dtype == "bf16" else w.v_cache.dtype))
                want = vrow.view(torch.bfloat16) if dtype == "bf16" else vrow
                assert torch.equal(got[s, h], want), f"seq {s} head {h}"
        assert_close(compare(out, oracle_step(w, append=False), dtype), dtype, f"{w.name} pt={pt}")


def test_full_table_context():
    """Context equal to the whole table (max_blocks * block_size), and clamping above it."""
    w = W.custom("full_table", "f16", [64, 128, 7], 8, 8, 128, 32, seed=6, append=False)
    log("[gpu] full table")
    g = upload(w)
    out = gpu_step(w, g, partition_tokens=-1, append=False)
    torch.cuda.synchronize()
    assert_close(compare(out, oracle_step(w, append=False), "f16"), "f16", "full table")
    over = g.ctx.clone()
    over[1] = 10_000                                  # beyond max_blocks * block_size: clamped
    g2 = dataclass_replace(g, ctx=over)
    out2 = gpu_step(w, g2, partition_tokens=32, append=False)
    torch.cuda.synchronize()
    assert torch.allclose(out2.float(), out.float(), atol=2e-3, rtol=0)


def dataclass_replace(g, **kw):
    import dataclasses
    return dataclasses.replace(g, **kw)


def test_empty_batch_touches_nothing():
    q = torch.empty((0, 8, 128), dtype=torch.float16, device="cuda")
    out = torch.empty_like(q)
    kc = torch.zeros((4, 8, 16, 128), dtype=torch.float16, device="cuda")
    B.pa_decode_ex(out, q, kc, kc, torch.zeros((0, 4), dtype=torch.int32, device="cuda"),
                   torch.zeros((0,), dtype=torch.int32, device="cuda"), 0.1)
    torch.cuda.synchronize()


def test_unmapped_block_contributes_nothing():
    """A table entry outside [0, num_blocks) is skipped, never read: with the
    last block of a sequence unmapped, the answer is attention over the earlier blocks."""
    w = W.custom("unmapped", "f16", [40, 70], 4, 4, 128, 16, seed=8, append=False)
    g = upload(w)
    last = (70 + 15) // 16 - 1
    tables = w.block_tables.copy()
    tables[1, last] = w.num_blocks + 123
    g2 = dataclass_replace(g, tables=torch.from_numpy(tables).cuda())
    log("[gpu] unmapped block")
    out = gpu_step(w, g2, partition_tokens=-1, append=False)
    torch.cuda.synchronize()
    ref = oracle_step(w, append=False, context_lens=np.array([40, last * 16], dtype=np.int32))
    assert_close(compare(out, ref, "f16"), "f16", "unmapped last block")


@pytest.mark.parametrize("name", ["llama7b", "llama70b_gqa"])
def test_placement_and_rerun_bit_identical(cache, name):
    """Moving every physical block elsewhere in the pool (same logical data) and
    running again must give identical bits: no atomics, fixed reduction order."""
    w = _workload(cache, name)
    log(f"[gpu] {name} placement permutation")
    g = upload(w)
    a = gpu_step(w, g, partition_tokens=w.partition_tokens)
    b = gpu_step(w, g, partition_tokens=w.partition_tokens, append=False)
    rng = np.random.default_rng(99)
    perm = rng.permutation(w.num_blocks)                  # old block i -> new block perm[i]
    inv = np.empty_like(perm)
    inv[perm] = np.arange(w.num_blocks)
    k2 = g.k_cache[torch.from_numpy(inv).cuda()]
    v2 = g.v_cache[torch.from_numpy(inv).cuda()]
    tables = w.block_tables.copy()
    m = tables >= 0
    tables[m] = perm[tables[m]]
    g2 = dataclass_replace(g, k_cache=k2, v_cache=v2, tables=torch.from_numpy(tables).cuda())
    c = gpu_step(w, g2, partition_tokens=w.partition_tokens, append=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(a, c)


@pytest.mark.parametrize("kernel", [B.PA_KERNEL_VECTOR, B.PA_KERNEL_MFMA])
@pytest.mark.parametrize("pt", [B.PA_PARTITION_SINGLE, B.PA_PARTITION_BALANCED, 64])
def test_shared_blocks_flag_changes_no_bit(kernel, pt):
    # PA_DECODE_SHARED_BLOCKS only changes the cache policy of the K/V loads:
    # on tables that share a prefix, both settings match the oracle and each other bit for bit
    w = W.shared_prefix(seed=41, num_seqs=12)
    g = upload(w)
    log(f"[gpu] shared prefix flag kernel {kernel} pt {pt}")
    a = gpu_step(w, g, partition_tokens=pt, kernel=kernel, shared_blocks=True)
    b = gpu_step(w, g, partition_tokens=pt, kernel=kernel, shared_blocks=False, append=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert_close(compare(a, oracle_step(w), w.dtype), w.dtype, f"shared blocks kernel={kernel} pt={pt}")


@pytest.mark.parametrize("kernel", [B.PA_KERNEL_VECTOR, B.PA_KERNEL_MFMA])
def test_longest_first_windows(kernel):
    """The grid kernels take each window of 64 sequences longest first: 150
    sequences (two full windows and a ragged one of 22), many equal lengths
    (ties go by index), a table long enough that the ordering is on; single
    pass and split-K write every sequence's own rows."""
    rng = np.random.default_rng(77)
    ctxs = [int(c) for c in rng.choice([1, 16, 17, 300, 700, 1000], size=150)]
    ctxs[149] = 1000        # the longest in the last, ragged window
    ctxs[64] = 1            # the second window opens on one of many equal short lengths
    w = W.custom(f"order_{kernel}", "bf16", ctxs, 16, 2, 128, 16, seed=78, append=True, table_pad=1)
    log(f"[gpu] {w.name}")
    g = upload(w)
    for pt in (-1, 512):
        out = gpu_step(w, g, partition_tokens=pt, kernel=kernel, append=(pt == -1))
        torch.cuda.synchronize()
        assert_close(compare(out, oracle_step(w), "bf16"), "bf16", f"{w.name} pt={pt}")
